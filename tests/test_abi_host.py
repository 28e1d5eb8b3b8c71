"""The C ABI on the host (no GPU needed): the library loads, exports every function that
include/subspec.h declares, and rejects bad arguments with the documented status before
it touches a device.

When the in-tree library has not been built yet, it is built into a temporary folder
first, so the check never silently passes on a missing library.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from bit_quantized_draft_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "subspec.h")


@pytest.fixture(scope="module")
def L(tmp_path_factory):
    path = _lib.LIB_PATH
    if not os.path.exists(path):
        from bit_quantized_draft_amd import build
        d = tmp_path_factory.mktemp("lib")
        path = build.build(verbose=False, out=str(d / "libsubspec.so"), build_dir=str(d / "obj"))
    lib = ctypes.CDLL(path)
    for name, (res, args) in _lib.SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:ss_status|size_t|int|const char\s*\*)\s*(ss_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("ss_quantize_substitute", "ss_draft_tree_step", "ss_tree_attention", "ss_tree_accept"):
        assert required in names
    assert len(names) >= 15, names


def test_every_declared_function_is_exported(L):
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, f"declared but not exported: {missing}"


def test_binding_signatures_cover_the_header():
    assert set(declared_functions()) == set(_lib.SIGNATURES), (
        set(declared_functions()) ^ set(_lib.SIGNATURES))


def test_version_and_last_error(L):
    assert L.ss_abi_version() >= 1
    assert isinstance(L.ss_last_error(), bytes)


def _parents(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def test_tree_validate_host(L):
    a, p = _parents([-1, 0, 1, 1, 0])
    assert L.ss_tree_validate(p, len(a)) == _lib.SS_OK
    a, p = _parents([-1] + list(range(63)))   # a chain
    assert L.ss_tree_validate(p, len(a)) == _lib.SS_OK
    a, p = _parents([0, 0])                   # root not -1
    assert L.ss_tree_validate(p, len(a)) == _lib.SS_ERR_BAD_TREE
    a, p = _parents([-1, 0, 2])               # parent not earlier
    assert L.ss_tree_validate(p, len(a)) == _lib.SS_ERR_BAD_TREE
    assert b"parents[2]" in L.ss_last_error()
    assert L.ss_tree_validate(None, 3) == _lib.SS_ERR_INVALID_ARG


def test_linear_argument_checks_before_any_device_call(L):
    dummy = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    # T out of range, k not a multiple of 128, n not a multiple of 16, null x
    assert L.ss_w4a16_linear(dummy, 0, dummy, dummy, dummy, 16, 128, dummy, None, None, 0, None) \
        == _lib.SS_ERR_UNSUPPORTED
    assert L.ss_w4a16_linear(dummy, 4, dummy, dummy, dummy, 16, 100, dummy, None, None, 0, None) \
        == _lib.SS_ERR_UNSUPPORTED
    assert L.ss_w4a16_linear(dummy, 4, dummy, dummy, dummy, 20, 128, dummy, None, None, 0, None) \
        == _lib.SS_ERR_UNSUPPORTED
    assert L.ss_w4a16_linear(None, 4, dummy, dummy, dummy, 16, 128, dummy, None, None, 0, None) \
        == _lib.SS_ERR_INVALID_ARG
    assert b"x_bf16" in L.ss_last_error() or b"null" in L.ss_last_error()


def test_workspace_queries_are_host_only(L):
    # sizes follow the work split: 0 when no block is split, else room for the partials
    assert L.ss_w4a16_linear_workspace(16, 512, 512) >= 0
    big = L.ss_w4a16_linear_workspace(64, 3584, 18944)   # split blocks: partials needed
    assert big > 0 and big % 256 == 0
    assert L.ss_tree_attention_workspace(64, 2048, 28, 4, 128) > 0
    assert L.ss_tree_attention_workspace(64, 2048, 28, 4, 96) == 0   # unsupported head dim


def test_attention_and_step_reject_null_arguments(L):
    assert L.ss_tree_attention(None, None, 0, None) == _lib.SS_ERR_INVALID_ARG
    assert L.ss_draft_tree_step(None, None, None, 0, None) == _lib.SS_ERR_INVALID_ARG


def test_kv_commit_argument_checks(L):
    arr = (ctypes.c_void_p * 1)(16)
    dummy = ctypes.c_void_p(16)
    # C + T beyond c_stride, unsupported hd, null arrays: rejected before any launch
    assert L.ss_kv_commit(arr, arr, arr, arr, 1, 1, 128, 100, 90, 16, dummy, dummy, None) == _lib.SS_ERR_INVALID_ARG
    assert b"c_stride" in L.ss_last_error()
    assert L.ss_kv_commit(arr, arr, arr, arr, 1, 1, 96, 100, 0, 16, dummy, dummy, None) == _lib.SS_ERR_UNSUPPORTED
    assert L.ss_kv_commit(None, arr, arr, arr, 1, 1, 128, 100, 0, 16, dummy, dummy, None) == _lib.SS_ERR_INVALID_ARG


def test_draft_select_workspace_checks(L):
    dummy = ctypes.c_void_p(16)
    # long rows are split across workgroups: the candidates need a workspace
    need = L.ss_draft_select_workspace(64, 152064, 6)
    assert need > 0
    assert L.ss_draft_select_workspace(2, 40, 6) == 0          # one pass per row
    assert L.ss_draft_select_workspace(2, 40, 17) == 0         # k out of range
    assert L.ss_draft_select(dummy, None, 64, 152064, 5.0, 6, dummy, None, 0, None) \
        == _lib.SS_ERR_WORKSPACE
    assert L.ss_draft_select(dummy, None, 64, 152064, 5.0, 6, dummy, dummy, need - 1, None) \
        == _lib.SS_ERR_WORKSPACE
    assert L.ss_draft_select(dummy, None, 64, 152064, 5.0, 0, dummy, dummy, need, None) \
        == _lib.SS_ERR_UNSUPPORTED


def _dummy_step(C):
    """A one-layer model and step arguments whose pointers are never dereferenced (the
    checks fail or stop at the workspace before any device call); no KV cache."""
    p = 4096   # aligned dummy address
    lin = _lib.SsLinear(kind=_lib.SS_W4G64_TILED, qweight=p)
    layers = (_lib.SsLayer * 1)()
    layers[0] = _lib.SsLayer(norm1=p, norm2=p, qkv=lin, o=lin, gate_up=lin, down=lin,
                             k_cache=None, v_cache=None)
    model = _lib.SsModel(H=256, I=512, nq=4, nkv=2, hd=64, L=1, V=0, rope_theta=1e6, rms_eps=1e-6,
                         c_stride=16, layers=layers)
    tk = (ctypes.c_void_p * 1)(p)
    args = _lib.SsStepArgs(parents=p, T=4, C=C, tree_k=tk, tree_v=tk, hidden_in=p, hidden_out=p)
    return model, args, layers, tk


def test_step_kv_cache_may_be_null_only_without_prefix(L):
    model, args, _keep1, _keep2 = _dummy_step(C=0)
    # passes every argument check and stops at the missing workspace
    assert L.ss_draft_tree_step(ctypes.byref(model), ctypes.byref(args), None, 0, None) == _lib.SS_ERR_WORKSPACE
    model, args, _keep1, _keep2 = _dummy_step(C=5)
    assert L.ss_draft_tree_step(ctypes.byref(model), ctypes.byref(args), None, 0, None) == _lib.SS_ERR_INVALID_ARG
    assert b"null KV cache" in L.ss_last_error()


def test_misaligned_pointers_are_rejected_on_the_host(L):
    """Device pointers must meet the alignment the kernels' vector loads assume (16 bytes for
    bf16 activations, code bytes and workspaces, 2 for bf16 outputs, 4 for fp32 outputs);
    a misaligned one is rejected with SS_ERR_INVALID_ARG before anything is launched."""
    ok = ctypes.c_void_p(1 << 20)
    for bad_x in (ctypes.c_void_p((1 << 20) + 2), ctypes.c_void_p((1 << 20) + 8)):
        assert L.ss_w4a16_linear_tiled(bad_x, 4, ok, 16, 128, ok, None, None, 0, None) == _lib.SS_ERR_INVALID_ARG
        assert b"align" in L.ss_last_error()
    # misaligned fp32 output
    assert L.ss_w4a16_linear_tiled(ok, 4, ok, 16, 128, None, ctypes.c_void_p((1 << 20) + 2), None, 0, None) \
        == _lib.SS_ERR_INVALID_ARG
    # misaligned tiled weight
    assert L.ss_w4a16_linear_tiled(ok, 4, ctypes.c_void_p((1 << 20) + 4), 16, 128, ok, None, None, 0, None) \
        == _lib.SS_ERR_INVALID_ARG
    # misaligned workspace on a shape that needs one
    T, n, k = 64, 3584, 18944
    need = L.ss_w4a16_linear_workspace(T, n, k)
    assert need > 0
    assert L.ss_w4a16_linear_tiled(ok, T, ok, n, k, ok, None, ctypes.c_void_p((1 << 20) + 8), need, None) \
        == _lib.SS_ERR_INVALID_ARG


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present: the no-device path is not reachable")
def test_no_device_is_reported_not_crashed(L):
    """Without a HIP device every compute entry point returns SS_ERR_DEVICE with a message
    once its arguments are valid (the pointers are never dereferenced)."""
    ok = ctypes.c_void_p(1 << 20)
    assert L.ss_w4a16_linear_tiled(ok, 4, ok, 16, 128, ok, None, None, 0, None) == _lib.SS_ERR_DEVICE
    assert b"device" in L.ss_last_error()
    assert L.ss_w4a16_linear_tiled_noalloc(ok, 4, ok, 16, 128, ok, None, None) == _lib.SS_ERR_DEVICE
    assert L.ss_row_argmax(ctypes.cast(ok, ctypes.POINTER(ctypes.c_float)), 4, 100,
                           ctypes.cast(ok, ctypes.POINTER(ctypes.c_int32)), None) == _lib.SS_ERR_DEVICE


# ------------------------------------------------------------------ sanitizers

def _sources_objects(tmp):
    """Objects of every source but the C ABI itself: the in-tree build's where they are at
    least as new as their sources, else compiled afresh into `tmp`."""
    from bit_quantized_draft_amd import build
    objs = []
    for src in build.SOURCES:
        if src == "api.cpp":
            continue
        o = os.path.join(build.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(o) or os.path.getmtime(o) < os.path.getmtime(os.path.join(build.CSRC, src)):
            o = build._compile(src, str(tmp))
        objs.append(o)
    return objs


def test_host_checks_under_sanitizers(tmp_path):
    """The host half of the C ABI (argument checks, messages, the no-device path) built
    with AddressSanitizer and UndefinedBehaviorSanitizer, driven by a C program that makes
    invalid calls; no call reaches a GPU. The device code is built as usual."""
    import shutil
    import subprocess
    from bit_quantized_draft_amd import build
    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(build.HIPCC) and os.path.exists(clang)):
        pytest.skip("hipcc / clang not available")
    objs = _sources_objects(tmp_path)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    api_o, drv_o, exe = str(tmp_path / "api_san.o"), str(tmp_path / "driver.o"), str(tmp_path / "driver")
    steps = [
        [build.HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC", *san,
         "-fno-omit-frame-pointer", "-c", os.path.join(build.CSRC, "api.cpp"), "-o", api_o],
        [clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-Wall", "-c",
         os.path.join(ROOT, "tests", "host_sanitize", "driver.c"), "-o", drv_o],
        [build.HIPCC, "--offload-arch=gfx950", *san, drv_o, api_o, *objs, "-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert r.returncode == 0 and "PASSED" in r.stdout, out
    shutil.rmtree(tmp_path, ignore_errors=True)
