"""Host-only tests of the Python binding's argument checks: every tensor's dtype, layout and
exact shape is checked before the library is called, so a mismatched tensor never reaches a
kernel (where it would be read or written out of bounds). CPU tensors stand in for device
tensors (the device test is patched out) and the library is replaced by a stub that fails
the test if a compute entry point is reached."""
import pytest
import torch

import bit_quantized_draft_amd.api as api
from bit_quantized_draft_amd._lib import SS_ERR_INVALID_ARG, SubspecError


class _NoLib:
    """Stands in for the shared library: only the pure size queries answer."""

    def ss_w4_tiled_bytes(self, n, k):
        return (n // 16) * (k // 128) * 1152

    def __getattr__(self, name):
        def call(*a, **kw):
            raise AssertionError(f"library entry point {name} reached with a bad argument")
        return call


@pytest.fixture(autouse=True)
def _host_only(monkeypatch):
    monkeypatch.setattr(api, "_on_device", lambda t: True)
    monkeypatch.setattr(api, "lib", lambda: _NoLib())
    monkeypatch.setattr(api, "_stream", lambda: None)


def bf(*s):
    return torch.zeros(s, dtype=torch.bfloat16)


def f32(*s):
    return torch.zeros(s, dtype=torch.float32)


def i32(*s):
    return torch.zeros(s, dtype=torch.int32)


def u8(*s):
    return torch.zeros(s, dtype=torch.uint8)


def f16(*s):
    return torch.zeros(s, dtype=torch.float16)


def _bad(fn, *a, **kw):
    with pytest.raises(SubspecError) as e:
        fn(*a, **kw)
    assert e.value.status == SS_ERR_INVALID_ARG


def test_w4_linear_shapes():
    T, n, k = 4, 32, 256
    _bad(api.w4a16_linear, bf(T, k), u8(n, k // 2 + 1), f16(n, k // 64), f16(n, k // 64))   # codes vs x's k
    _bad(api.w4a16_linear, bf(T, k), u8(n, k // 2), f16(n, k // 64 - 1), f16(n, k // 64))   # scales
    _bad(api.w4a16_linear, bf(T, k), u8(n, k // 2), f16(n, k // 64), f16(n + 16, k // 64))  # zeros
    _bad(api.w4a16_gate_up_swiglu, bf(T, k), u8(2 * n, k // 2), f16(2 * n, k // 64), f16(2 * n, k // 64),
         out=bf(T, n + 1))
    _bad(api.dequantize_substitute, u8(n, k // 2), f16(n, k // 64), f16(n, 1))


def test_tiled_shapes():
    T, n, k = 4, 32, 256
    tw = api.TiledW4(u8(api.lib().ss_w4_tiled_bytes(n, k)), n, k)
    _bad(api.w4a16_linear_tiled, bf(T, 2 * k), tw)                       # tw.k != x's k
    short = api.TiledW4(u8(100), n, k)
    _bad(api.w4a16_linear_tiled, bf(T, k), short)                        # data too small
    _bad(api.w4a16_linear_tiled_noalloc, bf(T, k), tw, bf(T, n + 16), None)
    _bad(api.w4a16_linear_tiled_noalloc, bf(T, k), tw, None, f32(T + 1, n))
    _bad(api.w4a16_gate_up_swiglu_tiled, bf(T, k), tw, out=bf(T, n))    # out is [T][n/2]


def test_attention_shapes():
    T, nq, nkv, hd, cs = 8, 4, 2, 64, 32
    q, kc, vc = bf(T, nq, hd), bf(nkv, cs, hd), bf(nkv, cs, hd)
    kt, vt, par = bf(nkv, T, hd), bf(nkv, T, hd), i32(T)
    _bad(api.tree_attention, q, kc, vc, bf(nkv, T - 1, hd), vt, par, 4)  # tree K sized for a smaller tree
    _bad(api.tree_attention, q, kc, bf(nkv, cs - 1, hd), kt, vt, par, 4)
    _bad(api.tree_attention, q, kc, vc, kt, vt, i32(T + 1), 4)
    _bad(api.tree_attention, q, kc, vc, kt, vt, par, cs + 1)             # C beyond the cache


def test_selection_shapes():
    R, V, k = 3, 50, 6
    _bad(api.draft_select, f32(R, V), f32(R, V - 1), 5.0, k)             # gumbel shape
    _bad(api.draft_select, f32(R, V), None, 5.0, k, out=i32(R, k + 1))
    _bad(api.row_argmax, f32(R, V), out=i32(R + 1))
    T = 6
    _bad(api.tree_accept, i32(T), i32(T), i32(T - 1))
    _bad(api.tree_accept, i32(T), i32(T + 1), i32(T))


def test_kv_commit_shapes():
    nkv, cs, hd, T = 2, 16, 64, 5
    kc, vc, kt, vt = [bf(nkv, cs, hd)], [bf(nkv, cs, hd)], [bf(nkv, T, hd)], [bf(nkv, T, hd)]
    _bad(api.kv_commit, kc, vc, [bf(nkv, T + 1, hd)], vt, 0, i32(T), i32(1))
    _bad(api.kv_commit, kc, vc, kt, vt, 0, i32(T - 1), i32(1))
    _bad(api.kv_commit, kc, vc, kt, vt + vt, 0, i32(T), i32(1))


def test_step_shapes():
    H, I, nq, nkv, hd, V, T = 128, 256, 2, 1, 64, 40, 4
    cache = bf(nkv, 8, hd)
    ly = dict(qkv=bf((nq + 2 * nkv) * hd, H), o=bf(H, nq * hd), gate_up=bf(2 * I, H), down=bf(H, I),
              norm1=bf(H), norm2=bf(H), k_cache=cache, v_cache=cache)
    m = api.SubstituteModel(H, I, nq, nkv, hd, [ly], V=V, embed=bf(V, H), final_norm=bf(H), lm_head=bf(V, H))
    par, tok = i32(T), i32(T)
    tk, tv = [bf(nkv, T, hd)], [bf(nkv, T, hd)]
    _bad(m.draft_tree_step, par, 0, [bf(nkv, T - 1, hd)], tv, tokens=tok)     # tree K for a smaller tree
    _bad(m.draft_tree_step, par, 0, tk, tv, tokens=i32(T + 1))
    _bad(m.draft_tree_step, par, 0, tk, tv, tokens=tok, logits=f32(T, V + 1))
    _bad(m.draft_tree_step, par, 0, tk, tv, tokens=tok, logits=f32(T, V), logit_rows=i32(2))
    _bad(m.draft_tree_step, par, 0, tk, tv, hidden_in=bf(T, H + 1))
    _bad(m.draft_tree_step, par, 0, tk, tv)                                   # neither tokens nor hidden_in


def test_wrong_dtype_is_a_type_error():
    with pytest.raises(TypeError):
        api.row_argmax(torch.zeros((2, 3), dtype=torch.float64))
