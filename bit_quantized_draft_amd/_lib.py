"""ctypes declarations of the C ABI in include/subspec.h (argument marshalling only)."""

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p, c_char_p

HERE = os.path.dirname(os.path.abspath(__file__))
# SS_LIB_PATH selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("SS_LIB_PATH") or os.path.join(HERE, "libsubspec.so")

SS_OK = 0
SS_ERR_INVALID_ARG = -1
SS_ERR_UNSUPPORTED = -2
SS_ERR_BAD_TREE = -3
SS_ERR_WORKSPACE = -4
SS_ERR_DEVICE = -5
STATUS_NAMES = {0: "SS_OK", -1: "SS_ERR_INVALID_ARG", -2: "SS_ERR_UNSUPPORTED",
                -3: "SS_ERR_BAD_TREE", -4: "SS_ERR_WORKSPACE", -5: "SS_ERR_DEVICE"}

SS_W4G64 = 0
SS_BF16 = 1
SS_W4G64_TILED = 2


class SsLinear(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("qweight", c_void_p), ("scale", c_void_p),
                ("zero", c_void_p), ("w", c_void_p)]


class SsLayer(ctypes.Structure):
    _fields_ = [("norm1", c_void_p), ("norm2", c_void_p), ("qkv", SsLinear), ("o", SsLinear),
                ("gate_up", SsLinear), ("down", SsLinear), ("k_cache", c_void_p),
                ("v_cache", c_void_p)]


class SsModel(ctypes.Structure):
    _fields_ = [("H", c_int32), ("I", c_int32), ("nq", c_int32), ("nkv", c_int32),
                ("hd", c_int32), ("L", c_int32), ("V", c_int32), ("rope_theta", c_float),
                ("rms_eps", c_float), ("c_stride", c_int32), ("embed", c_void_p),
                ("final_norm", c_void_p), ("lm_head", c_void_p), ("layers", POINTER(SsLayer))]


class SsStepArgs(ctypes.Structure):
    _fields_ = [("tokens", c_void_p), ("parents", c_void_p), ("T", c_int32), ("C", c_int32),
                ("tree_k", POINTER(c_void_p)), ("tree_v", POINTER(c_void_p)),
                ("hidden_in", c_void_p), ("hidden_out", c_void_p), ("logits", c_void_p),
                ("logit_rows", c_void_p), ("n_logit_rows", c_int32)]


class SsAttnArgs(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("k_cache", c_void_p), ("v_cache", c_void_p),
                ("k_tree", c_void_p), ("v_tree", c_void_p), ("parents", c_void_p),
                ("out", c_void_p), ("out_f32", c_void_p), ("mask_out", c_void_p),
                ("T", c_int32), ("C", c_int32), ("c_stride", c_int32), ("nq", c_int32),
                ("nkv", c_int32), ("hd", c_int32), ("sm_scale", c_float)]


# name -> (restype, argtypes)
SIGNATURES = {
    "ss_last_error": (c_char_p, []),
    "ss_abi_version": (c_int, []),
    "ss_quantize_substitute": (c_int, [c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p,
                                       c_void_p, c_void_p]),
    "ss_dequantize_substitute": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int32,
                                         c_void_p, c_void_p]),
    "ss_w4a16_linear_workspace": (c_size_t, [c_int32, c_int64, c_int64]),
    "ss_w4a16_linear": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "ss_w4a16_gate_up_swiglu_workspace": (c_size_t, [c_int32, c_int64, c_int64]),
    "ss_w4a16_gate_up_swiglu": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int64,
                                        c_int64, c_void_p, c_void_p, c_size_t, c_void_p]),
    "ss_w4_tiled_bytes": (c_size_t, [c_int64, c_int64]),
    "ss_w4_tile": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p]),
    "ss_w4a16_linear_tiled": (c_int, [c_void_p, c_int32, c_void_p, c_int64, c_int64, c_void_p, c_void_p,
                                      c_void_p, c_size_t, c_void_p]),
    "ss_tree_accept_stochastic_workspace": (c_size_t, [c_int32, c_int32]),
    "ss_tree_accept_stochastic": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_float,
                                          c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_size_t, c_void_p]),
    "ss_tree_expand_init": (c_int, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p]),
    "ss_tree_expand_workspace": (c_size_t, [c_int32, c_int32]),
    "ss_tree_expand": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_float, c_int32, c_int32, c_int32, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "ss_w4a16_linear_tiled_noalloc": (c_int, [c_void_p, c_int32, c_void_p, c_int64, c_int64, c_void_p,
                                              c_void_p, c_void_p]),
    "ss_w4a16_gate_up_swiglu_tiled": (c_int, [c_void_p, c_int32, c_void_p, c_int64, c_int64, c_void_p,
                                              c_void_p, c_size_t, c_void_p]),
    "ss_kv_commit": (c_int, [POINTER(c_void_p), POINTER(c_void_p), POINTER(c_void_p), POINTER(c_void_p),
                             c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                             c_void_p]),
    "ss_bf16_linear_workspace": (c_size_t, [c_int32, c_int64, c_int64]),
    "ss_bf16_linear": (c_int, [c_void_p, c_int32, c_void_p, c_int64, c_int64, c_void_p, c_void_p,
                               c_void_p, c_size_t, c_void_p]),
    "ss_tree_validate": (c_int, [POINTER(c_int32), c_int32]),
    "ss_tree_mask": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "ss_tree_attention_workspace": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32]),
    "ss_tree_attention": (c_int, [POINTER(SsAttnArgs), c_void_p, c_size_t, c_void_p]),
    "ss_draft_tree_step_workspace": (c_size_t, [POINTER(SsModel), c_int32, c_int32]),
    "ss_draft_tree_step": (c_int, [POINTER(SsModel), POINTER(SsStepArgs), c_void_p, c_size_t,
                                   c_void_p]),
    "ss_row_argmax": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "ss_tree_accept": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                               c_void_p, c_void_p]),
    "ss_draft_select_workspace": (c_size_t, [c_int32, c_int32, c_int32]),
    "ss_draft_select": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_float, c_int32, c_void_p,
                                c_void_p, c_size_t, c_void_p]),
}

_lib = None


def lib():
    """Load libsubspec.so (built in-tree); raise if it is missing. There is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with "
                              "`python -m bit_quantized_draft_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class SubspecError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status):
    if status != SS_OK:
        raise SubspecError(status, lib().ss_last_error().decode())
    return status
