"""Python binding of the substitute-draft hot path: the C ABI names over torch tensors.

Torch supplies device memory and the current stream; every step runs in the HIP
library (libsubspec.so). Functions allocate their outputs with torch.empty when the
caller passes none, check shapes/dtypes enough to marshal pointers, and raise
SubspecError with the library's message on any error status.
"""

import ctypes

import torch

from ._lib import (SS_BF16, SS_ERR_INVALID_ARG, SS_ERR_UNSUPPORTED, SS_W4G64, SS_W4G64_TILED, SsAttnArgs,
                   SsLayer, SsLinear, SsModel, SsStepArgs, SubspecError, check, lib)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_device(t):
    return t.is_cuda


def _bad(msg):
    return SubspecError(SS_ERR_INVALID_ARG, msg)


def _need(t, dtype, name, shape=None):
    """A contiguous device tensor of this dtype and, when given, exactly this shape (a
    mismatch would make the library read or write outside the tensor)."""
    dtypes = dtype if isinstance(dtype, tuple) else (dtype,)
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes or not _on_device(t) or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous CUDA tensor of dtype {' or '.join(map(str, dtypes))}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise _bad(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _need_2d(t, dtype, name):
    _need(t, dtype, name)
    if t.dim() != 2:
        raise _bad(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape


def _need_vec(t, dtype, name, n):
    _need(t, dtype, name)
    if t.numel() != n:
        raise _bad(f"{name} must hold {n} elements, got {t.numel()}")


def _need_w4(q, s, z, n, k, what):
    _need(q, torch.uint8, f"{what} qweight", (n, k // 2))
    _need(s, torch.float16, f"{what} scale", (n, k // 64))
    _need(z, torch.float16, f"{what} zero", (n, k // 64))


def _need_tiled(tw, n, k):
    if not isinstance(tw, TiledW4):
        raise TypeError("weight must be a TiledW4")
    if (tw.n, tw.k) != (n, k):
        raise _bad(f"tiled weight is [{tw.n}][{tw.k}], expected [{n}][{k}]")
    _need(tw.data, torch.uint8, "tiled weight data")
    if tw.data.numel() < lib().ss_w4_tiled_bytes(n, k):
        raise _bad(f"tiled weight data holds {tw.data.numel()} bytes, {lib().ss_w4_tiled_bytes(n, k)} needed")


def _workspace(nbytes, device, ws=None):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def abi_version():
    return lib().ss_abi_version()


# ------------------------------------------------------------------ substitute construction

def quantize_substitute(w, group=64):
    """bf16 W [n][k] -> (qweight u8 [n][k/2], scale fp16 [n][k/64], zero fp16 [n][k/64])."""
    n, k = _need_2d(w, torch.bfloat16, "w")
    q = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    s = torch.empty((n, k // 64), dtype=torch.float16, device=w.device)
    z = torch.empty((n, k // 64), dtype=torch.float16, device=w.device)
    check(lib().ss_quantize_substitute(_ptr(w), n, k, group, _ptr(q), _ptr(s), _ptr(z), _stream()))
    return q, s, z


def dequantize_substitute(q, s, z, group=64):
    n, kh = _need_2d(q, torch.uint8, "qweight")
    _need_w4(q, s, z, n, kh * 2, "dequantize")
    out = torch.empty((n, kh * 2), dtype=torch.float16, device=q.device)
    check(lib().ss_dequantize_substitute(_ptr(q), _ptr(s), _ptr(z), n, kh * 2, group, _ptr(out),
                                         _stream()))
    return out


class TiledW4:
    """An int4 weight [n][k] in the tiled layout the GEMMs stream (a relocation of the
    codes, scales and zeros; see ss_w4_tile in include/subspec.h)."""

    def __init__(self, data, n, k):
        self.data, self.n, self.k = data, n, k


def w4_tile(q, s, z):
    """(qweight, scale, zero) of an int4 weight [n][k] -> TiledW4."""
    n, kh = _need_2d(q, torch.uint8, "qweight")
    k = kh * 2
    _need_w4(q, s, z, n, k, "w4_tile")
    nbytes = lib().ss_w4_tiled_bytes(n, k)
    if nbytes == 0:
        raise SubspecError(SS_ERR_UNSUPPORTED, f"w4_tile: unsupported shape n={n} k={k}")
    t = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    check(lib().ss_w4_tile(_ptr(q), _ptr(s), _ptr(z), n, k, _ptr(t), _stream()))
    return TiledW4(t, n, k)


# ------------------------------------------------------------------ linear layers

def w4a16_linear(x, q, s, z, want_bf16=True, want_f32=True, workspace=None):
    """Y = X deq(W)^T; returns (y_bf16 or None, y_f32 or None)."""
    T, k = _need_2d(x, torch.bfloat16, "x")
    n = _need_2d(q, torch.uint8, "qweight")[0]
    _need_w4(q, s, z, n, k, "w4a16_linear")
    yb = torch.empty((T, n), dtype=torch.bfloat16, device=x.device) if want_bf16 else None
    yf = torch.empty((T, n), dtype=torch.float32, device=x.device) if want_f32 else None
    nbytes = lib().ss_w4a16_linear_workspace(T, n, k)
    ws = _workspace(nbytes, x.device, workspace)
    check(lib().ss_w4a16_linear(_ptr(x), T, _ptr(q), _ptr(s), _ptr(z), n, k, _ptr(yb), _ptr(yf),
                                _ptr(ws), nbytes, _stream()))
    return yb, yf


def w4a16_gate_up_swiglu(x, q, s, z, out=None, workspace=None):
    """u = silu(X Wg^T) * (X Wu^T) with the fused int4 gate_up weight [2I][k]; u bf16 [T][I]."""
    T, k = _need_2d(x, torch.bfloat16, "x")
    n2 = _need_2d(q, torch.uint8, "qweight")[0]
    if n2 % 2:
        raise _bad(f"gate_up weight has {n2} rows, an odd count")
    I = n2 // 2
    _need_w4(q, s, z, n2, k, "w4a16_gate_up_swiglu")
    if out is not None:
        _need(out, torch.bfloat16, "out", (T, I))
    u = torch.empty((T, I), dtype=torch.bfloat16, device=x.device) if out is None else out
    nbytes = lib().ss_w4a16_gate_up_swiglu_workspace(T, I, k)
    ws = _workspace(nbytes, x.device, workspace)
    check(lib().ss_w4a16_gate_up_swiglu(_ptr(x), T, _ptr(q), _ptr(s), _ptr(z), I, k, _ptr(u),
                                        _ptr(ws), nbytes, _stream()))
    return u


def w4a16_linear_tiled(x, tw, want_bf16=True, want_f32=True, workspace=None):
    """w4a16_linear on a TiledW4 weight."""
    T, k = _need_2d(x, torch.bfloat16, "x")
    n = tw.n
    _need_tiled(tw, n, k)
    yb = torch.empty((T, n), dtype=torch.bfloat16, device=x.device) if want_bf16 else None
    yf = torch.empty((T, n), dtype=torch.float32, device=x.device) if want_f32 else None
    nbytes = lib().ss_w4a16_linear_workspace(T, n, k)
    ws = _workspace(nbytes, x.device, workspace)
    check(lib().ss_w4a16_linear_tiled(_ptr(x), T, _ptr(tw.data), n, k, _ptr(yb), _ptr(yf), _ptr(ws),
                                      nbytes, _stream()))
    return yb, yf


def w4a16_linear_tiled_noalloc(x, tw, yb, yf):
    """w4a16_linear_tiled into caller-provided outputs (bf16 and/or fp32 [T][n], either may be
    None), with the library's device scratch for partial sums: no allocation anywhere."""
    T, k = _need_2d(x, torch.bfloat16, "x")
    n = tw.n
    _need_tiled(tw, n, k)
    if yb is not None:
        _need(yb, torch.bfloat16, "yb", (T, n))
    if yf is not None:
        _need(yf, torch.float32, "yf", (T, n))
    check(lib().ss_w4a16_linear_tiled_noalloc(_ptr(x), T, _ptr(tw.data), n, k, _ptr(yb), _ptr(yf), _stream()))
    return yb, yf


def w4a16_gate_up_swiglu_tiled(x, tw, out=None, workspace=None):
    """w4a16_gate_up_swiglu on a TiledW4 weight [2I][k]."""
    T, k = _need_2d(x, torch.bfloat16, "x")
    _need_tiled(tw, tw.n, k)
    if tw.n % 2:
        raise _bad(f"gate_up weight has {tw.n} rows, an odd count")
    I = tw.n // 2
    if out is not None:
        _need(out, torch.bfloat16, "out", (T, I))
    u = torch.empty((T, I), dtype=torch.bfloat16, device=x.device) if out is None else out
    nbytes = lib().ss_w4a16_gate_up_swiglu_workspace(T, I, k)
    ws = _workspace(nbytes, x.device, workspace)
    check(lib().ss_w4a16_gate_up_swiglu_tiled(_ptr(x), T, _ptr(tw.data), I, k, _ptr(u), _ptr(ws), nbytes,
                                              _stream()))
    return u


def bf16_linear(x, w, want_bf16=True, want_f32=True, workspace=None):
    T, k = _need_2d(x, torch.bfloat16, "x")
    n = _need_2d(w, torch.bfloat16, "w")[0]
    _need(w, torch.bfloat16, "w", (n, k))
    yb = torch.empty((T, n), dtype=torch.bfloat16, device=x.device) if want_bf16 else None
    yf = torch.empty((T, n), dtype=torch.float32, device=x.device) if want_f32 else None
    nbytes = lib().ss_bf16_linear_workspace(T, n, k)
    ws = _workspace(nbytes, x.device, workspace)
    check(lib().ss_bf16_linear(_ptr(x), T, _ptr(w), n, k, _ptr(yb), _ptr(yf), _ptr(ws), nbytes,
                               _stream()))
    return yb, yf


# ------------------------------------------------------------------ tree

def tree_validate(parents):
    """CPU check of a parent array (list / numpy / CPU tensor). Returns True or raises."""
    import numpy as np
    p = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
    check(lib().ss_tree_validate(p.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(p)))
    return True


def tree_mask(parents):
    """Ancestor-or-self mask (int64 view of the uint64 words) [T][ceil(T/64)] and depth [T]."""
    _need(parents, torch.int32, "parents")
    if parents.dim() != 1:
        raise _bad(f"parents must be 1-D, got shape {tuple(parents.shape)}")
    T = parents.numel()
    W = (T + 63) // 64
    mask = torch.empty((T, W), dtype=torch.int64, device=parents.device)
    depth = torch.empty(T, dtype=torch.int32, device=parents.device)
    check(lib().ss_tree_mask(_ptr(parents), T, _ptr(mask), _ptr(depth), _stream()))
    return mask, depth


def tree_attention(q, k_cache, v_cache, k_tree, v_tree, parents, C, sm_scale=0.0,
                   want_bf16=True, want_f32=False, want_mask=False, workspace=None):
    """Tree attention; q [T][nq][hd], caches [nkv][c_stride][hd], tree K/V [nkv][T][hd]."""
    _need(q, torch.bfloat16, "q")
    if q.dim() != 3:
        raise _bad(f"q must be [T][nq][hd], got shape {tuple(q.shape)}")
    T, nq, hd = q.shape
    _need(k_cache, torch.bfloat16, "k_cache")
    if k_cache.dim() != 3:
        raise _bad(f"k_cache must be [nkv][c_stride][hd], got shape {tuple(k_cache.shape)}")
    nkv, c_stride, _ = k_cache.shape
    _need(k_cache, torch.bfloat16, "k_cache", (nkv, c_stride, hd))
    _need(v_cache, torch.bfloat16, "v_cache", (nkv, c_stride, hd))
    _need(k_tree, torch.bfloat16, "k_tree", (nkv, T, hd))
    _need(v_tree, torch.bfloat16, "v_tree", (nkv, T, hd))
    _need_vec(parents, torch.int32, "parents", T)
    if not 0 <= C <= c_stride:
        raise _bad(f"C={C} outside 0..{c_stride}")
    dev = q.device
    out = torch.empty((T, nq, hd), dtype=torch.bfloat16, device=dev) if want_bf16 else None
    outf = torch.empty((T, nq, hd), dtype=torch.float32, device=dev) if want_f32 else None
    W = (T + 63) // 64
    mask = torch.empty((T, W), dtype=torch.int64, device=dev) if want_mask else None
    a = SsAttnArgs(q=q.data_ptr(), k_cache=k_cache.data_ptr(), v_cache=v_cache.data_ptr(),
                   k_tree=k_tree.data_ptr(), v_tree=v_tree.data_ptr(), parents=parents.data_ptr(),
                   out=None if out is None else out.data_ptr(),
                   out_f32=None if outf is None else outf.data_ptr(),
                   mask_out=None if mask is None else mask.data_ptr(),
                   T=T, C=C, c_stride=c_stride, nq=nq, nkv=nkv, hd=hd, sm_scale=sm_scale)
    nbytes = lib().ss_tree_attention_workspace(T, C, nq, nkv, hd)
    ws = _workspace(nbytes, dev, workspace)
    check(lib().ss_tree_attention(ctypes.byref(a), _ptr(ws), nbytes, _stream()))
    return out, outf, mask


# ------------------------------------------------------------------ verification / selection

def row_argmax(logits, out=None):
    R, V = _need_2d(logits, torch.float32, "logits")
    if out is not None:
        _need(out, torch.int32, "out", (R,))
    out = torch.empty(R, dtype=torch.int32, device=logits.device) if out is None else out
    check(lib().ss_row_argmax(_ptr(logits), R, V, _ptr(out), _stream()))
    return out


def tree_accept(parents, tokens, target_argmax, out=None):
    """Returns device tensors (path [T], accept_len [1], bonus [1])."""
    _need(parents, torch.int32, "parents")
    T = parents.numel()
    _need_vec(tokens, torch.int32, "tokens", T)
    _need_vec(target_argmax, torch.int32, "target_argmax", T)
    dev = parents.device
    if out is not None:
        _need_vec(out[0], torch.int32, "path", T)
        _need_vec(out[1], torch.int32, "accept_len", 1)
        _need_vec(out[2], torch.int32, "bonus", 1)
    if out is None:
        path = torch.empty(T, dtype=torch.int32, device=dev)
        ln = torch.empty(1, dtype=torch.int32, device=dev)
        bonus = torch.empty(1, dtype=torch.int32, device=dev)
    else:
        path, ln, bonus = out
    check(lib().ss_tree_accept(_ptr(parents), _ptr(tokens), _ptr(target_argmax), T, _ptr(path),
                               _ptr(ln), _ptr(bonus), _stream()))
    return path, ln, bonus


def draft_select(logits, gumbel, inv_temp, k, out=None, workspace=None):
    R, V = _need_2d(logits, torch.float32, "logits")
    if gumbel is not None:
        _need(gumbel, torch.float32, "gumbel", (R, V))
    if out is not None:
        _need(out, torch.int32, "out", (R, k))
    out = torch.empty((R, k), dtype=torch.int32, device=logits.device) if out is None else out
    nbytes = lib().ss_draft_select_workspace(R, V, k)
    ws = _workspace(nbytes, logits.device, workspace)
    check(lib().ss_draft_select(_ptr(logits), _ptr(gumbel), R, V, float(inv_temp), k, _ptr(out),
                                _ptr(ws), nbytes, _stream()))
    return out


def tree_accept_stochastic(parents, tokens, draft_logits, target_logits, inv_t_draft, inv_t_target, uniforms,
                           bonus_uniforms, out=None, workspace=None):
    """Multi-round speculative sampling over the tree; returns device tensors (path [T],
    accept_len [1], bonus [1]) as tree_accept."""
    _need(parents, torch.int32, "parents")
    T = parents.numel()
    _need_vec(tokens, torch.int32, "tokens", T)
    V = _need_2d(draft_logits, torch.float32, "draft_logits")[1]
    _need(draft_logits, torch.float32, "draft_logits", (T, V))
    _need(target_logits, torch.float32, "target_logits", (T, V))
    _need_vec(uniforms, torch.float64, "uniforms", T)
    _need_vec(bonus_uniforms, torch.float64, "bonus_uniforms", T)
    dev = parents.device
    if out is None:
        out = (torch.empty(T, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev))
    else:
        _need_vec(out[0], torch.int32, "path", T)
        _need_vec(out[1], torch.int32, "accept_len", 1)
        _need_vec(out[2], torch.int32, "bonus", 1)
    nbytes = lib().ss_tree_accept_stochastic_workspace(T, V)
    ws = _workspace(nbytes, dev, workspace)
    check(lib().ss_tree_accept_stochastic(_ptr(parents), _ptr(tokens), _ptr(draft_logits), _ptr(target_logits), T, V,
                                          float(inv_t_draft), float(inv_t_target), _ptr(uniforms),
                                          _ptr(bonus_uniforms), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(ws),
                                          nbytes, _stream()))
    return out


class TreeState:
    """Device state of the draft-tree expansion: parents / tokens int32 [T] (the draft
    step's inputs), cum fp32 [T], frontier int32 [R] (the next step's logit rows) and meta
    int32 [4] = {nodes, frontier size, step, 0}."""

    def __init__(self, T, D, R, k, device):
        self.T, self.D, self.R, self.k = T, D, R, k
        self.parents = torch.empty(T, dtype=torch.int32, device=device)
        self.tokens = torch.empty(T, dtype=torch.int32, device=device)
        self.cum = torch.empty(T, dtype=torch.float32, device=device)
        self.frontier = torch.empty(R, dtype=torch.int32, device=device)
        self.meta = torch.empty(4, dtype=torch.int32, device=device)
        self._ws = None

    def _args(self):
        return (_ptr(self.parents), _ptr(self.tokens), _ptr(self.cum), _ptr(self.frontier), _ptr(self.meta))


def tree_expand_init(state, root_token):
    """The template before step 0: the root alone."""
    check(lib().ss_tree_expand_init(int(root_token), state.T, state.D, state.R, state.k, *state._args(), _stream()))


def tree_expand(state, logits, children, inv_temp, workspace=None):
    """One expansion step from the frontier rows' logits [R][V] and their children [R][k]."""
    R, V = _need_2d(logits, torch.float32, "logits")
    if R != state.R:
        raise _bad(f"logits has {R} rows, the state's frontier {state.R}")
    _need(children, torch.int32, "children", (state.R, state.k))
    nbytes = lib().ss_tree_expand_workspace(state.R, V)
    ws = _workspace(nbytes, logits.device, workspace if workspace is not None else state._ws)
    state._ws = ws
    check(lib().ss_tree_expand(_ptr(logits), _ptr(children), state.R, V, float(inv_temp), state.k, state.T, state.D,
                               *state._args(), _ptr(ws), nbytes, _stream()))


def draft_select_workspace_bytes(rows, vocab, k):
    """Workspace bytes ss_draft_select needs for this shape (0: none)."""
    return lib().ss_draft_select_workspace(rows, vocab, k)


# ------------------------------------------------------------------ the draft step

def linear_desc(entry):
    """(qweight, scale, zero) tuple -> int4 descriptor; TiledW4 -> tiled int4 descriptor;
    a bf16 tensor -> dense descriptor."""
    if isinstance(entry, TiledW4):
        return SsLinear(kind=SS_W4G64_TILED, qweight=entry.data.data_ptr(), scale=None, zero=None, w=None)
    if isinstance(entry, tuple):
        q, s, z = entry
        return SsLinear(kind=SS_W4G64, qweight=q.data_ptr(), scale=s.data_ptr(), zero=z.data_ptr(),
                        w=None)
    return SsLinear(kind=SS_BF16, qweight=None, scale=None, zero=None, w=entry.data_ptr())


def kv_commit(k_caches, v_caches, tree_k, tree_v, C, path, accept_len):
    """Copy the root's and the accepted path's tree K/V rows of every layer into the
    caches at rows C .. C + L (path / accept_len: device outputs of tree_accept)."""
    L = len(k_caches)
    if L < 1 or not (len(v_caches) == len(tree_k) == len(tree_v) == L):
        raise _bad("kv_commit: one cache and one tree K/V per layer")
    b16 = (torch.bfloat16, torch.int16, torch.uint16)   # rows are copied as 2-byte words
    _need(k_caches[0], b16, "k_caches[0]")
    if k_caches[0].dim() != 3 or tree_k[0].dim() != 3:
        raise _bad("kv_commit: caches are [nkv][c_stride][hd] and tree K/V [nkv][T][hd]")
    nkv, c_stride, hd = k_caches[0].shape
    T = tree_k[0].shape[1]
    for l in range(L):
        _need(k_caches[l], b16, f"k_caches[{l}]", (nkv, c_stride, hd))
        _need(v_caches[l], b16, f"v_caches[{l}]", (nkv, c_stride, hd))
        _need(tree_k[l], b16, f"tree_k[{l}]", (nkv, T, hd))
        _need(tree_v[l], b16, f"tree_v[{l}]", (nkv, T, hd))
    _need_vec(path, torch.int32, "path", T)
    _need_vec(accept_len, torch.int32, "accept_len", 1)
    arr = lambda ts: (ctypes.c_void_p * L)(*[t.data_ptr() for t in ts])
    check(lib().ss_kv_commit(arr(k_caches), arr(v_caches), arr(tree_k), arr(tree_v), L, nkv, hd, c_stride,
                             C, T, _ptr(path), _ptr(accept_len), _stream()))


class SubstituteModel:
    """Borrowed descriptor of a stack: per-layer weights (int4 tuples or bf16), norms, KV caches.

    layers: list of dicts with keys qkv, o, gate_up, down, norm1, norm2, k_cache, v_cache.
    The tensors stay owned by the caller (this object only keeps references).
    """

    def __init__(self, H, I, nq, nkv, hd, layers, V=0, embed=None, final_norm=None,
                 lm_head=None, rope_theta=1e6, rms_eps=1e-6):
        self.layers = layers
        self.keep = (embed, final_norm, lm_head)
        L = len(layers)
        c_stride = layers[0]["k_cache"].shape[1]
        self._layer_arr = (SsLayer * L)()
        for i, ly in enumerate(layers):
            self._layer_arr[i] = SsLayer(
                norm1=ly["norm1"].data_ptr(), norm2=ly["norm2"].data_ptr(),
                qkv=linear_desc(ly["qkv"]), o=linear_desc(ly["o"]),
                gate_up=linear_desc(ly["gate_up"]), down=linear_desc(ly["down"]),
                k_cache=ly["k_cache"].data_ptr(), v_cache=ly["v_cache"].data_ptr())
        self.desc = SsModel(H=H, I=I, nq=nq, nkv=nkv, hd=hd, L=L, V=V, rope_theta=rope_theta,
                            rms_eps=rms_eps, c_stride=c_stride,
                            embed=None if embed is None else embed.data_ptr(),
                            final_norm=None if final_norm is None else final_norm.data_ptr(),
                            lm_head=None if lm_head is None else lm_head.data_ptr(),
                            layers=self._layer_arr)
        self.H, self.I, self.nq, self.nkv, self.hd, self.L, self.V = H, I, nq, nkv, hd, L, V
        self._ws = None

    def workspace_bytes(self, T, C):
        return lib().ss_draft_tree_step_workspace(ctypes.byref(self.desc), T, C)

    def draft_tree_step(self, parents, C, tree_k, tree_v, tokens=None, hidden_in=None,
                        hidden_out=None, logits=None, logit_rows=None, workspace=None):
        """One substitute-stack step over the T tree tokens (outputs written in place)."""
        _need(parents, torch.int32, "parents")
        T = parents.numel()
        L = self.L
        if len(tree_k) != L or len(tree_v) != L:
            raise _bad(f"tree_k / tree_v need one tensor per layer ({L})")
        for l in range(L):
            _need(tree_k[l], torch.bfloat16, f"tree_k[{l}]", (self.nkv, T, self.hd))
            _need(tree_v[l], torch.bfloat16, f"tree_v[{l}]", (self.nkv, T, self.hd))
        if tokens is not None:
            _need_vec(tokens, torch.int32, "tokens", T)
        if hidden_in is not None:
            _need(hidden_in, torch.bfloat16, "hidden_in", (T, self.H))
        if tokens is None and hidden_in is None:
            raise _bad("tokens or hidden_in is needed")
        if hidden_out is not None:
            _need(hidden_out, torch.bfloat16, "hidden_out", (T, self.H))
        if logit_rows is not None:
            _need(logit_rows, torch.int32, "logit_rows")
        if logits is not None:
            R = T if logit_rows is None else logit_rows.numel()
            _need(logits, torch.float32, "logits", (R, self.V))
        tk = (ctypes.c_void_p * L)(*[t.data_ptr() for t in tree_k])
        tv = (ctypes.c_void_p * L)(*[t.data_ptr() for t in tree_v])
        a = SsStepArgs(tokens=None if tokens is None else tokens.data_ptr(),
                       parents=parents.data_ptr(), T=T, C=C, tree_k=tk, tree_v=tv,
                       hidden_in=None if hidden_in is None else hidden_in.data_ptr(),
                       hidden_out=None if hidden_out is None else hidden_out.data_ptr(),
                       logits=None if logits is None else logits.data_ptr(),
                       logit_rows=None if logit_rows is None else logit_rows.data_ptr(),
                       n_logit_rows=0 if logit_rows is None else logit_rows.numel())
        nbytes = self.workspace_bytes(T, C)
        if workspace is None:
            if self._ws is None or self._ws.numel() < nbytes:
                self._ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=parents.device)
            workspace = self._ws
        check(lib().ss_draft_tree_step(ctypes.byref(self.desc), ctypes.byref(a),
                                       ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                       _stream()))


__all__ = ["abi_version", "quantize_substitute", "dequantize_substitute", "w4a16_linear",
           "w4a16_gate_up_swiglu", "TiledW4", "w4_tile", "w4a16_linear_tiled", "w4a16_linear_tiled_noalloc",
           "w4a16_gate_up_swiglu_tiled",
           "bf16_linear", "tree_validate", "tree_mask", "tree_attention", "row_argmax",
           "tree_accept", "kv_commit", "draft_select", "draft_select_workspace_bytes", "TreeState",
           "tree_expand_init", "tree_expand", "tree_accept_stochastic", "SubstituteModel", "SubspecError"]
