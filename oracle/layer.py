"""One substitute decoder layer and the substitute stack, in fp64.

TEST INFRASTRUCTURE ONLY (see the package header).

The substitute draft is the target's own architecture with its linear layers
replaced by their 4-bit copies, sharing the target's KV cache ([Summary]
"Approach"; [Abstract]). The pages do not restate the decoder layer; the plainest
reading is the pre-norm Qwen2.5 / Llama-3.1 layer of the model families they
evaluate ([Review] §3.2):

  x = RMSNorm1(h);  [q k v] = x Wqkv^T;  q, k rotated (RoPE) at position C + depth
  h = h + TreeAttention(q, k, v) Wo^T
  x = RMSNorm2(h);  [g u] = x Wgu^T;  h = h + (silu(g) * u) Wdown^T

Readings: no qkv bias; RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gain; RoPE in
rotate-half form with inverse frequency theta^(-2i/hd); the tree node at depth d
sits at position C + d (the root, depth 0, is the token right after the prefix).
Everything here is fp64 from the given bf16 inputs; nothing is rounded between
steps.
"""

import numpy as np

from .attention import tree_attention64
from .fp import bf16_to_f64
from .quant import dequant_exact64
from .tree import tree_depth


def rmsnorm64(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gain, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * g


def rope64(x, pos, theta):
    """Rotate-half RoPE on the last axis of x [T][heads][hd] at integer positions pos [T]."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]      # [T][half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu64(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu64(gate, up):
    return silu64(gate) * np.asarray(up, dtype=np.float64)


def weight64(entry, group=64):
    """A linear weight as fp64: (q, s, z) is a substitute (exact dequant); a uint16 array is bf16."""
    if isinstance(entry, tuple):
        q, s, z = entry
        return dequant_exact64(q, s, z, group)
    return bf16_to_f64(entry)


def layer64(h, lw, k_cache, v_cache, parents, C, cfg):
    """One layer over the T tree tokens.

    h fp64 [T][H]; lw dict with "qkv", "o", "gate_up", "down" (each (q, s, z) or bf16
    bits) and "norm1", "norm2" (bf16 bits [H]); k_cache / v_cache [nkv][>=C][hd].
    Returns (h_out [T][H], k_tree [nkv][T][hd], v_tree [nkv][T][hd]) in fp64.
    """
    h = np.asarray(h, dtype=np.float64)
    T = h.shape[0]
    nq, nkv, hd, I = cfg.nq, cfg.nkv, cfg.hd, cfg.I
    x = rmsnorm64(h, bf16_to_f64(lw["norm1"]), cfg.eps)
    qkv = x @ weight64(lw["qkv"]).T
    q = qkv[:, :nq * hd].reshape(T, nq, hd)
    k = qkv[:, nq * hd:(nq + nkv) * hd].reshape(T, nkv, hd)
    v = qkv[:, (nq + nkv) * hd:].reshape(T, nkv, hd)
    pos = C + tree_depth(parents)
    q = rope64(q, pos, cfg.rope_theta)
    k = rope64(k, pos, cfg.rope_theta)
    kt = np.ascontiguousarray(k.transpose(1, 0, 2))
    vt = np.ascontiguousarray(v.transpose(1, 0, 2))
    kc = bf16_to_f64(k_cache) if k_cache.dtype == np.uint16 else np.asarray(k_cache, np.float64)
    vc = bf16_to_f64(v_cache) if v_cache.dtype == np.uint16 else np.asarray(v_cache, np.float64)
    a = tree_attention64(q, kc, vc, kt, vt, parents, C).reshape(T, nq * hd)
    h = h + a @ weight64(lw["o"]).T
    x = rmsnorm64(h, bf16_to_f64(lw["norm2"]), cfg.eps)
    gu = x @ weight64(lw["gate_up"]).T
    m = swiglu64(gu[:, :I], gu[:, I:])
    h = h + m @ weight64(lw["down"]).T
    return h, kt, vt


def stack64(tokens, parents, C, embed, layers, k_caches, v_caches, final_norm, lm_head, cfg,
            logit_rows=None):
    """Embedding gather, every layer, then final RMSNorm and the bf16 LM head.

    Returns (h after the last layer [T][H], logits [R][V] or None) in fp64.
    """
    h = bf16_to_f64(np.asarray(embed)[np.asarray(tokens)])
    for li, lw in enumerate(layers):
        h, _, _ = layer64(h, lw, k_caches[li], v_caches[li], parents, C, cfg)
    logits = None
    if lm_head is not None:
        rows = np.arange(len(tokens)) if logit_rows is None else np.asarray(logit_rows)
        x = rmsnorm64(h[rows], bf16_to_f64(final_norm), cfg.eps)
        logits = x @ bf16_to_f64(lm_head).T
    return h, logits
