"""Pins of the oracle's RMSNorm, RoPE, SwiGLU and decoder-layer composition.

- RoPE: identity at position 0; norm preserved; scores depend only on the position
  difference; equal to multiplying (x_i, x_{i+hd/2}) pairs by e^{i pos theta^(-2i/hd)};
- RMSNorm: a constant vector maps to +-gain; invariant to positive rescaling;
- silu: x * expit(x) from scipy;
- layer: zero o/down weights leave the hidden state unchanged; a single root token
  with no prefix attends only to itself, so the layer reduces to plain matrix
  products, checked in closed form with all four projections;
- relabelling the tree nodes in another topological order permutes the layer output;
- stack: zero o/down weights reduce it to embedding, final norm and head; three
  non-trivial layers agree with an independent float64 torch implementation (torch
  RMSNorm, RoPE as a complex rotation, ancestor mask by walking parents, masked
  scaled-dot-product attention, SiLU).
"""

import types

import numpy as np
import scipy.special

import oracle
from synth import gen


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((3, 2, 16))
    np.testing.assert_array_equal(oracle.rope64(x, np.zeros(3), 1e6), x)


def test_rope_preserves_norm_and_matches_complex_form():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 32))
    pos = np.array([0, 1, 7, 2048, 16431])
    y = oracle.rope64(x, pos, 5e5)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    half = 16
    z = x[..., :half] + 1j * x[..., half:]
    freqs = 5e5 ** (-np.arange(half) * 2.0 / 32)
    w = z * np.exp(1j * pos[:, None, None] * freqs[None, None, :])
    np.testing.assert_allclose(y, np.concatenate([w.real, w.imag], axis=-1), rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_on_position_difference():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    a = np.sum(oracle.rope64(q, [100], 1e6) * oracle.rope64(k, [37], 1e6))
    b = np.sum(oracle.rope64(q, [1063], 1e6) * oracle.rope64(k, [1000], 1e6))
    np.testing.assert_allclose(a, b, rtol=1e-10)


def test_rmsnorm_constant_vector_and_scale_invariance():
    g = 1 + 0.1 * np.random.default_rng(3).standard_normal(64)
    np.testing.assert_allclose(oracle.rmsnorm64(np.full((1, 64), -3.0), g, 0.0)[0], -g, rtol=1e-15)
    x = np.random.default_rng(4).standard_normal((4, 64))
    np.testing.assert_allclose(oracle.rmsnorm64(x, g, 0.0), oracle.rmsnorm64(7.5 * x, g, 0.0),
                               rtol=1e-14)


def test_silu_is_x_times_logistic():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu64(x), x * scipy.special.expit(x), rtol=1e-14, atol=1e-300)


def _cfg(H=64, I=128, nq=4, nkv=2, hd=16):
    return types.SimpleNamespace(H=H, I=I, nq=nq, nkv=nkv, hd=hd, rope_theta=1e6, eps=1e-6)


def _layer_weights(cfg, seed, zero_o=False, zero_down=False):
    rng = np.random.default_rng(seed)
    qkv_n = (cfg.nq + 2 * cfg.nkv) * cfg.hd

    def w(n, k, zero=False):
        a = np.zeros((n, k)) if zero else rng.standard_normal((n, k)) * 0.1
        return oracle.quantize(gen.bf16_bits(a))

    return {"qkv": w(qkv_n, cfg.H), "o": w(cfg.H, cfg.nq * cfg.hd, zero_o),
            "gate_up": w(2 * cfg.I, cfg.H), "down": w(cfg.H, cfg.I, zero_down),
            "norm1": gen.norm_gain_bf16(cfg.H, seed=seed, which=0, random=True),
            "norm2": gen.norm_gain_bf16(cfg.H, seed=seed, which=1, random=True)}


def test_layer_with_zero_output_projections_is_identity():
    cfg = _cfg()
    lw = _layer_weights(cfg, 0, zero_o=True, zero_down=True)
    T, C = 9, 5
    rng = np.random.default_rng(1)
    h = rng.standard_normal((T, cfg.H))
    kc = rng.standard_normal((cfg.nkv, C, cfg.hd))
    vc = rng.standard_normal((cfg.nkv, C, cfg.hd))
    out, _, _ = oracle.layer64(h, lw, kc, vc, gen.tree_parents(T, "R"), C, cfg)
    np.testing.assert_array_equal(out, h)


def test_single_root_token_reduces_to_matrix_products():
    cfg = _cfg()
    lw = _layer_weights(cfg, 2)
    rng = np.random.default_rng(3)
    h = rng.standard_normal((1, cfg.H))
    kc = np.zeros((cfg.nkv, 0, cfg.hd))
    out, kt, vt = oracle.layer64(h, lw, kc, kc, np.array([-1]), 0, cfg)
    W = {n: oracle.dequant_exact64(*lw[n]) for n in ("qkv", "o", "gate_up", "down")}
    g1 = oracle.bf16_to_f64(lw["norm1"])
    g2 = oracle.bf16_to_f64(lw["norm2"])
    x = h[0] / np.sqrt(np.mean(h[0] ** 2) + cfg.eps) * g1
    nq_hd, nkv_hd = cfg.nq * cfg.hd, cfg.nkv * cfg.hd
    v = W["qkv"][nq_hd + nkv_hd:] @ x                          # rows of the v projection
    attn = np.concatenate([v[(hh // 2) * cfg.hd:(hh // 2 + 1) * cfg.hd] for hh in range(cfg.nq)])
    h1 = h[0] + W["o"] @ attn
    x2 = h1 / np.sqrt(np.mean(h1 ** 2) + cfg.eps) * g2
    gate, up = W["gate_up"][:cfg.I] @ x2, W["gate_up"][cfg.I:] @ x2
    h2 = h1 + W["down"] @ (gate * scipy.special.expit(gate) * up)
    np.testing.assert_allclose(out[0], h2, rtol=1e-12, atol=1e-12)
    # at position C + depth = 0, the stored tree key is the unrotated k projection
    k = W["qkv"][nq_hd:nq_hd + nkv_hd] @ x
    np.testing.assert_allclose(kt[:, 0, :].ravel(), k, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(vt[:, 0, :].ravel(), v, rtol=1e-12, atol=1e-13)


def test_layer_relabelling_permutes_outputs():
    cfg = _cfg()
    lw = _layer_weights(cfg, 4)
    T, C = 8, 3
    rng = np.random.default_rng(5)
    h = rng.standard_normal((T, cfg.H))
    kc = rng.standard_normal((cfg.nkv, C, cfg.hd))
    vc = rng.standard_normal((cfg.nkv, C, cfg.hd))
    par = np.array([-1, 0, 1, 0, 3, 1, 4, 2], dtype=np.int32)
    order = [0, 3, 4, 6, 1, 5, 2, 7]                  # another topological order
    new_of = {o: n for n, o in enumerate(order)}
    par2 = np.array([-1] + [new_of[int(par[o])] for o in order[1:]], dtype=np.int32)
    a, _, _ = oracle.layer64(h, lw, kc, vc, par, C, cfg)
    b, _, _ = oracle.layer64(h[order], lw, kc, vc, par2, C, cfg)
    np.testing.assert_allclose(b, a[order], rtol=1e-12, atol=1e-12)


def test_stack_with_zero_output_projections_is_embedding_then_head():
    cfg = _cfg()
    V = 50
    rng = np.random.default_rng(6)
    embed = gen.bf16_bits(rng.standard_normal((V, cfg.H)))
    head = gen.bf16_bits(rng.standard_normal((V, cfg.H)) * 0.05)
    fnorm = gen.norm_gain_bf16(cfg.H, seed=6, random=True)
    layers = [_layer_weights(cfg, 10 + i, zero_o=True, zero_down=True) for i in range(3)]
    T, C = 6, 2
    kcs = [rng.standard_normal((cfg.nkv, C, cfg.hd)) for _ in range(3)]
    tok = np.array([3, 49, 0, 7, 7, 21])
    par = gen.tree_parents(T, "R", seed=6)
    h, logits = oracle.stack64(tok, par, C, embed, layers, kcs, kcs, fnorm, head, cfg,
                               logit_rows=[1, 4])
    e = oracle.bf16_to_f64(embed)[tok]
    np.testing.assert_array_equal(h, e)
    g = oracle.bf16_to_f64(fnorm)
    for r, row in enumerate([1, 4]):
        x = e[row] / np.sqrt(np.mean(e[row] ** 2) + cfg.eps) * g
        np.testing.assert_allclose(logits[r], oracle.bf16_to_f64(head) @ x, rtol=1e-12, atol=1e-12)


def _torch_stack_reference(tok, par, C, embed, layers, kcs, vcs, fnorm, head, cfg, rows):
    """An independent float64 implementation of the substitute stack with torch primitives:
    torch's RMSNorm, RoPE as a complex rotation of (x_i, x_{i+hd/2}) pairs, the tree mask
    by walking parent pointers, torch's masked scaled-dot-product attention with the KV
    heads repeated per query group, and torch's SiLU."""
    import torch
    import torch.nn.functional as F
    f64 = torch.float64
    bf = lambda bits: torch.from_numpy(oracle.bf16_to_f64(bits))  # bf16 bits -> float64 tensor

    def deq(entry):
        q, s, z = entry
        q = torch.from_numpy(q.astype(np.float64))
        s = torch.from_numpy(s.astype(np.float64)).repeat_interleave(64, dim=1)
        z = torch.from_numpy(z.astype(np.float64)).repeat_interleave(64, dim=1)
        return (q - z) * s

    T = len(tok)
    depth = []
    for i in range(T):                      # depth by walking parents
        d, cur = 0, i
        while par[cur] >= 0:
            cur, d = int(par[cur]), d + 1
        depth.append(d)
    vis = torch.zeros((T, C + T), dtype=torch.bool)
    vis[:, :C] = True
    for i in range(T):                      # ancestors-or-self by walking parents
        cur = i
        while cur >= 0:
            vis[i, C + cur] = True
            cur = int(par[cur])
    pos = torch.tensor([C + d for d in depth], dtype=f64)
    half = cfg.hd // 2
    freq = cfg.rope_theta ** (-torch.arange(half, dtype=f64) * 2.0 / cfg.hd)
    rot = torch.polar(torch.ones(T, half, dtype=f64), pos[:, None] * freq[None, :])   # e^{i pos f}

    def rope(x):                            # x [T][heads][hd]
        c = torch.complex(x[..., :half], x[..., half:]) * rot[:, None, :]
        return torch.cat([c.real, c.imag], dim=-1)

    h = bf(embed)[torch.from_numpy(np.asarray(tok))]
    grp = cfg.nq // cfg.nkv
    for li, lw in enumerate(layers):
        x = F.rms_norm(h, (cfg.H,), weight=bf(lw["norm1"]), eps=cfg.eps)
        qkv = x @ deq(lw["qkv"]).T
        q = rope(qkv[:, :cfg.nq * cfg.hd].reshape(T, cfg.nq, cfg.hd))
        k = rope(qkv[:, cfg.nq * cfg.hd:(cfg.nq + cfg.nkv) * cfg.hd].reshape(T, cfg.nkv, cfg.hd))
        v = qkv[:, (cfg.nq + cfg.nkv) * cfg.hd:].reshape(T, cfg.nkv, cfg.hd)
        K = torch.cat([torch.from_numpy(np.asarray(kcs[li], np.float64)[:, :C]), k.transpose(0, 1)], dim=1)
        Vv = torch.cat([torch.from_numpy(np.asarray(vcs[li], np.float64)[:, :C]), v.transpose(0, 1)], dim=1)
        K = K.repeat_interleave(grp, dim=0)                                   # [nq][C+T][hd]
        Vv = Vv.repeat_interleave(grp, dim=0)
        a = F.scaled_dot_product_attention(q.transpose(0, 1), K, Vv, attn_mask=vis[None])
        h = h + a.transpose(0, 1).reshape(T, cfg.nq * cfg.hd) @ deq(lw["o"]).T
        x = F.rms_norm(h, (cfg.H,), weight=bf(lw["norm2"]), eps=cfg.eps)
        gu = x @ deq(lw["gate_up"]).T
        h = h + (F.silu(gu[:, :cfg.I]) * gu[:, cfg.I:]) @ deq(lw["down"]).T
    x = F.rms_norm(h[list(rows)], (cfg.H,), weight=bf(fnorm), eps=cfg.eps)
    return h.numpy(), (x @ bf(head).T).numpy()


def test_stack_matches_an_independent_torch_implementation():
    """Pins the whole-stack composition: layer order, each layer's own KV cache, positions
    C + depth, residual adds, final RMSNorm of the selected rows and the LM head."""
    cfg = _cfg(H=64, I=128, nq=4, nkv=2, hd=16)
    V, T, C = 40, 11, 7
    rng = np.random.default_rng(21)
    embed = gen.bf16_bits(rng.standard_normal((V, cfg.H)))
    head = gen.bf16_bits(rng.standard_normal((V, cfg.H)) * 0.05)
    fnorm = gen.norm_gain_bf16(cfg.H, seed=21, random=True)
    layers = [_layer_weights(cfg, 30 + i) for i in range(3)]
    kcs = [rng.standard_normal((cfg.nkv, C + 2, cfg.hd)) for _ in range(3)]   # c_stride > C
    vcs = [rng.standard_normal((cfg.nkv, C + 2, cfg.hd)) for _ in range(3)]
    tok = rng.integers(0, V, T)
    par = gen.tree_parents(T, "R", seed=21)
    rows = [10, 0, 4]
    h, logits = oracle.stack64(tok, par, C, embed, layers, kcs, vcs, fnorm, head, cfg, logit_rows=rows)
    h_ref, lg_ref = _torch_stack_reference(tok, par, C, embed, layers, kcs, vcs, fnorm, head, cfg, rows)
    np.testing.assert_allclose(h, h_ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(logits, lg_ref, rtol=1e-10, atol=1e-10)
    # swapping two layers changes the result: the composition order is observed
    h_sw, _ = oracle.stack64(tok, par, C, embed, [layers[1], layers[0], layers[2]],
                             [kcs[1], kcs[0], kcs[2]], [vcs[1], vcs[0], vcs[2]], fnorm, head, cfg)
    assert np.abs(h_sw - h).max() > 1e-3
