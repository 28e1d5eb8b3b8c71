"""Parity at the workloads' full sizes, on sampled outputs the oracle computes cheaply.

Every substitute linear shape of the three model families (Qwen2.5-7B, Qwen2.5-32B and
Llama-3.1-8B shaped layers) runs through the C ABI at the tree size its workload uses
(T = 64 / 48 for the 7B and 8B shapes, T = 256 for the 32B shapes), on the plain int4
layout (compared with the oracle on sampled rows) and on the tiled layout the bench
streams (compared bit for bit with the plain layout's output: the same arithmetic on
relocated codes). The bf16 LM heads of the 7B and 8B families (V = 152064 and 128256) are
compared with the oracle on sampled vocabulary rows. Weights and activations come from the seeded generators;
the GPU quantizes the whole bf16 matrix, the oracle quantizes only the sampled rows
(quantization is per row and group, so the rows are independent), and both the codes
and the outputs of those rows are compared. Attention at the 32B workload's size
(T = 256 random-branching tree, C = 4096, 40 / 8 heads) is compared on one KV head's
query heads, which the oracle can afford.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests.gpu_util import assert_close, bf16_bits, host, to_bf16, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_quantized_draft_amd")

N_SAMPLE = 48


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


# (name, N, K, T): the four fused linears of each family at its workload's tree size
SHAPES = [
    ("7b.qkv", 4608, 3584, 64), ("7b.o", 3584, 3584, 64), ("7b.down", 3584, 18944, 64),
    ("32b.qkv", 7168, 5120, 256), ("32b.o", 5120, 5120, 256), ("32b.down", 5120, 27648, 256),
    ("8b.qkv", 6144, 4096, 48), ("8b.o", 4096, 4096, 48), ("8b.down", 4096, 14336, 48),
]
GATE_UP = [("7b.gate_up", 18944, 3584, 64), ("32b.gate_up", 27648, 5120, 256),
           ("8b.gate_up", 14336, 4096, 48)]


def _rows(N, seed, n=N_SAMPLE):
    rng = np.random.default_rng(seed)
    # include both ends and a spread of interior rows
    return np.unique(np.concatenate([[0, N - 1], rng.choice(N, size=n - 2, replace=False)]))


def _check_rows_quant(q_dev, s_dev, z_dev, w_rows):
    q_o, s_o, z_o = oracle.quantize(w_rows)
    assert np.array_equal(host(q_dev), oracle.pack_int4(q_o)), "int4 codes differ on sampled rows"
    assert np.array_equal(host(s_dev).view(np.uint16), s_o.view(np.uint16)), "scales differ on sampled rows"
    assert np.array_equal(host(z_dev).view(np.uint16), z_o.view(np.uint16)), "zeros differ on sampled rows"
    return q_o, s_o, z_o


@pytest.mark.parametrize("name,N,K,T", SHAPES)
def test_w4a16_linear_fullsize_sampled(name, N, K, T):
    print(f"full-size linear {name}: N={N} K={K} T={T}", flush=True)
    seed = N + K
    w = gen.weight_bf16(N, K, 0.02, seed=seed, cid=11)
    x = gen.normal_bf16((T, K), 1.0, seed, 11, gen.TID_X)
    q, s, z = bq.quantize_substitute(to_bf16(w))
    _, yf = bq.w4a16_linear(to_bf16(x), q, s, z, want_bf16=False)
    torch.cuda.synchronize()
    rows = _rows(N, seed)
    ridx = torch.from_numpy(rows).to(q.device)
    q_o, s_o, z_o = _check_rows_quant(q[ridx], s[ridx], z[ridx], w[rows])
    ref = oracle.w4a16_matmul64(x, q_o, s_o, z_o)
    assert_close(host(yf)[:, rows], ref, what=f"{name} fp32 (sampled rows)")
    # the tiled layout the bench streams: bit-identical to the plain layout's output
    _, yt = bq.w4a16_linear_tiled(to_bf16(x), bq.w4_tile(q, s, z), want_bf16=False)
    torch.cuda.synchronize()
    assert torch.equal(yt, yf), f"{name}: tiled output differs from the plain layout's"


@pytest.mark.parametrize("name,I,K,T", GATE_UP)
def test_gate_up_swiglu_fullsize_sampled(name, I, K, T):
    print(f"full-size gate_up {name}: I={I} K={K} T={T}", flush=True)
    seed = I + K
    w = gen.weight_bf16(2 * I, K, 0.02, seed=seed, cid=12)
    x = gen.normal_bf16((T, K), 1.0, seed, 12, gen.TID_X)
    q, s, z = bq.quantize_substitute(to_bf16(w))
    u = bq.w4a16_gate_up_swiglu(to_bf16(x), q, s, z)
    torch.cuda.synchronize()
    g_rows = _rows(I, seed)
    both = np.concatenate([g_rows, g_rows + I])
    bidx = torch.from_numpy(both).to(q.device)
    q_o, s_o, z_o = _check_rows_quant(q[bidx], s[bidx], z[bidx], w[both])
    y = oracle.w4a16_matmul64(x, q_o, s_o, z_o)
    n = len(g_rows)
    ref = oracle.swiglu64(y[:, :n], y[:, n:])
    got = oracle.bf16_to_f64(bf16_bits(u))[:, g_rows]
    assert_close(got, ref, scale_abs=True, bf16_out=True, what=f"{name} u (sampled rows)")
    ut = bq.w4a16_gate_up_swiglu_tiled(to_bf16(x), bq.w4_tile(q, s, z))
    torch.cuda.synchronize()
    assert torch.equal(ut.view(torch.int16), u.view(torch.int16)), f"{name}: tiled u differs from the plain layout's"


@pytest.mark.parametrize("name,V,H,T", [("7b.lm_head", 152064, 3584, 64), ("8b.lm_head", 128256, 4096, 48)])
def test_lm_head_fullsize_sampled(name, V, H, T):
    """The dense bf16 LM head at the full vocabulary (the draft step's last GEMM and the
    verify pass's), against the oracle's fp64 product on sampled vocabulary rows."""
    print(f"full-size LM head {name}: V={V} H={H} T={T}", flush=True)
    seed = V + H
    w = gen.normal_bf16((V, H), 0.05, seed, 13, gen.TID_LMHEAD)
    x = gen.normal_bf16((T, H), 1.0, seed, 13, gen.TID_X)
    yb, yf = bq.bf16_linear(to_bf16(x), to_bf16(w))
    torch.cuda.synchronize()
    rows = _rows(V, seed, n=256)
    ref = oracle.matmul64(oracle.bf16_to_f64(x), oracle.bf16_to_f64(w[rows]))
    assert_close(host(yf)[:, rows], ref, scale_abs=True, what=f"{name} logits (sampled rows)")
    assert np.array_equal(bf16_bits(yb)[:, rows], oracle.f32_to_bf16(host(yf)[:, rows]))


def test_tree_attention_32b_workload_one_kv_head():
    T, C, nq, nkv, hd = 256, 4096, 40, 8, 128
    print(f"full-size attention T={T} C={C} nq={nq} nkv={nkv}", flush=True)
    seed = 4
    q = gen.normal_bf16((T, nq, hd), 1.0, seed, 4, gen.TID_Q)
    kc = gen.normal_bf16((nkv, C, hd), 1.0, seed, 4, gen.TID_KC)
    vc = gen.normal_bf16((nkv, C, hd), 1.0, seed, 4, gen.TID_VC)
    kt = gen.normal_bf16((nkv, T, hd), 1.0, seed, 4, gen.TID_KT)
    vt = gen.normal_bf16((nkv, T, hd), 1.0, seed, 4, gen.TID_VT)
    par = gen.tree_parents(T, "RB", seed=seed)
    out, outf, _ = bq.tree_attention(to_bf16(q), to_bf16(kc), to_bf16(vc), to_bf16(kt), to_bf16(vt),
                                     to_dev(par), C, want_f32=True)
    torch.cuda.synchronize()
    kvh = 5   # one KV head and its query heads
    grp = nq // nkv
    hs = slice(kvh * grp, (kvh + 1) * grp)
    ref = oracle.tree_attention64(oracle.bf16_to_f64(q[:, hs]), oracle.bf16_to_f64(kc[kvh:kvh + 1]),
                                  oracle.bf16_to_f64(vc[kvh:kvh + 1]), oracle.bf16_to_f64(kt[kvh:kvh + 1]),
                                  oracle.bf16_to_f64(vt[kvh:kvh + 1]), par, C)
    assert_close(host(outf)[:, hs], ref, what="attention fp32 (KV head 5)")
    assert np.array_equal(bf16_bits(out)[:, hs], oracle.f32_to_bf16(host(outf)[:, hs]))
