"""Parity of the HIP kernels (through the C ABI) with the CPU oracle, kernel by kernel.

Integer outputs (int4 codes, fp16 dequant, masks, argmax, selections, acceptance) must
match bit for bit. Float outputs: rel-L2 <= 1e-2 and max-abs <= 2e-2 on the fp32 result
against the fp64 oracle, and the bf16 output equal to the round-to-nearest-even of the
fp32 result (this reading of the tolerance is documented with the oracle).
"""

import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests.gpu_util import assert_close, bf16_bits, dev, host, to_bf16, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_quantized_draft_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _q_gpu(w_bits):
    q, s, z = bq.quantize_substitute(to_bf16(w_bits))
    torch.cuda.synchronize()
    return host(q), host(s), host(z)


def _check_quant(w_bits):
    q, s, z = _q_gpu(w_bits)
    q_o, s_o, z_o = oracle.quantize(w_bits)
    bad_s = np.argwhere(s.view(np.uint16) != s_o.view(np.uint16))
    bad_z = np.argwhere(z.view(np.uint16) != z_o.view(np.uint16))
    assert len(bad_s) == 0, f"scale mismatch at {bad_s[:4].tolist()}: gpu {s[tuple(bad_s[0])]} oracle {s_o[tuple(bad_s[0])]}"
    assert len(bad_z) == 0, f"zero mismatch at {bad_z[:4].tolist()}: gpu {z[tuple(bad_z[0])]} oracle {z_o[tuple(bad_z[0])]}"
    bad_q = np.argwhere(q != oracle.pack_int4(q_o))
    assert len(bad_q) == 0, f"code mismatch at {bad_q[:4].tolist()}"
    return q_o, s_o, z_o


# ------------------------------------------------------------------ quantization

@pytest.mark.parametrize("N,K,std", [(512, 512, 0.02), (48, 192, 1.0), (16, 64, 0.02)])
def test_quantize_bitexact(N, K, std):
    print(f"quantize N={N} K={K}", flush=True)
    _check_quant(gen.weight_bf16(N, K, std, seed=0, cid=1))


def test_quantize_edge_groups_bitexact():
    from tests.test_oracle_quant import _groups_mix
    _check_quant(_groups_mix(seed=1))


@pytest.mark.parametrize("edge", [False, True])
def test_dequantize_bitexact(edge):
    if edge:
        from tests.test_oracle_quant import _groups_mix
        w = _groups_mix(seed=2)
    else:
        w = gen.weight_bf16(256, 512, 0.05, seed=3, cid=1)
    q_o, s_o, z_o = oracle.quantize(w)
    d = bq.dequantize_substitute(to_dev(oracle.pack_int4(q_o)), to_dev(s_o), to_dev(z_o))
    ref = oracle.dequantize_f16(q_o, s_o, z_o)
    assert np.array_equal(host(d).view(np.uint16), ref.view(np.uint16))


# ------------------------------------------------------------------ W4A16 / bf16 linear

def _linear_case(T, N, K, seed, std=0.02):
    w = gen.weight_bf16(N, K, std, seed=seed, cid=1)
    x = gen.normal_bf16((T, K), 1.0, seed=seed, cid=1, tid=gen.TID_X)
    return w, x


@pytest.mark.parametrize("T,N,K", [(16, 512, 512), (1, 256, 384), (5, 256, 384), (33, 144, 640),
                                   (48, 512, 1024), (64, 384, 512), (100, 256, 256),
                                   (256, 128, 384), (64, 3584, 2048)])
def test_w4a16_linear_parity(T, N, K):
    print(f"w4a16 T={T} N={N} K={K}", flush=True)
    w, x = _linear_case(T, N, K, seed=T + N + K)
    q_o, s_o, z_o = _check_quant(w)
    yb, yf = bq.w4a16_linear(to_bf16(x), to_dev(oracle.pack_int4(q_o)), to_dev(s_o), to_dev(z_o))
    torch.cuda.synchronize()
    ref = oracle.w4a16_matmul64(x, q_o, s_o, z_o)
    assert_close(host(yf), ref, what="w4a16 fp32")
    assert np.array_equal(bf16_bits(yb), oracle.f32_to_bf16(host(yf)))


@pytest.mark.parametrize("T,N,K", [(16, 512, 512), (7, 272, 384), (64, 1024, 1024), (130, 256, 512)])
def test_bf16_linear_parity(T, N, K):
    w, x = _linear_case(T, N, K, seed=7 * T + N, std=0.05)
    yb, yf = bq.bf16_linear(to_bf16(x), to_bf16(w))
    torch.cuda.synchronize()
    ref = oracle.matmul64(oracle.bf16_to_f64(x), oracle.bf16_to_f64(w))
    assert_close(host(yf), ref, what="bf16 linear")
    assert np.array_equal(bf16_bits(yb), oracle.f32_to_bf16(host(yf)))


def test_w4a16_linear_deterministic():
    w, x = _linear_case(48, 3584, 3584, seed=11)
    q, s, z = bq.quantize_substitute(to_bf16(w))
    xd = to_bf16(x)
    a = bq.w4a16_linear(xd, q, s, z)[1].clone()
    b = bq.w4a16_linear(xd, q, s, z)[1]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ tree

@pytest.mark.parametrize("kind,T", [("R", 1), ("R", 16), ("CB", 48), ("CB", 64), ("R", 65),
                                    ("RB", 200), ("RB", 256), ("chain", 256)])
def test_tree_mask_bitexact(kind, T):
    par = gen.tree_parents(T, kind, seed=T)
    mask, depth = bq.tree_mask(to_dev(par))
    torch.cuda.synchronize()
    assert np.array_equal(host(mask).view(np.uint64), oracle.tree_mask(par))
    assert np.array_equal(host(depth), oracle.tree_depth(par))


def test_tree_validate_host():
    assert bq.tree_validate([-1, 0, 0, 1])
    with pytest.raises(bq.SubspecError):
        bq.tree_validate([-1, 0, 3, 1])


# ------------------------------------------------------------------ attention

def _attn_case(T, C, nq, nkv, hd, kind, seed, c_stride=None):
    c_stride = C if c_stride is None else c_stride
    q = gen.normal_bf16((T, nq, hd), 1.0, seed, 1, gen.TID_Q)
    kc = gen.normal_bf16((nkv, c_stride, hd), 1.0, seed, 1, gen.TID_KC)
    vc = gen.normal_bf16((nkv, c_stride, hd), 1.0, seed, 1, gen.TID_VC)
    kt = gen.normal_bf16((nkv, T, hd), 1.0, seed, 1, gen.TID_KT)
    vt = gen.normal_bf16((nkv, T, hd), 1.0, seed, 1, gen.TID_VT)
    par = gen.tree_parents(T, kind, seed=seed)
    return q, kc, vc, kt, vt, par


@pytest.mark.parametrize("T,C,nq,nkv,hd,kind", [
    (16, 128, 1, 1, 64, "R"),          # the small unit case
    (1, 0, 2, 1, 64, "R"),             # root only, no prefix
    (48, 1024, 28, 4, 128, "CB"),      # 7B-shaped layer
    (64, 2048, 28, 4, 128, "CB"),      # 7B-shaped stack step
    (37, 77, 8, 2, 128, "RB"),         # ragged key tiles
    (256, 300, 40, 8, 128, "RB"),      # 32B-shaped head groups, 256-node tree
    (48, 16384, 32, 8, 128, "CB"),     # long context (Llama-8B-shaped)
    # one workgroup shape each past 4K keys: up to 192 query rows per KV head, and more
    (40, 4500, 8, 2, 64, "CB"),        # 160 rows, hd 64
    (64, 4200, 16, 4, 64, "RB"),       # 256 rows, hd 64
    (64, 4200, 16, 4, 128, "CB"),      # 256 rows, hd 128
    (256, 200, 16, 4, 64, "RB"),       # 4096 (row, KV head) pairs: the wide merge, hd 64
])
def test_tree_attention_parity(T, C, nq, nkv, hd, kind):
    print(f"attention T={T} C={C} nq={nq} nkv={nkv} hd={hd}", flush=True)
    q, kc, vc, kt, vt, par = _attn_case(T, C, nq, nkv, hd, kind, seed=T + C, c_stride=C + 5)
    out, outf, mask = bq.tree_attention(to_bf16(q), to_bf16(kc), to_bf16(vc), to_bf16(kt),
                                        to_bf16(vt), to_dev(par), C, want_f32=True, want_mask=True)
    torch.cuda.synchronize()
    ref = oracle.tree_attention64(oracle.bf16_to_f64(q), oracle.bf16_to_f64(kc),
                                  oracle.bf16_to_f64(vc), oracle.bf16_to_f64(kt),
                                  oracle.bf16_to_f64(vt), par, C)
    assert np.array_equal(host(mask).view(np.uint64), oracle.tree_mask(par))
    assert_close(host(outf), ref, what="attention fp32")
    assert np.array_equal(bf16_bits(out), oracle.f32_to_bf16(host(outf)))


# ------------------------------------------------------------------ verification / selection

@pytest.mark.parametrize("R,V", [(1, 7), (16, 1000), (64, 152064), (3, 128256)])
def test_row_argmax_bitexact(R, V):
    rng = np.random.default_rng(R + V)
    lg = np.round(rng.standard_normal((R, V)) * 3).astype(np.float32)   # many ties
    got = host(bq.row_argmax(to_dev(lg)))
    assert np.array_equal(got, oracle.row_argmax(lg))


# Rows of 4096+ elements are split across workgroups and merged: (48, 128256) and
# (64, 152064) take 11 and 8 parts, (3, 50001) 12 parts of an odd-length row (scalar
# loads) with k = 16, (64, 152064, k = 1) the two-entry lists; the short rows one pass.
@pytest.mark.parametrize("R,V,t,k,noise", [(48, 128256, 0.2, 6, True), (48, 128256, 0.6, 6, True),
                                           (64, 152064, 1.0, 6, False), (5, 40, 0.5, 16, True),
                                           (2, 6, 0.2, 6, True), (3, 50001, 0.3, 16, True),
                                           (64, 152064, 0.2, 1, True)])
def test_draft_select_bitexact(R, V, t, k, noise):
    rng = np.random.default_rng(V + k)
    lg = (rng.standard_normal((R, V)) * 2).astype(np.float32)
    lg[:, ::97] = lg[:, :1]                                   # planted ties
    g = gen.gumbel_f32(R, V, seed=k) if noise else None
    inv_t = np.float32(1.0) / np.float32(t)
    got = host(bq.draft_select(to_dev(lg), None if g is None else to_dev(g), inv_t, k))
    assert np.array_equal(got, oracle.draft_select(lg, g, inv_t, k))


@pytest.mark.parametrize("where", ["first", "last", "spread"])
def test_draft_select_split_extremes(where):
    """All k winners inside one part (first or last), or one per part: the merge must take
    every candidate a part offers, and the order of equal values across parts is by index."""
    R, V, k = 4, 152064, 6
    rng = np.random.default_rng(7)
    lg = (rng.standard_normal((R, V))).astype(np.float32)
    if where == "first":
        lg[:, 3:3 + k] = 50.0                     # k equal winners in part 0: by index
    elif where == "last":
        lg[:, V - k:] = np.arange(k, dtype=np.float32)[::-1] + 40.0
    else:
        idx = np.linspace(0, V - 1, k).astype(int)
        lg[:, idx] = 45.0                         # equal values in different parts
    got = host(bq.draft_select(to_dev(lg), None, np.float32(1.0), k))
    want = oracle.draft_select(lg, None, np.float32(1.0), k)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kind,T,L_star", [("CB", 64, 27), ("CB", 48, 0), ("RB", 256, 5),
                                           ("R", 16, 3), ("CB", 64, 48)])
def test_tree_accept_bitexact(kind, T, L_star):
    V = 5000
    par = gen.tree_parents(T, kind, seed=T)
    tok = gen.tree_tokens(par, V, seed=T)
    lg = gen.target_logits(par, tok, V, L_star, seed=T)
    tgt = oracle.row_argmax(lg)
    path, ln, bonus = bq.tree_accept(to_dev(par), to_dev(tok), to_dev(tgt))
    torch.cuda.synchronize()
    p_o, L_o, b_o = oracle.accept(par, tok, tgt)
    L = int(host(ln)[0])
    assert L == L_o
    assert host(path)[:L].tolist() == p_o and np.all(host(path)[L:] == -1)
    assert int(host(bonus)[0]) == b_o


def test_tree_accept_small_trees_exhaustive():
    from tests.test_oracle_tree import all_trees
    rng = np.random.default_rng(0)
    for T in range(1, 7):
        for par in all_trees(T):
            tok = rng.integers(0, 3, T).astype(np.int32)
            tgt = rng.integers(0, 3, T).astype(np.int32)
            path, ln, bonus = bq.tree_accept(to_dev(par), to_dev(tok), to_dev(tgt))
            p_o, L_o, b_o = oracle.accept(par, tok, tgt)
            assert int(host(ln)[0]) == L_o and host(path)[:L_o].tolist() == p_o
            assert int(host(bonus)[0]) == b_o
