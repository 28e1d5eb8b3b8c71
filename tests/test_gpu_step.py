"""Parity of the whole substitute-draft step (ss_draft_tree_step) with the oracle.

One layer is compared with the oracle's fp64 layer from the same bf16 hidden input
(tolerance: rel-L2 <= 1e-2, max-abs <= 2e-2 * max(1, rms(ref)) plus, for outputs stored
in bf16, the storage rounding of half a bf16 ulp of each reference value); the tree K/V
it writes are compared too. Small stacks with an LM head are compared end to end, including the
logits of selected rows. Weights run as plain int4, tiled int4 (the draft) and dense bf16 (the
target's verify pass).
"""

import types

import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests.gpu_util import assert_close, bf16_bits, host, to_bf16, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_quantized_draft_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def make_layer(cfg, li, C, seed=0, random_norm=True, kind="int4"):
    """Oracle-side weights (bf16 bits and their quantization) and the device copies
    (kind "int4": (qweight, scale, zero) tuples; "tiled": the tiled layout of the same
    codes; "bf16": dense weights)."""
    shapes = {"qkv": ((cfg.nq + 2 * cfg.nkv) * cfg.hd, cfg.H), "o": (cfg.H, cfg.nq * cfg.hd),
              "gate_up": (2 * cfg.I, cfg.H), "down": (cfg.H, cfg.I)}
    o_lw, d_lw = {}, {}
    for name, (N, K) in shapes.items():
        w = gen.weight_bf16(N, K, 0.02, seed=seed, cid=cfg.cid, layer=li, slot=gen.SLOT[name])
        if kind in ("int4", "tiled"):
            q, s, z = oracle.quantize(w)
            o_lw[name] = (q, s, z)
            d_lw[name] = (to_dev(oracle.pack_int4(q)), to_dev(s), to_dev(z))
            if kind == "tiled":
                d_lw[name] = bq.w4_tile(*d_lw[name])
        else:
            o_lw[name] = w
            d_lw[name] = to_bf16(w)
    for which, key in ((0, "norm1"), (1, "norm2")):
        g = gen.norm_gain_bf16(cfg.H, seed=seed, cid=cfg.cid, layer=li, which=which, random=random_norm)
        o_lw[key] = g
        d_lw[key] = to_bf16(g)
    kc = gen.normal_bf16((cfg.nkv, C, cfg.hd), 1.0, seed, cfg.cid, gen.TID_KC, li)
    vc = gen.normal_bf16((cfg.nkv, C, cfg.hd), 1.0, seed, cfg.cid, gen.TID_VC, li)
    d_lw["k_cache"], d_lw["v_cache"] = to_bf16(kc), to_bf16(vc)
    return o_lw, d_lw, kc, vc


def small_cfg(**kw):
    base = dict(cid=9, H=512, I=1024, nq=8, nkv=2, hd=128, rope_theta=1e6, eps=1e-6)
    base.update(kw)
    return types.SimpleNamespace(**base)


@pytest.mark.parametrize("cfgkw,T,C,kind,wl", [
    (dict(), 48, 256, "CB", "int4"),
    (dict(), 48, 256, "CB", "tiled"),
    (dict(nq=4, nkv=4, hd=64, H=256, I=512), 17, 100, "R", "int4"),
    (dict(nq=4, nkv=4, hd=64, H=256, I=512), 17, 100, "R", "tiled"),
    (dict(H=3584, I=18944, nq=28, nkv=4, hd=128, cid=2), 48, 1024, "CB", "int4"),   # Qwen2.5-7B-shaped layer
    (dict(H=3584, I=18944, nq=28, nkv=4, hd=128, cid=2), 64, 2048, "CB", "tiled"),
    (dict(nq=4, nkv=4, hd=64, H=256, I=512), 1, 0, "R", "tiled"),       # root only, no prefix
    (dict(nq=4, nkv=2, hd=64, H=256, I=512), 256, 64, "RB", "tiled"),   # largest tree: 4 token blocks
    (dict(H=3584, I=18944, nq=28, nkv=4, hd=128, cid=2), 64, 2048, "CB", "bf16"),   # target verify layer
])
def test_one_layer_parity(cfgkw, T, C, kind, wl):
    cfg = small_cfg(**cfgkw)
    print(f"layer H={cfg.H} I={cfg.I} T={T} C={C} weights={wl}", flush=True)
    o_lw, d_lw, kc, vc = make_layer(cfg, 0, C, seed=1, kind=wl)
    par = gen.tree_parents(T, kind, seed=T)
    h_in = gen.normal_bf16((T, cfg.H), 1.0, 1, cfg.cid, gen.TID_HIDDEN)
    model = bq.SubstituteModel(cfg.H, cfg.I, cfg.nq, cfg.nkv, cfg.hd, [d_lw],
                               rope_theta=cfg.rope_theta, rms_eps=cfg.eps)
    dev = torch.device("cuda:0")
    tk = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev)]
    tv = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev)]
    hout = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
    model.draft_tree_step(to_dev(par), C, tk, tv, hidden_in=to_bf16(h_in), hidden_out=hout)
    torch.cuda.synchronize()
    ref_h, ref_k, ref_v = oracle.layer64(oracle.bf16_to_f64(h_in), o_lw, kc, vc, par, C, cfg)
    assert_close(oracle.bf16_to_f64(bf16_bits(hout)), ref_h, scale_abs=True, bf16_out=True, what="layer hidden")
    assert_close(oracle.bf16_to_f64(bf16_bits(tk[0])), ref_k, scale_abs=True, bf16_out=True, what="tree K")
    assert_close(oracle.bf16_to_f64(bf16_bits(tv[0])), ref_v, scale_abs=True, bf16_out=True, what="tree V")


@pytest.mark.parametrize("L,T,C,V,kind,rows,wl", [(2, 16, 64, 4096, "R", None, "int4"),
                                                  (3, 64, 128, 2048, "CB", [0, 5, 63, 5], "int4"),
                                                  (3, 64, 128, 2048, "CB", [0, 5, 63, 5], "tiled"),
                                                  (3, 64, 128, 2048, "CB", None, "bf16")])
def test_small_stack_with_lm_head(L, T, C, V, kind, rows, wl):
    cfg = small_cfg(cid=8, H=256, I=512, nq=4, nkv=2, hd=64)
    layers = [make_layer(cfg, li, C, seed=2, kind=wl) for li in range(L)]
    embed = gen.normal_bf16((V, cfg.H), 1.0, 2, cfg.cid, gen.TID_EMBED)
    head = gen.normal_bf16((V, cfg.H), 0.05, 2, cfg.cid, gen.TID_LMHEAD)
    fnorm = gen.norm_gain_bf16(cfg.H, seed=2, cid=cfg.cid, layer=99, random=True)
    par = gen.tree_parents(T, kind, seed=3)
    tok = gen.tree_tokens(par, V, seed=3)
    model = bq.SubstituteModel(cfg.H, cfg.I, cfg.nq, cfg.nkv, cfg.hd, [d for _, d, _, _ in layers],
                               V=V, embed=to_bf16(embed), final_norm=to_bf16(fnorm),
                               lm_head=to_bf16(head), rope_theta=cfg.rope_theta, rms_eps=cfg.eps)
    dev = torch.device("cuda:0")
    tk = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    tv = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    R = T if rows is None else len(rows)
    logits = torch.empty((R, V), dtype=torch.float32, device=dev)
    hout = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
    model.draft_tree_step(to_dev(par), C, tk, tv, tokens=to_dev(tok), hidden_out=hout, logits=logits,
                          logit_rows=None if rows is None else to_dev(np.array(rows, dtype=np.int32)))
    torch.cuda.synchronize()
    ref_h, ref_lg = oracle.stack64(tok, par, C, embed, [o for o, _, _, _ in layers],
                                   [kc for _, _, kc, _ in layers], [vc for _, _, _, vc in layers],
                                   fnorm, head, cfg, logit_rows=rows)
    assert_close(oracle.bf16_to_f64(bf16_bits(hout)), ref_h, scale_abs=True, bf16_out=True, what="stack hidden")
    assert_close(host(logits), ref_lg, scale_abs=True, what="logits")


def test_step_rejects_bad_tree_under_debug_sync():
    # validation on the host side of the binding: a non-topological parent array
    with pytest.raises(bq.SubspecError):
        bq.tree_validate([-1, 2, 0])


def test_tiled_step_is_bit_identical_to_plain():
    """The tiled weights change where the codes live, not the arithmetic: the whole
    step's outputs match the plain layout's bit for bit (7B-shaped layer, T = 64)."""
    cfg = small_cfg(H=3584, I=18944, nq=28, nkv=4, hd=128, cid=2)
    T, C = 64, 512
    _, d_plain, _, _ = make_layer(cfg, 0, C, seed=5)
    d_tiled = dict(d_plain)
    for name in ("qkv", "o", "gate_up", "down"):
        d_tiled[name] = bq.w4_tile(*d_plain[name])
    par = to_dev(gen.tree_parents(T, "CB", seed=5))
    h_in = to_bf16(gen.normal_bf16((T, cfg.H), 1.0, 5, cfg.cid, gen.TID_HIDDEN))
    dev = torch.device("cuda:0")
    outs = []
    for lw in (d_plain, d_tiled):
        model = bq.SubstituteModel(cfg.H, cfg.I, cfg.nq, cfg.nkv, cfg.hd, [lw],
                                   rope_theta=cfg.rope_theta, rms_eps=cfg.eps)
        tk = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev)]
        tv = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev)]
        hout = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
        model.draft_tree_step(par, C, tk, tv, hidden_in=h_in, hidden_out=hout)
        torch.cuda.synchronize()
        outs.append((hout, tk[0], tv[0]))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
