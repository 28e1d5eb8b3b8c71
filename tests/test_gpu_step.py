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
    # Llama-3.1-8B-shaped long-context layer (theta 5e5, eps 1e-5), the workload's tree and prefix
    (dict(H=4096, I=14336, nq=32, nkv=8, hd=128, cid=5, rope_theta=5e5, eps=1e-5), 48, 16384, "CB", "tiled"),
    # Qwen2.5-32B-shaped layer at the 256-token random-branching tree, C = 4096
    (dict(H=5120, I=27648, nq=40, nkv=8, hd=128, cid=4), 256, 4096, "RB", "tiled"),
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


def test_tree_validate_rejects_non_topological_parents_on_the_host():
    with pytest.raises(bq.SubspecError):
        bq.tree_validate([-1, 2, 0])


_DEBUG_SYNC_SCRIPT = r"""
import json, sys, torch
sys.path.insert(0, sys.argv[1])
import bit_quantized_draft_amd as bq
from bit_quantized_draft_amd._lib import STATUS_NAMES
torch.manual_seed(0)
dev = torch.device("cuda:0")
H, I, nq, nkv, hd, V, T, cs = 128, 256, 2, 1, 64, 64, 4, 16
r = lambda *s: (0.05 * torch.randn(*s)).to(torch.bfloat16).to(dev)
ly = dict(qkv=r((nq + 2 * nkv) * hd, H), o=r(H, nq * hd), gate_up=r(2 * I, H), down=r(H, I),
          norm1=r(H) + 1, norm2=r(H) + 1, k_cache=r(nkv, cs, hd), v_cache=r(nkv, cs, hd))
m = bq.SubstituteModel(H, I, nq, nkv, hd, [ly], V=V, embed=r(V, H), final_norm=r(H) + 1, lm_head=r(V, H))
tk = [torch.empty((nkv, T, hd), dtype=torch.bfloat16, device=dev)]
tv = [torch.empty((nkv, T, hd), dtype=torch.bfloat16, device=dev)]
i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=dev)
good_par, good_tok = i32([-1, 0, 0, 1]), i32([1, 2, 3, 4])
cases = {"ok": (good_par, good_tok, None),
         "bad_tree": (i32([-1, 2, 0, 1]), good_tok, None),
         "bad_token": (good_par, i32([1, 2, V, 4]), None),
         "bad_logit_row": (good_par, good_tok, i32([0, T]))}
out = {}
for name, (par, tok, rows) in cases.items():
    print("case", name, flush=True)
    R = T if rows is None else rows.numel()
    logits = torch.empty((R, V), dtype=torch.float32, device=dev)
    try:
        m.draft_tree_step(par, 8, tk, tv, tokens=tok, logits=logits, logit_rows=rows)
        torch.cuda.synchronize()
        out[name] = "SS_OK"
    except bq.SubspecError as e:
        out[name] = STATUS_NAMES.get(e.status, str(e.status)) + " " + str(e)
print("RESULT " + json.dumps(out), flush=True)
"""


def test_step_error_word_under_debug_sync():
    """With SS_DEBUG_SYNC=1 (set in a fresh process before any GPU call) the step reports
    the device-side checks: a non-topological parent array (SS_ERR_BAD_TREE), a token id
    outside [0, V) and a logit row outside [0, T) (SS_ERR_INVALID_ARG). The kernels that
    detect them are bounds-safe on such input (the mask walk is bounded, the embedding and
    the final norm write zeros for the bad rows), so nothing faults."""
    import json
    import os
    import subprocess
    import sys
    env = dict(os.environ, SS_DEBUG_SYNC="1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, "-c", _DEBUG_SYNC_SCRIPT, root], env=env, capture_output=True, text=True,
                       timeout=240)
    print(p.stdout[-2000:], p.stderr[-2000:], flush=True)
    assert p.returncode == 0
    res = json.loads([l for l in p.stdout.splitlines() if l.startswith("RESULT ")][-1][7:])
    assert res["ok"] == "SS_OK"
    assert res["bad_tree"].startswith("SS_ERR_BAD_TREE")
    assert res["bad_token"].startswith("SS_ERR_INVALID_ARG") and "token id" in res["bad_token"]
    assert res["bad_logit_row"].startswith("SS_ERR_INVALID_ARG") and "logit row" in res["bad_logit_row"]


def test_28_layer_stack_drift():
    """Drift over the depth of a 7B-sized stack: 28 substitute layers (a narrower width,
    H=512, I=1536, so that the fp64 oracle stays quick) with the LM head, T=64 CB tree,
    C=256. Reported (DRIFT line) and held to a bound twice the single-layer one; the
    per-layer parity tests above carry the real gate."""
    L, T, C, V = 28, 64, 256, 4096
    cfg = small_cfg(cid=10, H=512, I=1536, nq=8, nkv=2, hd=64)
    print(f"stack drift L={L} T={T} C={C} H={cfg.H}", flush=True)
    layers = [make_layer(cfg, li, C, seed=4, kind="tiled") for li in range(L)]
    embed = gen.normal_bf16((V, cfg.H), 1.0, 4, cfg.cid, gen.TID_EMBED)
    head = gen.normal_bf16((V, cfg.H), 0.05, 4, cfg.cid, gen.TID_LMHEAD)
    fnorm = gen.norm_gain_bf16(cfg.H, seed=4, cid=cfg.cid, layer=99, random=True)
    par = gen.tree_parents(T, "CB", seed=4)
    tok = gen.tree_tokens(par, V, seed=4)
    model = bq.SubstituteModel(cfg.H, cfg.I, cfg.nq, cfg.nkv, cfg.hd, [d for _, d, _, _ in layers],
                               V=V, embed=to_bf16(embed), final_norm=to_bf16(fnorm),
                               lm_head=to_bf16(head), rope_theta=cfg.rope_theta, rms_eps=cfg.eps)
    dev = torch.device("cuda:0")
    tk = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    tv = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    logits = torch.empty((T, V), dtype=torch.float32, device=dev)
    hout = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
    model.draft_tree_step(to_dev(par), C, tk, tv, tokens=to_dev(tok), hidden_out=hout, logits=logits)
    torch.cuda.synchronize()
    ref_h, ref_lg = oracle.stack64(tok, par, C, embed, [o for o, _, _, _ in layers],
                                   [kc for _, _, kc, _ in layers], [vc for _, _, _, vc in layers],
                                   fnorm, head, cfg)
    got_h = oracle.bf16_to_f64(bf16_bits(hout))
    got_lg = host(logits).astype(np.float64)
    rel = lambda g, r: float(np.linalg.norm(g - r) / np.linalg.norm(r))
    agree = float(np.mean(np.argmax(got_lg, axis=1) == np.argmax(ref_lg, axis=1)))
    print(f"DRIFT 28 layers: hidden rel-L2 {rel(got_h, ref_h):.3e}, logits rel-L2 {rel(got_lg, ref_lg):.3e}, "
          f"top-1 agreement {agree:.3f}", flush=True)
    assert_close(got_h, ref_h, rel_l2=2e-2, max_abs=4e-2, scale_abs=True, bf16_out=True, what="28-layer hidden")
    assert_close(got_lg, ref_lg, rel_l2=2e-2, max_abs=4e-2, scale_abs=True, what="28-layer logits")


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
