#!/usr/bin/env python3
"""Throughput of the SubSpec substitute-draft hot path on one MI355X.

Workload: the full 28-layer Qwen2.5-7B-shaped substitute stack (hidden 3584, MLP 18944,
28/4 heads, head dim 128, vocab 152064), random-init int4 group-64 substitute weights
quantized on the GPU from random-init bf16 weights, a 64-token chain-plus-branches draft
tree of depth 48, KV context 2048. One measured step is one decode cycle of that
workload: 48 draft expansion steps over the 64 tree slots (substitute stack + bf16 LM
head + greedy top-6 child selection each), one bf16-weight target verify pass over the
tree, row argmax of the seeded target logits, the greedy acceptance walk and the commit of
the accepted tokens' K/V to the cache, with the accept length read back by the host.

Printed: one JSON line. `value` is draft-tree tokens per second (48 * 64 tree tokens per
cycle over the cycle time). The `roofline` object covers the dominant kernel, the fused
int4 gate_up + SwiGLU GEMM, timed with HIP events on its own stream; `cpu_baseline` is the
CPU oracle on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DRAFT_STEPS = 48
TOPK = 6
DRAFT_TEMP = 0.2
L_STAR = 27
ROOT_TOKEN = 1234


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (debug only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run only the dominant kernel over rotated weights, then a 256 MiB "
                         "negation as the counter calibration (for rocprofv3 --pmc passes)")
    ap.add_argument("--attn-probe", action="store_true",
                    help="run only the tree attention (attention kernel + split merge) at the "
                         "Qwen2.5-7B (T=64, C=2048) and Llama-3.1-8B (T=48, C=16384) shapes over "
                         "rotated KV caches, then the 256 MiB negation (for rocprofv3 passes)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="MFMA utilisation at the large-tree workload: the four tiled int4 linears "
                         "of a Qwen2.5-32B-shaped layer at T=256, timed against the dense bf16 peak")
    ap.add_argument("--extra-steps", type=int, default=10,
                    help="timed step replays of the Qwen2.5-32B and Llama-3.1-8B shaped stacks")
    ap.add_argument("--no-extra", action="store_true", help="skip the 32B and 8B stack steps")
    ap.add_argument("--extra-only", type=int, choices=(4, 5), default=None,
                    help="run only the step of workload 4 (Qwen2.5-32B stack) or 5 (Llama-3.1-8B "
                         "long-context stack) and print its entry (for kernel traces)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of "
                         "--pmc-probe into the traffic summary under profiles/ (CPU only)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ model construction

def build_model(cfg, dev, n_layers):
    import torch
    import bit_quantized_draft_amd as bq
    from synth import gen
    from synth.configs import layer_shapes
    torch.manual_seed(0)
    draft_layers, target_layers = [], []
    ones = torch.ones(cfg.H, dtype=torch.bfloat16, device=dev)
    for li in range(n_layers):
        d, t = {}, {}
        for name, N, K in layer_shapes(cfg):
            w = gen.torch_normal_bf16((N, K), cfg.w_std, 0, cfg.cid, gen.TID_W, li * 16 + gen.SLOT[name], dev)
            d[name] = bq.w4_tile(*bq.quantize_substitute(w))   # the tiled layout the GEMMs stream
            t[name] = w
        # C committed rows, plus room for the T rows a cycle may commit
        pad = torch.zeros((cfg.nkv, cfg.T, cfg.hd), dtype=torch.bfloat16, device=dev)
        kc = torch.cat([gen.torch_normal_bf16((cfg.nkv, cfg.C, cfg.hd), 1.0, 0, cfg.cid, gen.TID_KC, li, dev), pad], 1)
        vc = torch.cat([gen.torch_normal_bf16((cfg.nkv, cfg.C, cfg.hd), 1.0, 0, cfg.cid, gen.TID_VC, li, dev), pad], 1)
        for x in (d, t):
            x.update(norm1=ones, norm2=ones, k_cache=kc, v_cache=vc)
        draft_layers.append(d)
        target_layers.append(t)
        if li % 7 == 0:
            log(f"  layer {li} built")
    embed = gen.torch_normal_bf16((cfg.V, cfg.H), cfg.w_std, 0, cfg.cid, gen.TID_EMBED, 0, dev)
    head = gen.torch_normal_bf16((cfg.V, cfg.H), cfg.w_std, 0, cfg.cid, gen.TID_LMHEAD, 0, dev)
    kw = dict(V=cfg.V, embed=embed, final_norm=ones, lm_head=head, rope_theta=cfg.rope_theta,
              rms_eps=cfg.eps)
    draft = bq.SubstituteModel(cfg.H, cfg.I, cfg.nq, cfg.nkv, cfg.hd, draft_layers, **kw)
    target = bq.SubstituteModel(cfg.H, cfg.I, cfg.nq, cfg.nkv, cfg.hd, target_layers, **kw)
    torch.cuda.synchronize()
    return draft, target


def algorithmic_bytes_step(cfg, n_layers, logit_rows=None):
    """Bytes one draft step must move: int4 weights + fp16 scale/zero, prefix KV once per
    layer, activations at kernel boundaries, bf16 LM head and the fp32 logits of the rows
    that need them (all T, or the expansion frontier's logit_rows)."""
    from synth.configs import layer_shapes
    T, C = cfg.T, cfg.C
    w_params = sum(N * K for _, N, K in layer_shapes(cfg))
    per_layer = 0.5625 * w_params
    per_layer += 2 * cfg.nkv * C * cfg.hd * 2                        # prefix K and V, bf16
    qkvN = (cfg.nq + 2 * cfg.nkv) * cfg.hd
    per_layer += T * (cfg.H * 2 * 2 + qkvN * 2 * 2 + cfg.nq * cfg.hd * 2 * 2 + cfg.I * 2 * 2)
    per_layer += 2 * cfg.nkv * T * cfg.hd * 2                        # tree K/V written
    rows = T if logit_rows is None else logit_rows
    head = cfg.V * cfg.H * 2 + rows * cfg.V * 4 + rows * cfg.H * 2
    return n_layers * per_layer + head


# ------------------------------------------------------------------ the 32B and 8B stacks

def step_flops(cfg, n_layers):
    """Multiply-add flops of one draft step: the four linears over all T tree tokens, the
    tree attention (scores and values over C + T keys) and the LM head."""
    from synth.configs import layer_shapes
    T, C = cfg.T, cfg.C
    lin = sum(N * K for _, N, K in layer_shapes(cfg))
    per_layer = 2.0 * T * lin + 4.0 * T * (C + T) * cfg.nq * cfg.hd
    return n_layers * per_layer + (2.0 * T * cfg.V * cfg.H if cfg.V else 0.0)


def extra_config(cid, args, dev):
    """One draft step of workload cid (4: 64-layer Qwen2.5-32B-shaped stack, T = 256, C =
    4096; 5: 32-layer Llama-3.1-8B-shaped stack, T = 48, C = 16384, bf16 LM head and child
    selection at temperatures 0.2 and 0.6), captured in a HIP graph, checked against its
    eager run and timed over args.extra_steps replays with HIP events."""
    import torch
    import bit_quantized_draft_amd as bq
    from synth import gen
    from synth.configs import get_config, layer_shapes
    cfg = get_config(cid)
    L, T, C, V = cfg.L, cfg.T, cfg.C, cfg.V
    log(f"building {cfg.name}: {L} layers, T={T}, C={C}")
    ones = torch.ones(cfg.H, dtype=torch.bfloat16, device=dev)
    layers = []
    for li in range(L):
        d = {}
        for name, N, K in layer_shapes(cfg):
            w = gen.torch_normal_bf16((N, K), cfg.w_std, 0, cfg.cid, gen.TID_W, li * 16 + gen.SLOT[name], dev)
            d[name] = bq.w4_tile(*bq.quantize_substitute(w))
            del w
        kc = gen.torch_normal_bf16((cfg.nkv, C, cfg.hd), 1.0, 0, cfg.cid, gen.TID_KC, li, dev)
        vc = gen.torch_normal_bf16((cfg.nkv, C, cfg.hd), 1.0, 0, cfg.cid, gen.TID_VC, li, dev)
        d.update(norm1=ones, norm2=ones, k_cache=kc, v_cache=vc)
        layers.append(d)
        if li % 16 == 0:
            log(f"  layer {li} built")
    kw = dict(rope_theta=cfg.rope_theta, rms_eps=cfg.eps)
    if V:
        kw.update(V=V, embed=gen.torch_normal_bf16((V, cfg.H), cfg.w_std, 0, cfg.cid, gen.TID_EMBED, 0, dev),
                  final_norm=ones,
                  lm_head=gen.torch_normal_bf16((V, cfg.H), cfg.w_std, 0, cfg.cid, gen.TID_LMHEAD, 0, dev))
    model = bq.SubstituteModel(cfg.H, cfg.I, cfg.nq, cfg.nkv, cfg.hd, layers, **kw)
    par_np = gen.tree_parents(T, cfg.tree, cfg.depth_cap, seed=0, cid=cfg.cid)
    par = torch.from_numpy(par_np).to(dev)
    # with a vocabulary the step starts from token ids (embedding gather); without one (the
    # 32B workload names no head) it starts from seeded hidden states
    tok = torch.from_numpy(gen.tree_tokens(par_np, V, seed=0, cid=cfg.cid)).to(dev) if V else None
    h_in = None if V else gen.torch_normal_bf16((T, cfg.H), 1.0, 0, cfg.cid, gen.TID_HIDDEN, 0, dev)
    tk = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    tv = [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    hout = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((T, V), dtype=torch.float32, device=dev) if V else None
    ws = torch.empty(model.workspace_bytes(T, C), dtype=torch.uint8, device=dev)
    temps = cfg.temps if V else ()
    kids = {t: torch.empty((T, TOPK), dtype=torch.int32, device=dev) for t in temps}
    ws_s = torch.empty(max(1, bq.draft_select_workspace_bytes(T, V, TOPK)) if V else 1, dtype=torch.uint8,
                       device=dev)
    inv = {t: float(np.float32(1.0) / np.float32(t)) for t in temps}

    def step():
        model.draft_tree_step(par, C, tk, tv, tokens=tok, hidden_in=h_in, hidden_out=hout, logits=logits,
                              workspace=ws)

    def select(t):
        bq.draft_select(logits, None, inv[t], TOPK, out=kids[t], workspace=ws_s)

    step()
    for t in temps:
        select(t)
    torch.cuda.synchronize()
    ref_h = hout.clone()
    ref_k = {t: kids[t].clone() for t in temps}
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g_step = torch.cuda.CUDAGraph()
    g_sel = {t: torch.cuda.CUDAGraph() for t in temps}
    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g_step, stream=stream):
            step()
        for t in temps:
            with torch.cuda.graph(g_sel[t], stream=stream):
                select(t)
    torch.cuda.synchronize()
    for _ in range(2):
        g_step.replay()
        for t in temps:
            g_sel[t].replay()
        torch.cuda.synchronize()
        assert torch.equal(hout, ref_h), f"{cfg.name}: graph replay differs from the eager step"
        for t in temps:
            assert torch.equal(kids[t], ref_k[t]), f"{cfg.name}: selection replay differs at t={t}"
        step()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g_step.replay()   # steady state
    e0.record()
    for _ in range(args.extra_steps):
        g_step.replay()
    e1.record(); torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.extra_steps
    ms_sel = {}
    for t in temps:
        e0.record()
        for _ in range(args.extra_steps):
            g_sel[t].replay()
        e1.record(); torch.cuda.synchronize()
        ms_sel[t] = e0.elapsed_time(e1) / args.extra_steps
    alg = algorithmic_bytes_step(cfg, L)
    flops = step_flops(cfg, L)
    entry = {"workload": f"{cfg.name}: {L}-layer substitute stack, T={T} tree tokens ({cfg.tree} tree), C={C}"
                         + (f", bf16 LM head (vocab {V}) + child selection" if V else ""),
             "step_ms": round(ms_step, 4), "tree_tokens_per_s": round(T / (ms_step * 1e-3), 1),
             "alg_bytes": int(alg), "hbm_frac": round(alg / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
             "mfma_flops": int(flops), "mfma_frac": round(flops / (ms_step * 1e-3) / (MFMA_PEAK_TFLOPS * 1e12), 4),
             "steps_timed": args.extra_steps}
    for t in temps:
        entry[f"select_t{t}_ms"] = round(ms_sel[t], 4)
        entry[f"tree_tokens_per_s_t{t}"] = round(T / ((ms_step + ms_sel[t]) * 1e-3), 1)
    del layers, model, ws
    torch.cuda.empty_cache()
    return entry


# ------------------------------------------------------------------ CPU oracle baseline

def cpu_baseline(cfg, n_layers, R):
    """The oracle timed on the host, as a whole decode cycle like the GPU's `value`: 48
    draft steps (n_layers substitute layers + the LM head on R frontier rows) and one
    verify pass (n_layers bf16 target layers + the LM head on all T rows). Each layer kind
    is timed once per repeat (3 repeats: mean and std); the LM head on 1/16 of its rows,
    scaled. Also one 7B-shaped substitute layer at T=48, C=1024 (the one-layer workload)
    and the 512-wide linear + attention case (T=16, C=128) on one thread."""
    import oracle
    from synth import gen
    from synth.configs import get_config, layer_shapes
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    T, C = cfg.T, cfg.C
    log("cpu baseline: generating and quantizing one layer with the oracle (untimed)")
    sub, tgt = {}, {}
    for name, N, K in layer_shapes(cfg):
        w = gen.weight_bf16(N, K, cfg.w_std, seed=0, cid=cfg.cid, layer=0, slot=gen.SLOT[name])
        sub[name] = oracle.quantize(w)
        tgt[name] = w
    for lw in (sub, tgt):
        lw["norm1"] = gen.norm_gain_bf16(cfg.H)
        lw["norm2"] = gen.norm_gain_bf16(cfg.H)
    kc = gen.normal_bf16((cfg.nkv, C, cfg.hd), 1.0, 0, cfg.cid, gen.TID_KC, 0)
    vc = gen.normal_bf16((cfg.nkv, C, cfg.hd), 1.0, 0, cfg.cid, gen.TID_VC, 0)
    par = gen.tree_parents(T, cfg.tree, seed=0, cid=cfg.cid)
    h = oracle.bf16_to_f64(gen.normal_bf16((T, cfg.H), 1.0, 0, cfg.cid, gen.TID_HIDDEN))
    head_rows = cfg.V // 16
    head = oracle.bf16_to_f64(gen.normal_bf16((head_rows, cfg.H), cfg.w_std, 0, cfg.cid, gen.TID_LMHEAD))

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    values, parts = [], []
    for _ in range(3):
        t_sub = timed(lambda: oracle.layer64(h, sub, kc, vc, par, C, cfg))
        t_tgt = timed(lambda: oracle.layer64(h, tgt, kc, vc, par, C, cfg))
        x = oracle.rmsnorm64(h, np.ones(cfg.H), cfg.eps)
        t_head = timed(lambda: oracle.matmul64(x, head)) * (cfg.V / head_rows)   # all T rows
        cycle = cfg.steps * (n_layers * t_sub + t_head * R / T) + (n_layers * t_tgt + t_head)
        values.append(cfg.steps * T / cycle)
        parts.append((t_sub, t_tgt, t_head, cycle))
    t_sub, t_tgt, t_head, cycle = (float(np.mean([p[i] for p in parts])) for i in range(4))
    single = {}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            c2 = get_config(2)
            par2 = gen.tree_parents(c2.T, c2.tree, seed=0, cid=c2.cid)
            h2 = h[:c2.T]
            t2 = timed(lambda: oracle.layer64(h2, sub, kc[:, :c2.C], vc[:, :c2.C], par2, c2.C, cfg))
            single["qwen2.5-7b-layer (T=48, C=1024)"] = {"tree_tokens_per_s": round(c2.T / t2, 3),
                                                         "seconds": round(t2, 3)}
            c1 = get_config(1)
            w1 = oracle.quantize(gen.weight_bf16(c1.H, c1.H, 0.02, seed=0, cid=c1.cid))
            x1 = gen.normal_bf16((c1.T, c1.H), 1.0, 0, c1.cid, gen.TID_X)
            t1 = timed(lambda: oracle.w4a16_matmul64(x1, *w1))
            single["linear512 (T=16)"] = {"tree_tokens_per_s": round(c1.T / t1, 3), "seconds": round(t1, 5)}
    return {"value": float(np.mean(values)), "unit": "draft-tree tokens/s", "cores": int(threads),
            "kind": "oracle", "std": float(np.std(values)), "repeats": len(values),
            "single_thread": single,
            "sample": (f"one decode cycle estimated from timed parts, like the GPU value: "
                       f"{cfg.steps} x ({n_layers} substitute layers at {t_sub:.2f} s + the LM head "
                       f"on {R} frontier rows) + one verify pass ({n_layers} bf16 target layers at "
                       f"{t_tgt:.2f} s + the LM head on all {T} rows, {t_head:.2f} s scaled from 1/16 "
                       f"of its rows); T={T}, C={C}, fp64; {cycle:.0f} s per cycle; mean of 3 repeats")}


# ------------------------------------------------------------------ profiling data

def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("gemm_w4.hip", "gemm_w4_kernel.h", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "bit_quantized_draft_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


PMC_JSON = os.path.join(ROOT, "profiles", "gate_up_swiglu_qwen7b_T64_pmc.json")
PMC_MD = os.path.join(ROOT, "profiles", "gate_up_swiglu_qwen7b_T64_pmc.md")
CAL_BYTES = 256 << 20          # calibration: fp32 negation reads and writes this many bytes


def gate_up_bytes(cfg, T=None):
    """Algorithmic bytes of one gate_up launch: int4 codes + fp16 scale/zero (0.5625 B per
    weight), bf16 activations in, bf16 SwiGLU output."""
    T = cfg.T if T is None else T
    return 0.5625 * 2 * cfg.I * cfg.H + T * cfg.H * 2 + T * cfg.I * 2


def pmc_probe(args):
    """The dominant kernel alone: tiled gate_up + SwiGLU (int4, T=64) over 8 weight copies in
    rotation (more than the 256 MB Infinity Cache), then the calibration negation."""
    import torch
    import bit_quantized_draft_amd as bq
    from synth import gen
    from synth.configs import get_config
    cfg = get_config(3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rot = []
    for li in range(8):
        w = gen.torch_normal_bf16((2 * cfg.I, cfg.H), cfg.w_std, 0, cfg.cid, gen.TID_W,
                                  li * 16 + gen.SLOT["gate_up"], dev)
        rot.append(bq.w4_tile(*bq.quantize_substitute(w)))
        del w
    x = gen.torch_normal_bf16((cfg.T, cfg.H), 1.0, 0, cfg.cid, gen.TID_X, 0, dev)
    u = torch.empty((cfg.T, cfg.I), dtype=torch.bfloat16, device=dev)
    a = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for r in range(args.kernel_reps):
        for tw in rot:
            bq.w4a16_gate_up_swiglu_tiled(x, tw, out=u)
    torch.cuda.synchronize()
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(f"pmc probe done: {8 * args.kernel_reps} gate_up launches, one {CAL_BYTES >> 20} MiB negation",
          flush=True)


def attn_probe(args):
    """Tree attention alone at two shapes, each over enough KV-cache copies in rotation to
    exceed the 256 MB Infinity Cache (as in the draft step, where a layer's cache was last
    read a whole step earlier): Qwen2.5-7B (28 query / 4 KV heads, T=64 CB tree, C=2048,
    64 copies of 4.3 MB) and Llama-3.1-8B (32 / 8 heads, T=48 CB tree, C=16384, 5 copies of
    67 MB). kernel_reps launches of each, then the calibration negation."""
    import torch
    import bit_quantized_draft_amd as bq
    from synth import gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for name, T, C, nq, nkv, copies, cid in (("qwen2.5-7b", 64, 2048, 28, 4, 64, 3),
                                            ("llama3.1-8b", 48, 16384, 32, 8, 5, 5)):
        hd = 128
        rnd = lambda shape, tid, layer: gen.torch_normal_bf16(shape, 1.0, 0, cid, tid, layer, dev)
        q = rnd((T, nq, hd), gen.TID_Q, 0)
        kv = [(rnd((nkv, C, hd), gen.TID_KC, i), rnd((nkv, C, hd), gen.TID_VC, i)) for i in range(copies)]
        kt = rnd((nkv, T, hd), gen.TID_KT, 0)
        vt = rnd((nkv, T, hd), gen.TID_VT, 0)
        par = torch.from_numpy(gen.tree_parents(T, "CB", seed=0, cid=cid)).to(dev)
        torch.cuda.synchronize()
        for r in range(args.kernel_reps):
            for kc, vc in kv:
                bq.tree_attention(q, kc, vc, kt, vt, par, C)
        torch.cuda.synchronize()
        print(f"attn probe {name}: {args.kernel_reps * copies} launches", flush=True)
        del kv
    a = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(f"attn probe done: one {CAL_BYTES >> 20} MiB negation", flush=True)


MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def mfma_probe(args):
    """The substitute GEMMs of one Qwen2.5-32B-shaped layer at T=256 (the large-tree
    workload, MFMA-bound: 2T/0.5625 = 910 FLOP/B > the 312 FLOP/B ridge), tiled int4
    weights of two layers in rotation (> 256 MB Infinity Cache), each linear timed with
    HIP events on its own stream. Reports TFLOP/s against the dense bf16 MFMA peak."""
    import torch
    import bit_quantized_draft_amd as bq
    from synth import gen
    from synth.configs import get_config, layer_shapes
    cfg = get_config(4)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = cfg.T
    copies = 2
    ws = {}
    for name, N, K in layer_shapes(cfg):
        ws[name] = []
        for li in range(copies):
            w = gen.torch_normal_bf16((N, K), cfg.w_std, 0, cfg.cid, gen.TID_W, li * 16 + gen.SLOT[name], dev)
            ws[name].append(bq.w4_tile(*bq.quantize_substitute(w)))
            del w
    torch.cuda.empty_cache()
    res = {}
    tot_flop, tot_us = 0.0, 0.0
    ks = torch.cuda.Stream()
    for name, N, K in layer_shapes(cfg):
        x = gen.torch_normal_bf16((T, K), 1.0, 0, cfg.cid, gen.TID_X, 0, dev)
        if name == "gate_up":
            out = torch.empty((T, N // 2), dtype=torch.bfloat16, device=dev)
            run = lambda tw: bq.w4a16_gate_up_swiglu_tiled(x, tw, out=out)
        else:
            run = lambda tw: bq.w4a16_linear_tiled(x, tw, want_bf16=False)
        with torch.cuda.stream(ks):
            for tw in ws[name]:
                run(tw)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(ks)
            n = 0
            for _ in range(args.kernel_reps):
                for tw in ws[name]:
                    run(tw)
                    n += 1
            e1.record(ks)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        flop = 2.0 * T * N * K
        tot_flop += flop
        tot_us += us
        res[name] = {"N": N, "K": K, "us": round(us, 2), "tflops": round(flop / us / 1e6, 1),
                     "mfma_frac": round(flop / us / 1e6 / MFMA_PEAK_TFLOPS, 4),
                     "hbm_gbs": round(0.5625 * N * K / us / 1e3, 1)}
    line = {"probe": "mfma", "workload": f"{cfg.name} layer GEMMs (tiled int4), T={T}", "peak_tflops": MFMA_PEAK_TFLOPS,
            "layer_us": round(tot_us, 2), "layer_tflops": round(tot_flop / tot_us / 1e6, 1),
            "layer_mfma_frac": round(tot_flop / tot_us / 1e6 / MFMA_PEAK_TFLOPS, 4), "gemms": res}
    print(json.dumps(line), flush=True)


def _counter_rows(folder, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Kernel_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def pmc_summary(fetch_dir, write_dir):
    from synth.configs import get_config
    cfg = get_config(3)
    out = {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(folder, counter)
        gemm = [v for (_, k), v in rows.items() if "w4k_kernel" in k]
        red = [v for (_, k), v in rows.items() if "w4_reduce_kernel" in k]
        cal = [v for (_, k), v in rows.items() if "neg" in k.lower()]
        if not gemm or len(cal) != 1:
            raise SystemExit(f"{counter}: expected gate_up dispatches and one calibration dispatch, "
                             f"found {len(gemm)} and {len(cal)}")
        factor = CAL_BYTES / (cal[0] * 1024.0)
        g = sum(gemm) / len(gemm) * 1024.0 * factor
        r = (sum(red) / len(red) * 1024.0 * factor) if red else 0.0
        out[counter] = {"kib_per_dispatch_gemm": sum(gemm) / len(gemm),
                        "kib_per_dispatch_reduce": (sum(red) / len(red)) if red else 0.0,
                        "kib_calibration": cal[0], "scale_factor": factor,
                        "bytes_gemm": g, "bytes_reduce": r, "dispatches": len(gemm)}
    alg = gate_up_bytes(cfg)
    hbm = sum(v["bytes_gemm"] + v["bytes_reduce"] for v in out.values())
    d = {"kernel": "w4k_kernel<TT=4, EPI_SWIGLU, tiled> (tiled int4 gate_up 37888x3584, T=64)",
         "source_hash": kernel_source_hash(), "alg_bytes_per_launch": int(alg),
         "hbm_bytes_per_launch": int(hbm), "hbm_over_alg": round(hbm / alg, 4), "counters": out}
    with open(PMC_JSON, "w") as fh:
        json.dump(d, fh, indent=1)
    lines = [
        "# Tiled int4 gate_up + SwiGLU (g64, 37888 x 3584, T=64): HBM traffic from PMC counters",
        "",
        "Commands (from the repository root on the GPU host; each pass its own run):",
        "",
        "```",
        "cd /tmp && timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o run -- python3 <repo>/bench.py --pmc-probe --kernel-reps 2",
        "cd /tmp && timeout -s KILL 90 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o run -- python3 <repo>/bench.py --pmc-probe --kernel-reps 2",
        "python3 bench.py --pmc-summary <out>/fetch <out>/write",
        "```",
        "",
        f"Kernel sources hash (gemm_w4.hip, gemm_w4_kernel.h, common.h, kernels.h): `{d['source_hash']}`",
        "",
        "| counter | KiB/dispatch GEMM | KiB/dispatch reduce | KiB calibration (256 MiB) | factor | bytes/launch |",
        "|---|---|---|---|---|---|",
    ]
    for c, v in out.items():
        lines.append(f"| {c} | {v['kib_per_dispatch_gemm']:.1f} | {v['kib_per_dispatch_reduce']:.1f} | "
                     f"{v['kib_calibration']:.1f} | {v['scale_factor']:.3f} | "
                     f"{v['bytes_gemm'] + v['bytes_reduce']:.0f} |")
    lines += ["", f"Algorithmic bytes per launch: {int(alg)}; measured HBM bytes per launch: {int(hbm)} "
              f"({hbm / alg:.3f} x algorithmic).", ""]
    with open(PMC_MD, "w") as fh:
        fh.write("\n".join(lines))
    print(json.dumps(d))


def traffic_from_profile(bytes_alg):
    """HBM bytes per launch of the dominant kernel from committed PMC summaries, or None."""
    path = PMC_JSON
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)
    if args.pmc_probe:
        pmc_probe(args)
        return
    if args.mfma_probe:
        mfma_probe(args)
        return
    if args.attn_probe:
        attn_probe(args)
        return
    if args.extra_only:
        import torch
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        print(json.dumps({f"workload_{args.extra_only}": extra_config(args.extra_only, args, dev)}), flush=True)
        return
    import torch
    import bit_quantized_draft_amd as bq
    from synth import gen
    from synth.configs import get_config
    cfg = get_config(3)
    n_layers = args.layers or cfg.L
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, C, V = cfg.T, cfg.C, cfg.V
    log(f"building {cfg.name}: {n_layers} layers, T={T}, C={C}")
    draft, target = build_model(cfg, dev, n_layers)

    # the draft tree is grown on the device: each draft step runs the stack over the T slots
    # (static shape), takes the LM head on the frontier rows only, selects their k children
    # and appends the step's quota of best children (ss_tree_expand); 48 steps fill the
    # k=6 / depth-48 template
    R = -(-(T - 1) // DRAFT_STEPS)
    state = bq.TreeState(T, DRAFT_STEPS, R, TOPK, dev)
    mk = lambda: [torch.empty((cfg.nkv, T, cfg.hd), dtype=torch.bfloat16, device=dev) for _ in range(n_layers)]
    tk_d, tv_d, tk_t, tv_t = mk(), mk(), mk(), mk()
    logits = torch.empty((R, V), dtype=torch.float32, device=dev)
    vlogits = torch.empty((T, V), dtype=torch.float32, device=dev)
    children = torch.empty((R, TOPK), dtype=torch.int32, device=dev)
    seeded_logits = torch.empty((T, V), dtype=torch.float32, device=dev)
    tgt = torch.empty(T, dtype=torch.int32, device=dev)
    acc_out = (torch.empty(T, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev))
    inv_t = float(np.float32(1.0) / np.float32(DRAFT_TEMP))
    ws_d = torch.empty(draft.workspace_bytes(T, C), dtype=torch.uint8, device=dev)
    ws_t = torch.empty(target.workspace_bytes(T, C), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(max(1, bq.draft_select_workspace_bytes(R, V, TOPK)), dtype=torch.uint8, device=dev)
    parents, tokens = state.parents, state.tokens

    def tree_init():
        bq.tree_expand_init(state, ROOT_TOKEN)

    def draft_step():
        draft.draft_tree_step(parents, C, tk_d, tv_d, tokens=tokens, logits=logits, logit_rows=state.frontier,
                              workspace=ws_d)
        bq.draft_select(logits, None, inv_t, TOPK, out=children, workspace=ws_s)
        bq.tree_expand(state, logits, children, inv_t)

    kc_all = [ly["k_cache"] for ly in target.layers]
    vc_all = [ly["v_cache"] for ly in target.layers]

    def verify():
        target.draft_tree_step(parents, C, tk_t, tv_t, tokens=tokens, logits=vlogits, workspace=ws_t)
        bq.row_argmax(seeded_logits, out=tgt)
        bq.tree_accept(parents, tokens, tgt, out=acc_out)
        # commit the root and the accepted path's target K/V at rows C .. C + L (the next
        # cycle would advance C by L + 1; the timed cycles keep C fixed and read rows < C)
        bq.kv_commit(kc_all, vc_all, tk_t, tv_t, C, acc_out[0], acc_out[1])

    # eager cycle: grow the tree, then seed the target's argmax on the finished tree so the
    # acceptance walk accepts L_STAR nodes (the draft and target weights are random); the
    # tree is the same every cycle (the draft reads cache rows < C only)
    tree_init()
    for _ in range(DRAFT_STEPS):
        draft_step()
    torch.cuda.synchronize()
    par_np, tok_np = parents.cpu().numpy(), tokens.cpu().numpy()
    depth = np.zeros(T, dtype=np.int64)
    assert par_np[0] == -1 and all(0 <= par_np[i] < i for i in range(1, T)), "expanded tree is not topological"
    for i in range(1, T):
        depth[i] = depth[par_np[i]] + 1
    assert depth.max() == DRAFT_STEPS, f"expanded tree depth {depth.max()}, expected {DRAFT_STEPS}"
    seeded_logits.copy_(torch.from_numpy(gen.target_logits(par_np, tok_np, V, L_STAR, seed=0, cid=cfg.cid,
                                                           path=gen.deepest_path(par_np))))
    verify()
    torch.cuda.synchronize()
    ref_len = int(acc_out[1].item())
    assert ref_len == L_STAR, f"acceptance walk returned {ref_len}, expected {L_STAR}"
    ref_par, ref_tok, ref_cum = parents.clone(), tokens.clone(), state.cum.clone()

    # capture the three phases in HIP graphs
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g_init, g_draft, g_verify = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        tree_init(); draft_step(); verify()          # warm the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g_init, stream=stream):
            tree_init()
        with torch.cuda.graph(g_draft, stream=stream):
            draft_step()
        with torch.cuda.graph(g_verify, stream=stream):
            verify()
    torch.cuda.synchronize()

    def cycle():
        g_init.replay()
        for _ in range(DRAFT_STEPS):
            g_draft.replay()
        g_verify.replay()
        return int(acc_out[1].item())      # the one host read-back per cycle

    # every replayed cycle checked against the eager one, with eager work in between
    for _ in range(2):
        assert cycle() == L_STAR
        assert torch.equal(parents, ref_par) and torch.equal(tokens, ref_tok), "graph cycle grew another tree"
        assert torch.equal(state.cum, ref_cum), "graph cycle's path scores differ from the eager cycle's"
        tree_init()
        for _ in range(DRAFT_STEPS):
            draft_step()
        torch.cuda.synchronize()
        assert torch.equal(parents, ref_par) and torch.equal(tokens, ref_tok)

    log(f"warmup {args.warmup} cycles")
    for _ in range(args.warmup):
        cycle()
    torch.cuda.synchronize()
    log(f"timing {args.steps} cycles")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L = cycle()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert L == L_STAR
    ms_cycle = elapsed / args.steps * 1e3
    value = DRAFT_STEPS * T * args.steps / elapsed

    # phase split (outside the timed region): draft step alone and the verify phase alone
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g_init.replay()
    e0.record()
    for _ in range(DRAFT_STEPS):
        g_draft.replay()
    e1.record(); torch.cuda.synchronize()
    ms_draft_step = e0.elapsed_time(e1) / DRAFT_STEPS
    e0.record(); g_verify.replay(); e1.record(); torch.cuda.synchronize()
    ms_verify = e0.elapsed_time(e1)
    step_bytes = algorithmic_bytes_step(cfg, n_layers, logit_rows=R)

    # stochastic verification at target temperature 0.6 on the cycle's finished tree (outside
    # the timed cycle): the verify pass's target logits, the draft's logits of every node
    # from one extra all-rows draft step, seeded uniforms
    d_all = torch.empty((T, V), dtype=torch.float32, device=dev)
    draft.draft_tree_step(parents, C, tk_d, tv_d, tokens=tokens, logits=d_all, workspace=ws_d)
    rng_u = np.random.default_rng(7)
    uni = torch.from_numpy(rng_u.random(T)).to(dev)
    buni = torch.from_numpy(rng_u.random(T)).to(dev)
    inv_tt = float(np.float32(1.0) / np.float32(0.6))
    sv_out = bq.tree_accept_stochastic(parents, tokens, d_all, vlogits, inv_t, inv_tt, uni, buni)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        bq.tree_accept_stochastic(parents, tokens, d_all, vlogits, inv_t, inv_tt, uni, buni, out=sv_out)
    e1.record(); torch.cuda.synchronize()
    ms_stochastic = e0.elapsed_time(e1) / 5
    sv_len = int(sv_out[1].item())
    del d_all
    step_gbs = step_bytes / (ms_draft_step * 1e-3) / 1e9

    # dominant kernel: fused int4 gate_up + SwiGLU, 8 layers' weights in rotation (> 256 MB
    # Infinity Cache), timed with HIP events recorded on the stream it runs on. The sweep
    # over tree sizes runs first and also brings the GPU to a steady state; the T = 64
    # figure of the roofline object is measured last.
    x = gen.torch_normal_bf16((T, cfg.H), 1.0, 0, cfg.cid, gen.TID_X, 0, dev)
    u = torch.empty((T, cfg.I), dtype=torch.bfloat16, device=dev)
    rot = [draft.layers[i % n_layers]["gate_up"] for i in range(8)]
    ks = torch.cuda.Stream()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the same kernel over the tree sizes the HBM-bound target covers (16 to 64 tokens),
    # same weights, same timing method
    by_tokens = {}
    for tn in (16, 32, 48, 64):
        xt = gen.torch_normal_bf16((tn, cfg.H), 1.0, 0, cfg.cid, gen.TID_X, 0, dev)
        ut = torch.empty((tn, cfg.I), dtype=torch.bfloat16, device=dev)
        with torch.cuda.stream(ks):
            for tw in rot:
                bq.w4a16_gate_up_swiglu_tiled(xt, tw, out=ut)
            k0.record(ks)
            for _ in range(args.kernel_reps):
                for tw in rot:
                    bq.w4a16_gate_up_swiglu_tiled(xt, tw, out=ut)
            k1.record(ks)
        torch.cuda.synchronize()
        us_t = k0.elapsed_time(k1) * 1e3 / (args.kernel_reps * len(rot))
        gbs_t = gate_up_bytes(cfg, tn) / (us_t * 1e-6) / 1e9
        by_tokens[str(tn)] = {"avg_launch_us": round(us_t, 3), "achieved": round(gbs_t, 1),
                              "frac": round(gbs_t / HBM_PEAK_GBS, 4)}

    with torch.cuda.stream(ks):
        for tw in rot:
            bq.w4a16_gate_up_swiglu_tiled(x, tw, out=u)
        k0.record(ks)
        n_launch = 0
        for _ in range(args.kernel_reps):
            for tw in rot:
                bq.w4a16_gate_up_swiglu_tiled(x, tw, out=u)
                n_launch += 1
        k1.record(ks)
    torch.cuda.synchronize()
    us_launch = k0.elapsed_time(k1) * 1e3 / n_launch
    gu_bytes = gate_up_bytes(cfg)
    achieved = gu_bytes / (us_launch * 1e-6) / 1e9

    # the other single-GPU workloads: the 32B stack at T = 256 and the 8B long-context stack
    extra = {}
    if not args.no_extra:
        del draft, target, ws_d, ws_t, g_draft, g_verify
        torch.cuda.empty_cache()
        for cid in (4, 5):
            extra[f"workload_{cid}"] = extra_config(cid, args, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, n_layers, state.R)

    line = {
        "metric": "draft-tree tokens/s per substitute-stack step; % of MI355X HBM roofline",
        "value": round(value, 1), "unit": "draft-tree tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_cycle, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16+int4",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {n_layers}-layer substitute stack, T={T} tree tokens "
                               f"grown on the device to depth {DRAFT_STEPS} (k={TOPK}, {R} nodes per level at most), "
                               f"C={C}, vocab {V}; cycle = {DRAFT_STEPS} draft steps (stack over all T slots, LM "
                               f"head on the frontier rows, child selection at t={DRAFT_TEMP}, tree expansion) + bf16 "
                               f"verify pass + argmax + greedy accept + KV commit",
                   "tree_tokens_per_cycle": DRAFT_STEPS * T, "accept_len": L,
                   "draft_step_ms": round(ms_draft_step, 4), "verify_ms": round(ms_verify, 4),
                   "draft_step_alg_bytes": int(step_bytes),
                   "draft_step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
                   "stochastic_verify_ms": round(ms_stochastic, 4), "stochastic_accept_len": sv_len,
                   "other_workloads": extra},
        "roofline": {"kernel": "w4k_kernel<TT=4, EPI_SWIGLU, tiled> (tiled int4 gate_up 37888x3584, T=64)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(gu_bytes),
                     "alg_bytes_per_launch": int(gu_bytes), "avg_launch_us": round(us_launch, 3),
                     "by_tree_tokens": by_tokens},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
