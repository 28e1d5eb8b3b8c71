"""Run-to-run determinism of the float kernels: every result is computed in a fixed order
(fixed split and reduction orders, no atomics on values), so two calls on the same inputs
agree bit for bit, also with other work on the GPU in between.

Covered: tree attention at each workgroup shape and both merge kernels, the tiled int4
linear with K splits (partials added by the reduce pass), the tiled gate_up + SwiGLU, and
the bf16 linear of the LM head (split over K).
"""

import pytest
import torch

from synth import gen
from tests.gpu_util import to_bf16, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_quantized_draft_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _perturb():
    """Unrelated GPU work between the calls (other cache contents, other timing)."""
    a = torch.randn(1 << 22, device="cuda")
    (a * 2).sum().item()


def _attn(T, C, nq, nkv, hd, kind, seed):
    q = to_bf16(gen.normal_bf16((T, nq, hd), 1.0, seed, 2, gen.TID_Q))
    kc = to_bf16(gen.normal_bf16((nkv, C, hd), 1.0, seed, 2, gen.TID_KC))
    vc = to_bf16(gen.normal_bf16((nkv, C, hd), 1.0, seed, 2, gen.TID_VC))
    kt = to_bf16(gen.normal_bf16((nkv, T, hd), 1.0, seed, 2, gen.TID_KT))
    vt = to_bf16(gen.normal_bf16((nkv, T, hd), 1.0, seed, 2, gen.TID_VT))
    par = to_dev(gen.tree_parents(T, kind, seed=seed))
    return lambda: bq.tree_attention(q, kc, vc, kt, vt, par, C, want_f32=True)[:2]


@pytest.mark.parametrize("T,C,nq,nkv,hd,kind", [
    (64, 2048, 28, 4, 128, "CB"),     # one tile per wave, two key groups; one-row merge
    (48, 5000, 32, 8, 128, "CB"),     # one tile per wave, four key groups
    (64, 4200, 16, 4, 128, "RB"),     # two tiles per wave
    (256, 300, 40, 8, 128, "RB"),     # the wide merge
])
def test_tree_attention_deterministic(T, C, nq, nkv, hd, kind):
    print(f"attention determinism T={T} C={C} nq={nq} nkv={nkv}", flush=True)
    run = _attn(T, C, nq, nkv, hd, kind, seed=T + C)
    a = [t.clone() for t in run()]
    _perturb()
    b = run()
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("T,N,K", [(64, 3584, 3584), (64, 3584, 18944), (16, 4608, 3584)])
def test_w4a16_linear_tiled_deterministic(T, N, K):
    print(f"tiled linear determinism T={T} N={N} K={K}", flush=True)
    w = to_bf16(gen.weight_bf16(N, K, 0.02, seed=N + K, cid=2))
    x = to_bf16(gen.normal_bf16((T, K), 1.0, seed=N + K, cid=2, tid=gen.TID_X))
    tw = bq.w4_tile(*bq.quantize_substitute(w))
    del w
    a = bq.w4a16_linear_tiled(x, tw)[1].clone()
    _perturb()
    b = bq.w4a16_linear_tiled(x, tw)[1]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gate_up_tiled_deterministic():
    T, I, K = 64, 4096, 3584
    print(f"gate_up determinism T={T} I={I} K={K}", flush=True)
    w = to_bf16(gen.weight_bf16(2 * I, K, 0.02, seed=5, cid=2))
    x = to_bf16(gen.normal_bf16((T, K), 1.0, seed=5, cid=2, tid=gen.TID_X))
    tw = bq.w4_tile(*bq.quantize_substitute(w))
    del w
    a = bq.w4a16_gate_up_swiglu_tiled(x, tw).clone()
    _perturb()
    b = bq.w4a16_gate_up_swiglu_tiled(x, tw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_lm_head_bf16_deterministic():
    R, V, H = 2, 32768, 3584
    print(f"bf16 LM-head determinism R={R} V={V} H={H}", flush=True)
    w = to_bf16(gen.weight_bf16(V, H, 0.02, seed=9, cid=2))
    x = to_bf16(gen.normal_bf16((R, H), 1.0, seed=9, cid=2, tid=gen.TID_X))
    a = bq.bf16_linear(x, w)[1].clone()
    _perturb()
    b = bq.bf16_linear(x, w)[1]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
