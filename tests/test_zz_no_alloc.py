"""The no-allocation linear (ss_w4a16_linear_tiled_noalloc, partial sums in the library's
device scratch) against ss_w4a16_linear_tiled (caller workspace) on the same inputs: the same
plan and kernels, so the outputs must be bit-identical. Two calls in a row, the second
smaller, show that the scratch's leftover contents from the first call do not leak into the
second."""
import pytest
import torch

import bit_quantized_draft_amd as bq
from bit_quantized_draft_amd._lib import lib
from synth import gen
from tests.gpu_util import to_bf16

pytestmark = pytest.mark.gpu


def _case(T, n, k, seed):
    w = gen.weight_bf16(n, k, 0.02, seed=seed, cid=7)
    x = gen.normal_bf16((T, k), 1.0, seed=seed, cid=7, tid=gen.TID_X)
    q, s, z = bq.quantize_substitute(to_bf16(w))
    return to_bf16(x), bq.w4_tile(q, s, z)


@pytest.mark.parametrize("first,second", [((64, 3584, 18944), (16, 512, 4096)),
                                          ((33, 1024, 4096), (16, 512, 4096))])
def test_noalloc_matches_workspace_linear(first, second):
    for (T, n, k), seed in ((first, 1), (second, 2)):
        print(f"noalloc T={T} n={n} k={k}", flush=True)
        print(f"  partial-sum bytes {lib().ss_w4a16_linear_workspace(T, n, k)}", flush=True)
        x, tw = _case(T, n, k, seed)
        ref_b, ref_f = bq.w4a16_linear_tiled(x, tw)
        yb = torch.full((T, n), float("nan"), dtype=torch.bfloat16, device=x.device)
        yf = torch.full((T, n), float("nan"), dtype=torch.float32, device=x.device)
        bq.w4a16_linear_tiled_noalloc(x, tw, yb, yf)
        torch.cuda.synchronize()
        assert torch.equal(yf, ref_f), (T, n, k)
        assert torch.equal(yb.view(torch.int16), ref_b.view(torch.int16)), (T, n, k)


def test_noalloc_rejects_oversized_partials():
    # a shape whose K-range partial sums would exceed the 16 MiB device scratch
    T, n, k = 192, 8192, 65536
    need = lib().ss_w4a16_linear_workspace(T, n, k)
    if need <= 16 << 20:
        pytest.skip(f"the plan for this shape needs only {need} bytes")
    x = torch.zeros((T, k), dtype=torch.bfloat16, device="cuda:0")
    tw = bq.TiledW4(torch.zeros(lib().ss_w4_tiled_bytes(n, k), dtype=torch.uint8, device="cuda:0"), n, k)
    yf = torch.empty((T, n), dtype=torch.float32, device="cuda:0")
    with pytest.raises(bq.SubspecError) as e:
        bq.w4a16_linear_tiled_noalloc(x, tw, None, yf)
    assert "scratch" in str(e.value)
