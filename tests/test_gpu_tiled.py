"""The tiled int4 layout the GEMMs stream (ss_w4_tile in include/subspec.h).

The relocation is checked byte for byte against the layout's definition, restated here
with numpy reshapes; the tiled linears are checked against the oracle and against the
untiled linears on the same weights, which they must match bit for bit (same codes,
same scales and zeros, same order of every operation).
"""

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


def tiled_reference(qp, s, z):
    """Layout definition: block (tile i, chunk c) = 64 lanes x 16 code bytes (lane l:
    row 16 i + l % 16, bytes 64 c + 16 (l / 16) ..), then words 2 j + h = scale | zero << 16
    of row 16 i + j, group 2 c + h."""
    n, kh = qp.shape
    nc = 2 * kh // 128
    codes = qp.reshape(n // 16, 16, nc, 4, 16).transpose(0, 2, 3, 1, 4).reshape(n // 16, nc, 1024)
    sb = s.view(np.uint16).astype(np.uint32).reshape(n // 16, 16, nc, 2).transpose(0, 2, 1, 3)
    zb = z.view(np.uint16).astype(np.uint32).reshape(n // 16, 16, nc, 2).transpose(0, 2, 1, 3)
    words = np.ascontiguousarray(sb | (zb << 16)).astype("<u4").reshape(n // 16, nc, 32)
    sz = words.view(np.uint8).reshape(n // 16, nc, 128)
    return np.concatenate([codes, sz], axis=2).reshape(-1)


def _case(N, K, seed):
    w = gen.weight_bf16(N, K, 0.02, seed=seed, cid=21)
    q, s, z = bq.quantize_substitute(to_bf16(w))
    return w, q, s, z


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 1024)])
def test_tile_relocation_matches_definition(N, K):
    print(f"tile relocation N={N} K={K}", flush=True)
    _, q, s, z = _case(N, K, seed=N + K)
    tw = bq.w4_tile(q, s, z)
    torch.cuda.synchronize()
    assert tw.data.numel() == N * K * 9 // 16
    assert np.array_equal(host(tw.data), tiled_reference(host(q), host(s), host(z)))


@pytest.mark.parametrize("T,N,K", [(16, 512, 512), (5, 256, 384), (33, 144, 640), (64, 384, 512),
                                   (100, 256, 256), (256, 128, 384), (64, 3584, 2048)])
def test_tiled_linear_parity(T, N, K):
    print(f"tiled w4a16 T={T} N={N} K={K}", flush=True)
    w, q, s, z = _case(N, K, seed=3 * T + N + K)
    x = gen.normal_bf16((T, K), 1.0, seed=T + K, cid=21, tid=gen.TID_X)
    xd = to_bf16(x)
    tw = bq.w4_tile(q, s, z)
    yb_t, yf_t = bq.w4a16_linear_tiled(xd, tw)
    yb_u, yf_u = bq.w4a16_linear(xd, q, s, z)
    torch.cuda.synchronize()
    assert torch.equal(yf_t, yf_u), "tiled and untiled fp32 outputs differ"
    assert torch.equal(yb_t, yb_u), "tiled and untiled bf16 outputs differ"
    q_o, s_o, z_o = oracle.quantize(w)
    ref = oracle.w4a16_matmul64(x, q_o, s_o, z_o)
    assert_close(host(yf_t), ref, what="tiled w4a16 fp32")
    assert np.array_equal(bf16_bits(yb_t), oracle.f32_to_bf16(host(yf_t)))


@pytest.mark.parametrize("T,I,K", [(64, 640, 512), (7, 272, 384), (48, 1024, 1024), (200, 128, 256)])
def test_tiled_gate_up_parity(T, I, K):
    print(f"tiled gate_up T={T} I={I} K={K}", flush=True)
    w, q, s, z = _case(2 * I, K, seed=5 * T + I + K)
    x = gen.normal_bf16((T, K), 1.0, seed=T + I, cid=22, tid=gen.TID_X)
    xd = to_bf16(x)
    tw = bq.w4_tile(q, s, z)
    u_t = bq.w4a16_gate_up_swiglu_tiled(xd, tw)
    u_u = bq.w4a16_gate_up_swiglu(xd, q, s, z)
    torch.cuda.synchronize()
    assert torch.equal(u_t, u_u), "tiled and untiled SwiGLU outputs differ"
    q_o, s_o, z_o = oracle.quantize(w)
    y = oracle.w4a16_matmul64(x, q_o, s_o, z_o)
    ref = oracle.swiglu64(y[:, :I], y[:, I:])
    assert_close(oracle.bf16_to_f64(bf16_bits(u_t)), ref, scale_abs=True, bf16_out=True, what="tiled gate_up u")
