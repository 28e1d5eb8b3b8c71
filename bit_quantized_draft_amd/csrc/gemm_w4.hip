// W4A16 substitute linear layers on gfx950: Y[T][N] = X[T][K] * deq(W)[N][K]^T over all
// draft-tree tokens at once (Summary page "Speculate Deep and Accurate ...", "Approach":
// the draft's layers are 4-bit copies of the target's; Abstract: they run in place of the
// offloaded layers), 4-bit codes with one fp16 scale and zero per 64 inputs, bf16
// activations, bf16 MFMA with fp32 accumulation.
//
// Design (MI355X, 256 CUs, one workgroup per CU):
//  * Workgroup = 4 waves, one per SIMD, each a K phase with 512 registers (accumulation
//    registers included) for up to 6-8 logical tiles; inside a wave the MFMAs of one tile
//    overlap the dequantization of the next on gfx950 (MFMA and VALU issue together).
//  * A unit of work is (token block of 64, group of logical tiles, K range). A logical tile
//    is 32 weight rows (two 16-row MFMA tiles; for SwiGLU 16 gate rows and their 16 up
//    rows). Every wave holds all of the group's tiles; K phase kp takes chunk kp of every
//    super-chunk of 4 chunks (512 k).
//  * Weights go straight from HBM into the registers of the wave that multiplies them
//    (one 16-byte load per lane per 16-row tile and 128-wide chunk on the tiled layout:
//    1 KB contiguous per wave instruction), two super-chunks ahead; no hand-off through
//    LDS and no cross-wave protocol for weights.
//  * Activations of a super-chunk are staged in an LDS double buffer by all four waves
//    with direct-to-LDS loads (global_load_lds_dwordx4, no registers), one barrier per
//    super-chunk; each wave reads its phase's fragments once and uses them for all its
//    tiles.
//  * The four K phases are added at the end of a unit through LDS in a fixed tree
//    ((p0 + p2) + (p1 + p3)); results do not depend on timing.
//  * The planner picks the tile groups and K ranges: large N (gate_up) runs one unit per
//    CU over all of K with tile counts within one tile of each other (no partial sums);
//    small N (qkv, o, down) also splits K, and the K ranges' fp32 partials are added in
//    range order by the consumer (RoPE scatter, residual + RMSNorm inputs) or by a reduce
//    kernel.
//
// Dequantization of 8 codes (one 32-bit word): a nibble OR-ed into the mantissa of fp16
// 1024.0 is 1024 + q exactly (odd nibbles masked in place give 1024 + 16 q); v_fma_mix_f32
// evaluates (1024 + q) s + c straight from that fp16 half with c = -(1024 + z) s rounded
// once to fp32, which gives (q - z) s up to that rounding (about 2^-14 s, far below the
// bf16 step of the result); v_cvt_pk_bf16_f32 rounds pairs to bf16.
#include "gemm_w4_kernel.h"

#include <algorithm>
#include <cmath>
#include <mutex>

namespace ss {

using w4::CHK;
using w4::MAX_WGS;

int w4_tpw_max(int TT, int epi) { return w4::tpw_max(TT, epi); }

namespace {
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }
}  // namespace

// K ranges' partials [splits][T][nout] added in range order (fixed), then the epilogue:
// EPI_STORE y, EPI_SWIGLU u = silu(gate) * up. One thread per output column and token.
template <int EPI>
__global__ __launch_bounds__(256) void w4_reduce_kernel(const float* __restrict__ part, int splits, int T,
                                                        int nout, int ncols, float* __restrict__ y_f32,
                                                        uint16_t* __restrict__ y_bf16,
                                                        uint16_t* __restrict__ u_bf16, int I) {
  const int tok = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= ncols) return;
  const size_t slice = (size_t)T * nout;
  const float* src = part + (size_t)tok * nout + n;
  float v0 = 0.f, v1 = 0.f;
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float a[8], c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = s0 + i < splits;
      a[i] = ok ? src[(size_t)(s0 + i) * slice] : 0.f;
      c[i] = (ok && EPI == EPI_SWIGLU) ? src[(size_t)(s0 + i) * slice + I] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (s0 + i < splits) {
        v0 += a[i];
        v1 += c[i];
      }
    }
  }
  if (EPI == EPI_SWIGLU) {
    u_bf16[(size_t)tok * I + n] = f32_to_bf16(silu_f32(v0) * v1);
  } else {
    if (y_f32) y_f32[(size_t)tok * nout + n] = v0;
    if (y_bf16) y_bf16[(size_t)tok * nout + n] = f32_to_bf16(v0);
  }
}

// ------------------------------------------------------------------ host side

namespace {
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// cost model of a plan (seconds), fitted to per-wave timelines of the kernel on MI355X:
// a unit is a pipeline fill, S super-chunks and the K-phase reduction plus epilogue. A
// super-chunk costs the larger of its math (per SIMD: two waves x TPW tiles x 4 k-steps of
// one 17-instruction dequantization plus TT MFMAs, about 74 + 11.4 TT cycles, plus about
// 1000 cycles of barrier skew) and its weight bytes at the CU's share of HBM bandwidth.
// Split K ranges add their fp32 partial sums written and read back, and a reduce launch
// when no consumer adds them.
double plan_cost(const W4Plan& pl, int T, int nout, bool reduce_launch) {
  const double clk = 2.3e9, bw = 7.5e12;
  const int active = std::min(pl.units, MAX_WGS);
  const int rounds = (pl.units + MAX_WGS - 1) / MAX_WGS;
  const int tpw = (pl.NL + pl.n_groups - 1) / pl.n_groups;
  const int chunks = (pl.nch + pl.splits - 1) / pl.splits;
  const int S = (chunks + w4::KP - 1) / w4::KP;
  const double step_math = 1000.0 + 2.0 * tpw * 4 * (74.0 + 11.4 * pl.TT);
  const double step_mem = (double)w4::KP * 2 * tpw * TILE_BLOCK_BYTES / (bw / active / clk);
  const double fill = 4000.0 + step_mem;
  const double epi = 1000.0 + 450.0 * tpw * pl.TT;
  double t = rounds * (fill + S * std::max(step_math, step_mem) + epi) / clk;
  if (pl.splits > 1) t += 2.0 * pl.splits * T * (double)nout * 4 / 5.0e12 + (reduce_launch ? 3e-6 : 0.0);
  return t;
}
}  // namespace

W4Plan plan_w4(int T, int N, int K, int epi, int swiglu_I, bool reduce_launch) {
  W4Plan best{};
  best.TT = T >= 64 ? 4 : (T + 15) / 16;
  best.tb_count = (T + 63) / 64;
  best.nch = std::max(1, K / CHK);
  best.NL = epi == EPI_SWIGLU ? swiglu_I / 16 : (N + 31) / 32;
  best.nout = epi == EPI_SWIGLU ? 2 * swiglu_I : N;
  const int tpw_max = w4_tpw_max(best.TT, epi);
  double best_t = 1e30;
  bool found = false;
  for (int tpw = 1; tpw <= tpw_max; ++tpw) {
    const int ng = (best.NL + tpw - 1) / tpw;
    if (tpw > 1 && (best.NL + ng - 1) / ng < tpw) continue;   // the same groups as a smaller tpw
    for (int splits = 1; splits <= std::min(best.nch, 64); ++splits) {
      W4Plan pl = best;
      pl.splits = splits;
      pl.n_groups = ng;
      pl.units = best.tb_count * ng * splits;
      if (splits > 1 && (double)splits * T * best.nout * sizeof(float) > 256.0 * (1 << 20)) break;
      const double t = plan_cost(pl, T, best.nout, reduce_launch);
      // equal cost: fewer K splits (less partial-sum traffic)
      if (t < best_t * 0.999) {
        best_t = t;
        best = pl;
        found = true;
      }
    }
  }
  if (!found) {
    best.splits = 1;
    best.n_groups = (best.NL + tpw_max - 1) / tpw_max;
    best.units = best.tb_count * best.n_groups;
  }
  best.G = std::min(best.units, MAX_WGS);
  best.ws_bytes = best.splits > 1 ? align256((size_t)best.splits * T * best.nout * sizeof(float)) : 0;
  return best;
}

// ------------------------------------------------------------------ no-allocation scratch

// Partial sums of the no-allocation entry point: one array per device, held until the
// process ends. Host code passes its device address (scratch_ptrs), never the symbol.
static __device__ __align__(256) unsigned char scratch[W4_SCRATCH_BYTES];

hipError_t w4_scratch(void** out) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static void* scratch_ptrs[MAX_DEV] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!scratch_ptrs[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptrs[dev] = ptr;
  }
  *out = scratch_ptrs[dev];
  return hipSuccess;
}

hipError_t launch_w4(const W4Args& a, const W4Plan& pl, void* ws, hipStream_t st) {
  if (!a.qw || (!a.tiled && (!a.sc || !a.zp))) return hipErrorInvalidValue;
  if (a.K % CHK || a.N % 16 || a.T < 1 || a.T > 256) return hipErrorInvalidValue;
  if (pl.NL != (a.epi == EPI_SWIGLU ? a.swiglu_I / 16 : (a.N + 31) / 32) || pl.nch != a.K / CHK)
    return hipErrorInvalidValue;   // a plan for another shape
  {
    // the plan's groups must fit the registers of a wave
    const int maxg = (pl.NL + pl.n_groups - 1) / pl.n_groups;
    if (maxg < 1 || maxg > w4_tpw_max(pl.TT, a.epi)) return hipErrorInvalidValue;
  }
  if (pl.splits > 1 && !ws) return hipErrorInvalidValue;
  if (a.ssq_in && (a.epi == EPI_RESID || a.ssq_n < 1 || a.ssq_n > w4::SSQ_MAX)) return hipErrorInvalidValue;
  if (pl.splits > 1 && a.epi == EPI_RESID && !a.defer_reduce) return hipErrorInvalidValue;
  W4Params p{};
  p.x = a.x; p.qw = a.qw; p.sc = a.sc; p.zp = a.zp;
  p.T = a.T; p.N = a.N; p.K = a.K; p.nch = pl.nch;
  p.swiglu_I = a.swiglu_I;
  p.NL = pl.NL; p.n_groups = pl.n_groups; p.splits = pl.splits; p.tb_count = pl.tb_count; p.units = pl.units;
  p.nout = pl.nout;
  p.y_f32 = a.y_f32; p.y_bf16 = a.y_bf16; p.resid = a.resid; p.u_bf16 = a.u_bf16;
  p.part = pl.splits > 1 ? static_cast<float*>(ws) : nullptr;
  p.ssq_in = a.ssq_in; p.ssq_n = a.ssq_n; p.rms_H = a.rms_H; p.rms_eps = a.rms_eps;
  const int maxg = (pl.NL + pl.n_groups - 1) / pl.n_groups;
  switch (pl.TT) {
    case 1: launch_w4_tt1(p, maxg, a.epi, a.tiled, pl.G, st); break;
    case 2: launch_w4_tt2(p, maxg, a.epi, a.tiled, pl.G, st); break;
    case 3: launch_w4_tt3(p, maxg, a.epi, a.tiled, pl.G, st); break;
    default: launch_w4_tt4(p, maxg, a.epi, a.tiled, pl.G, st); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1 || a.defer_reduce) return e;
  // a K-split GEMM that nobody consumes deferred: add the ranges here
  const int ncols = a.epi == EPI_SWIGLU ? a.swiglu_I : a.N;
  const dim3 grid((ncols + 255) / 256, a.T);
  if (a.epi == EPI_SWIGLU)
    hipLaunchKernelGGL(w4_reduce_kernel<EPI_SWIGLU>, grid, dim3(256), 0, st, p.part, pl.splits, a.T, pl.nout, ncols,
                       nullptr, nullptr, a.u_bf16, a.swiglu_I);
  else
    hipLaunchKernelGGL(w4_reduce_kernel<EPI_STORE>, grid, dim3(256), 0, st, p.part, pl.splits, a.T, pl.nout, ncols,
                       a.y_f32, a.y_bf16, nullptr, 0);
  return hipGetLastError();
}

}  // namespace ss
