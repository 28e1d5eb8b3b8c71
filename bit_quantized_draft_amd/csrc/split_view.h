// Where a GEMM left the fp32 partial sums of its split blocks, for kernels that finish
// the reduction themselves (residual add + RMSNorm, RoPE scatter) instead of a separate
// reduce launch. Layout and piece order are those of w4_gemm_kernel (gemm.hip): block
// b = token block + row block * tb_count; blocks below sk_first and blocks covered by a
// single workgroup were stored by the GEMM itself; a split block's pieces belong to the
// workgroups g0 .. g1 that own its stream-K units, summed in that (K) order.
#pragma once

#include "kernels.h"

namespace ss {

struct SvBlock {
  int g0, g1;    // owning workgroups; g0 == g1: not split (the GEMM stored the value)
  int slot0;     // partial slot of the first piece (the others use slot 2 gk)
};

// Ownership arithmetic in 32 bits: the launchers check sk_units * G_sk < 2^31.
__device__ __forceinline__ int sv_owner(const SplitView& v, uint32_t u) {
  return (int)(((u + 1) * (uint32_t)v.G_sk - 1) / (uint32_t)v.sk_units);
}

__device__ __forceinline__ SvBlock sv_block(const SplitView& v, int b) {
  SvBlock r{0, 0, 0};
  if (b < v.sk_first) return r;
  const int sb = b - v.sk_first;
  const uint32_t u0 = (uint32_t)sb * (uint32_t)v.nsteps;
  r.g0 = sv_owner(v, u0);
  r.g1 = sv_owner(v, u0 + v.nsteps - 1);
  const uint32_t lo = (uint32_t)r.g0 * (uint32_t)v.sk_units / (uint32_t)v.G_sk;
  r.slot0 = 2 * r.g0 + ((int)(lo / (uint32_t)v.nsteps) == sb ? 0 : 1);
  return r;
}

// Offset of output element (token t, row n) inside one partial slot; row n lies in row
// block n / rows_per_block (non-SwiGLU layout: 32 rows per row group, two 16-row tiles).
__device__ __forceinline__ size_t sv_offset(const SplitView& v, int t, int n) {
  const int nn = n % v.rows_per_block;
  const int rg = nn >> 5, r = (nn >> 4) & 1, j = nn & 15;
  const int tl = t & 63, tt = tl >> 4, bq = (tl & 15) >> 2, e = tl & 3;
  return (size_t)rg * (2 * v.TT * 256) + ((r * v.TT + tt) * 4 + e) * 64 + 16 * bq + j;
}

// Final values of one token row's elements n = c0 + k * blockDim.x + threadIdx.x (k < KM,
// n < c1). blk holds the row's block table (one entry per row block). A split element is
// the sum of its pieces in K order from 0, plus row[n] when add_row (a residual); any
// other element is row[n] as the GEMM left it. Piece loads go out SV_BATCH at a time per
// element, all independent, and are added afterwards in order.
#ifndef SS_SV_BATCH
#define SS_SV_BATCH 8
#endif
constexpr int SV_BATCH = SS_SV_BATCH;

template <int KM>
__device__ __forceinline__ void sv_row(const SplitView& v, const SvBlock* blk, int t, int c0, int c1,
                                       const float* __restrict__ row, bool add_row, float (&val)[KM]) {
  const size_t se = (size_t)v.RG * 2 * v.TT * 256;   // floats per partial slot
  float s[KM];
  int g0[KM], np[KM], s0[KM];
  size_t off[KM];
  int pmax = 0;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int n = c0 + k * (int)blockDim.x + (int)threadIdx.x;
    const bool in = n < c1;
    SvBlock b{0, 0, 0};
    if (in) b = blk[n / v.rows_per_block];
    g0[k] = b.g0;
    s0[k] = b.slot0;
    np[k] = b.g1 != b.g0 ? b.g1 - b.g0 + 1 : 0;   // pieces to add (0: stored by the GEMM)
    off[k] = in ? sv_offset(v, t, n) : 0;
    val[k] = in ? row[n] : 0.f;
    s[k] = 0.f;
    pmax = max(pmax, np[k]);
  }
  for (int p0 = 0; p0 < pmax; p0 += SV_BATCH) {
    float x[KM][SV_BATCH];
#pragma unroll
    for (int k = 0; k < KM; ++k)
#pragma unroll
      for (int i = 0; i < SV_BATCH; ++i) {
        const int pi = p0 + i;
        const size_t slot = pi == 0 ? (size_t)s0[k] : (size_t)(2 * (g0[k] + pi));
        x[k][i] = pi < np[k] ? v.partials[slot * se + off[k]] : 0.f;
      }
#pragma unroll
    for (int k = 0; k < KM; ++k)
#pragma unroll
      for (int i = 0; i < SV_BATCH; ++i)
        if (p0 + i < np[k]) s[k] += x[k][i];
  }
#pragma unroll
  for (int k = 0; k < KM; ++k)
    if (np[k] > 0) val[k] = add_row ? val[k] + s[k] : s[k];
}

}  // namespace ss
