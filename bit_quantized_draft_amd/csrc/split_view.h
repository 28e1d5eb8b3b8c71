// Where a GEMM left the fp32 partial sums of its split blocks, for kernels that finish
// the reduction themselves (residual add + RMSNorm inputs, RoPE scatter) instead of a separate
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

// Partial loads a finisher keeps in flight per element before adding them in order.
#ifndef SS_SV_BATCH
#define SS_SV_BATCH 8
#endif
constexpr int SV_BATCH = SS_SV_BATCH;

}  // namespace ss
