// Skinny GEMMs of the substitute draft: Y[T][N] = X[T][K] * W[N][K]^T for the small
// token counts of a draft tree (T <= 64 per token block), on gfx950 MFMA.
//
// W4A16 path (the substitute linear layer: 4-bit weights, bf16 activations, fp32
// accumulation). Packed int4 weights stream from HBM with 128-bit loads: lane (j, b) of
// a wave reads 32 consecutive nibbles (one 64-group half) of weight row j. A nibble q is
// OR-ed into the mantissa of fp16 1024.0 (0x6400), which is the fp16 value 1024 + q
// exactly; v_fma_mix_f32 then evaluates (1024 + q) * s + c in fp32 straight from that
// fp16 half, with c = -(1024 + z) * s precomputed per group, so it yields the exact
// substitute weight (q - z) * s up to one fp32 rounding. v_cvt_pk_bf16_f32 rounds pairs
// to bf16 and bf16 MFMA (v_mfma_f32_16x16x32_bf16) accumulates in fp32 across all of K.
// About 2.4 ALU ops per weight, independent of the token count.
//
// MFMA roles: A = activations (16 tokens x 32 k), B = weights (32 k x 16 rows); lane
// (j, b) supplies k = 32b + 8m .. 32b + 8m + 7 of the 128-wide chunk to MFMA m, so the
// activations are staged in LDS in exactly that fragment order. Loads are branch-free
// (out-of-range rows and tokens read a clamped address and are discarded), which lets
// the compiler count outstanding loads precisely and keep PF chunks in flight.
//
// bf16-weight path: the same engine with dense bf16 weights (LM head, verify pass).
//
// Work split: a workgroup of NW waves owns NW*NR*16 weight rows and all tokens of its
// token block; waves split rows and share the staged activation chunk. Split-K across
// workgroups writes fp32 partials that a second kernel sums in fixed order.
#include "common.h"
#include "kernels.h"

namespace ss {

constexpr int CHUNK_K = 128;

// 16-byte block blk (k = 8 blk .. 8 blk + 7) of a 128-wide chunk feeds MFMA m = blk % 4
// from lane group b = blk / 4.
struct GemmParams {
  const uint16_t* x;   // bf16 [T][K]
  const uint8_t* qw;   // int4 [N][K/2]
  const uint16_t* sc;  // fp16 [N][K/64]
  const uint16_t* zp;  // fp16 [N][K/64]
  const uint16_t* wb;  // bf16 [N][K]
  int T, N, K;
  int chunks_per_split;  // 128-wide K chunks per split
  int splits;
  int swiglu_I;        // rows [0,I) gate, [I,2I) up
  float* partial;      // fp32 [splits][T][N] when splits > 1
  float* y_f32;        // [T][N]
  uint16_t* y_bf16;    // [T][N]
  float* resid;        // fp32 [T][N] residual stream (EPI_RESID)
  uint16_t* u_bf16;    // bf16 [T][I] (EPI_SWIGLU)
};

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

template <int NR, int NW, int EPI>
__device__ __forceinline__ int row_of(const GemmParams& p, int wave, int r, int j) {
  if (EPI == EPI_SWIGLU) {
    constexpr int HALF = NR / 2;
    const int base = (blockIdx.x * NW + wave) * HALF * 16;
    return (r < HALF) ? base + r * 16 + j : p.swiglu_I + base + (r - HALF) * 16 + j;
  }
  return (blockIdx.x * NW + wave) * NR * 16 + r * 16 + j;
}

// Final store of one output element for STORE / RESID.
template <int EPI>
__device__ __forceinline__ void store_out(const GemmParams& p, int t, int n, float v) {
  const size_t o = (size_t)t * p.N + n;
  if (EPI == EPI_RESID) {
    p.resid[o] += v;
  } else {
    if (p.y_f32) p.y_f32[o] = v;
    if (p.y_bf16) p.y_bf16[o] = f32_to_bf16(v);
  }
}

__device__ __forceinline__ float f16lo(uint32_t x) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t x) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  typedef __bf16 b2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, b2v));
}

// 8 nibbles (k = e, e = 0..7 of one 8-block) -> 8 bf16 weights (q - z) s, natural order
__device__ __forceinline__ u32x4_t dequant8(uint32_t q, float s, float c) {
  const uint32_t h04 = (q & 0x000F000Fu) | 0x64006400u;          // 1024+q0 | 1024+q4
  const uint32_t h15 = ((q >> 4) & 0x000F000Fu) | 0x64006400u;   // q1 | q5
  const uint32_t h26 = ((q >> 8) & 0x000F000Fu) | 0x64006400u;   // q2 | q6
  const uint32_t h37 = ((q >> 12) & 0x000F000Fu) | 0x64006400u;  // q3 | q7
  const float w0 = __builtin_fmaf(f16lo(h04), s, c), w4 = __builtin_fmaf(f16hi(h04), s, c);
  const float w1 = __builtin_fmaf(f16lo(h15), s, c), w5 = __builtin_fmaf(f16hi(h15), s, c);
  const float w2 = __builtin_fmaf(f16lo(h26), s, c), w6 = __builtin_fmaf(f16hi(h26), s, c);
  const float w3 = __builtin_fmaf(f16lo(h37), s, c), w7 = __builtin_fmaf(f16hi(h37), s, c);
  return u32x4_t{pk_bf16(w0, w1), pk_bf16(w2, w3), pk_bf16(w4, w5), pk_bf16(w6, w7)};
}

// Loader -> compute hand-off through LDS counters. Only LDS ordering is needed: a wave's
// LDS instructions execute in order, so waiting for its own LDS operations
// (lgkmcnt(0)) before touching a counter orders them. Release/acquire atomics would
// also wait for every outstanding global load (vmcnt(0)), draining the weight prefetch
// each chunk, so the counters use relaxed atomics plus explicit LDS waits.
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Bounded waits on LDS counters. A correct pipeline never comes near the limit; the
// bound guarantees that every wave exits even if it were wrong.
constexpr int kSpinLimit = 1 << 20;
__device__ __forceinline__ void wait_eq(int* flag, int want) {
  for (int it = 0; it < kSpinLimit; ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == want) break;
    __builtin_amdgcn_s_sleep(1);
  }
  compiler_fence();
}
__device__ __forceinline__ void wait_ge(int* flag, int want) {
  for (int it = 0; it < kSpinLimit; ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= want) break;
    __builtin_amdgcn_s_sleep(1);
  }
  compiler_fence();
}

// SZV: scale and zero of 4 consecutive chunks (8 groups) arrive in one 16-byte load per
// row tile (needs K % 512 == 0 and split boundaries on multiples of 4 chunks).
template <int NR, int TT, int NW, bool INT4, int PF, bool SZV, int EPI>
__global__ __launch_bounds__((NW + 1) * 64) void skinny_gemm_kernel(GemmParams p) {
  // Waves 0..NW-1 compute; wave NW streams activation chunks into an NB-deep LDS ring.
  // The hand-off uses LDS counters instead of workgroup barriers: ready[b] holds the
  // chunk index last written to buffer b, done[b] counts compute waves that finished
  // reading it. Compute waves never wait for each other, and their in-order load
  // counters only track their own weight prefetches.
  constexpr int NB = 4;              // LDS ring depth
  constexpr int LA = 2;              // chunks the loader holds in registers
  static_assert(8 % PF == 0, "the main loop is unrolled by 8 chunks (two scale/zero quads)");
  __shared__ u32x4_t xfrag[NB][4][TT][64];
  __shared__ int ready[NB];
  __shared__ int done[NB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 15;       // weight row within a 16-row tile / output column
  const int b = lane >> 4;       // k lane group
  const int tok0 = blockIdx.z * 64;
  const int Tb = min(64, p.T - tok0);
  const int split = blockIdx.y;
  const int c_begin = split * p.chunks_per_split;
  const int c_end = min(p.K / CHUNK_K, c_begin + p.chunks_per_split);
  const int G = p.K >> 6;
  const int nchunks = c_end - c_begin;
  const int c_last = max(c_end - 1, c_begin);

  if (tid < NB) {
    ready[tid] = -1;
    done[tid] = 0;
  }
  __syncthreads();   // the only workgroup barrier

  if (wave == NW) {
    // ---------------- loader wave. Pass (m, tt) fills fragment block [m][tt] of a chunk:
    // lane l = 16 b + i loads token tt*16 + i, k = 32 b + 8 m .. +7, so every LDS store
    // instruction writes one contiguous 1 KB block.
    constexpr int PASSES = TT * 4;
    u32x4_t v[LA][PASSES];
    const int li = lane & 15, lb = lane >> 4;
    auto load = [&](int slot, int c) {
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        const int m = ps & 3, tt = ps >> 2;
        const int tl = min(tt * 16 + li, Tb - 1);
        v[slot][ps] = *reinterpret_cast<const u32x4_t*>(p.x + (size_t)(tok0 + tl) * p.K + c * CHUNK_K +
                                                        lb * 32 + m * 8);
      }
    };
    auto store = [&](int slot, int bufi) {
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        const int m = ps & 3, tt = ps >> 2;
        const bool live = tt * 16 + li < Tb;       // padded tokens contribute zeros
        const u32x4_t x = v[slot][ps];
        xfrag[bufi][m][tt][lane] = u32x4_t{live ? x.x : 0u, live ? x.y : 0u, live ? x.z : 0u, live ? x.w : 0u};
      }
    };
#pragma unroll
    for (int a = 0; a < LA; ++a) load(a, min(c_begin + a, c_last));
    for (int q0 = 0; q0 < nchunks; q0 += LA) {
#pragma unroll
      for (int a = 0; a < LA; ++a) {
        const int q = q0 + a;
        if (q < nchunks) {
          const int bq = q % NB;
          if (q >= NB) wait_ge(&done[bq], NW * (q / NB));   // chunk q - NB fully read
          store(a, bq);
          compiler_fence();
          lds_wait();                                        // fragment stores done
          if (lane == 0) __hip_atomic_store(&ready[bq], q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          load(a, min(c_begin + q + LA, c_last));
        }
      }
    }
    return;
  }

  // ---------------- compute waves
  int rows[NR];
  bool rvalid[NR];
  size_t rbase[NR];   // element offset of the (clamped) row
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    rows[r] = row_of<NR, NW, EPI>(p, wave, r, j);
    const int lim = (EPI == EPI_SWIGLU) ? ((r < NR / 2) ? p.swiglu_I : 2 * p.swiglu_I) : p.N;
    // tiles are 16 rows and N (or I) is a multiple of 16: a tile is all valid or all invalid
    rvalid[r] = rows[r] < lim;
    rbase[r] = (size_t)(rvalid[r] ? rows[r] : 0);
  }

  // ---- weight prefetch ring (PF chunks) and scale/zero ring (per chunk, or per 4 chunks)
  constexpr int QF = 2;   // scale/zero quads in flight: the next quad's is always loaded
  u32x4_t wreg[PF][NR][INT4 ? 1 : 4];
  uint32_t szreg[INT4 && !SZV ? PF : 1][NR];   // fp16 scale (low) | zero (high), one chunk
  u32x4_t sq[QF][NR], zq[QF][NR];               // 8 fp16 scales / zeros = 4 chunks x 2 groups
  const int c_last4 = c_begin + ((nchunks - 1) >> 2) * 4;
  auto w_load = [&](int slot, int c) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (INT4) {
        wreg[slot][r][0] = *reinterpret_cast<const u32x4_t*>(p.qw + rbase[r] * (p.K >> 1) + c * 64 + b * 16);
        if (!SZV) {
          const size_t gi = rbase[r] * G + 2 * c + (b >> 1);
          szreg[SZV ? 0 : slot][r] = (uint32_t)p.sc[gi] | ((uint32_t)p.zp[gi] << 16);
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          wreg[slot][r][m] = *reinterpret_cast<const u32x4_t*>(p.wb + rbase[r] * p.K + c * CHUNK_K + b * 32 + m * 8);
      }
    }
  };
  auto sz_load = [&](int qs, int c4) {   // c4: first chunk of a 4-chunk quad
    if (INT4 && SZV) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        sq[qs][r] = *reinterpret_cast<const u32x4_t*>(p.sc + rbase[r] * G + 2 * c4);
        zq[qs][r] = *reinterpret_cast<const u32x4_t*>(p.zp + rbase[r] * G + 2 * c4);
      }
    }
  };

  f32x4_t acc[NR][TT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // chunk q of this split: wait for its activation buffer; per k-step m, read the
  // fragments, dequantize the matching weight words and multiply (few live registers);
  // release the buffer after the last read
  auto compute = [&](int slot, int qslot, int q) {
    const int bq = q % NB;
    wait_eq(&ready[bq], q);
    float sf[NR], cf[NR];
    if (INT4) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        uint32_t sz;
        if (SZV) {
          const int q4 = slot & 3;   // chunk within the quad (quads start on multiples of 4)
          const u32x4_t s4 = sq[qslot][r], z4 = zq[qslot][r];
          const uint32_t sw = q4 == 0 ? s4.x : q4 == 1 ? s4.y : q4 == 2 ? s4.z : s4.w;
          const uint32_t zw = q4 == 0 ? z4.x : q4 == 1 ? z4.y : q4 == 2 ? z4.z : z4.w;
          const int sh = (b >> 1) * 16;   // group 2 c + (b >> 1) of the lane
          sz = ((sw >> sh) & 0xFFFFu) | (((zw >> sh) & 0xFFFFu) << 16);
        } else {
          sz = szreg[SZV ? 0 : slot][r];
        }
        sf[r] = f16lo(sz);
        const float zf = f16hi(sz);
        cf[r] = __builtin_fmaf(-1024.0f, sf[r], -(zf * sf[r]));   // -(1024 + z) s
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      bf16x8_t xa[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) xa[t] = __builtin_bit_cast(bf16x8_t, xfrag[bq][m][t][lane]);
      if (m == 3) {
        // the fragment reads have returned (their values are in registers) before the
        // buffer is released; one increment per wave (atomics run once per active lane)
        compiler_fence();
        lds_wait();
        if (lane == 0) __hip_atomic_fetch_add(&done[bq], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        u32x4_t wv;
        if (INT4) {
          const u32x4_t w = wreg[slot][r][0];
          wv = dequant8(m == 0 ? w.x : m == 1 ? w.y : m == 2 ? w.z : w.w, sf[r], cf[r]);
        } else {
          wv = wreg[slot][r][m];
        }
#pragma unroll
        for (int t = 0; t < TT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[t], __builtin_bit_cast(bf16x8_t, wv),
                                                             acc[r][t], 0, 0, 0);
      }
    }
  };

  // The main loop is unrolled by 8 chunks: weight slot s % PF holds chunk q0 + s, scale
  // / zero quad slot s / 4 holds chunks q0 + 4 (s / 4) .. +3, so all ring indices are
  // compile-time registers and the body is straight-line (prefetch indices are clamped
  // at the end instead of guarded): the load counters stay exact, PF chunks of weights
  // and the next scale/zero quad stay in flight. A guarded tail handles the last
  // (chunks mod 8) chunks.
  constexpr int UNR = 8;
#pragma unroll
  for (int s = 0; s < PF; ++s) w_load(s, min(c_begin + s, c_last));
  sz_load(0, c_begin);
  sz_load(1, min(c_begin + 4, c_last4));
  int q0 = 0;
  for (; q0 + UNR <= nchunks; q0 += UNR) {
#pragma unroll
    for (int s = 0; s < UNR; ++s) {
      const int c = c_begin + q0 + s;
      compute(s % PF, s >> 2, q0 + s);
      w_load(s % PF, min(c + PF, c_last));
      if ((s & 3) == 3) sz_load(s >> 2, min(c + 5, c_last4));   // quad two ahead
    }
  }
#pragma unroll
  for (int s = 0; s < UNR; ++s) {
    if (q0 + s < nchunks) {
      const int c = c_begin + q0 + s;
      compute(s % PF, s >> 2, q0 + s);
      w_load(s % PF, min(c + PF, c_last));
      if ((s & 3) == 3) sz_load(s >> 2, min(c + 5, c_last4));
    }
  }

  // ---- epilogue: lane holds tokens t*16 + 4b + e of row tile r, column j
  if (p.splits > 1) {
    float* part = p.partial + (size_t)split * p.T * p.N;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (!rvalid[r]) continue;
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = t * 16 + 4 * b + e;
          if (tok < Tb) part[(size_t)(tok0 + tok) * p.N + rows[r]] = acc[r][t][e];
        }
    }
    return;
  }
  if (EPI == EPI_SWIGLU) {
    constexpr int HALF = NR / 2;
#pragma unroll
    for (int r = 0; r < HALF; ++r) {
      if (!rvalid[r]) continue;
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = t * 16 + 4 * b + e;
          if (tok < Tb) {
            const float g = acc[r][t][e], u = acc[r + HALF][t][e];
            p.u_bf16[(size_t)(tok0 + tok) * p.swiglu_I + rows[r]] = f32_to_bf16(silu_f32(g) * u);
          }
        }
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (!rvalid[r]) continue;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = t * 16 + 4 * b + e;
        if (tok < Tb) store_out<EPI>(p, tok0 + tok, rows[r], acc[r][t][e]);
      }
  }
}

// Fixed-order sum of split-K partials followed by the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p) {
  const int ncols = (EPI == EPI_SWIGLU) ? p.swiglu_I : p.N;
  const size_t total = (size_t)p.T * ncols;
  const size_t stride = (size_t)p.T * p.N;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / ncols), n = (int)(i % ncols);
    if (EPI == EPI_SWIGLU) {
      float g = 0.f, u = 0.f;
      for (int s = 0; s < p.splits; ++s) {
        g += p.partial[s * stride + (size_t)t * p.N + n];
        u += p.partial[s * stride + (size_t)t * p.N + p.swiglu_I + n];
      }
      p.u_bf16[(size_t)t * p.swiglu_I + n] = f32_to_bf16(silu_f32(g) * u);
    } else {
      float v = 0.f;
      for (int s = 0; s < p.splits; ++s) v += p.partial[s * stride + (size_t)t * p.N + n];
      store_out<EPI>(p, t, n, v);
    }
  }
}

// ------------------------------------------------------------------ host side

namespace {
#ifndef SS_GEMM_NW
#define SS_GEMM_NW 4
#endif
#ifndef SS_GEMM_NR
#define SS_GEMM_NR 2
#endif
#ifndef SS_GEMM_PF
#define SS_GEMM_PF 4
#endif
#ifndef SS_GEMM_PFB
#define SS_GEMM_PFB 2
#endif
constexpr int kNW = SS_GEMM_NW;   // compute waves per workgroup
constexpr int kNR = SS_GEMM_NR;   // 16-row weight tiles per compute wave
constexpr int kPF = SS_GEMM_PF;   // int4 weight chunks in flight per wave (multiple of 4)
constexpr int kPFB = SS_GEMM_PFB; // bf16 weight chunks in flight per wave
constexpr int kRowsPerBlock = kNW * kNR * 16;

int choose_splits(int row_blocks, int chunks, int tok_blocks) {
  const int target = 256;
  const int units = std::max(1, row_blocks * tok_blocks);
  int s = (target + units - 1) / units;
  s = std::max(1, std::min(s, chunks / 4));
  return std::max(1, std::min(s, chunks));
}

template <int TT, bool INT4, bool SZV, int EPI>
hipError_t launch_tt(const GemmParams& p, dim3 grid, hipStream_t st) {
  constexpr int PF = INT4 ? kPF : kPFB;
  hipLaunchKernelGGL((skinny_gemm_kernel<kNR, TT, kNW, INT4, PF, SZV, EPI>), grid, dim3((kNW + 1) * 64), 0, st, p);
  return hipGetLastError();
}

template <bool INT4, bool SZV, int EPI>
hipError_t launch_tt_any(const GemmParams& p, int TT, dim3 grid, hipStream_t st) {
  switch (TT) {
    case 1: return launch_tt<1, INT4, SZV, EPI>(p, grid, st);
    case 2: return launch_tt<2, INT4, SZV, EPI>(p, grid, st);
    case 3: return launch_tt<3, INT4, SZV, EPI>(p, grid, st);
    default: return launch_tt<4, INT4, SZV, EPI>(p, grid, st);
  }
}

template <int EPI>
hipError_t launch_epi(const GemmParams& p, bool int4, bool szv, int TT, dim3 grid, hipStream_t st) {
  if (!int4) return launch_tt_any<false, false, EPI>(p, TT, grid, st);
  return szv ? launch_tt_any<true, true, EPI>(p, TT, grid, st) : launch_tt_any<true, false, EPI>(p, TT, grid, st);
}
}  // namespace

GemmPlan plan_gemm(int T, int N, int K, int epi, int swiglu_I) {
  GemmPlan pl;
  const int rows = (epi == EPI_SWIGLU) ? 2 * swiglu_I : N;
  const int half_rows = (epi == EPI_SWIGLU) ? swiglu_I : N;
  const int per_block = (epi == EPI_SWIGLU) ? kRowsPerBlock / 2 : kRowsPerBlock;
  pl.row_blocks = (half_rows + per_block - 1) / per_block;
  (void)rows;
  pl.tok_blocks = (T + 63) / 64;
  pl.chunks = std::max(1, K / CHUNK_K);
  pl.splits = choose_splits(pl.row_blocks, pl.chunks, pl.tok_blocks);
  pl.chunks_per_split = (pl.chunks + pl.splits - 1) / pl.splits;
  if (pl.chunks % 4 == 0) pl.chunks_per_split = (pl.chunks_per_split + 3) / 4 * 4;   // whole quads
  pl.splits = (pl.chunks + pl.chunks_per_split - 1) / pl.chunks_per_split;
  pl.ws_bytes = pl.splits > 1 ? (size_t)pl.splits * T * N * sizeof(float) : 0;
  return pl;
}

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& pl, void* ws, hipStream_t st) {
  GemmParams p{};
  p.x = a.x; p.qw = a.qw; p.sc = a.sc; p.zp = a.zp; p.wb = a.wb;
  p.T = a.T; p.N = a.N; p.K = a.K;
  p.chunks_per_split = pl.chunks_per_split;
  p.splits = pl.splits;
  p.swiglu_I = a.swiglu_I;
  p.partial = reinterpret_cast<float*>(ws);
  p.y_f32 = a.y_f32; p.y_bf16 = a.y_bf16; p.resid = a.resid; p.u_bf16 = a.u_bf16;
  dim3 grid(pl.row_blocks, pl.splits, pl.tok_blocks);
  const int TT = (a.T >= 64) ? 4 : (a.T + 15) / 16;
  const bool int4 = a.qw != nullptr;
  hipError_t e;
  // vector scale/zero loads: 16-byte aligned quads of groups and whole quads per split
  const bool szv = int4 && (a.K % 512 == 0) && (pl.chunks_per_split % 4 == 0);
  switch (a.epi) {
    case EPI_RESID: e = launch_epi<EPI_RESID>(p, int4, szv, TT, grid, st); break;
    case EPI_SWIGLU: e = launch_epi<EPI_SWIGLU>(p, int4, szv, TT, grid, st); break;
    default: e = launch_epi<EPI_STORE>(p, int4, szv, TT, grid, st); break;
  }
  if (e != hipSuccess || pl.splits == 1) return e;
  const int ncols = (a.epi == EPI_SWIGLU) ? a.swiglu_I : a.N;
  const size_t total = (size_t)a.T * ncols;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
  switch (a.epi) {
    case EPI_RESID: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_RESID>, dim3(blocks), dim3(256), 0, st, p); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_SWIGLU>, dim3(blocks), dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_STORE>, dim3(blocks), dim3(256), 0, st, p); break;
  }
  return hipGetLastError();
}

}  // namespace ss
