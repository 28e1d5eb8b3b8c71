// Skinny GEMMs of the substitute draft: Y[T][N] = X[T][K] * W[N][K]^T for the small
// token counts of a draft tree (T <= 64 per token block), on gfx950 MFMA.
//
// W4A16 path (the substitute linear layer: 4-bit weights, bf16 activations, fp32
// accumulation). A nibble q is OR-ed into the mantissa of fp16 1024.0 (0x6400), which
// is the fp16 value 1024 + q exactly; v_fma_mix_f32 evaluates (1024 + q) * s + c in fp32
// straight from that fp16 half, with c = -(1024 + z) * s precomputed per group, giving
// the substitute weight (q - z) * s up to one fp32 rounding (odd nibbles are masked in
// place as 1024 + 16 q, see dequant8). v_cvt_pk_bf16_f32 rounds pairs to bf16 and
// v_mfma_f32_16x16x32_bf16 accumulates in fp32 across all of K. On gfx950 MFMA and VALU
// work of one SIMD do not overlap, so the ALU time per weight is the dequantization
// (about 2.1 VALU ops per weight) plus T/16 MFMA passes.
//
// Workgroup: NWC compute waves (one per SIMD by default; two per SIMD measured slower,
// an MFMA wave and a VALU wave on one SIMD interfere) and NLD = 2 loader waves.
//  * Compute wave w works on row group rg = w % RG and K phase ph = w / RG (KS phases,
//    RG = NWC / KS row groups of 32 weight rows). Each holds PF chunks (128 k) of its own
//    int4 weights in registers, loaded branch-free with 16-byte loads.
//  * Loader waves copy, per chunk, the activation fragments (and, when K % 512 != 0, the
//    block rows' fp16 scale / zero pairs) global -> LDS with gfx950's direct-to-LDS
//    loads (global_load_lds_dwordx4 / _dword: no registers, no conversion) into a ring
//    of NS chunk slots. Otherwise a third loader wave stages scale / zero per octet of
//    chunks with 16-byte loads (one cache line per row instead of one per row and chunk:
//    the address unit, shared with the weight loads, was the bottleneck). Hand-off through LDS counters: ready[slot] is the sequence number of
//    the chunk in the slot, done[slot] counts the compute waves that finished reading it.
//  * MFMA roles: A = activations (16 tokens x 32 k), B = weights (32 k x 16 rows); lane
//    (j, b) supplies k = 32 b + 8 m .. +7 of the chunk to k-step m, so a fragment block
//    [m][token tile] is 1 KB, contiguous by lane: exactly one direct-to-LDS load.
//
// Work split (data parallel + stream-K): a block is (token block of 64, row block of
// RG * 32 rows) over all of K, cut into steps of KS chunks. With G workgroups (one per
// CU), workgroup g first takes whole blocks g, g + G, ... (dp_rounds of them), then an
// even share of the remaining blocks' steps. A block split between workgroups leaves
// one fp32 partial per piece; a small second kernel adds them in K order (a fixed
// order: results do not depend on timing) and runs the epilogue.
#include "common.h"
#include "kernels.h"

namespace ss {

constexpr int CHUNK_K = 128;
#ifndef SS_GEMM_NWC
#define SS_GEMM_NWC 4
#endif
constexpr int NWC = SS_GEMM_NWC;   // compute waves
#ifndef SS_GEMM_NLD
#define SS_GEMM_NLD 2
#endif
constexpr int NLD = SS_GEMM_NLD;   // loader waves
constexpr int NR = 2;    // 16-row weight tiles per compute wave
constexpr int NS = 6;    // activation chunk slots in LDS

#ifndef SS_GEMM_MIN_PIECE
#define SS_GEMM_MIN_PIECE 3
#endif
#ifndef SS_GEMM_WGS
#define SS_GEMM_WGS 256
#endif

struct GemmParams {
  const uint16_t* x;   // bf16 [T][K]
  const uint8_t* qw;   // int4 [N][K/2]
  const uint16_t* sc;  // fp16 [N][K/64]
  const uint16_t* zp;  // fp16 [N][K/64]
  const uint16_t* wb;  // bf16 [N][K]
  int T, N, K;
  int swiglu_I;        // rows [0,I) gate, [I,2I) up
  float* y_f32;        // [T][N]
  uint16_t* y_bf16;    // [T][N]
  float* resid;        // fp32 [T][N] residual stream (EPI_RESID)
  uint16_t* u_bf16;    // bf16 [T][I] (EPI_SWIGLU)
  int nchunks, nsteps, tb_count;
  int G, dp_rounds, sk_first, G_sk;
  long long sk_units;
  float* partials;     // [2 G_sk][RG][NR][TT][4][64]
  // RMSNorm folded into the consumer: x holds bf16(h * gain); output row t is scaled by
  // rs[t] = 1 / sqrt(sum_i ssq_in[t][i] / rms_H + rms_eps), i < ssq_n
  const float* ssq_in;
  int ssq_n, rms_H;
  float rms_eps;
  // RMSNorm inputs made by a residual GEMM (EPI_RESID): hg_out = bf16(h * hg_gain) and
  // ssq_out[t][n / 32] = sum of h^2 over each 32-column group (ssq_n columns groups)
  uint16_t* hg_out;
  const uint16_t* hg_gain;
  float* ssq_out;
};

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

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

// (a & m) | c in one VOP3 instruction. gfx9 VOP3 encodings take no literal constants, so
// with both constants written as literals the compiler splits this into v_and + v_or;
// passing them in registers keeps the single v_and_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// 8 nibbles (k = e, e = 0..7 of one 8-block) -> 8 bf16 weights (q - z) s, natural order.
// Even nibbles (bits 0-3 of each half) OR-ed into fp16 1024.0 give 1024 + q; odd nibbles
// (bits 4-7) masked in place give 1024 + 16 q, both exact. With c = -(1024 + z) s and,
// for the odd ones, s16 = s / 16 and c16 = -(64 + z) s, one fp32 FMA on the fp16 half
// (v_fma_mix_f32) yields (q - z) s up to one rounding of c; one shift per 32-bit word
// brings nibbles 2, 3, 6, 7 down.
__device__ __forceinline__ u32x4_t dequant8(uint32_t q, float s, float c, float s16, float c16) {
  const uint32_t ME = 0x000F000Fu, MO = 0x00F000F0u, X = 0x64006400u;
  const uint32_t qh = q >> 8;
  const uint32_t h04 = and_or(q, ME, X);     // 1024 + q0      | 1024 + q4
  const uint32_t h15 = and_or(q, MO, X);     // 1024 + 16 q1   | 1024 + 16 q5
  const uint32_t h26 = and_or(qh, ME, X);    // 1024 + q2      | 1024 + q6
  const uint32_t h37 = and_or(qh, MO, X);    // 1024 + 16 q3   | 1024 + 16 q7
  const float w0 = __builtin_fmaf(f16lo(h04), s, c), w4 = __builtin_fmaf(f16hi(h04), s, c);
  const float w1 = __builtin_fmaf(f16lo(h15), s16, c16), w5 = __builtin_fmaf(f16hi(h15), s16, c16);
  const float w2 = __builtin_fmaf(f16lo(h26), s, c), w6 = __builtin_fmaf(f16hi(h26), s, c);
  const float w3 = __builtin_fmaf(f16lo(h37), s16, c16), w7 = __builtin_fmaf(f16hi(h37), s16, c16);
  return u32x4_t{pk_bf16(w0, w1), pk_bf16(w2, w3), pk_bf16(w4, w5), pk_bf16(w6, w7)};
}

// LDS hand-off. Only LDS ordering is needed: a wave's LDS operations complete in order,
// so waiting for them (lgkmcnt(0)) before touching a counter orders them; relaxed
// atomics avoid the vmcnt(0) that release/acquire would add (it would drain the
// weight prefetch every chunk).
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Bounded waits on LDS counters: a correct pipeline never comes near the limit; the
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
__device__ __forceinline__ void lds_store(int* flag, int v) {
  __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// A workgroup's work is a list of segments (block, steps [s0, s1)): its dp_rounds whole
// blocks g, g + G, ..., then the blocks its stream-K unit range [lo, hi) touches.
struct SegList {
  int nd, nsk;         // whole blocks, stream-K segments
  int sb_lo, s_lo;     // first stream-K block and its first step
  long long hi;
};

__device__ __forceinline__ SegList make_segs(const GemmParams& p, int g) {
  SegList L;
  L.nd = p.dp_rounds;
  L.nsk = 0;
  L.sb_lo = L.s_lo = 0;
  L.hi = 0;
  if (g < p.G_sk) {
    const long long lo = (long long)g * p.sk_units / p.G_sk;
    L.hi = (long long)(g + 1) * p.sk_units / p.G_sk;
    if (L.hi > lo) {
      L.sb_lo = (int)(lo / p.nsteps);
      L.s_lo = (int)(lo % p.nsteps);
      L.nsk = (int)((L.hi - 1) / p.nsteps) - L.sb_lo + 1;
    }
  }
  return L;
}

__device__ __forceinline__ void seg_of(const GemmParams& p, const SegList& L, int g, int k, int& block,
                                       int& s0, int& s1) {
  if (k < L.nd) {
    block = g + k * p.G;
    s0 = 0;
    s1 = p.nsteps;
  } else {
    const int sb = L.sb_lo + (k - L.nd);
    block = p.sk_first + sb;
    s0 = (k == L.nd) ? L.s_lo : 0;
    s1 = (int)min((long long)p.nsteps, L.hi - (long long)sb * p.nsteps);
  }
}

// Prefetch cursor over the segments, each padded to a multiple of PF positions so that
// position p of every segment uses ring slot p % PF; padding positions (and positions
// past the last segment) reload the segment's last step, which stays in bounds and is
// never used.
struct PCur {
  int k, pos, len, plen, s0, rb;
};

template <int PF>
__device__ __forceinline__ void pcur_set(PCur& c, const GemmParams& p, const SegList& L, int g, int k) {
  int block, s0, s1;
  seg_of(p, L, g, k, block, s0, s1);
  c.k = k;
  c.pos = 0;
  c.s0 = s0;
  c.len = s1 - s0;
  c.plen = (c.len + PF - 1) / PF * PF;
  c.rb = block / p.tb_count;
}

template <int PF>
__device__ __forceinline__ void pcur_next(PCur& c, const GemmParams& p, const SegList& L, int g) {
  if (++c.pos < c.plen) return;
  if (c.k + 1 < L.nd + L.nsk) pcur_set<PF>(c, p, L, g, c.k + 1);
  else c.pos = c.plen - 1;
}

// workgroup index that owns stream-K unit u
__device__ __forceinline__ int sk_owner(const GemmParams& p, long long u) {
  return (int)(((u + 1) * p.G_sk - 1) / p.sk_units);
}
// partial slot of workgroup gk's piece of stream-K block sb (a workgroup's range has a
// partial piece at most at its first and at its last block)
__device__ __forceinline__ int sk_slot(const GemmParams& p, int gk, int sb) {
  const long long lo = (long long)gk * p.sk_units / p.G_sk;
  return 2 * gk + ((int)(lo / p.nsteps) == sb ? 0 : 1);
}

template <int EPI, int RG>
__device__ __forceinline__ int tile_row(const GemmParams& p, int rb, int rg, int r, int j) {
  if (EPI == EPI_SWIGLU) {
    const int g = rb * RG * 16 + rg * 16 + j;
    return r == 0 ? g : p.swiglu_I + g;
  }
  return rb * RG * 32 + rg * 32 + r * 16 + j;
}
template <int EPI, int RG>
__device__ __forceinline__ bool tile_valid(const GemmParams& p, int rb, int rg, int r) {
  if (EPI == EPI_SWIGLU) return rb * RG * 16 + rg * 16 < p.swiglu_I;
  return rb * RG * 32 + rg * 32 + r * 16 < p.N;   // N is a multiple of 16
}

// Final values of a wave's tiles -> outputs. Lane (j, b) holds tokens t*16 + 4b + e of
// row j of each tile.
template <int TT, int EPI, int RG>
__device__ __forceinline__ void final_store(const GemmParams& p, const f32x4_t (&acc)[NR][TT], int block,
                                            int rg, int lane) {
  const int j = lane & 15, b = lane >> 4;
  const int tb = block % p.tb_count, rb = block / p.tb_count;
  if (EPI == EPI_SWIGLU) {
    if (!tile_valid<EPI, RG>(p, rb, rg, 0)) return;
    const int g = tile_row<EPI, RG>(p, rb, rg, 0, j);
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = tb * 64 + t * 16 + 4 * b + e;
        if (tok < p.T)
          p.u_bf16[(size_t)tok * p.swiglu_I + g] = f32_to_bf16(silu_f32(acc[0][t][e]) * acc[1][t][e]);
      }
    return;
  }
  float ss[TT][4];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) ss[t][e] = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (!tile_valid<EPI, RG>(p, rb, rg, r)) continue;
    const int n = tile_row<EPI, RG>(p, rb, rg, r, j);
    const float gn = (EPI == EPI_RESID && p.hg_out) ? bf16_to_f32(p.hg_gain[n]) : 0.f;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = tb * 64 + t * 16 + 4 * b + e;
        if (tok >= p.T) continue;
        const size_t o = (size_t)tok * p.N + n;
        const float v = acc[r][t][e];
        if (EPI == EPI_RESID) {
          const float h = p.resid[o] + v;
          p.resid[o] = h;
          if (p.hg_out) {
            p.hg_out[o] = f32_to_bf16(h * gn);
            ss[t][e] += h * h;
          }
        } else {
          if (p.y_f32) p.y_f32[o] = v;
          if (p.y_bf16) p.y_bf16[o] = f32_to_bf16(v);
        }
      }
  }
  if (EPI == EPI_RESID && p.hg_out) {
    // sums of squares of the wave's 32 rows (one 32-column group of the next layer's
    // input) per token: the two tiles are in ss already, the 16 rows j across lanes
    const int grp = (rb * RG * 32 + rg * 32) >> 5;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = ss[t][e];
        x += __shfl_xor(x, 1, 16);
        x += __shfl_xor(x, 2, 16);
        x += __shfl_xor(x, 4, 16);
        x += __shfl_xor(x, 8, 16);
        const int tok = tb * 64 + t * 16 + 4 * b + e;
        if (j == 0 && tok < p.T && rb * RG * 32 + rg * 32 < p.N) p.ssq_out[(size_t)tok * p.ssq_n + grp] = x;
      }
  }
}

// Row scales of RMSNorm folded into a consumer GEMM, for all T tokens, computed once per
// workgroup by its nw compute waves together: wave w takes tokens [w per, (w + 1) per),
// lpt lanes per token each add a strided share of the token's partial sums (eight float4
// loads in flight), the lpt shares are combined by an xor tree (a fixed order), and the
// result goes to rs_all in LDS; each wave then counts itself in rs_done.
__device__ __forceinline__ void row_scales(const GemmParams& p, int wave, int nw, int lane, float* rs_all,
                                           int* rs_done) {
  const int per = (p.T + nw - 1) / nw;
  int lpt = 64;
  while (lpt > 1 && lpt * per > 64) lpt >>= 1;   // lanes per token
  const int tpw = 64 / lpt;                       // tokens per pass
  const int n4 = p.ssq_n >> 2;
  const int part = lane % lpt;
  for (int base = 0; base < per; base += tpw) {   // uniform trip count
    const int tl = base + lane / lpt;
    const int tok = wave * per + tl;
    const bool ok = tl < per && tok < p.T;
    float s = 0.f;
    if (ok) {
      const float4* src = reinterpret_cast<const float4*>(p.ssq_in + (size_t)tok * p.ssq_n);
      for (int i0 = part; i0 < n4; i0 += 8 * lpt) {
        float4 x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = i0 + k * lpt;
          x[k] = i < n4 ? src[i] : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) s += (x[k].x + x[k].y) + (x[k].z + x[k].w);
      }
    }
    for (int o = 1; o < lpt; o <<= 1) s += __shfl_xor(s, o, 64);
    if (ok && part == 0) rs_all[tok] = 1.0f / sqrtf(s / (float)p.rms_H + p.rms_eps);
  }
  compiler_fence();
  lds_wait();
  if (lane == 0) __hip_atomic_fetch_add(rs_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// acc[r][t][e] (token t * 16 + 4 b + e of the token block) times its row scale
template <int TT>
__device__ __forceinline__ void apply_row_scales(f32x4_t (&acc)[NR][TT], const float* rsl, int lane) {
  const int b = lane >> 4;
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sc = rsl[t * 16 + 4 * b + e];
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r][t][e] *= sc;
    }
}

// SZO: scale / zero staged per octet of chunks (8 chunks = 16 groups, 32 bytes per row
// per array, 16-byte loads) by one more loader wave into a 2-slot LDS ring, instead of
// per chunk with 4-byte loads; needs KS == 1 and K % 512 == 0 (16-byte aligned rows).
template <int TT, bool INT4, int EPI, int KS, int PF, bool SZO>
__global__ __launch_bounds__((NWC + NLD + 1) * 64) void w4_gemm_kernel(GemmParams p) {
  constexpr int RG = NWC / KS;
  constexpr int NCB = KS > 1 ? RG * (KS - 1) : 1;   // phase-combine buffers
  constexpr int FRAG = TT * 4;                     // 1 KB fragment blocks per chunk
  constexpr int ROWS = RG * 32;                    // weight rows of a block
  static_assert(!SZO || (INT4 && KS == 1), "octet staging: int4, one K phase");
  constexpr int SZL = (INT4 && !SZO) ? 2 * ROWS / 64 : 0;   // scale / zero loads per chunk
  constexpr int LOADS = FRAG + SZL;                // loader instructions per chunk
  constexpr int LA = (63 / LOADS) < 3 ? (63 / LOADS) : 3;   // chunks in flight per loader
  static_assert(ROWS % 64 == 0, "scale / zero staging uses whole waves of rows");
  static_assert(NS % KS == 0 && NS % NLD == 0, "slot ring must split evenly");
  __shared__ u32x4_t xfrag[NS][4][TT][64];
  __shared__ uint32_t szs[NS][2][(INT4 && !SZO) ? ROWS : 1];   // per row: fp16 scale pair, zero pair
  __shared__ __align__(16) uint16_t szo[2][2][SZO ? ROWS : 1][16];   // octet ring: [slot][s|z][row][group]
  __shared__ int oct_ready[2], oct_done[2];
  __shared__ f32x4_t comb[NCB][NR][TT][64];
  __shared__ int ready[NS], done[NS];
  __shared__ int comb_ready[NCB], comb_done[NCB];
  __shared__ float rs_all[256];    // RMSNorm row scales of all tokens (consumer GEMMs)
  __shared__ int rs_done;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = blockIdx.x;
  const SegList L = make_segs(p, g);
  const int nsegs = L.nd + L.nsk;

  if (tid < NS) {
    ready[tid] = -1;
    done[tid] = 0;
  }
  if (tid < NCB) {
    comb_ready[tid] = 0;
    comb_done[tid] = 0;
  }
  if (tid < 2) {
    oct_ready[tid] = -1;
    oct_done[tid] = 0;
  }
  if (tid < 256) rs_all[tid] = 0.f;
  if (tid == 0) rs_done = 0;
  __syncthreads();   // the only workgroup barrier

  if (SZO && wave == NWC + NLD) {
    // ---------------- scale / zero loader: at every octet start in the sequence (chunk a
    // multiple of 8, or a segment's first chunk) it copies the block rows' 16 scales and
    // 16 zeros of that octet into slot oseq % 2, after all compute waves left the slot's
    // previous octet. Load i covers rows 32 i .. 32 i + 31, lane l -> row 32 i + l / 2,
    // groups 8 (l % 2) .. +7 of the octet (16 bytes; the LDS order is the row order).
    const int Gq = p.K >> 6;
    int oseq = 0;
    for (int k = 0; k < nsegs; ++k) {
      int block, s0, s1;
      seg_of(p, L, g, k, block, s0, s1);
      const int rb = block / p.tb_count;
      for (int st = s0; st < s1; ++st) {
        if ((st & 7) != 0 && st != s0) continue;
        const int slot = oseq & 1;
        if (oseq >= 2) wait_ge(&oct_done[slot], RG * (oseq >> 1));
        const int g0 = (st & ~7) * 2;
#pragma unroll
        for (int i = 0; i < ROWS / 32; ++i) {
          const int rl = i * 32 + (lane >> 1);
          const int rgl = rl >> 5, rr = (rl >> 4) & 1, jl = rl & 15;
          const size_t row = tile_valid<EPI, RG>(p, rb, rgl, rr) ? (size_t)tile_row<EPI, RG>(p, rb, rgl, rr, jl) : 0;
          int gi = g0 + 8 * (lane & 1);
          if (gi + 8 > Gq) gi = 0;   // octet past the end of K: never read, kept in bounds
          __builtin_amdgcn_global_load_lds((const void*)(p.sc + row * Gq + gi),
                                           (__attribute__((address_space(3))) void*)&szo[slot][0][i * 32][0], 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)(p.zp + row * Gq + gi),
                                           (__attribute__((address_space(3))) void*)&szo[slot][1][i * 32][0], 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        if (lane == 0) lds_store(&oct_ready[slot], oseq);
        ++oseq;
      }
    }
    return;
  }

  if (wave >= NWC) {
    // ---------------- loader wave l copies the chunks with sequence number qc = 2 k + l
    // (k = 0, 1, ...), keeping LA chunks in flight. Before it waits for a slot to be
    // released it drains and publishes everything it has issued, so no consumer can be
    // waiting on a chunk the loader holds back.
    const int l = wave - NWC;
    const int li = lane & 15, lb = lane >> 4;
    int n = 0;    // chunks issued by this loader
    int ns = 0;   // chunks published (ready) by this loader
    int qs = 0;   // steps before the current segment
    auto publish = [&](int upto) {
      for (; ns < upto; ++ns) {
        const int qd = 2 * ns + l;
        if (lane == 0) lds_store(&ready[qd % NS], qd);
      }
    };
    for (int k = 0; k < nsegs; ++k) {
      int block, s0, s1;
      seg_of(p, L, g, k, block, s0, s1);
      const int tb = block % p.tb_count, rb = block / p.tb_count;
      for (int st = s0; st < s1; ++st, ++qs) {
#pragma unroll
        for (int ph = 0; ph < KS; ++ph) {
          const int qc = qs * KS + ph;
          if ((qc & 1) != l) continue;
          const int slot = qc % NS;
          if (qc >= NS) {
            const int need = RG * (qc / NS);   // the previous occupant was read by all its waves
            if (__hip_atomic_load(&done[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
              __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
              publish(n);
              wait_ge(&done[slot], need);
            }
          }
          const int ch = min(st * KS + ph, p.nchunks - 1);
          const uint16_t* src = p.x + (size_t)ch * CHUNK_K + lb * 32;
#pragma unroll
          for (int ps = 0; ps < FRAG; ++ps) {
            const int m = ps & 3, tt = ps >> 2;
            const int tok = min(tb * 64 + tt * 16 + li, p.T - 1);   // padded tokens: clamped copies
            __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)tok * p.K + m * 8),
                                             (__attribute__((address_space(3))) void*)&xfrag[slot][m][tt][0],
                                             16, 0, 0);
          }
          if (INT4 && !SZO) {
            // scale and zero pairs (groups 2 ch, 2 ch + 1) of the block's rows; row
            // rl = 32 rg + 16 r + j of the block is lane rl % 64 of load rl / 64
            const int Gq = p.K >> 6;
#pragma unroll
            for (int i = 0; i < ROWS / 64; ++i) {
              const int rl = i * 64 + lane;
              const int rgl = rl >> 5, rr = (rl >> 4) & 1, jl = rl & 15;
              const size_t row = tile_valid<EPI, RG>(p, rb, rgl, rr) ? (size_t)tile_row<EPI, RG>(p, rb, rgl, rr, jl) : 0;
              __builtin_amdgcn_global_load_lds((const void*)(p.sc + row * Gq + 2 * ch),
                                               (__attribute__((address_space(3))) void*)&szs[slot][0][i * 64], 4, 0, 0);
              __builtin_amdgcn_global_load_lds((const void*)(p.zp + row * Gq + 2 * ch),
                                               (__attribute__((address_space(3))) void*)&szs[slot][1][i * 64], 4, 0, 0);
            }
          }
          ++n;
          if (n - ns > LA) {
            // all but the newest LA chunks have landed in LDS
            __builtin_amdgcn_s_waitcnt(((LA * LOADS) & 0xF) | 0x0F70 | (((LA * LOADS) >> 4) << 14));
            publish(n - LA);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    publish(n);
    return;
  }

  // ---------------- compute waves
  const int rg = wave % RG, ph = wave / RG;
  const int j = lane & 15, b = lane >> 4;

  u32x4_t wreg[PF][NR][INT4 ? 1 : 4];

  auto w_load = [&](int slot, const PCur& c) {
    const int ch = min((c.s0 + min(c.pos, c.len - 1)) * KS + ph, p.nchunks - 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const size_t row = tile_valid<EPI, RG>(p, c.rb, rg, r) ? (size_t)tile_row<EPI, RG>(p, c.rb, rg, r, j) : 0;
      if (INT4) {
        wreg[slot][r][0] = *reinterpret_cast<const u32x4_t*>(p.qw + row * (p.K >> 1) + ch * 64 + b * 16);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          wreg[slot][r][m] = *reinterpret_cast<const u32x4_t*>(p.wb + row * p.K + ch * CHUNK_K + b * 32 + m * 8);
      }
    }
  };

  f32x4_t acc[NR][TT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one chunk: wait for its activation slot; per k-step m read the fragments, dequantize
  // the matching weight word and multiply; release the slot after the last read
  auto compute = [&](int slot, int step, int qc, int os) {
    const int xs = qc % NS;
    wait_eq(&ready[xs], qc);
    if (step * KS + ph < p.nchunks) {   // uniform; false only past the end of K
      float sf[NR], cf[NR], sf16[NR], cf16[NR];
      if (INT4) {
        const int sh = (b >> 1) * 16;   // group 2 ch + (b >> 1) of the lane
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int rl = rg * 32 + r * 16 + j;
          float zf;
          if (SZO) {
            const int gsel = 2 * (step & 7) + (b >> 1);
            sf[r] = (float)__builtin_bit_cast(_Float16, szo[os][0][rl][gsel]);
            zf = (float)__builtin_bit_cast(_Float16, szo[os][1][rl][gsel]);
          } else {
            sf[r] = f16lo(szs[xs][0][rl] >> sh);
            zf = f16lo(szs[xs][1][rl] >> sh);
          }
          cf[r] = -(1024.0f + zf) * sf[r];   // 1024 + z is exact in fp32
          sf16[r] = sf[r] * 0.0625f;         // exact
          cf16[r] = -(64.0f + zf) * sf[r];
        }
      }
      // all fragments of the chunk first: the slot is released before the math, and the
      // LDS latency overlaps the first dequantization
      bf16x8_t xa[4][TT];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t) xa[m][t] = __builtin_bit_cast(bf16x8_t, xfrag[xs][m][t][lane]);
      // fragment values are in registers before the slot is released; one increment per
      // wave (atomics run once per active lane)
      compiler_fence();
      lds_wait();
      if (lane == 0) __hip_atomic_fetch_add(&done[xs], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          u32x4_t wv;
          if (INT4) {
            const u32x4_t w = wreg[slot][r][0];
            wv = dequant8(m == 0 ? w.x : m == 1 ? w.y : m == 2 ? w.z : w.w, sf[r], cf[r], sf16[r], cf16[r]);
          } else {
            wv = wreg[slot][r][m];
          }
#pragma unroll
          for (int t = 0; t < TT; ++t)
            acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[m][t], __builtin_bit_cast(bf16x8_t, wv),
                                                               acc[r][t], 0, 0, 0);
        }
      }
    } else {
      compiler_fence();
      if (lane == 0) __hip_atomic_fetch_add(&done[xs], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  };

  // Segments in order; the weight prefetch runs PF positions ahead along the padded
  // position sequence (across segment boundaries) and is issued unconditionally, so
  // the load counters stay exact and ring slots are compile-time registers.
  PCur pc;
  pcur_set<PF>(pc, p, L, g, 0);
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    w_load(u, pc);
    pcur_next<PF>(pc, p, L, g);
  }
  int qs = 0;         // steps before the current segment
  int oseq = -1;      // scale / zero octet in use (SZO)
  auto octet = [&](int st, int s0) {
    if (SZO && ((st & 7) == 0 || st == s0)) {
      if (oseq >= 0) {
        // this wave's reads of the old octet have returned before the slot is released
        compiler_fence();
        lds_wait();
        if (lane == 0) __hip_atomic_fetch_add(&oct_done[oseq & 1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      ++oseq;
      wait_eq(&oct_ready[oseq & 1], oseq);
    }
  };
  if (p.ssq_in) row_scales(p, wave, NWC, lane, rs_all, &rs_done);
  bool rs_seen = false;
  for (int k = 0; k < nsegs; ++k) {
    int block, s0, s1;
    seg_of(p, L, g, k, block, s0, s1);
    const int len = s1 - s0;
    for (int p0 = 0; p0 < len; p0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        if (p0 + u < len) {
          octet(s0 + p0 + u, s0);
          compute(u, s0 + p0 + u, (qs + p0 + u) * KS + ph, oseq & 1);
        }
        w_load(u, pc);
        pcur_next<PF>(pc, p, L, g);
      }
    }
    qs += len;

    // ---- end of segment: combine the K phases in LDS (fixed order), then store the
    // result, or the partial of a block split between workgroups
    if (KS > 1) {
      if (ph > 0) {
        const int cb = rg * (KS - 1) + ph - 1;
        wait_ge(&comb_done[cb], k);
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int t = 0; t < TT; ++t) comb[cb][r][t][lane] = acc[r][t];
        compiler_fence();
        lds_wait();
        if (lane == 0) lds_store(&comb_ready[cb], k + 1);
      } else {
#pragma unroll
        for (int q = 1; q < KS; ++q) {
          const int cb = rg * (KS - 1) + q - 1;
          wait_ge(&comb_ready[cb], k + 1);
#pragma unroll
          for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[r][t] += comb[cb][r][t][lane];
          compiler_fence();
          lds_wait();
          if (lane == 0) lds_store(&comb_done[cb], k + 1);
        }
      }
    }
    if (ph == 0) {
      if (p.ssq_in) {
        if (!rs_seen) {
          wait_ge(&rs_done, NWC);
          rs_seen = true;
        }
        apply_row_scales<TT>(acc, rs_all + (block % p.tb_count) * 64, lane);
      }
      if (s0 == 0 && s1 == p.nsteps) {
        final_store<TT, EPI, RG>(p, acc, block, rg, lane);
      } else {
        float* part = p.partials + ((size_t)sk_slot(p, g, block - p.sk_first) * RG + rg) * (NR * TT * 4 * 64);
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[((r * TT + t) * 4 + e) * 64 + lane] = acc[r][t][e];
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Tiled int4 weights (TILE_BLOCK_BYTES per 16-row tile and chunk, contiguous): the
// loader waves stream each chunk's activation fragments AND the block's 8 weight tiles
// (1 KB of codes each, plus one load for their (scale, zero) words) into the LDS ring
// with direct-to-LDS loads, so compute waves issue no global loads at all: a compute
// wave never stalls at a load instruction that the busy address unit has not accepted
// (waves issue in order, so such a stall would hold back its math). K phases: one.
// Chunk slots (activations + weights) of the tiled kernel: 4 (about 100 KB of LDS at 64
// tokens) measured faster than 2 or 6 at every token count.
#ifndef SS_TILED_NS
#define SS_TILED_NS 4
#endif
constexpr int NS_T = SS_TILED_NS;

template <int TT, int EPI>
__global__ __launch_bounds__((NWC + NLD) * 64) void w4t_gemm_kernel(GemmParams p) {
  constexpr int RG = NWC;
  constexpr int FRAG = TT * 4;         // 1 KB activation fragment blocks per chunk
  constexpr int NT = RG * NR;          // weight tiles per block
  constexpr int LOADS = FRAG + NT + 1; // loader instructions per chunk
#ifndef SS_TILED_LA
#define SS_TILED_LA 8
#endif
  constexpr int LA1 = 63 / LOADS < NS_T / NLD ? 63 / LOADS : NS_T / NLD;
  constexpr int LA0 = LA1 < SS_TILED_LA ? LA1 : SS_TILED_LA;
  constexpr int LA = LA0 < 1 ? 1 : LA0;   // chunks in flight per loader
  static_assert(NT * 8 == 64, "one load carries the (scale, zero) words of all tiles");
  static_assert(NS_T % NLD == 0, "slot ring must split evenly");
  __shared__ u32x4_t xfrag[NS_T][4][TT][64];
  __shared__ u32x4_t wfrag[NS_T][NT][64];
  __shared__ uint32_t wsz[NS_T][NT * 32];
  __shared__ int ready[NS_T], done[NS_T];
  __shared__ float rs_all[256];    // RMSNorm row scales of all tokens (consumer GEMMs)
  __shared__ int rs_done;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = blockIdx.x;
  const SegList L = make_segs(p, g);
  const int nsegs = L.nd + L.nsk;

  if (tid < NS_T) {
    ready[tid] = -1;
    done[tid] = 0;
  }
  if (tid < 256) rs_all[tid] = 0.f;
  if (tid == 0) rs_done = 0;
  __syncthreads();   // the only workgroup barrier

  if (wave >= NWC) {
    // ---------------- loader wave l copies the chunks with sequence number qc = 2 k + l,
    // keeping LA chunks in flight; before waiting for a slot it drains and publishes
    // everything it has issued (no consumer can be waiting on a chunk it holds back)
    const int l = wave - NWC;
    const int li = lane & 15, lb = lane >> 4;
    int n = 0, ns = 0, qs = 0;
    auto publish = [&](int upto) {
      for (; ns < upto; ++ns) {
        const int qd = NLD * ns + l;
        if (lane == 0) lds_store(&ready[qd % NS_T], qd);
      }
    };
    for (int k = 0; k < nsegs; ++k) {
      int block, s0, s1;
      seg_of(p, L, g, k, block, s0, s1);
      const int tb = block % p.tb_count, rb = block / p.tb_count;
      // global tile of each of the block's weight tiles (rows past N: tile 0, never used)
      size_t tile_off[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int rgi = i / NR, ri = i % NR;
        const size_t tile = tile_valid<EPI, RG>(p, rb, rgi, ri) ? (size_t)(tile_row<EPI, RG>(p, rb, rgi, ri, 0) >> 4) : 0;
        tile_off[i] = tile * p.nchunks * TILE_BLOCK_BYTES;
      }
      for (int st = s0; st < s1; ++st, ++qs) {
        const int qc = qs;
        if (qc % NLD != l) continue;
        const int slot = qc % NS_T;
        if (qc >= NS_T) {
          const int need = RG * (qc / NS_T);   // the previous occupant was read by all compute waves
          if (__hip_atomic_load(&done[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            publish(n);
            wait_ge(&done[slot], need);
          }
        }
        const int ch = st;
        const uint16_t* src = p.x + (size_t)ch * CHUNK_K + lb * 32;
#pragma unroll
        for (int ps = 0; ps < FRAG; ++ps) {
          const int m = ps & 3, tt = ps >> 2;
          const int tok = min(tb * 64 + tt * 16 + li, p.T - 1);   // padded tokens: clamped copies
          __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)tok * p.K + m * 8),
                                           (__attribute__((address_space(3))) void*)&xfrag[slot][m][tt][0],
                                           16, 0, 0);
        }
        const size_t cb = (size_t)ch * TILE_BLOCK_BYTES;
#pragma unroll
        for (int i = 0; i < NT; ++i)
          __builtin_amdgcn_global_load_lds((const void*)(p.qw + tile_off[i] + cb + lane * 16),
                                           (__attribute__((address_space(3))) void*)&wfrag[slot][i][0], 16, 0, 0);
        // (scale, zero) words: lane -> tile lane / 8, 16-byte piece lane % 8
        size_t so = tile_off[0];
#pragma unroll
        for (int i = 1; i < NT; ++i)
          if ((lane >> 3) == i) so = tile_off[i];
        __builtin_amdgcn_global_load_lds((const void*)(p.qw + so + cb + 1024 + (lane & 7) * 16),
                                         (__attribute__((address_space(3))) void*)&wsz[slot][0], 16, 0, 0);
        ++n;
        if (n - ns > LA) {
          // all but the newest LA chunks have landed in LDS
          __builtin_amdgcn_s_waitcnt(((LA * LOADS) & 0xF) | 0x0F70 | (((LA * LOADS) >> 4) << 14));
          publish(n - LA);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    publish(n);
    return;
  }

  // ---------------- compute waves: row group rg = wave
  const int rg = wave;
  const int j = lane & 15, b = lane >> 4;
  f32x4_t acc[NR][TT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (p.ssq_in) row_scales(p, rg, NWC, lane, rs_all, &rs_done);
  bool rs_seen = false;
  int qs = 0;
  for (int k = 0; k < nsegs; ++k) {
    int block, s0, s1;
    seg_of(p, L, g, k, block, s0, s1);
    for (int st = s0; st < s1; ++st, ++qs) {
      const int xs = qs % NS_T;
      wait_eq(&ready[xs], qs);
      bf16x8_t xa[4][TT];
      u32x4_t wv[NR];
      uint32_t szv[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        wv[r] = wfrag[xs][rg * NR + r][lane];
        szv[r] = wsz[xs][(rg * NR + r) * 32 + j * 2 + (b >> 1)];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t) xa[m][t] = __builtin_bit_cast(bf16x8_t, xfrag[xs][m][t][lane]);
      float sf[NR], cf[NR], sf16[NR], cf16[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        sf[r] = f16lo(szv[r]);
        const float zf = f16hi(szv[r]);
        cf[r] = -(1024.0f + zf) * sf[r];   // 1024 + z is exact in fp32
        sf16[r] = sf[r] * 0.0625f;         // exact
        cf16[r] = -(64.0f + zf) * sf[r];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const u32x4_t w = wv[r];
          const u32x4_t d = dequant8(m == 0 ? w.x : m == 1 ? w.y : m == 2 ? w.z : w.w, sf[r], cf[r], sf16[r], cf16[r]);
#pragma unroll
          for (int t = 0; t < TT; ++t)
            acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[m][t], __builtin_bit_cast(bf16x8_t, d), acc[r][t], 0, 0, 0);
        }
      }
      // the slot is released after the chunk's math: its reads land while the first k-steps
      // are multiplied (the compiler waits for each fragment at its first use); every read
      // has returned before the release; one increment per wave
      compiler_fence();
      lds_wait();
      if (lane == 0) __hip_atomic_fetch_add(&done[xs], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // end of segment: the result, or the partial of a block split between workgroups
    // (partials carry the row scales too: the reduce adds scaled pieces)
    if (p.ssq_in) {
      if (!rs_seen) {
        wait_ge(&rs_done, NWC);
        rs_seen = true;
      }
      apply_row_scales<TT>(acc, rs_all + (block % p.tb_count) * 64, lane);
    }
    if (s0 == 0 && s1 == p.nsteps) {
      final_store<TT, EPI, RG>(p, acc, block, rg, lane);
    } else {
      float* part = p.partials + ((size_t)sk_slot(p, g, block - p.sk_first) * RG + rg) * (NR * TT * 4 * 64);
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) part[((r * TT + t) * 4 + e) * 64 + lane] = acc[r][t][e];
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Blocks split between workgroups: every thread owns one output element (for SwiGLU,
// one gate / up pair) of one block, adds the pieces' partials in K order (a fixed
// order, so results do not depend on timing) and applies the epilogue. A block that
// one workgroup covered whole was stored by the GEMM kernel itself.
template <int TT, int EPI, int KS>
__global__ __launch_bounds__(256) void sk_reduce_kernel(GemmParams p) {
  constexpr int RG = NWC / KS;
  constexpr int NRE = (EPI == EPI_SWIGLU) ? 1 : NR;   // tiles handled per thread set
  constexpr int PER_BLOCK = RG * NRE * TT * 4 * 64;
  const int sb = blockIdx.x;
  const int idx = blockIdx.y * 256 + threadIdx.x;
  if (idx >= PER_BLOCK) return;
  const long long u0 = (long long)sb * p.nsteps;
  const int g0 = sk_owner(p, u0), g1 = sk_owner(p, u0 + p.nsteps - 1);
  if (g0 == g1) return;
  const int lane = idx & 63;
  const int e = (idx >> 6) & 3;
  const int t = (idx >> 8) % TT;
  const int r = (idx >> 8) / TT % NRE;
  const int rg = (idx >> 8) / TT / NRE;
  const int block = p.sk_first + sb;
  const int tb = block % p.tb_count, rb = block / p.tb_count;
  const int j = lane & 15, bq = lane >> 4;
  const int tok = tb * 64 + t * 16 + 4 * bq + e;
  if (tok >= p.T || !tile_valid<EPI, RG>(p, rb, rg, r)) return;
  // piece slots: every piece after the first starts its workgroup's range inside this
  // block (slot 2 gk); the first piece is its workgroup's first or second block
  const size_t slot_elems = (size_t)RG * NR * TT * 4 * 64;
  const size_t off = (size_t)rg * (NR * TT * 4 * 64) + ((r * TT + t) * 4 + e) * 64 + lane;
  const size_t off1 = (size_t)rg * (NR * TT * 4 * 64) + ((1 * TT + t) * 4 + e) * 64 + lane;
  auto piece = [&](int gk) { return p.partials + (gk == g0 ? sk_slot(p, g0, sb) : 2 * gk) * slot_elems; };
  float v0 = 0.f, v1 = 0.f;
  int gk = g0;
  for (; gk + 4 <= g1 + 1; gk += 4) {   // four independent loads in flight, added in order
    float a[4], c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = piece(gk + i)[off];
      c[i] = EPI == EPI_SWIGLU ? piece(gk + i)[off1] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v0 += a[i];
      v1 += c[i];
    }
  }
  for (; gk <= g1; ++gk) {
    v0 += piece(gk)[off];
    if (EPI == EPI_SWIGLU) v1 += piece(gk)[off1];
  }
  const int n = tile_row<EPI, RG>(p, rb, rg, r, j);
  if (EPI == EPI_SWIGLU) {
    p.u_bf16[(size_t)tok * p.swiglu_I + n] = f32_to_bf16(silu_f32(v0) * v1);
  } else {
    const size_t o = (size_t)tok * p.N + n;
    if (EPI == EPI_RESID) {
      p.resid[o] += v0;
    } else {
      if (p.y_f32) p.y_f32[o] = v0;
      if (p.y_bf16) p.y_bf16[o] = f32_to_bf16(v0);
    }
  }
}

// ------------------------------------------------------------------ host side

namespace {
#ifndef SS_GEMM_PF
#define SS_GEMM_PF 4
#endif
#ifndef SS_GEMM_PFB
#define SS_GEMM_PFB 2
#endif
#ifndef SS_GEMM_KS
#define SS_GEMM_KS 1
#endif
constexpr int kPF = SS_GEMM_PF;     // int4 weight steps in flight per wave
constexpr int kPFB = SS_GEMM_PFB;   // bf16 weight steps in flight per wave

template <int TT, bool INT4, int EPI, int KS>
hipError_t launch_k(const GemmParams& p, int sk_blocks, bool defer, bool tiled, hipStream_t st) {
  constexpr int PF = INT4 ? kPF : kPFB;
  constexpr bool CAN_SZO = INT4 && KS == 1;
  const bool aligned16 = (reinterpret_cast<uintptr_t>(p.sc) % 16 == 0) && (reinterpret_cast<uintptr_t>(p.zp) % 16 == 0);
  if (INT4 && KS == 1 && tiled)
    hipLaunchKernelGGL((w4t_gemm_kernel<TT, EPI>), dim3(p.G), dim3((NWC + NLD) * 64), 0, st, p);
  else if (CAN_SZO && p.K % 512 == 0 && aligned16)
    hipLaunchKernelGGL((w4_gemm_kernel<TT, INT4, EPI, KS, PF, CAN_SZO>), dim3(p.G), dim3((NWC + NLD + 1) * 64), 0, st, p);
  else
    hipLaunchKernelGGL((w4_gemm_kernel<TT, INT4, EPI, KS, PF, false>), dim3(p.G), dim3((NWC + NLD) * 64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sk_blocks == 0 || defer) return e;
  constexpr int per_block = (NWC / KS) * (EPI == EPI_SWIGLU ? 1 : NR) * TT * 4 * 64;
  hipLaunchKernelGGL((sk_reduce_kernel<TT, EPI, KS>), dim3(sk_blocks, (per_block + 255) / 256), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <bool INT4, int EPI, int KS>
hipError_t launch_tt(const GemmParams& p, int TT, int skb, bool defer, bool tiled, hipStream_t st) {
  switch (TT) {
    case 1: return launch_k<1, INT4, EPI, KS>(p, skb, defer, tiled, st);
    case 2: return launch_k<2, INT4, EPI, KS>(p, skb, defer, tiled, st);
    case 3: return launch_k<3, INT4, EPI, KS>(p, skb, defer, tiled, st);
    default: return launch_k<4, INT4, EPI, KS>(p, skb, defer, tiled, st);
  }
}

template <int EPI>
hipError_t launch_epi(const GemmParams& p, bool int4, int TT, int KS, int skb, bool defer, bool tiled, hipStream_t st) {
  if (KS == 1) return int4 ? launch_tt<true, EPI, 1>(p, TT, skb, defer, tiled, st) : launch_tt<false, EPI, 1>(p, TT, skb, defer, tiled, st);
  return int4 ? launch_tt<true, EPI, 2>(p, TT, skb, defer, tiled, st) : launch_tt<false, EPI, 2>(p, TT, skb, defer, tiled, st);
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
}  // namespace

GemmPlan plan_gemm(int T, int N, int K, int epi, int swiglu_I) {
  GemmPlan pl{};
  pl.KS = SS_GEMM_KS;
  const int RG = NWC / pl.KS;
  pl.TT = (T >= 64) ? 4 : (T + 15) / 16;
  const int rows_per_block = (epi == EPI_SWIGLU) ? RG * 16 : RG * 32;
  const int span = (epi == EPI_SWIGLU) ? swiglu_I : N;
  pl.rb_count = std::max(1, (span + rows_per_block - 1) / rows_per_block);
  pl.tb_count = std::max(1, (T + 63) / 64);
  pl.nchunks = std::max(1, K / CHUNK_K);
  pl.nsteps = (pl.nchunks + pl.KS - 1) / pl.KS;
  const int blocks = pl.rb_count * pl.tb_count;
  const int G = SS_GEMM_WGS;
  pl.dp_rounds = blocks / G;
  pl.sk_first = pl.dp_rounds * G;
  pl.sk_blocks = blocks - pl.sk_first;
  pl.sk_units = (long long)pl.sk_blocks * pl.nsteps;
  const long long min_piece = std::max(1, SS_GEMM_MIN_PIECE);
  pl.G_sk = pl.sk_units > 0 ? (int)std::min<long long>(G, std::max<long long>(1, pl.sk_units / min_piece)) : 0;
  pl.G = pl.dp_rounds > 0 ? G : std::max(1, pl.G_sk);
  const size_t slot_bytes = (size_t)RG * NR * pl.TT * 4 * 64 * sizeof(float);
  pl.ws_bytes = pl.sk_blocks > 0 ? align256(2 * (size_t)pl.G_sk * slot_bytes) : 0;
  return pl;
}

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& pl, void* ws, hipStream_t st) {
  GemmParams p{};
  p.x = a.x; p.qw = a.qw; p.sc = a.sc; p.zp = a.zp; p.wb = a.wb;
  p.T = a.T; p.N = a.N; p.K = a.K;
  p.swiglu_I = a.swiglu_I;
  p.y_f32 = a.y_f32; p.y_bf16 = a.y_bf16; p.resid = a.resid; p.u_bf16 = a.u_bf16;
  p.nchunks = pl.nchunks;
  p.nsteps = pl.nsteps;
  p.tb_count = pl.tb_count;
  p.G = pl.G;
  p.dp_rounds = pl.dp_rounds;
  p.sk_first = pl.sk_first;
  p.G_sk = pl.G_sk;
  p.sk_units = pl.sk_units;
  p.partials = pl.sk_blocks > 0 ? reinterpret_cast<float*>(ws) : nullptr;
  p.ssq_in = a.ssq_in;
  p.ssq_n = a.ssq_n;
  p.rms_H = a.rms_H;
  p.rms_eps = a.rms_eps;
  p.hg_out = a.hg_out;
  p.hg_gain = a.hg_gain;
  p.ssq_out = a.ssq_out;
  // producers of RMSNorm inputs leave split blocks to resid_finish (deferred reduce);
  // consumers need a 16-byte aligned sum table of whole float4s
  if (a.hg_out && (a.epi != EPI_RESID || !a.ssq_out || !a.hg_gain || (pl.sk_blocks > 0 && !a.defer_reduce)))
    return hipErrorInvalidValue;
  if (a.ssq_in && ((a.ssq_n & 3) || (reinterpret_cast<uintptr_t>(a.ssq_in) & 15) || a.epi == EPI_RESID))
    return hipErrorInvalidValue;
  const bool int4 = a.qw != nullptr;
  const bool defer = a.defer_reduce && a.epi != EPI_SWIGLU;
  // the tiled kernel has one K phase; plan_gemm's default (KS = 1) is what it needs
  const bool tiled = int4 && a.tiled;
  if (tiled && pl.KS != 1) return hipErrorInvalidValue;
  switch (a.epi) {
    case EPI_RESID: return launch_epi<EPI_RESID>(p, int4, pl.TT, pl.KS, pl.sk_blocks, defer, tiled, st);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(p, int4, pl.TT, pl.KS, pl.sk_blocks, false, tiled, st);
    default: return launch_epi<EPI_STORE>(p, int4, pl.TT, pl.KS, pl.sk_blocks, defer, tiled, st);
  }
}

SplitView gemm_split_view(const GemmPlan& pl, const void* ws) {
  SplitView v{};
  v.partials = pl.sk_blocks > 0 ? static_cast<const float*>(ws) : nullptr;
  v.RG = NWC / pl.KS;
  v.TT = pl.TT;
  v.tb_count = pl.tb_count;
  v.rows_per_block = v.RG * 32;
  v.rb_count = pl.rb_count;
  v.nsteps = pl.nsteps;
  v.G_sk = pl.G_sk;
  v.sk_first = pl.sk_first;
  v.sk_units = pl.sk_units;
  return v;
}

}  // namespace ss
