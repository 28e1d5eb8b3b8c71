// The W4A16 GEMM kernel of gemm_w4.hip (its design notes are there), instantiated per
// token-tile count in gemm_w4_tt{1,2,3,4}.hip so the instantiations compile in parallel.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ss {

namespace w4 {
constexpr int KP = 4;           // K phases; wave w runs on SIMD w % 4
constexpr int RGW = 2;          // row groups: two waves per SIMD, each its own tiles
constexpr int NWV = KP * RGW;
constexpr int CHK = 128;        // chunk width (k)
constexpr int MAX_WGS = 256;    // one workgroup per CU
constexpr int SSQ_MAX = 32;     // folded RMSNorm: at most 32 partial sums per token (H <= 8192)

// 16-row tiles a wave can hold (= logical tiles of a unit: each row group takes one half of
// every logical tile): the 256 registers of each of the two waves of a SIMD (accumulation
// registers included) hold the accumulators, three super-chunks of weights and the
// dequantization operands.
constexpr int tpw_max(int TT, int) { return TT <= 2 ? 6 : 5; }
// weight register slots: super-chunk s (math) and PD = SLOTS - 1 ahead of it
constexpr int slots_of(int) { return 3; }
}  // namespace w4

struct W4Params {
  const uint16_t* x;    // bf16 [T][K]
  const uint8_t* qw;    // tiled blocks, or plain codes [N][K/2]
  const uint16_t* sc;   // plain layout: fp16 [N][K/64]
  const uint16_t* zp;
  int T, N, K, nch;
  int swiglu_I;
  int NL, n_groups, splits, tb_count, units;
  int nout;             // columns of a partial slice: N, or 2 I for SwiGLU
  float* y_f32;
  uint16_t* y_bf16;
  float* resid;
  uint16_t* u_bf16;
  float* part;          // splits > 1: fp32 [splits][T][nout]
  const float* ssq_in;  // folded RMSNorm: rows scaled by 1/sqrt(sum ssq_in[t][:] / rms_H + eps)
  int ssq_n, rms_H;
  float rms_eps;
};

// launchers of the instantiations (one per token-tile count)
void launch_w4_tt1(const W4Params& p, int tpw, int epi, bool tiled, int G, hipStream_t st);
void launch_w4_tt2(const W4Params& p, int tpw, int epi, bool tiled, int G, hipStream_t st);
void launch_w4_tt3(const W4Params& p, int tpw, int epi, bool tiled, int G, hipStream_t st);
void launch_w4_tt4(const W4Params& p, int tpw, int epi, bool tiled, int G, hipStream_t st);

namespace w4 {

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
// (a & m) | c, one v_and_or_b32: m and c come from opaque_vgpr, so the compiler cannot
// fold them into literals (a VOP3 instruction takes none; it would split the operation in
// an AND and an OR)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) { return (a & m) | c; }
// a constant in a VGPR whose value the compiler does not know
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(v));
  return r;
}
// VALU instructions of one dequant8 (one shift, four and-or, eight fma_mix, four packs)
constexpr int DQV = 17;

// Issue order for the scheduler over one super-chunk's math (four k-steps): per k-step its
// share of the pipeline's register loads, the next fragments' LDS reads, the first tile's
// dequantization, then each MFMA followed by its share of the next tile's dequantization
// (MFMA and VALU of one wave overlap only when interleaved). The masks are LLVM's
// scheduling-group classes: 0x2 VALU, 0x8 MFMA, 0x20 VMEM read, 0x100 LDS read. Pipeline
// list: NA direct-to-LDS loads (inline asm, not counted), then TPW register loads.
template <int TT, int TPW, int X>
__device__ __forceinline__ void sched_tiles() {
  if constexpr (X < TPW * TT) {
    constexpr int i = X / TT, t = X % TT;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (i + 1 < TPW) __builtin_amdgcn_sched_group_barrier(0x002, DQV / TT + (t < DQV % TT ? 1 : 0), 0);
    sched_tiles<TT, TPW, X + 1>();
  }
}
template <int TT, int TPW, int NA, int NLA, int M>
__device__ __forceinline__ void sched_compute() {
  if constexpr (M < 4) {
    constexpr int lo = M * NLA / 4, hi = (M + 1) * NLA / 4;
    constexpr int vlo = lo > NA ? lo : NA, vhi = hi < NA + TPW ? hi : NA + TPW;
    if constexpr (vhi > vlo) __builtin_amdgcn_sched_group_barrier(0x020, vhi - vlo, 0);
    if constexpr (M < 3) __builtin_amdgcn_sched_group_barrier(0x100, TT, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, M == 0 ? DQV + 6 * TPW : DQV, 0);
    sched_tiles<TT, TPW, 0>();
    sched_compute<TT, TPW, NA, NLA, M + 1>();
  }
}
// Masks and fp16 bases of the dequantization, kept in registers.
struct DqConst {
  uint32_t me, mo, x1024, x64;
};
// 8 codes of one 32-bit word (k = e for nibble e) -> 8 bf16 weights (q - z) s. Even
// nibbles (bits 0-3 of each half) OR-ed into fp16 1024.0 give 1024 + q; odd nibbles
// (bits 4-7) OR-ed into fp16 64.0, whose mantissa unit there is 1/16 * 16 = 1, give 64 + q;
// both exact. v_fma_mix_f32 evaluates (base + q) s + c straight from the fp16 half with
// c = -(base + z) s rounded once to fp32; one shift per word brings nibbles 2, 3, 6, 7 down.
__device__ __forceinline__ u32x4_t dequant8(uint32_t q, float s, float c1024, float c64, const DqConst& k) {
  const uint32_t qh = q >> 8;
  const uint32_t h04 = and_or(q, k.me, k.x1024);    // 1024 + q0 | 1024 + q4
  const uint32_t h15 = and_or(q, k.mo, k.x64);      //   64 + q1 |   64 + q5
  const uint32_t h26 = and_or(qh, k.me, k.x1024);   // 1024 + q2 | 1024 + q6
  const uint32_t h37 = and_or(qh, k.mo, k.x64);     //   64 + q3 |   64 + q7
  const float w0 = __builtin_fmaf(f16lo(h04), s, c1024), w4 = __builtin_fmaf(f16hi(h04), s, c1024);
  const float w1 = __builtin_fmaf(f16lo(h15), s, c64), w5 = __builtin_fmaf(f16hi(h15), s, c64);
  const float w2 = __builtin_fmaf(f16lo(h26), s, c1024), w6 = __builtin_fmaf(f16hi(h26), s, c1024);
  const float w3 = __builtin_fmaf(f16lo(h37), s, c64), w7 = __builtin_fmaf(f16hi(h37), s, c64);
  return u32x4_t{pk_bf16(w0, w1), pk_bf16(w2, w3), pk_bf16(w4, w5), pk_bf16(w6, w7)};
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)
// workgroup barrier without the vmcnt(0) drain a full fence would add (weights stay in flight)
__device__ __forceinline__ void wg_barrier() {
  compiler_fence();
  lds_wait();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}
// Direct-to-LDS loads (global_load_lds_dword / _dwordx4: lane l's bytes land at LDS address
// m0 + 4 l / 16 l), written as inline asm. The compiler's wait insertion treats a pending
// builtin LDS load as a possible alias of every later LDS read and drains all loads before
// it (vmcnt(0)), which would stop the weight prefetch at every super-chunk. These loads have
// no output registers, so hiding them from the compiler is safe: its own waits for the
// register loads can only be stricter than needed, and the explicit vmcnt waits plus the
// workgroup barrier order every LDS read after the data has landed. m0 is written one wait
// state before the load reads it.
// m0 is saved and restored around the load (the compiler owns it).
__device__ __forceinline__ void dma16(const void* gptr, const void* lds) {
  const uint32_t l = (uint32_t)(uintptr_t)lds;
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(gptr), "s"(l) : "memory");
}
__device__ __forceinline__ void dma4(const void* gptr, const void* lds) {
  const uint32_t l = (uint32_t)(uintptr_t)lds;
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(gptr), "s"(l) : "memory");
}
// A wave-uniform 64-bit address kept in scalar registers, so loads use it as the base with
// a 32-bit per-lane offset (no 64-bit address arithmetic per lane).
__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}
template <int N>
__device__ __forceinline__ void vm_wait_c() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | 0x0F70 | ((N >> 4) << 14));
}

// TPW 16-row tiles per wave (the planner's largest group of logical tiles), TT token tiles.
// Row group 0 takes the first 16-row tile of every logical tile of the unit (for SwiGLU the
// gate tiles), row group 1 the second (the up tiles), so the two waves of a SIMD carry the
// same work.
template <int TT, int EPI, bool TILED, int TPW>
__global__ __launch_bounds__(NWV * 64) void w4k_kernel(W4Params p) {
  constexpr int SLOTS = slots_of(TT);
  constexpr int PD = SLOTS - 1;
  constexpr int NTOK = TT * 16;
  constexpr int NSZ = (TPW + 1) / 2;   // (scale, zero) loads per super-chunk: two tiles each
  // activation rows of a super-chunk: [buffer][chunk][token][16 units of 16 bytes], unit u of
  // token t stored at position u ^ (t % 16) (no LDS bank conflicts for the fragment reads)
  __shared__ __align__(16) u32x4_t act[2][KP][NTOK][16];
  __shared__ __align__(16) uint32_t szl[NWV][SLOTS][NSZ][2][32];   // scale / zero words, two tiles a load
  __shared__ float rs_all[64];                                      // folded RMSNorm scales of a token block

  // the wave index is the same for all lanes of a wave: keep it (and all that derives from
  // it: tiles, chunks, branches) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kp = wave % KP, rg = wave / KP;
  const int j = lane & 15, b = lane >> 4;
  const int nt16 = p.N >> 4;                 // 16-row tiles of the weight
  const int swI16 = p.swiglu_I >> 4;
  DqConst dk;
  dk.me = opaque_vgpr(0x000F000Fu);
  dk.mo = opaque_vgpr(0x00F000F0u);
  dk.x1024 = opaque_vgpr(0x64006400u);
  dk.x64 = opaque_vgpr(0x54005400u);


  // per-lane part of the weight addresses (plain layout): row j of a tile, k slice of b
  const uint32_t lane_q = (uint32_t)j * (uint32_t)(p.K >> 1) + (uint32_t)b * 16;

  for (int u = blockIdx.x; u < p.units; u += gridDim.x) {
    const int sp = u % p.splits;
    const int grp = (u / p.splits) % p.n_groups;
    const int tb = u / (p.splits * p.n_groups);
    const int L0 = (int)((long long)grp * p.NL / p.n_groups);
    const int cnt = (int)((long long)(grp + 1) * p.NL / p.n_groups) - L0;   // <= TPW (planner)
    const int c0 = (int)((long long)sp * p.nch / p.splits);
    const int c1 = (int)((long long)(sp + 1) * p.nch / p.splits);
    const int S = (c1 - c0 + KP - 1) / KP;

    // the wave's 16-row tiles: tile i is the rg-th half of logical tile L0 + i. Index and
    // validity are wave-uniform. Every wave issues the same, compile-time number of loads
    // per super-chunk (missing tiles and the steps past the end re-load a tile or chunk it
    // already reads, which the L2 serves), so the compiler's own wait counts stay exact and
    // never drain the prefetch; a missing tile multiplies a duplicate (never stored).
    int pt[TPW];
    bool pv[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int L = L0 + i;
      const int t = EPI == EPI_SWIGLU ? (rg == 0 ? L : swI16 + L) : 2 * L + rg;
      pv[i] = i < cnt && t < nt16;
      pt[i] = pv[i] ? t : (EPI == EPI_SWIGLU ? (rg == 0 ? L0 : swI16 + L0) : min(2 * L0, nt16 - 1));
    }

    f32x4_t acc[TPW][TT];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wq[SLOTS][TPW];

    // wave-uniform bases of the wave's tiles at chunk 0 (scalar registers): tiled, the tile's
    // first block; plain, its first row of codes
    const uint8_t* tbase[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      tbase[i] = uniform_ptr(TILED ? p.qw + (size_t)pt[i] * p.nch * TILE_BLOCK_BYTES
                                   : p.qw + (size_t)pt[i] * 16 * (size_t)(p.K >> 1));
    // (scale, zero) words of two tiles go straight into LDS in one 4-byte-per-lane load,
    // lanes 0-31 tile 2 n, 32-63 tile 2 n + 1 (the last load of an odd count repeats).
    // Tiled: word 2 j + h = (scale | zero << 16) of row j, group 2 c + h. Plain: lane
    // (r, half, jj) = (l / 32, l / 16 % 2, l % 16) carries the scale (half 0) or zero
    // (half 1) pair of groups 2 c, 2 c + 1 of row jj. Tiled, per-lane byte offset from the
    // first tile's base at chunk 0 (signed: a missing tile repeats an earlier one):
    int szoff[NSZ];
#pragma unroll
    for (int n = 0; n < NSZ; ++n) {
      const int i0 = 2 * n, i1 = min(2 * n + 1, TPW - 1);
      szoff[n] = (lane < 32 ? 0 : (int)(tbase[i1] - tbase[i0])) + 1024 + 4 * (lane & 31);
    }
    // the loads that keep the pipeline full, in the order they are issued during a
    // super-chunk's math: NA activation loads of super-chunk s + 1, then the TPW weight
    // loads and NSZ (scale, zero) loads of super-chunk s + PD
    constexpr int NA = KP * 4 * TT / NWV;
    constexpr int NL_ALL = NA + TPW + NSZ;
    // activation load x of super-chunk s into buffer s & 1: per chunk q of the super-chunk,
    // one 1 KB load per group of 4 tokens (4 rows x 256 contiguous bytes: whole cache
    // lines), 16 TT loads in all, wave w taking loads w, w + 8, ...; lane i of a load
    // carries token 4 g + i / 16, unit (i % 16) ^ (token % 16). A chunk past the unit's
    // range is replaced by its last chunk (never read); padded tokens are clamped copies.
    auto load_a1 = [&](int s, int x) {
      const int buf = s & 1;
      const int sc = min(s, S - 1);
      const int l = wave + NWV * x;
      const int q = l / (4 * TT), g = l % (4 * TT);
      const int c = min(c0 + sc * KP + q, c1 - 1);
      const int t = 4 * g + (lane >> 4);
      const int unit = (lane & 15) ^ (t & 15);
      const int tok = min(tb * 64 + t, p.T - 1);
      const uint16_t* src = p.x + (size_t)tok * p.K + (size_t)c * CHK + unit * 8;
      dma16(src, &act[buf][q][4 * g][0]);
    };
    // weight load i (i < TPW: codes of tile i; else scale / zero load i - TPW) of this
    // wave's chunk of super-chunk s (clamped into the unit's range) into slot q
    auto load_w1 = [&](int s, int i, auto slot_c) {
      constexpr int q = decltype(slot_c)::value;
      const int c = min(c0 + min(s, S - 1) * KP + kp, c1 - 1);
      if (i < TPW) {
        const uint32_t off = TILED ? (uint32_t)c * TILE_BLOCK_BYTES + lane * 16 : (uint32_t)c * 64 + lane_q;
        wq[q][i] = *reinterpret_cast<const u32x4_t*>(tbase[i] + off);
      } else {
        const int n = i - TPW;
        if (TILED) {
          dma4(tbase[2 * n] + (long long)szoff[n] + (size_t)c * TILE_BLOCK_BYTES, &szl[wave][q][n][0][0]);
        } else {
          const int half = (lane >> 4) & 1, jj = lane & 15;
          const size_t row = (size_t)(lane < 32 ? pt[2 * n] : pt[min(2 * n + 1, TPW - 1)]) * 16 + jj;
          dma4((half ? p.zp : p.sc) + row * (size_t)(p.K >> 6) + (size_t)c * 2, &szl[wave][q][n][0][0]);
        }
      }
    };
    // load y of the pipeline list during super-chunk s's math (slot q of super-chunk s)
    auto issue = [&](int s, int y, auto slot_c) {
      constexpr int q = decltype(slot_c)::value;
      if (y < NA) load_a1(s + 1, y);
      else load_w1(s + PD, y - NA, std::integral_constant<int, (q + PD) % SLOTS>{});
    };
    auto compute = [&](int s, auto slot_c) {
      constexpr int q = decltype(slot_c)::value;
      const int c = c0 + s * KP + kp;
      if (c >= c1) {
        // no math for this wave in super-chunk s (past the unit's range): loads only
#pragma unroll
        for (int y = 0; y < NL_ALL; ++y) issue(s, y, slot_c);
        return;
      }
      const int buf = s & 1;
      // scale and the two offsets per tile, once per super-chunk (a missing tile multiplies
      // a duplicate of another tile's data; its sums are never stored)
      float sf[TPW], c1k[TPW], c64[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        float sv, zf;
        const int n = i >> 1, r = i & 1;
        if (TILED) {
          const uint32_t w = szl[wave][q][n][r][2 * j + (b >> 1)];
          sv = f16lo(w);
          zf = f16hi(w);
        } else {
          const int sh = (b >> 1) * 16;   // group 2 c + (b >> 1)
          sv = f16lo(szl[wave][q][n][r][j] >> sh);
          zf = f16lo(szl[wave][q][n][r][16 + j] >> sh);
        }
        sf[i] = sv;
        c1k[i] = -(1024.0f + zf) * sv;
        c64[i] = -(64.0f + zf) * sv;
      }
      // fragments of k-step m: token row 16 t + j, unit 4 b + m (k = 32 b + 8 m .. + 7 of
      // the chunk); the next k-step's are read while this one is multiplied
      auto frag = [&](int m, int t) {
        const int tok = 16 * t + j;
        return __builtin_bit_cast(bf16x8_t, act[buf][kp][tok][(4 * b + m) ^ j]);
      };
      constexpr int XB = TT >= 3 ? 1 : 2;
      bf16x8_t xa[2][TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) xa[0][t] = frag(0, t);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // this k-step's share of the pipeline loads (the memory path works on them while
        // the VALU dequantizes; a burst at the super-chunk start would stall every wave)
#pragma unroll
        for (int y = m * NL_ALL / 4; y < (m + 1) * NL_ALL / 4; ++y) issue(s, y, slot_c);
        if (XB == 1 && m > 0) {
#pragma unroll
          for (int t = 0; t < TT; ++t) xa[m & 1][t] = frag(m, t);
        }
        if (XB == 2 && m + 1 < 4) {
#pragma unroll
          for (int t = 0; t < TT; ++t) xa[(m + 1) & 1][t] = frag(m + 1, t);
        }
        // the tiles of this k-step, software-pipelined: tile i + 1 is dequantized while
        // tile i's MFMAs run. Every tile slot is computed (a group one tile smaller than the
        // largest multiplies a duplicate, never stored), so the k-step is straight-line code
        auto deq = [&](int i) {
          const u32x4_t w = wq[q][i];
          return dequant8(m == 0 ? w.x : m == 1 ? w.y : m == 2 ? w.z : w.w, sf[i], c1k[i], c64[i], dk);
        };
        u32x4_t dcur = deq(0);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          u32x4_t dnext = dcur;
          if (i + 1 < TPW) dnext = deq(i + 1);
#pragma unroll
          for (int t = 0; t < TT; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[m & 1][t], __builtin_bit_cast(bf16x8_t, dcur),
                                                                acc[i][t], 0, 0, 0);
          dcur = dnext;
        }
      }
#ifndef W4_NO_SCHED
      // (three or four token tiles: the interleaving costs more registers than the 256 a
      // wave has, and the MFMAs already keep the VALU work between them)
      if constexpr (TT <= 2) sched_compute<TT, TPW, NA, NL_ALL, 0>();
#endif
    };
    auto load_a = [&](int s) {
#pragma unroll
      for (int x = 0; x < NA; ++x) load_a1(s, x);
    };
    auto load_w = [&](int s, auto slot_c) {
#pragma unroll
      for (int i = 0; i < TPW + NSZ; ++i) load_w1(s, i, slot_c);
    };
    // one super-chunk: wait for its activations and weights, barrier, then its math with
    // the loads of act(s + 1) and w(s + PD) spread over it. The loads issued after act(s)
    // are those of w(s + PD - 1) (none left outstanding when PD == 1).
    auto step = [&](int s, auto slot_c) {
      if constexpr (PD >= 2) vm_wait_c<TPW + NSZ>();
      else vm_wait_c<0>();
      wg_barrier();   // every wave's share of act(s) has landed; buffer (s + 1) & 1 is free
      compute(s, slot_c);
    };

    load_a(0);
    load_w(0, std::integral_constant<int, 0>{});
    if constexpr (PD >= 2) load_w(1, std::integral_constant<int, 1>{});
    if (p.ssq_in && wave == 0) {
      // folded RMSNorm scales of the block's 64 tokens, lane = token: the partial sums in
      // order (fixed), loads issued after the first super-chunks' so their latency hides in
      // the pipeline fill; read in the epilogue, several barriers later. Loads are of
      // clamped in-bounds addresses with the unused values selected away (no branch around
      // a load, which would be waited for before the next is issued).
      const float* src = p.ssq_in + (size_t)min(tb * 64 + lane, p.T - 1) * p.ssq_n;
      float sum = 0.f;
#pragma unroll
      for (int e0 = 0; e0 < SSQ_MAX; e0 += 8) {
        if (e0 >= p.ssq_n) break;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = src[min(e0 + e, p.ssq_n - 1)];
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += e0 + e < p.ssq_n ? v[e] : 0.f;
      }
      rs_all[lane] = 1.0f / sqrtf(sum / (float)p.rms_H + p.rms_eps);
    }
    // rounds of SLOTS steps (the weight slot of a step is a compile-time index); the loads
    // issued during the last steps for super-chunks past S are clamped re-reads, drained below
    for (int s = 0; s < S; s += SLOTS) {
      step(s, std::integral_constant<int, 0>{});
      if (s + 1 >= S) break;
      step(s + 1, std::integral_constant<int, 1>{});
      if constexpr (SLOTS > 2) {
        if (s + 2 >= S) break;
        step(s + 2, std::integral_constant<int, 2 % SLOTS>{});
      }
    }
    vm_wait_c<0>();   // the loads past the end have landed before the LDS is reused


    // ---- K phases added through LDS (the activation buffers are free once every wave
    // has passed this barrier), per row group: (p0 + p2) + (p1 + p3)
    wg_barrier();
    f32x4_t* red = reinterpret_cast<f32x4_t*>(&act[0][0][0][0]);
    constexpr int SL = TPW * TT;   // f32x4 slices per wave
    static_assert(RGW * 2 * SL * 64 * 16 <= (int)sizeof(act), "reduction slots fit the activation buffers");
    auto slot_at = [&](int qq, int i, int t) { return red + ((size_t)((qq * 2 + rg) * SL + i * TT + t)) * 64 + lane; };
    // (a compiler fence per tile keeps the scheduler from hoisting every tile's LDS
    // traffic at once, which would need registers for all of it)
    auto put = [&](int qq) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
#pragma unroll
        for (int t = 0; t < TT; ++t) *slot_at(qq, i, t) = acc[i][t];
        compiler_fence();
      }
    };
    auto add = [&](int qq) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[i][t] += *slot_at(qq, i, t);
        compiler_fence();
      }
    };
    if (kp >= 2) put(kp - 2);
    wg_barrier();
    if (kp < 2) add(kp);
    wg_barrier();
    if (kp == 1) put(0);
    wg_barrier();
    // the sums of both row groups, scaled by the folded RMSNorm, to LDS in the layout
    // fin[logical tile i][half r][token tile t] (f32x4 per lane), over the slots of the
    // second level (free since the barrier before last): the epilogue is shared by all
    // eight waves
    f32x4_t* fin = red + (size_t)2 * SL * 64;
    auto fin_at = [&](int i, int r, int t) { return fin + ((size_t)((i * 2 + r) * TT + t)) * 64 + lane; };
    if (kp == 0) {
      add(0);
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          f32x4_t v = acc[i][t];
          if (p.ssq_in) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= rs_all[t * 16 + 4 * b + e];
          }
          *fin_at(i, rg, t) = v;
        }
        compiler_fence();
      }
    }
    wg_barrier();

    // ---- epilogue: wave w takes (logical tile i, token tile t) = (x / TT, x % TT) for
    // x = w, w + 8, ... Lane (j, b) holds tokens 16 t + 4 b + e of row j of each half.
    for (int x = wave; x < cnt * TT; x += NWV) {
      const int i = x / TT, t = x % TT;
      const int L = L0 + i;
      const f32x4_t v0 = *fin_at(i, 0, t), v1 = *fin_at(i, 1, t);
      const bool has1 = EPI == EPI_SWIGLU || 2 * L + 1 < nt16;
      if (p.splits > 1) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (r == 1 && !has1) continue;
          const int n = EPI == EPI_SWIGLU ? (r == 0 ? 16 * L + j : p.swiglu_I + 16 * L + j) : 32 * L + 16 * r + j;
          float* dst = p.part + (size_t)sp * p.T * p.nout + n;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = tb * 64 + t * 16 + 4 * b + e;
            if (tok < p.T) dst[(size_t)tok * p.nout] = r ? v1[e] : v0[e];
          }
        }
      } else if (EPI == EPI_SWIGLU) {
        const int g = 16 * L + j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = tb * 64 + t * 16 + 4 * b + e;
          if (tok < p.T) p.u_bf16[(size_t)tok * p.swiglu_I + g] = f32_to_bf16(silu_f32(v0[e]) * v1[e]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (r == 1 && !has1) continue;
          const int n = 32 * L + 16 * r + j;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = tb * 64 + t * 16 + 4 * b + e;
            if (tok >= p.T) continue;
            const size_t o = (size_t)tok * p.N + n;
            const float v = r ? v1[e] : v0[e];
            if (EPI == EPI_RESID) {
              p.resid[o] += v;
            } else {
              if (p.y_f32) p.y_f32[o] = v;
              if (p.y_bf16) p.y_bf16[o] = f32_to_bf16(v);
            }
          }
        }
      }
    }
    wg_barrier();   // the LDS reads above are done before the next unit's loads land there
  }
}

// Launch of one instantiation: tpw is the planner's largest group of logical tiles (1 .. tpw_max).
template <int TT, int EPI, bool TILED>
void launch_tpw(const W4Params& p, int tpw, int G, hipStream_t st) {
  constexpr int M = tpw_max(TT, EPI);
  const dim3 grid(G), block(NWV * 64);
#define W4K(n) \
  case n: if constexpr (n <= M) hipLaunchKernelGGL((w4k_kernel<TT, EPI, TILED, n>), grid, block, 0, st, p); break;
  switch (tpw) { W4K(1) W4K(2) W4K(3) W4K(4) W4K(5) W4K(6) default: break; }
#undef W4K
}

template <int TT>
void launch_tt(const W4Params& p, int tpw, int epi, bool tiled, int G, hipStream_t st) {
  // the plain layout runs the widest instantiation (results do not depend on the tile count)
  if (epi == EPI_RESID) {
    if (tiled) launch_tpw<TT, EPI_RESID, true>(p, tpw, G, st);
    else launch_tpw<TT, EPI_RESID, false>(p, tpw_max(TT, EPI_RESID), G, st);
  } else if (epi == EPI_SWIGLU) {
    if (tiled) launch_tpw<TT, EPI_SWIGLU, true>(p, tpw, G, st);
    else launch_tpw<TT, EPI_SWIGLU, false>(p, tpw_max(TT, EPI_SWIGLU), G, st);
  } else {
    if (tiled) launch_tpw<TT, EPI_STORE, true>(p, tpw, G, st);
    else launch_tpw<TT, EPI_STORE, false>(p, tpw_max(TT, EPI_STORE), G, st);
  }
}

}  // namespace w4
}  // namespace ss
