// Dense bf16-weight GEMMs for the layers the draft shares with the target unquantized
// (Review page "SubSpec: Using the Target Model's Own Low-Bit Shadow as Its Draft Model",
// §2.2 step 4: the layers that fit stay shared; here the LM head) and for the target's
// verify pass over the tree: Y[T][N] = X[T][K] * W[N][K]^T, bf16 MFMA, fp32 accumulation.
//
// Workgroup: NWC = 4 compute waves (one per SIMD) and NLD = 2 loader waves.
//  * Compute wave rg owns 32 weight rows (two 16-row MFMA tiles) of the workgroup's
//    128-row block and keeps PF chunks (128 k) of its bf16 weights in registers, loaded
//    branch-free with 16-byte loads.
//  * Loader waves copy each chunk's activation fragments global -> LDS with gfx950's
//    direct-to-LDS loads (global_load_lds_dwordx4) into a ring of NS slots. Hand-off
//    through LDS counters: ready[slot] is the sequence number of the chunk in the slot,
//    done[slot] counts the compute waves that finished reading it.
//  * MFMA roles: A = activations (16 tokens x 32 k), B = weights (32 k x 16 rows); lane
//    (j, b) supplies k = 32 b + 8 m .. +7 of the chunk to k-step m.
//
// Work split (data parallel + stream-K): a block is (token block of 64, row block of 128
// rows) over all of K, cut into 128-wide chunks. With G workgroups (one per CU),
// workgroup g first takes whole blocks g, g + G, ..., then an even share of the remaining
// blocks' chunks. A block split between workgroups leaves one fp32 partial per piece; a
// second kernel adds them in K order (fixed order) and runs the epilogue.
#include "common.h"
#include "kernels.h"

namespace ss {

namespace {
constexpr int CHUNK_K = 128;
constexpr int NWC = 4;   // compute waves
constexpr int NLD = 2;   // loader waves
constexpr int NR = 2;    // 16-row weight tiles per compute wave
constexpr int NS = 6;    // activation chunk slots in LDS
constexpr int RG = NWC;  // row groups (one K phase)
constexpr int PF = 2;    // bf16 weight chunks in flight per compute wave
constexpr int MIN_PIECE = 3;
constexpr int WGS = 256;
}  // namespace

// Set when a bounded hand-off wait gave up (read and cleared by gemm_bf16_wait_expired).
__device__ int g_bf16_wait_expired;

namespace {

struct GemmParams {
  const uint16_t* x;   // bf16 [T][K]
  const uint16_t* wb;  // bf16 [N][K]
  int T, N, K;
  int swiglu_I;        // rows [0,I) gate, [I,2I) up
  float* y_f32;        // [T][N]
  uint16_t* y_bf16;    // [T][N]
  float* resid;        // fp32 [T][N] residual stream (EPI_RESID)
  uint16_t* u_bf16;    // bf16 [T][I] (EPI_SWIGLU)
  int nchunks, tb_count;
  int G, dp_rounds, sk_first, G_sk;
  long long sk_units;
  float* partials;     // [2 G_sk][RG][NR][TT][4][64]
  const float* ssq_in;
  int ssq_n, rms_H;
  float rms_eps;
};

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// LDS hand-off. Only LDS ordering is needed: a wave's LDS operations complete in order,
// so waiting for them (lgkmcnt(0)) before touching a counter orders them; relaxed
// atomics avoid the vmcnt(0) that release/acquire would add.
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Bounded waits on LDS counters: a correct pipeline never comes near the limit. If one
// ever expired the wave would go on with stale data, so the expiry is recorded in a
// device flag that the library reports (SS_ERR_DEVICE under SS_DEBUG_SYNC).
constexpr int kSpinLimit = 1 << 20;
__device__ __forceinline__ void note_expiry() {
  __hip_atomic_store(&g_bf16_wait_expired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_eq(int* flag, int want) {
  for (int it = 0;; ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == want) break;
    if (it == kSpinLimit) { note_expiry(); break; }
    __builtin_amdgcn_s_sleep(1);
  }
  compiler_fence();
}
__device__ __forceinline__ void wait_ge(int* flag, int want) {
  for (int it = 0;; ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= want) break;
    if (it == kSpinLimit) { note_expiry(); break; }
    __builtin_amdgcn_s_sleep(1);
  }
  compiler_fence();
}
__device__ __forceinline__ void lds_store(int* flag, int v) {
  __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// A workgroup's work is a list of segments (block, chunks [s0, s1)): its dp_rounds whole
// blocks g, g + G, ..., then the blocks its stream-K unit range [lo, hi) touches.
struct SegList {
  int nd, nsk;
  int sb_lo, s_lo;
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
      L.sb_lo = (int)(lo / p.nchunks);
      L.s_lo = (int)(lo % p.nchunks);
      L.nsk = (int)((L.hi - 1) / p.nchunks) - L.sb_lo + 1;
    }
  }
  return L;
}

__device__ __forceinline__ void seg_of(const GemmParams& p, const SegList& L, int g, int k, int& block, int& s0,
                                       int& s1) {
  if (k < L.nd) {
    block = g + k * p.G;
    s0 = 0;
    s1 = p.nchunks;
  } else {
    const int sb = L.sb_lo + (k - L.nd);
    block = p.sk_first + sb;
    s0 = (k == L.nd) ? L.s_lo : 0;
    s1 = (int)min((long long)p.nchunks, L.hi - (long long)sb * p.nchunks);
  }
}

// Prefetch cursor over the segments, each padded to a multiple of PF positions so that
// position p of every segment uses register slot p % PF; padding positions (and positions
// past the last segment) reload the segment's last chunk, which stays in bounds and is
// never used.
struct PCur {
  int k, pos, len, plen, s0, rb;
};

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

__device__ __forceinline__ void pcur_next(PCur& c, const GemmParams& p, const SegList& L, int g) {
  if (++c.pos < c.plen) return;
  if (c.k + 1 < L.nd + L.nsk) pcur_set(c, p, L, g, c.k + 1);
  else c.pos = c.plen - 1;
}

__device__ __forceinline__ int sk_owner(const GemmParams& p, long long u) {
  return (int)(((u + 1) * p.G_sk - 1) / p.sk_units);
}
// partial slot of workgroup gk's piece of stream-K block sb (a workgroup's range has a
// partial piece at most at its first and at its last block)
__device__ __forceinline__ int sk_slot(const GemmParams& p, int gk, int sb) {
  const long long lo = (long long)gk * p.sk_units / p.G_sk;
  return 2 * gk + ((int)(lo / p.nchunks) == sb ? 0 : 1);
}

template <int EPI>
__device__ __forceinline__ int tile_row(const GemmParams& p, int rb, int rg, int r, int j) {
  if (EPI == EPI_SWIGLU) {
    const int g = rb * RG * 16 + rg * 16 + j;
    return r == 0 ? g : p.swiglu_I + g;
  }
  return rb * RG * 32 + rg * 32 + r * 16 + j;
}
template <int EPI>
__device__ __forceinline__ bool tile_valid(const GemmParams& p, int rb, int rg, int r) {
  if (EPI == EPI_SWIGLU) return rb * RG * 16 + rg * 16 < p.swiglu_I;
  return rb * RG * 32 + rg * 32 + r * 16 < p.N;   // N is a multiple of 16
}

// Final values of a wave's tiles -> outputs. Lane (j, b) holds tokens t*16 + 4b + e of
// row j of each tile.
template <int TT, int EPI>
__device__ __forceinline__ void final_store(const GemmParams& p, const f32x4_t (&acc)[NR][TT], int block, int rg,
                                            int lane) {
  const int j = lane & 15, b = lane >> 4;
  const int tb = block % p.tb_count, rb = block / p.tb_count;
  if (EPI == EPI_SWIGLU) {
    if (!tile_valid<EPI>(p, rb, rg, 0)) return;
    const int g = tile_row<EPI>(p, rb, rg, 0, j);
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
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (!tile_valid<EPI>(p, rb, rg, r)) continue;
    const int n = tile_row<EPI>(p, rb, rg, r, j);
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = tb * 64 + t * 16 + 4 * b + e;
        if (tok >= p.T) continue;
        const size_t o = (size_t)tok * p.N + n;
        const float v = acc[r][t][e];
        if (EPI == EPI_RESID) {
          p.resid[o] += v;
        } else {
          if (p.y_f32) p.y_f32[o] = v;
          if (p.y_bf16) p.y_bf16[o] = f32_to_bf16(v);
        }
      }
  }
}

// Row scales of RMSNorm folded into a consumer GEMM, for all T tokens, computed once per
// workgroup by its compute waves together (fixed summation order), shared through LDS.
__device__ __forceinline__ void row_scales(const GemmParams& p, int wave, int lane, float* rs_all, int* rs_done) {
  for (int t = wave; t < p.T; t += NWC) {
    float s = 0.f;
    for (int i = lane; i < p.ssq_n; i += 64) s += p.ssq_in[(size_t)t * p.ssq_n + i];
    s = wave_sum(s);
    if (lane == 0) rs_all[t] = 1.0f / sqrtf(s / (float)p.rms_H + p.rms_eps);
  }
  compiler_fence();
  lds_wait();
  if (lane == 0) __hip_atomic_fetch_add(rs_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

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

}  // namespace

template <int TT, int EPI>
__global__ __launch_bounds__((NWC + NLD) * 64) void bf16_gemm_kernel(GemmParams p) {
  constexpr int FRAG = TT * 4;   // 1 KB fragment blocks per chunk
  constexpr int LOADS = FRAG;    // loader instructions per chunk
  constexpr int LA = (63 / LOADS) < 3 ? (63 / LOADS) : 3;   // chunks in flight per loader
  __shared__ u32x4_t xfrag[NS][4][TT][64];
  __shared__ int ready[NS], done[NS];
  __shared__ float rs_all[256];
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
  if (tid < 256) rs_all[tid] = 0.f;
  if (tid == 0) rs_done = 0;
  __syncthreads();   // the only workgroup barrier

  if (wave >= NWC) {
    // ---------------- loader wave l copies the chunks with sequence number qc = 2 k + l
    // (k = 0, 1, ...), keeping LA chunks in flight; before it waits for a slot to be
    // released it drains and publishes everything it has issued, so no consumer can be
    // waiting on a chunk the loader holds back.
    const int l = wave - NWC;
    const int li = lane & 15, lb = lane >> 4;
    int n = 0, ns = 0, qs = 0;
    auto publish = [&](int upto) {
      for (; ns < upto; ++ns) {
        const int qd = NLD * ns + l;
        if (lane == 0) lds_store(&ready[qd % NS], qd);
      }
    };
    for (int k = 0; k < nsegs; ++k) {
      int block, s0, s1;
      seg_of(p, L, g, k, block, s0, s1);
      const int tb = block % p.tb_count;
      for (int st = s0; st < s1; ++st, ++qs) {
        const int qc = qs;
        if (qc % NLD != l) continue;
        const int slot = qc % NS;
        if (qc >= NS) {
          const int need = RG * (qc / NS);   // the previous occupant was read by all its waves
          if (__hip_atomic_load(&done[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            publish(n);
            wait_ge(&done[slot], need);
          }
        }
        const uint16_t* src = p.x + (size_t)st * CHUNK_K + lb * 32;
#pragma unroll
        for (int ps = 0; ps < FRAG; ++ps) {
          const int m = ps & 3, tt = ps >> 2;
          const int tok = min(tb * 64 + tt * 16 + li, p.T - 1);   // padded tokens: clamped copies
          __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)tok * p.K + m * 8),
                                           (__attribute__((address_space(3))) void*)&xfrag[slot][m][tt][0],
                                           16, 0, 0);
        }
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

  // ---------------- compute waves
  const int rg = wave;
  const int j = lane & 15, b = lane >> 4;
  u32x4_t wreg[PF][NR][4];

  auto w_load = [&](int slot, const PCur& c) {
    const int ch = min(c.s0 + min(c.pos, c.len - 1), p.nchunks - 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const size_t row = tile_valid<EPI>(p, c.rb, rg, r) ? (size_t)tile_row<EPI>(p, c.rb, rg, r, j) : 0;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        wreg[slot][r][m] = *reinterpret_cast<const u32x4_t*>(p.wb + row * p.K + ch * CHUNK_K + b * 32 + m * 8);
    }
  };

  f32x4_t acc[NR][TT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot, int qc) {
    const int xs = qc % NS;
    wait_eq(&ready[xs], qc);
    bf16x8_t xa[4][TT];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int t = 0; t < TT; ++t) xa[m][t] = __builtin_bit_cast(bf16x8_t, xfrag[xs][m][t][lane]);
    compiler_fence();
    lds_wait();
    if (lane == 0) __hip_atomic_fetch_add(&done[xs], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < TT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[m][t], __builtin_bit_cast(bf16x8_t, wreg[slot][r][m]),
                                                             acc[r][t], 0, 0, 0);
  };

  PCur pc;
  pcur_set(pc, p, L, g, 0);
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    w_load(u, pc);
    pcur_next(pc, p, L, g);
  }
  int qs = 0;
  if (p.ssq_in) row_scales(p, wave, lane, rs_all, &rs_done);
  bool rs_seen = false;
  for (int k = 0; k < nsegs; ++k) {
    int block, s0, s1;
    seg_of(p, L, g, k, block, s0, s1);
    const int len = s1 - s0;
    for (int p0 = 0; p0 < len; p0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        if (p0 + u < len) compute(u, qs + p0 + u);
        w_load(u, pc);
        pcur_next(pc, p, L, g);
      }
    }
    qs += len;
    if (p.ssq_in) {
      if (!rs_seen) {
        wait_ge(&rs_done, NWC);
        rs_seen = true;
      }
      apply_row_scales<TT>(acc, rs_all + (block % p.tb_count) * 64, lane);
    }
    if (s0 == 0 && s1 == p.nchunks) {
      final_store<TT, EPI>(p, acc, block, rg, lane);
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

// Blocks split between workgroups: every thread owns one output element (for SwiGLU, one
// gate / up pair) of one block and adds the pieces' partials in K order (fixed order).
template <int TT, int EPI>
__global__ __launch_bounds__(256) void bf16_reduce_kernel(GemmParams p) {
  constexpr int NRE = (EPI == EPI_SWIGLU) ? 1 : NR;
  constexpr int PER_BLOCK = RG * NRE * TT * 4 * 64;
  const int sb = blockIdx.x;
  const int idx = blockIdx.y * 256 + threadIdx.x;
  if (idx >= PER_BLOCK) return;
  const long long u0 = (long long)sb * p.nchunks;
  const int g0 = sk_owner(p, u0), g1 = sk_owner(p, u0 + p.nchunks - 1);
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
  if (tok >= p.T || !tile_valid<EPI>(p, rb, rg, r)) return;
  const size_t slot_elems = (size_t)RG * NR * TT * 4 * 64;
  const size_t off = (size_t)rg * (NR * TT * 4 * 64) + ((r * TT + t) * 4 + e) * 64 + lane;
  const size_t off1 = (size_t)rg * (NR * TT * 4 * 64) + ((1 * TT + t) * 4 + e) * 64 + lane;
  auto piece = [&](int gk) { return p.partials + (gk == g0 ? sk_slot(p, g0, sb) : 2 * gk) * slot_elems; };
  float v0 = 0.f, v1 = 0.f;
  int gk = g0;
  for (; gk + 4 <= g1 + 1; gk += 4) {
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
  const int n = tile_row<EPI>(p, rb, rg, r, j);
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
template <int TT, int EPI>
hipError_t launch_k(const GemmParams& p, int sk_blocks, hipStream_t st) {
  hipLaunchKernelGGL((bf16_gemm_kernel<TT, EPI>), dim3(p.G), dim3((NWC + NLD) * 64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sk_blocks == 0) return e;
  constexpr int per_block = RG * (EPI == EPI_SWIGLU ? 1 : NR) * TT * 4 * 64;
  hipLaunchKernelGGL((bf16_reduce_kernel<TT, EPI>), dim3(sk_blocks, (per_block + 255) / 256), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_tt(const GemmParams& p, int TT, int skb, hipStream_t st) {
  switch (TT) {
    case 1: return launch_k<1, EPI>(p, skb, st);
    case 2: return launch_k<2, EPI>(p, skb, st);
    case 3: return launch_k<3, EPI>(p, skb, st);
    default: return launch_k<4, EPI>(p, skb, st);
  }
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
}  // namespace

GemmPlan plan_gemm(int T, int N, int K, int epi, int swiglu_I) {
  GemmPlan pl{};
  pl.TT = (T >= 64) ? 4 : (T + 15) / 16;
  const int rows_per_block = (epi == EPI_SWIGLU) ? RG * 16 : RG * 32;
  const int span = (epi == EPI_SWIGLU) ? swiglu_I : N;
  pl.rb_count = std::max(1, (span + rows_per_block - 1) / rows_per_block);
  pl.tb_count = std::max(1, (T + 63) / 64);
  pl.nchunks = std::max(1, K / CHUNK_K);
  pl.nsteps = pl.nchunks;
  const int blocks = pl.rb_count * pl.tb_count;
  const int G = WGS;
  pl.dp_rounds = blocks / G;
  pl.sk_first = pl.dp_rounds * G;
  pl.sk_blocks = blocks - pl.sk_first;
  pl.sk_units = (long long)pl.sk_blocks * pl.nchunks;
  pl.G_sk = pl.sk_units > 0 ? (int)std::min<long long>(G, std::max<long long>(1, pl.sk_units / MIN_PIECE)) : 0;
  pl.G = pl.dp_rounds > 0 ? G : std::max(1, pl.G_sk);
  const size_t slot_bytes = (size_t)RG * NR * pl.TT * 4 * 64 * sizeof(float);
  pl.ws_bytes = pl.sk_blocks > 0 ? align256(2 * (size_t)pl.G_sk * slot_bytes) : 0;
  return pl;
}

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& pl, void* ws, hipStream_t st) {
  if (!a.wb || a.K % CHUNK_K || a.N % 16) return hipErrorInvalidValue;
  if (a.ssq_in && (a.ssq_n < 1 || a.epi == EPI_RESID)) return hipErrorInvalidValue;
  if (pl.sk_blocks > 0 && !ws) return hipErrorInvalidValue;
  if (pl.sk_units * (long long)std::max(pl.G_sk, 1) >= (1LL << 62)) return hipErrorInvalidValue;
  GemmParams p{};
  p.x = a.x; p.wb = a.wb;
  p.T = a.T; p.N = a.N; p.K = a.K;
  p.swiglu_I = a.swiglu_I;
  p.y_f32 = a.y_f32; p.y_bf16 = a.y_bf16; p.resid = a.resid; p.u_bf16 = a.u_bf16;
  p.nchunks = pl.nchunks;
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
  switch (a.epi) {
    case EPI_RESID: return launch_tt<EPI_RESID>(p, pl.TT, pl.sk_blocks, st);
    case EPI_SWIGLU: return launch_tt<EPI_SWIGLU>(p, pl.TT, pl.sk_blocks, st);
    default: return launch_tt<EPI_STORE>(p, pl.TT, pl.sk_blocks, st);
  }
}

hipError_t gemm_bf16_wait_expired(int* expired) {
  int v = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_bf16_wait_expired), sizeof v, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *expired = v;
  if (v) {
    const int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_bf16_wait_expired), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
  }
  return e;
}

}  // namespace ss
