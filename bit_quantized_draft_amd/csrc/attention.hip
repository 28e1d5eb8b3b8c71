// Tree mask and tree-masked grouped-query attention over the KV cache shared with the target.
//
// The draft reads the target's KV cache for the committed prefix, so draft and target
// attend over the same context (Review page "SubSpec: Using the Target Model's Own
// Low-Bit Shadow as Its Draft Model", §4.1; Summary page "Speculate Deep and Accurate
// ...", "Approach"). Each tree node additionally sees the tree keys of its own root
// path (Review §6.3, token-tree verification).
//
// Key sequence of query token t: prefix keys 0..C-1 (always visible), then tree keys
// C..C+T-1, tree key C+j visible iff bit j of t's ancestor-or-self mask is set.
//
// Layout on gfx950: all query rows of one KV head (grp = nq/nkv heads x T tokens) are
// packed as the columns of one MFMA operand, so each K/V tile is read once per KV
// head. Scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16 with
// keys as rows), which leaves every lane holding one query row's scores for 8 keys:
// exactly the B operand that O^T = V^T P^T needs, so P never leaves registers. V is
// staged transposed in LDS. The online softmax runs in fp32 per query row (exp2 with
// the scale folded in); the key sequence is split across workgroups and a second
// kernel merges the partial (max, sum, O) triples in fixed order.
#include "common.h"
#include "kernels.h"

namespace ss {

// ------------------------------------------------------------------ tree mask

// T <= 256, so a row has at most 4 mask words; the parent array is staged in LDS.
__global__ __launch_bounds__(256) void tree_mask_kernel(const int32_t* __restrict__ parents, int T,
                                                        uint64_t* __restrict__ mask,
                                                        int32_t* __restrict__ depth,
                                                        int32_t* __restrict__ err) {
  __shared__ int par[256];
  const int W = (T + 63) >> 6;
  // this kernel opens every call that uses the error word: clear it first (no memset
  // node, so the call sequence can be captured in a graph)
  if (err && threadIdx.x == 0) *err = 0;
  for (int i = threadIdx.x; i < T; i += blockDim.x) par[i] = parents[i];
  __syncthreads();
  // One thread per node walks its parent chain in LDS (at most T steps). Invalid parents
  // stop the walk and raise the error word, so an invalid tree never reads out of bounds.
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    uint64_t words[4] = {0, 0, 0, 0};
    int cur = i, d = 0, steps = 0;
    bool bad = (i == 0) ? (par[0] != -1) : false;
    while (true) {
      words[cur >> 6] |= 1ull << (cur & 63);
      if (cur == 0) break;
      const int pp = par[cur];
      if (pp < 0 || pp >= cur || ++steps > T) { bad = true; break; }
      cur = pp;
      ++d;
    }
    for (int w = 0; w < W; ++w) mask[(size_t)i * W + w] = words[w];
    if (depth) depth[i] = d;
    if (bad && err) atomicOr(err, 1);
  }
}

hipError_t launch_tree_mask(const int32_t* parents, int T, uint64_t* mask, int32_t* depth,
                            int32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(tree_mask_kernel, dim3(1), dim3(256), 0, st, parents, T, mask, depth, err);
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention

// Two floats to packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16_rne(float a, float b) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  typedef __bf16 b2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, b2v));
}

// Three workgroup shapes, all with 128-key tiles: (query tiles per row wave, 32-key
// sub-tiles per key group, key groups) = (1, 2, 2) for contexts up to 4K keys, (1, 1, 4)
// for up to 192 query rows per KV head over longer contexts, (2, 2, 2) otherwise.
constexpr int ATT_KT = 128;
struct AttnShape {
  int qc, nsub, nkq;
};

struct AttnParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const uint16_t* kt;
  const uint16_t* vt;
  const uint64_t* mask;
  int T, C, c_stride, nq, nkv, grp, rows;  // rows = grp * T query rows per KV head
  int keys_per_split, splits;
  float scale_log2;                        // sm_scale * log2(e)
  float* o_part;                           // [splits][nkv][rows][HD]
  float* ml_part;                          // [splits][nkv][rows][2]  (max in log2 units, sum)
};

// Workgroup = NR row waves x NKQ key groups. Row wave rw owns QC 16-row query tiles; key
// group kq takes sub-tiles kq NSUB .. kq NSUB + NSUB - 1 (32 keys each) of every K/V tile,
// with its own online-softmax state. The key groups of a row wave are combined in LDS at
// the end, in fixed order, so more waves share the work of a tile without adding partials.
template <int HD, int QC, int NSUB, int NKQ>
__global__ __launch_bounds__(256 * NKQ) void tree_attn_kernel(AttnParams p) {
  constexpr int NR = 4;
  constexpr int NW = NR * NKQ;
  constexpr int KT = 32 * NSUB * NKQ;       // keys per tile: NSUB sub-tiles of 32 per key group
  constexpr int VT_STRIDE = KT + 2;         // halfs per transposed-V row: (KT + 2) / 2 words,
                                            // odd, so key-pair writes of a wave spread over banks
  constexpr int HC = HD / 32;               // 32-wide hd chunks
  constexpr int DT = HD / 16;               // 16-wide d tiles of the output
  constexpr int K_STRIDE = HD + 8;          // halfs per K row in LDS (pad against bank conflicts)
  constexpr int KV_BYTES = 2 * (KT * K_STRIDE + HD * VT_STRIDE) * 2;
  constexpr int XC_FLOATS = (NKQ - 1) * NR * QC * (DT * 256 + 128);   // key-group exchange
  constexpr int SMEM = KV_BYTES > XC_FLOATS * 4 ? KV_BYTES : XC_FLOATS * 4;
  __shared__ __align__(16) char smem[SMEM];
  auto k_lds = reinterpret_cast<uint16_t(*)[KT * K_STRIDE]>(smem);
  auto vt_lds = reinterpret_cast<uint16_t(*)[HD * VT_STRIDE]>(smem + 2 * KT * K_STRIDE * 2);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rw = wave % NR, kq = wave / NR;
  const int j = lane & 15, b = lane >> 4;
  const int kv = blockIdx.y;
  const int split = blockIdx.z;
  const int row_block = blockIdx.x * NR * QC * 16 + rw * QC * 16;
  const int W = (p.T + 63) >> 6;   // mask words per row
  const int key_begin = split * p.keys_per_split;
  const int key_end = min(p.C + p.T, key_begin + p.keys_per_split);

  // Q fragments (B operand of S^T = K Q^T): lane (j, b) holds Q[row j][hd 8b..8b+7] per chunk
  bf16x8_t qf[QC][HC];
  uint64_t mw0[QC], mw1[QC], mw2[QC], mw3[QC];   // the row's ancestor mask (T <= 256: 4 words)
  bool qvalid[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    const int r = row_block + c * 16 + j;
    qvalid[c] = r < p.rows;
    const int t = qvalid[c] ? r / p.grp : 0;
    const int h = kv * p.grp + (qvalid[c] ? r % p.grp : 0);
    const uint64_t* mr = p.mask + (size_t)t * W;
    mw0[c] = mr[0];
    mw1[c] = W > 1 ? mr[1] : 0ull;
    mw2[c] = W > 2 ? mr[2] : 0ull;
    mw3[c] = W > 3 ? mr[3] : 0ull;
#pragma unroll
    for (int hc = 0; hc < HC; ++hc) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (qvalid[c]) v = *reinterpret_cast<const u32x4_t*>(p.q + ((size_t)t * p.nq + h) * HD + hc * 32 + b * 8);
      qf[c][hc] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x4_t o[QC][DT];
  float m_run[QC], l_run[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) o[c][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // ---- K / V tile staging, software-pipelined: the next tile's global loads are issued
  // before the current tile is computed and land in the other LDS buffer afterwards.
  // K: thread -> (key, 8-wide hd chunk), 16-byte rows. V: thread -> (key pair, 8-wide hd
  // chunk); the pair is written transposed as 4-byte words vt[d][key, key + 1], the 64
  // lanes of a wave covering 8 key pairs x 8 hd chunks (2-way banked at worst).
  constexpr int KCH = KT * HD / 8 / (NW * 64);          // K chunks per thread
  constexpr int VU = (KT / 2) * (HD / 8);                // V key-pair chunks per tile
  constexpr int VCH = (VU + NW * 64 - 1) / (NW * 64);   // per thread
  constexpr int KPW = KT / 16;                           // waves along the key pairs
  static_assert(KCH >= 1 && VU % 64 == 0, "tile / workgroup shape");
  u32x4_t kreg[KCH], vreg[VCH][2];
  // Keys past the split's end are clamped to its last key: branch-free loads of finite
  // data whose scores the mask turns into -inf (P = 0).
  auto key_src = [&](int kk, const uint16_t* cache, const uint16_t* tree, int d0) -> const uint16_t* {
    kk = min(kk, key_end - 1);
    const uint16_t* a = cache + ((size_t)kv * p.c_stride + kk) * HD + d0;
    const uint16_t* t = tree + ((size_t)kv * p.T + max(kk - p.C, 0)) * HD + d0;
    return kk < p.C ? a : t;
  };
  auto v_unit = [&](int i, int& kp, int& dc) -> bool {
    const int u = tid + i * NW * 64;
    const int w = u >> 6, l = u & 63;
    kp = (l & 7) + 8 * (w % KPW);
    dc = (l >> 3) + 8 * (w / KPW);
    return u < VU;   // whole waves
  };
  // per-thread element offsets of the tile's K / V chunks (loop-invariant)
  int koff[KCH], voff[VCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int ci = tid + i * NW * 64;
    koff[i] = (ci / (HD / 8)) * HD + (ci % (HD / 8)) * 8;
  }
#pragma unroll
  for (int i = 0; i < VCH; ++i) {
    int kp, dc;
    v_unit(i, kp, dc);
    voff[i] = 2 * kp * HD + dc * 8;
  }
  auto load_tile = [&](int k0) {
    if (k0 + KT <= min(p.C, key_end)) {
      // the whole tile lies in the prefix cache and in the split: one uniform base
      const size_t row0 = ((size_t)kv * p.c_stride + k0) * HD;
      const uint16_t* kb = p.kc + row0;
      const uint16_t* vb = p.vc + row0;
#pragma unroll
      for (int i = 0; i < KCH; ++i) kreg[i] = *reinterpret_cast<const u32x4_t*>(kb + koff[i]);
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        int kp, dc;
        if (v_unit(i, kp, dc)) {
#pragma unroll
          for (int h = 0; h < 2; ++h) vreg[i][h] = *reinterpret_cast<const u32x4_t*>(vb + voff[i] + h * HD);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = tid + i * NW * 64;
      const int key = ci / (HD / 8), d0 = (ci % (HD / 8)) * 8;
      const int kk = k0 + key;
      kreg[i] = *reinterpret_cast<const u32x4_t*>(key_src(kk, p.kc, p.kt, d0));
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      int kp, dc;
      if (v_unit(i, kp, dc)) {
        const int kk = k0 + 2 * kp;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          vreg[i][h] = *reinterpret_cast<const u32x4_t*>(key_src(kk + h, p.vc, p.vt, dc * 8));
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = tid + i * NW * 64;
      const int key = ci / (HD / 8), d0 = (ci % (HD / 8)) * 8;
      *reinterpret_cast<u32x4_t*>(&k_lds[buf][key * K_STRIDE + d0]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      int kp, dc;
      if (v_unit(i, kp, dc)) {
        const uint32_t a[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
        const uint32_t c[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // d = 8 dc + 2e (low halves) and 8 dc + 2e + 1 (high halves) of keys 2kp, 2kp+1
          uint32_t* row0 = reinterpret_cast<uint32_t*>(&vt_lds[buf][(dc * 8 + 2 * e) * VT_STRIDE]);
          uint32_t* row1 = reinterpret_cast<uint32_t*>(&vt_lds[buf][(dc * 8 + 2 * e + 1) * VT_STRIDE]);
          row0[kp] = (a[e] & 0xFFFFu) | (c[e] << 16);
          row1[kp] = (a[e] >> 16) | (c[e] & 0xFFFF0000u);
        }
      }
    }
  };

  int buf = 0;
  if (key_begin < key_end) {
    load_tile(key_begin);
    store_tile(0);
  }
  __syncthreads();
  for (int k0 = key_begin; k0 < key_end; k0 += KT) {
    const bool has_next = k0 + KT < key_end;
    if (has_next) load_tile(k0 + KT);
    const uint16_t* kl = k_lds[buf];
    const uint16_t* vl = vt_lds[buf];

    // ---- S^T tiles: keys (rows) x query rows (cols); 2 NSUB 16-key tiles
    f32x4_t s[QC][2 * NSUB];
#pragma unroll
    for (int c = 0; c < QC; ++c)
#pragma unroll
      for (int kt = 0; kt < 2 * NSUB; ++kt) s[c][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2 * NSUB; ++kt) {
#pragma unroll
      for (int hc = 0; hc < HC; ++hc) {
        const u32x4_t kf =
            *reinterpret_cast<const u32x4_t*>(&kl[((kq * 2 * NSUB + kt) * 16 + j) * K_STRIDE + hc * 32 + b * 8]);
        const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, kf);
#pragma unroll
        for (int c = 0; c < QC; ++c)
          s[c][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[c][hc], s[c][kt], 0, 0, 0);
      }
    }

    // ---- mask + online softmax. Lane (j, b) holds keys kt*16 + 4b + e of query row j.
    // tiles wholly inside the prefix and the split need no mask (wave-uniform test)
    const bool masked = (k0 + KT > p.C) || (k0 + KT > key_end);
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      float mx = -INFINITY;
      if (!masked) {
#pragma unroll
        for (int kt = 0; kt < 2 * NSUB; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[c][kt][e] *= p.scale_log2;
            mx = fmaxf(mx, s[c][kt][e]);
          }
      } else {
#pragma unroll
        for (int kt = 0; kt < 2 * NSUB; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int kk = k0 + (kq * 2 * NSUB + kt) * 16 + 4 * b + e;
            const int jn = kk - p.C;   // tree index (negative in the prefix)
            const uint64_t mw = jn < 64 ? mw0[c] : jn < 128 ? mw1[c] : jn < 192 ? mw2[c] : mw3[c];
            const bool vis = kk < key_end && (jn < 0 || ((mw >> (jn & 63)) & 1ull));
            const float v = vis ? s[c][kt][e] * p.scale_log2 : -INFINITY;
            s[c][kt][e] = v;
            mx = fmaxf(mx, v);
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Lazy rescaling: the reference max of a row moves only when the tile's max exceeds
      // it by more than 8 (log2 units), so P stays <= 2^8 and O / l are rescaled only in
      // the (wave-uniform) case that some row moved.
      const bool move = mx > m_run[c] + 8.0f;   // always true on a row's first finite tile
      const float m_new = move ? fmaxf(m_run[c], mx) : m_run[c];
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      // v_exp_f32 straight (no denormal range scaling): arguments are <= 8 or -inf, and
      // results below 2^-126, which it may flush to zero, are far below the row sum (>= 1)
      const float alpha = __builtin_amdgcn_exp2f(m_run[c] - m_use);   // 0 on the first tile
      const bool any_move = __builtin_amdgcn_ballot_w64(move) != 0;
      float psum = 0.f;
      uint32_t pk[NSUB][4];
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pv[e] = __builtin_amdgcn_exp2f(s[c][2 * sub + h][e] - m_use);
            psum += pv[e];
          }
          pk[sub][h * 2 + 0] = pk_bf16_rne(pv[0], pv[1]);
          pk[sub][h * 2 + 1] = pk_bf16_rne(pv[2], pv[3]);
        }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      m_run[c] = m_new;
      if (any_move) {
        l_run[c] = l_run[c] * alpha + psum;
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[c][d][e] *= alpha;
      } else {
        l_run[c] += psum;
      }
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        // P^T operand of sub-tile sub: lane (j, b) element e' <-> key 32 sub +
        // (e' < 4 ? 4b + e' : 16 + 4b + e' - 4)
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[sub][0], pk[sub][1], pk[sub][2], pk[sub][3]});
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          // A operand V^T: lane (i = d row, b) element e' <-> the same key permutation
          const uint32_t* vrow =
              reinterpret_cast<const uint32_t*>(&vl[(d * 16 + j) * VT_STRIDE + 32 * (kq * NSUB + sub)]);
          const u32x2_t lo = {vrow[2 * b], vrow[2 * b + 1]};
          const u32x2_t hi = {vrow[8 + 2 * b], vrow[8 + 2 * b + 1]};
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
          o[c][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[c][d], 0, 0, 0);
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);   // the other buffer: last read before the previous barrier
    __syncthreads();
    buf ^= 1;
  }

  // ---- combine the key groups of each row wave, fixed order kq = 0, 1, ...; the loop's
  // last barrier has passed, so the K / V buffers are free for the exchange
  if constexpr (NKQ > 1) {
    float* xo = reinterpret_cast<float*>(smem);          // [NKQ-1][NR][QC][DT][64][4]
    float* xml = xo + (NKQ - 1) * NR * QC * DT * 256;    // [NKQ-1][NR][QC][64][2]
    if (kq > 0) {
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const int slot = ((kq - 1) * NR + rw) * QC + c;
#pragma unroll
        for (int d = 0; d < DT; ++d) *reinterpret_cast<f32x4_t*>(&xo[(slot * DT + d) * 256 + lane * 4]) = o[c][d];
        xml[slot * 128 + lane * 2 + 0] = m_run[c];
        xml[slot * 128 + lane * 2 + 1] = l_run[c];
      }
    }
    __syncthreads();
    if (kq > 0) return;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      float mq[NKQ], lq[NKQ];
      mq[0] = m_run[c];
      lq[0] = l_run[c];
      float M = mq[0];
#pragma unroll
      for (int q = 1; q < NKQ; ++q) {
        const int slot = ((q - 1) * NR + rw) * QC + c;
        mq[q] = xml[slot * 128 + lane * 2 + 0];
        lq[q] = xml[slot * 128 + lane * 2 + 1];
        M = fmaxf(M, mq[q]);
      }
      const float Mu = (M == -INFINITY) ? 0.f : M;
      float f[NKQ], L = 0.f;
#pragma unroll
      for (int q = 0; q < NKQ; ++q) {
        f[q] = exp2f(mq[q] - Mu);   // 0 for a group that saw no visible key
        L += lq[q] * f[q];
      }
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        f32x4_t acc = o[c][d] * f[0];
#pragma unroll
        for (int q = 1; q < NKQ; ++q) {
          const int slot = ((q - 1) * NR + rw) * QC + c;
          acc += *reinterpret_cast<const f32x4_t*>(&xo[(slot * DT + d) * 256 + lane * 4]) * f[q];
        }
        o[c][d] = acc;
      }
      m_run[c] = M;
      l_run[c] = L;
    }
  }

  // ---- partials: lane (j, b) holds O^T[d = dt*16 + 4b + e][row j]
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    const int r = row_block + c * 16 + j;
    if (!qvalid[c]) continue;
    const size_t base = ((size_t)split * p.nkv + kv) * p.rows + r;
    float* op = p.o_part + base * HD;
#pragma unroll
    for (int d = 0; d < DT; ++d)
      *reinterpret_cast<f32x4_t*>(op + d * 16 + 4 * b) = o[c][d];
    if (b == 0) {
      p.ml_part[base * 2 + 0] = m_run[c];
      p.ml_part[base * 2 + 1] = l_run[c];
    }
  }
}

// Merge the split partials of one (KV head, query row): fixed split order.
template <int HD>
__global__ __launch_bounds__(HD) void attn_merge_kernel(AttnParams p, uint16_t* out, float* out_f32) {
  const int r = blockIdx.x, kv = blockIdx.y, d = threadIdx.x;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < p.splits; ++s)
    M = fmaxf(M, p.ml_part[(((size_t)s * p.nkv + kv) * p.rows + r) * 2]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float L = 0.f, acc = 0.f;
#pragma unroll 8
  for (int s = 0; s < p.splits; ++s) {
    const size_t base = ((size_t)s * p.nkv + kv) * p.rows + r;
    const float w = exp2f(p.ml_part[base * 2] - Mu);
    L += w * p.ml_part[base * 2 + 1];
    acc += w * p.o_part[base * HD + d];
  }
  const float v = acc / L;
  const int t = r / p.grp, h = kv * p.grp + r % p.grp;
  const size_t o = ((size_t)t * p.nq + h) * HD + d;
  if (out) out[o] = f32_to_bf16(v);
  if (out_f32) out_f32[o] = v;
}

// The same merge with a workgroup of 256 threads over MR query rows, a thread taking 4
// consecutive d of one row; faster when there are many rows (10240 (row, KV head) pairs:
// 6.1 us against 9.4 us), slower with few (1792 pairs: 6.4 against 5.1 us).
constexpr int MERGE_WIDE_THREADS = 256;
template <int HD>
__global__ __launch_bounds__(MERGE_WIDE_THREADS) void attn_merge_wide_kernel(AttnParams p, uint16_t* out,
                                                                           float* out_f32) {
  constexpr int TPR = HD / 4;                        // threads per row
  constexpr int MR = MERGE_WIDE_THREADS / TPR;       // rows per workgroup
  const int kv = blockIdx.y;
  const int r = blockIdx.x * MR + threadIdx.x / TPR;
  const int d = (threadIdx.x % TPR) * 4;
  if (r >= p.rows) return;
  const size_t stride = (size_t)p.nkv * p.rows;      // between splits, in rows
  const size_t row0 = (size_t)kv * p.rows + r;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.ml_part[(row0 + s * stride) * 2]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = 0; s < p.splits; ++s) {
    const size_t base = row0 + s * stride;
    const float w = exp2f(p.ml_part[base * 2] - Mu);
    L += w * p.ml_part[base * 2 + 1];
    const f32x4_t o4 = *reinterpret_cast<const f32x4_t*>(p.o_part + base * HD + d);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += w * o4[e];
  }
  const int t = r / p.grp, h = kv * p.grp + r % p.grp;
  const size_t o = ((size_t)t * p.nq + h) * HD + d;
  // element stores: the outputs need only their element alignment
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v = acc[e] / L;
    if (out) out[o + e] = f32_to_bf16(v);
    if (out_f32) out_f32[o + e] = v;
  }
}

// Measured on MI355X (attention kernel alone): up to 4K keys, (1, 2, 2) beats (1, 1, 4) by
// about 1 us (288 rows over 1072 keys: 12.1 us against 13.1 us; 448 rows over 2112 keys:
// 14.1 against 15.1). Longer contexts with up to 192 rows per KV head: (1, 1, 4), 44 us for
// 192 rows over 16432 keys, against 49 us with (1, 2, 2) and 62 us with three tiles per wave
// and one workgroup per KV head. Many rows over long contexts: (2, 2, 2), 65 us for 1280
// rows over 4352 keys, against 112 us with one key group and 108 us with one tile per wave.
// SS_ATTN_WGS (build-time) is the workgroup count the key split aims for; at the
// Qwen2.5-7B / Llama-3.1-8B shapes 128 and 512 are no faster than 256.
#ifndef SS_ATTN_WGS
#define SS_ATTN_WGS 256
#endif
static AttnShape attn_shape(int rows, int keys) {
  if (keys <= 4096) return {1, 2, 2};
  if (rows <= 192) return {1, 1, 4};
  return {2, 2, 2};
}

AttnPlan plan_attention(int T, int C, int nq, int nkv, int hd) {
  AttnPlan pl;
  const int grp = nq / nkv;
  const int rows = grp * T;
  // query-row blocks of 4 row waves x QC x 16 rows
  const int qc = attn_shape(rows, C + T).qc;
  const int KT = ATT_KT;
  pl.qblocks = (rows + 4 * qc * 16 - 1) / (4 * qc * 16);
  const int keys = C + T;
  const int units = pl.qblocks * nkv;
  // aim for ~256 workgroups (one per compute unit), at least one key tile per split
  int splits = std::max(1, SS_ATTN_WGS / std::max(1, units));
  const int max_splits = std::max(1, keys / KT);
  splits = std::min(splits, max_splits);
  int kps = (keys + splits - 1) / splits;
  kps = (kps + KT - 1) / KT * KT;
  pl.keys_per_split = kps;
  pl.splits = (keys + kps - 1) / kps;
  pl.ws_bytes = (size_t)pl.splits * nkv * rows * (hd + 2) * sizeof(float);
  return pl;
}

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& pl, void* ws, hipStream_t st) {
  AttnParams p{};
  p.q = a.q; p.kc = a.kc; p.vc = a.vc; p.kt = a.kt; p.vt = a.vt; p.mask = a.mask;
  p.T = a.T; p.C = a.C; p.c_stride = a.c_stride; p.nq = a.nq; p.nkv = a.nkv;
  p.grp = a.nq / a.nkv;
  p.rows = p.grp * a.T;
  p.keys_per_split = pl.keys_per_split;
  p.splits = pl.splits;
  p.scale_log2 = a.sm_scale * 1.4426950408889634f;
  p.o_part = reinterpret_cast<float*>(ws);
  p.ml_part = p.o_part + (size_t)pl.splits * a.nkv * p.rows * a.hd;
  const AttnShape sh = attn_shape(p.rows, a.C + a.T);
  dim3 grid(pl.qblocks, a.nkv, pl.splits);
  if (pl.keys_per_split % ATT_KT) return hipErrorInvalidValue;   // a plan for another shape
  const dim3 blk(256 * sh.nkq);
#define ATT_LAUNCH(HD)                                                                                     \
  do {                                                                                                    \
    if (sh.qc == 2) hipLaunchKernelGGL((tree_attn_kernel<HD, 2, 2, 2>), grid, blk, 0, st, p);             \
    else if (sh.nkq == 4) hipLaunchKernelGGL((tree_attn_kernel<HD, 1, 1, 4>), grid, blk, 0, st, p);      \
    else hipLaunchKernelGGL((tree_attn_kernel<HD, 1, 2, 2>), grid, blk, 0, st, p);                        \
  } while (0)
  if (a.hd == 128) ATT_LAUNCH(128);
  else ATT_LAUNCH(64);
#undef ATT_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((long long)p.rows * a.nkv >= 4096) {
    if (a.hd == 128)
      hipLaunchKernelGGL((attn_merge_wide_kernel<128>), dim3((p.rows + 7) / 8, a.nkv), dim3(MERGE_WIDE_THREADS), 0,
                         st, p, a.out, a.out_f32);
    else
      hipLaunchKernelGGL((attn_merge_wide_kernel<64>), dim3((p.rows + 15) / 16, a.nkv), dim3(MERGE_WIDE_THREADS), 0,
                         st, p, a.out, a.out_f32);
  } else if (a.hd == 128) {
    hipLaunchKernelGGL((attn_merge_kernel<128>), dim3(p.rows, a.nkv), dim3(128), 0, st, p, a.out, a.out_f32);
  } else {
    hipLaunchKernelGGL((attn_merge_kernel<64>), dim3(p.rows, a.nkv), dim3(64), 0, st, p, a.out, a.out_f32);
  }
  return hipGetLastError();
}

}  // namespace ss
