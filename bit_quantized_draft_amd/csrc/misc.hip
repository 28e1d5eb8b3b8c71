// Layer glue (embedding gather, RMSNorm, RoPE + q/k/v scatter), row argmax, draft child
// selection and the greedy tree-acceptance walk.
//
// Acceptance follows greedy token-tree verification (Review page "SubSpec: Using the
// Target Model's Own Low-Bit Shadow as Its Draft Model", §6.3 and §3.2): from the root,
// accept the child whose token is the target's argmax at the current node, repeat.
// Child selection sharpens the draft distribution with a temperature (Summary page
// "Speculate Deep and Accurate ...", "Approach": 0.2) and keeps k = 6 children per node
// (Review §6.3); read as Gumbel-top-k sampling without replacement.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace ss {

// ------------------------------------------------------------------ glue

__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const uint16_t* __restrict__ embed, int T, int H,
                                                    int V, float* __restrict__ h32,
                                                    int32_t* __restrict__ err) {
  const int t = blockIdx.x;
  const int tok = tokens[t];
  const bool ok = tok >= 0 && tok < V;
  if (!ok && threadIdx.x == 0 && err) atomicOr(err, 2);
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    h32[(size_t)t * H + i] = ok ? bf16_to_f32(embed[(size_t)tok * H + i]) : 0.f;
}

__global__ __launch_bounds__(256) void bf16_to_f32_kernel(const uint16_t* __restrict__ in, size_t n,
                                                          float* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    out[i] = bf16_to_f32(in[i]);
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ in, size_t n,
                                                          uint16_t* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    out[i] = f32_to_bf16(in[i]);
}

// out[r] = bf16(h[row] * rsqrt(mean(h[row]^2) + eps) * gain), one workgroup per output row.
// H % 4 == 0; each thread keeps up to RMS_CACHE float4s of its row in registers (one read
// of h for H <= 256 * 4 * RMS_CACHE), re-reading only beyond that.
constexpr int RMS_CACHE = 8;
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h32,
                                                      const uint16_t* __restrict__ gain, int H,
                                                      float eps, uint16_t* __restrict__ out,
                                                      const int32_t* __restrict__ rows, int src_rows,
                                                      int32_t* __restrict__ err) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int row = rows ? rows[r] : r;
  const int H4 = H >> 2;
  uint2* o4 = reinterpret_cast<uint2*>(out + (size_t)r * H);
  if (row < 0 || row >= src_rows) {   // invalid row index: zeros, error word
    if (threadIdx.x == 0 && err) atomicOr(err, 4);
    for (int i = threadIdx.x; i < H4; i += blockDim.x) o4[i] = uint2{0u, 0u};
    return;
  }
  const float4* x4 = reinterpret_cast<const float4*>(h32 + (size_t)row * H);
  float4 cache[RMS_CACHE];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < RMS_CACHE; ++u) {
    const int i = u * 256 + threadIdx.x;
    cache[u] = (i < H4) ? x4[i] : float4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < RMS_CACHE; ++u)
    ss += cache[u].x * cache[u].x + cache[u].y * cache[u].y + cache[u].z * cache[u].z + cache[u].w * cache[u].w;
  for (int i = RMS_CACHE * 256 + threadIdx.x; i < H4; i += 256) {
    const float4 v = x4[i];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float rs = 1.0f / sqrtf(tot / (float)H + eps);
  const uint2* g4 = reinterpret_cast<const uint2*>(gain);
  auto emit = [&](int i, float4 v) {
    const uint2 g = g4[i];
    o4[i] = uint2{pack_bf16x2(v.x * rs * bf16lo_to_f32(g.x), v.y * rs * bf16hi_to_f32(g.x)),
                  pack_bf16x2(v.z * rs * bf16lo_to_f32(g.y), v.w * rs * bf16hi_to_f32(g.y))};
  };
#pragma unroll
  for (int u = 0; u < RMS_CACHE; ++u) {
    const int i = u * 256 + threadIdx.x;
    if (i < H4) emit(i, cache[u]);
  }
  for (int i = RMS_CACHE * 256 + threadIdx.x; i < H4; i += 256) emit(i, x4[i]);
}


// ------------------------------------------------------------------ split-K finish

// Finish of a residual GEMM: workgroup (column block blockIdx.x of 256, token blockIdx.y).
// With K split into ranges (splits > 1) each thread adds the ranges' partials of its column
// in range order (a fixed order) to h32; with splits <= 1 h32 is already final. With a gain
// it then writes the next RMSNorm's inputs: hg = bf16(h * gain) and ssq[t][blockIdx.x], the
// block's sum of h^2 (each wave's xor tree, then the four waves in order).
__global__ __launch_bounds__(256) void resid_finish_kernel(const float* __restrict__ part, int splits, int T,
                                                           int H, float* __restrict__ h32,
                                                           const uint16_t* __restrict__ gain,
                                                           uint16_t* __restrict__ hg, float* __restrict__ ssq) {
  __shared__ float wsum[4];
  const int tok = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const size_t o = (size_t)tok * H + n;
  float h = 0.f;
  if (n < H) {
    h = h32[o];
    if (splits > 1) {
      const size_t slice = (size_t)T * H;
      const float* src = part + o;
      float sum = 0.f;
      for (int s0 = 0; s0 < splits; s0 += 8) {   // eight independent loads in flight, added in order
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = s0 + i < splits ? src[(size_t)(s0 + i) * slice] : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (s0 + i < splits) sum += x[i];
      }
      h += sum;
      h32[o] = h;
    }
  }
  if (!gain) return;
  if (n < H) hg[o] = f32_to_bf16(h * bf16_to_f32(gain[n]));
  const float x = wave_sum(n < H ? h * h : 0.f);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0)
    ssq[(size_t)tok * gridDim.x + blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// RoPE table of a step (every layer uses the same positions): rope[t][i] = (cos, sin) of
// (C + depth[t]) * theta^(-2i/hd), angles in fp64, rounded to fp32 once.
__global__ __launch_bounds__(64) void rope_table_kernel(const int32_t* __restrict__ depth, int C, int hd,
                                                        double theta, float2* __restrict__ rope) {
  const int t = blockIdx.x, i = threadIdx.x, half = hd >> 1;
  if (i >= half) return;
  const double pos = (double)(C + depth[t]);
  const double inv = pow(theta, -2.0 * (double)i / (double)hd);
  double sd, cd;
  sincos(pos * inv, &sd, &cd);
  rope[(size_t)t * half + i] = float2{(float)cd, (float)sd};
}

// qkv GEMM output -> q bf16 [T][nq][hd] and tree K / V bf16 [nkv][T][hd]. Thread (token
// blockIdx.y, head h, i < hd / 2) takes the pair of columns (h hd + i, h hd + i + hd / 2):
// each value is the sum of the K ranges' partials in range order (splits > 1) or the
// GEMM's output; q and k heads are rotated by the step's RoPE table (rotate-half), v heads
// are copied.
__device__ __forceinline__ float qkv_value(const float* __restrict__ part, int splits, const float* __restrict__ qkv32,
                                           int T, int W, int tok, int n) {
  if (splits <= 1) return qkv32[(size_t)tok * W + n];
  const size_t slice = (size_t)T * W;
  const float* src = part + (size_t)tok * W + n;
  float x = 0.f;
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = s0 + i < splits ? src[(size_t)(s0 + i) * slice] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < splits) x += y[i];
  }
  return x;
}

__global__ __launch_bounds__(256) void qkv_finish_kernel(const float* __restrict__ part, int splits,
                                                         const float* __restrict__ qkv32,
                                                         const float2* __restrict__ rope, int T, int nq, int nkv,
                                                         int hd, uint16_t* __restrict__ q, uint16_t* __restrict__ kt,
                                                         uint16_t* __restrict__ vt) {
  const int tok = blockIdx.y;
  const int half = hd >> 1;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int heads = nq + 2 * nkv;
  if (idx >= heads * half) return;
  const int h = idx / half, i = idx - h * half;
  const int W = heads * hd;
  const float a = qkv_value(part, splits, qkv32, T, W, tok, h * hd + i);
  const float bb = qkv_value(part, splits, qkv32, T, W, tok, h * hd + i + half);
  if (h >= nq + nkv) {   // value head: no rotation
    uint16_t* dst = vt + ((size_t)(h - nq - nkv) * T + tok) * hd;
    dst[i] = f32_to_bf16(a);
    dst[i + half] = f32_to_bf16(bb);
    return;
  }
  const float2 cs = rope[(size_t)tok * half + i];
  uint16_t* dst = (h < nq) ? q + ((size_t)tok * nq + h) * hd : kt + ((size_t)(h - nq) * T + tok) * hd;
  dst[i] = f32_to_bf16(a * cs.x - bb * cs.y);
  dst[i + half] = f32_to_bf16(bb * cs.x + a * cs.y);
}

hipError_t launch_resid_finish(const float* part, int splits, float* h32, int T, int H, const uint16_t* gain,
                               uint16_t* hg, float* ssq, hipStream_t st) {
  if (splits <= 1 && !gain) return hipSuccess;   // nothing to add, no norm inputs wanted
  if ((splits > 1 && !part) || !h32 || H < 1 || (gain && (!hg || !ssq))) return hipErrorInvalidValue;
  hipLaunchKernelGGL(resid_finish_kernel, dim3(ssq_groups(H), T), dim3(256), 0, st, part, splits, T, H, h32, gain,
                     hg, ssq);
  return hipGetLastError();
}

hipError_t launch_row_stats(const float* h32, int T, int H, const uint16_t* gain, uint16_t* hg, float* ssq,
                            hipStream_t st) {
  return launch_resid_finish(nullptr, 0, const_cast<float*>(h32), T, H, gain, hg, ssq, st);
}

hipError_t launch_rope_table(const int32_t* depth, int T, int C, int hd, float theta, float2* rope,
                             hipStream_t st) {
  if (hd > 128 || (hd & 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_table_kernel, dim3(T), dim3(64), 0, st, depth, C, hd, (double)theta, rope);
  return hipGetLastError();
}

hipError_t launch_qkv_finish(const float* part, int splits, const float* qkv32, const float2* rope, int T,
                             int nq, int nkv, int hd, uint16_t* q, uint16_t* kt, uint16_t* vt, hipStream_t st) {
  if ((hd != 64 && hd != 128) || (splits > 1 ? !part : !qkv32)) return hipErrorInvalidValue;
  const int pairs = (nq + 2 * nkv) * (hd / 2);
  hipLaunchKernelGGL(qkv_finish_kernel, dim3((pairs + 255) / 256, T), dim3(256), 0, st, part, splits, qkv32, rope, T,
                     nq, nkv, hd, q, kt, vt);
  return hipGetLastError();
}

// ------------------------------------------------------------------ KV commit

// Grid (layers, nkv, 2): workgroup (l, h, kv) copies the root's and the accepted path's
// tree rows of layer l, KV head h, K (kv = 0) or V (kv = 1) to cache rows C .. C + L,
// 16 bytes per thread and step. L comes from the device (the acceptance walk's output);
// L and the path entries are clamped into the tree, so no access leaves the buffers.
__global__ __launch_bounds__(256) void kv_commit_kernel(KvCommitPtrs a, int nkv, int hd, int c_stride, int C,
                                                        int T, const int32_t* __restrict__ path,
                                                        const int32_t* __restrict__ accept_len) {
  const int l = blockIdx.x, h = blockIdx.y, kv = blockIdx.z;
  const int L = min(max(*accept_len, 0), T - 1);
  const int units = hd >> 3;   // 16-byte units per row
  const uint16_t* src = (kv ? a.vt[l] : a.kt[l]) + (size_t)h * T * hd;
  uint16_t* dst = (kv ? a.vc[l] : a.kc[l]) + ((size_t)h * c_stride + C) * hd;
  for (int idx = threadIdx.x; idx < (L + 1) * units; idx += blockDim.x) {
    const int r = idx / units, u = idx - r * units;
    const int node = r == 0 ? 0 : min(max(path[r - 1], 0), T - 1);
    *reinterpret_cast<u32x4_t*>(dst + (size_t)r * hd + u * 8) =
        *reinterpret_cast<const u32x4_t*>(src + (size_t)node * hd + u * 8);
  }
}

hipError_t launch_kv_commit(const KvCommitPtrs& a, int layers, int nkv, int hd, int c_stride, int C, int T,
                            const int32_t* path, const int32_t* accept_len, hipStream_t st) {
  if (layers < 1 || layers > KVC_MAX_LAYERS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_commit_kernel, dim3(layers, nkv, 2), dim3(256), 0, st, a, nkv, hd, c_stride, C, T,
                     path, accept_len);
  return hipGetLastError();
}

hipError_t launch_embed(const int32_t* tokens, const uint16_t* embed, int T, int H, int V, float* h32,
                        int32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(T), dim3(256), 0, st, tokens, embed, T, H, V, h32, err);
  return hipGetLastError();
}
hipError_t launch_bf16_to_f32(const uint16_t* in, size_t n, float* out, hipStream_t st) {
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3(blocks), dim3(256), 0, st, in, n, out);
  return hipGetLastError();
}
hipError_t launch_f32_to_bf16(const float* in, size_t n, uint16_t* out, hipStream_t st) {
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks), dim3(256), 0, st, in, n, out);
  return hipGetLastError();
}
hipError_t launch_rmsnorm(const float* h32, const uint16_t* gain, int R, int H, float eps,
                          uint16_t* out, const int32_t* rows, int src_rows, int32_t* err,
                          hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(R), dim3(256), 0, st, h32, gain, H, eps, out, rows,
                     src_rows, err);
  return hipGetLastError();
}

// ------------------------------------------------------------------ argmax

struct ArgBest {
  float v;
  int i;
};
// total order: larger value first, equal values by lower index
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ ArgBest block_best(float v, int i) {
  __shared__ float sv[16];
  __shared__ int si[16];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(i, o, 64);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sv[w] = v; si[w] = i; }
  __syncthreads();
  ArgBest r{sv[0], si[0]};
  for (int k = 1; k < (int)(blockDim.x >> 6); ++k)
    if (better(sv[k], si[k], r.v, r.i)) { r.v = sv[k]; r.i = si[k]; }
  return r;
}

// Batched loads: each thread has SCAN_U independent float4 (or scalar) loads in flight.
constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_U = 4;

template <typename F>
__device__ __forceinline__ void scan_row(const float* __restrict__ x, const float* __restrict__ g,
                                         int vocab, float scale, F&& visit) {
  const bool vec = ((vocab & 3) == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
                   (!g || ((reinterpret_cast<uintptr_t>(g) & 15) == 0));
  if (vec) {
    const int V4 = vocab >> 2;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    const float4* g4 = reinterpret_cast<const float4*>(g);
    for (int base = threadIdx.x; base < V4; base += SCAN_THREADS * SCAN_U) {
      float4 v[SCAN_U], n[SCAN_U];
#pragma unroll
      for (int u = 0; u < SCAN_U; ++u) {
        const int i = min(base + u * SCAN_THREADS, V4 - 1);
        v[u] = x4[i];
        n[u] = g ? g4[i] : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < SCAN_U; ++u) {
        const int i = base + u * SCAN_THREADS;
        if (i < V4) {
          visit(v[u].x * scale + n[u].x, 4 * i + 0);
          visit(v[u].y * scale + n[u].y, 4 * i + 1);
          visit(v[u].z * scale + n[u].z, 4 * i + 2);
          visit(v[u].w * scale + n[u].w, 4 * i + 3);
        }
      }
    }
  } else {
    for (int base = threadIdx.x; base < vocab; base += SCAN_THREADS * SCAN_U) {
      float v[SCAN_U], n[SCAN_U];
#pragma unroll
      for (int u = 0; u < SCAN_U; ++u) {
        const int i = min(base + u * SCAN_THREADS, vocab - 1);
        v[u] = x[i];
        n[u] = g ? g[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < SCAN_U; ++u) {
        const int i = base + u * SCAN_THREADS;
        if (i < vocab) visit(v[u] * scale + n[u], i);
      }
    }
  }
}

__global__ __launch_bounds__(SCAN_THREADS) void row_argmax_kernel(const float* __restrict__ logits, int vocab,
                                                                  int32_t* __restrict__ out) {
  const float* x = logits + (size_t)blockIdx.x * vocab;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  // scale 1 and no noise: the visited value is the logit itself (x * 1 + 0 is exact)
  scan_row(x, nullptr, vocab, 1.0f, [&](float v, int i) {
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  });
  const ArgBest r = block_best(bv, bi);
  if (threadIdx.x == 0) out[blockIdx.x] = r.i;
}

// ------------------------------------------------------------------ draft selection

constexpr int SEL_MAX = 16;
constexpr int SELECT_MAX_PARTS = 32;   // parts per row of the split selection

// KM: length of each thread's sorted candidate list (>= k); the kernel is instantiated
// for a few list lengths so the common k = 6 does not pay for 16-entry insertions.
template <int KM>
__global__ __launch_bounds__(SCAN_THREADS) void draft_select_kernel(const float* __restrict__ logits,
                                                                    const float* __restrict__ gumbel,
                                                                    int vocab, float inv_temp, int k,
                                                                    int32_t* __restrict__ out) {
  const size_t off = (size_t)blockIdx.x * vocab;
  float tv[KM];
  int ti[KM];
#pragma unroll
  for (int s = 0; s < KM; ++s) { tv[s] = -INFINITY; ti[s] = 0x7FFFFFFF; }
  // y = fp32(fp32(logit * inv_temp) + g): two roundings (the library is built without
  // contraction); with no noise, y + 0 is y
  scan_row(logits + off, gumbel ? gumbel + off : nullptr, vocab, inv_temp, [&](float y, int i) {
    if (!better(y, i, tv[KM - 1], ti[KM - 1])) return;
    float cv = y;
    int ci = i;
#pragma unroll
    for (int s = 0; s < KM; ++s) {
      if (better(cv, ci, tv[s], ti[s])) {
        const float xv = tv[s];
        const int xi = ti[s];
        tv[s] = cv; ti[s] = ci;
        cv = xv; ci = xi;
      }
    }
  });
  for (int r = 0; r < k; ++r) {
    const ArgBest w = block_best(tv[0], ti[0]);
    if (threadIdx.x == 0) out[(size_t)blockIdx.x * k + r] = w.i;
    if (ti[0] == w.i) {   // the owner pops its head
#pragma unroll
      for (int s = 0; s < KM - 1; ++s) { tv[s] = tv[s + 1]; ti[s] = ti[s + 1]; }
      tv[KM - 1] = -INFINITY;
      ti[KM - 1] = 0x7FFFFFFF;
    }
  }
}

// Rows split across workgroups: a row needs ~1.2 MB of logits and noise per draft step
// at Qwen2.5's vocabulary, and one workgroup per row (64 rows: 64 CUs) is bound by one
// CU's load rate. Part p of a row scans elements [p seg, (p + 1) seg) and writes its k
// best (value, index) pairs, best first; a missing entry is (-inf, INT_MAX), which every
// element beats under the same total order. The k best of a row are among the union of
// its parts' k best, so the merge reproduces the single-pass result exactly.
template <int KM>
__global__ __launch_bounds__(SCAN_THREADS) void draft_select_part_kernel(const float* __restrict__ logits,
                                                                         const float* __restrict__ gumbel,
                                                                         int vocab, float inv_temp, int k, int seg,
                                                                         float* __restrict__ cand_v,
                                                                         int32_t* __restrict__ cand_i) {
  const int row = blockIdx.y, part = blockIdx.x, parts = gridDim.x;
  const int lo = part * seg;
  const int n = min(vocab, lo + seg) - lo;   // >= 1: the host sizes parts to cover the row
  const size_t off = (size_t)row * vocab + lo;
  float tv[KM];
  int ti[KM];
#pragma unroll
  for (int s = 0; s < KM; ++s) { tv[s] = -INFINITY; ti[s] = 0x7FFFFFFF; }
  scan_row(logits + off, gumbel ? gumbel + off : nullptr, n, inv_temp, [&](float y, int i) {
    i += lo;
    if (!better(y, i, tv[KM - 1], ti[KM - 1])) return;
    float cv = y;
    int ci = i;
#pragma unroll
    for (int s = 0; s < KM; ++s) {
      if (better(cv, ci, tv[s], ti[s])) {
        const float xv = tv[s];
        const int xi = ti[s];
        tv[s] = cv; ti[s] = ci;
        cv = xv; ci = xi;
      }
    }
  });
  const size_t o = ((size_t)row * parts + part) * k;
  for (int r = 0; r < k; ++r) {
    const ArgBest w = block_best(tv[0], ti[0]);
    if (threadIdx.x == 0) { cand_v[o + r] = w.v; cand_i[o + r] = w.i; }
    if (ti[0] == w.i) {
#pragma unroll
      for (int s = 0; s < KM - 1; ++s) { tv[s] = tv[s + 1]; ti[s] = ti[s + 1]; }
      tv[KM - 1] = -INFINITY;
      ti[KM - 1] = 0x7FFFFFFF;
    }
  }
}

// One wave per row: k rounds of picking the best remaining candidate of the row's parts.
// Candidate indices are distinct (the parts cover disjoint ranges) except for the
// (-inf, INT_MAX) fillers, which only win once every real candidate is taken.
__global__ __launch_bounds__(64) void draft_select_merge_kernel(const float* __restrict__ cand_v,
                                                                const int32_t* __restrict__ cand_i, int parts,
                                                                int k, int32_t* __restrict__ out) {
  constexpr int CM = SELECT_MAX_PARTS * SEL_MAX / 64;   // candidates per lane
  const int row = blockIdx.x, lane = threadIdx.x;
  const int n = parts * k;
  const size_t o = (size_t)row * n;
  float cv[CM];
  int ci[CM];
#pragma unroll
  for (int c = 0; c < CM; ++c) {
    const int e = lane + 64 * c;
    cv[c] = e < n ? cand_v[o + e] : -INFINITY;
    ci[c] = e < n ? cand_i[o + e] : 0x7FFFFFFF;
  }
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF, bc = -1;
#pragma unroll
    for (int c = 0; c < CM; ++c)
      if (bc < 0 || better(cv[c], ci[c], bv, bi)) { bv = cv[c]; bi = ci[c]; bc = c; }
    float wv = bv;
    int wi = bi;
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) {
      const float ov = __shfl_xor(wv, sh, 64);
      const int oi = __shfl_xor(wi, sh, 64);
      if (better(ov, oi, wv, wi)) { wv = ov; wi = oi; }
    }
    if (lane == 0) out[(size_t)row * k + r] = wi;
    // the owner retires the winner; a filler winner (index INT_MAX) leaves only fillers
    if (bi == wi && bv == wv) {
#pragma unroll
      for (int c = 0; c < CM; ++c)
        if (c == bc) { cv[c] = -INFINITY; ci[c] = 0x7FFFFFFF; }
    }
  }
}

#ifndef SS_SELECT_WGS
#define SS_SELECT_WGS 512
#endif
int select_parts(int rows, int vocab, int k) {
  // about SS_SELECT_WGS workgroups in all, parts of at least 4096 elements and at least k
  int parts = std::max(1, std::min(SELECT_MAX_PARTS, (SS_SELECT_WGS + rows - 1) / rows));
  parts = std::min(parts, std::max(1, vocab / std::max(4096, k)));
  return parts;
}

size_t draft_select_ws_bytes(int rows, int vocab, int k) {
  const int parts = select_parts(rows, vocab, k);
  if (parts == 1) return 0;
  const size_t n = (size_t)rows * parts * k;
  return ((n * sizeof(float) + 255) & ~(size_t)255) + n * sizeof(int32_t);
}

// ------------------------------------------------------------------ draft-tree expansion

// Log-sum-exp partials of the frontier rows' sharpened logits y = fp32(l * inv_temp):
// workgroup (part blockIdx.x, row blockIdx.y) writes the (max, sum of exp(y - max)) of its
// range, each thread's elements in order, then the threads in a fixed tree. Rows at or past
// the frontier size (meta[1]) are skipped.
__global__ __launch_bounds__(256) void expand_lse_part_kernel(const float* __restrict__ logits, int vocab,
                                                              float inv_temp, int seg,
                                                              const int32_t* __restrict__ meta,
                                                              float2* __restrict__ part) {
  __shared__ float sm[256], ss[256];
  const int row = blockIdx.y, p = blockIdx.x;
  if (row >= meta[1]) return;
  const int lo = p * seg, hi = min(vocab, lo + seg);
  const float* x = logits + (size_t)row * vocab;
  float m = -INFINITY, sum = 0.f;
  for (int i = lo + threadIdx.x; i < hi; i += 256) {
    const float y = x[i] * inv_temp;
    if (y > m) {
      sum = sum * expf(m - y) + 1.f;
      m = y;
    } else {
      sum += expf(y - m);
    }
  }
  sm[threadIdx.x] = m;
  ss[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      const float m0 = sm[threadIdx.x], m1 = sm[threadIdx.x + w];
      const float M = fmaxf(m0, m1);
      const float a = m0 == -INFINITY ? 0.f : ss[threadIdx.x] * expf(m0 - M);
      const float b = m1 == -INFINITY ? 0.f : ss[threadIdx.x + w] * expf(m1 - M);
      sm[threadIdx.x] = M;
      ss[threadIdx.x] = a + b;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) part[(size_t)row * gridDim.x + p] = float2{sm[0], ss[0]};
}

// One expansion step (one wave): the frontier's children (ss_draft_select's top-k of the
// same rows) scored cum[parent] + (y - lse), the B best appended at slots n .. n + B - 1
// (ties: lower frontier position, then lower child rank), which become the frontier.
// meta = {nodes n, frontier size, step}; a step at or past D changes nothing.
__global__ __launch_bounds__(64) void expand_select_kernel(const float* __restrict__ logits,
                                                           const int32_t* __restrict__ children, int R,
                                                           int vocab, float inv_temp, int k, int T, int D,
                                                           int parts, const float2* __restrict__ part,
                                                           int32_t* __restrict__ parents, int32_t* __restrict__ tokens,
                                                           float* __restrict__ cum, int32_t* __restrict__ frontier,
                                                           int32_t* __restrict__ meta) {
  const int lane = threadIdx.x;
  const int n = meta[0], nf = min(meta[1], R), s = meta[2];
  if (s >= D || n >= T) return;
  const int B = min((T - n + (D - s) - 1) / (D - s), R);
  // candidate lane = r * k + rank (r < nf, rank < k); k * R <= 64 (host check)
  const int r = lane / k, rank = lane - r * k;
  const bool live = r < nf;
  float score = -INFINITY;
  int token = 0, par = 0;
  if (live) {
    float M = -INFINITY;
    for (int q = 0; q < parts; ++q) M = fmaxf(M, part[(size_t)r * parts + q].x);
    float S = 0.f;
    for (int q = 0; q < parts; ++q) {
      const float2 v = part[(size_t)r * parts + q];
      S += v.x == -INFINITY ? 0.f : v.y * expf(v.x - M);
    }
    const float lse = M + logf(S);
    token = children[(size_t)r * k + rank];
    par = frontier[r];
    const float y = logits[(size_t)r * vocab + token] * inv_temp;
    score = cum[par] + (y - lse);
  }
  // B rounds of a wave-wide best (score desc, then lower candidate index)
  int chosen = -1;   // the output slot offset this lane's candidate takes
  float cs = live ? score : -INFINITY;
  int ci = live ? lane : 0x7FFFFFFF;
  for (int b = 0; b < B; ++b) {
    float bv = cs;
    int bi = ci;
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) {
      const float ov = __shfl_xor(bv, sh, 64);
      const int oi = __shfl_xor(bi, sh, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (bi == lane && live && chosen < 0) {
      chosen = b;
      cs = -INFINITY;
      ci = 0x7FFFFFFF;
    }
  }
  __syncthreads();   // every lane has read frontier[] before it is rewritten
  if (chosen >= 0) {
    const int slot = n + chosen;
    parents[slot] = par;
    tokens[slot] = token;
    cum[slot] = score;
  }
  if (lane < R) frontier[lane] = n + (lane < B ? lane : 0);
  if (lane == 0) {
    meta[0] = n + B;
    meta[1] = B;
    meta[2] = s + 1;
  }
}

// The template before step 0: the root alone (cum 0, frontier {0}); other slots hold
// parent 0 and the root's token (valid inputs that no real node attends to).
__global__ __launch_bounds__(256) void expand_init_kernel(int root_token, int T, int R, int32_t* __restrict__ parents,
                                                          int32_t* __restrict__ tokens, float* __restrict__ cum,
                                                          int32_t* __restrict__ frontier, int32_t* __restrict__ meta) {
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    parents[i] = i == 0 ? -1 : 0;
    tokens[i] = root_token;
    cum[i] = 0.f;
  }
  for (int i = threadIdx.x; i < R; i += blockDim.x) frontier[i] = 0;
  if (threadIdx.x == 0) {
    meta[0] = 1;
    meta[1] = 1;
    meta[2] = 0;
    meta[3] = 0;
  }
}

int expand_parts(int vocab) { return std::max(1, std::min(64, vocab / 2048)); }

size_t expand_ws_bytes(int R, int vocab) { return (size_t)R * expand_parts(vocab) * sizeof(float2); }

hipError_t launch_expand_init(int root_token, int T, int R, int32_t* parents, int32_t* tokens, float* cum,
                              int32_t* frontier, int32_t* meta, hipStream_t st) {
  hipLaunchKernelGGL(expand_init_kernel, dim3(1), dim3(256), 0, st, root_token, T, R, parents, tokens, cum,
                     frontier, meta);
  return hipGetLastError();
}

hipError_t launch_expand(const float* logits, const int32_t* children, int R, int vocab, float inv_temp, int k,
                         int T, int D, int32_t* parents, int32_t* tokens, float* cum, int32_t* frontier,
                         int32_t* meta, void* ws, hipStream_t st) {
  if (k * R > 64 || R < 1 || k < 1) return hipErrorInvalidValue;
  const int parts = expand_parts(vocab);
  const int seg = (vocab + parts - 1) / parts;
  float2* part = static_cast<float2*>(ws);
  hipLaunchKernelGGL(expand_lse_part_kernel, dim3(parts, R), dim3(256), 0, st, logits, vocab, inv_temp, seg, meta,
                     part);
  hipLaunchKernelGGL(expand_select_kernel, dim3(1), dim3(64), 0, st, logits, children, R, vocab, inv_temp, k, T, D,
                     parts, part, parents, tokens, cum, frontier, meta);
  return hipGetLastError();
}

hipError_t launch_row_argmax(const float* logits, int rows, int vocab, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(row_argmax_kernel, dim3(rows), dim3(SCAN_THREADS), 0, st, logits, vocab, out);
  return hipGetLastError();
}
hipError_t launch_draft_select(const float* logits, const float* gumbel, int rows, int vocab,
                               float inv_temp, int k, int32_t* out, void* ws, hipStream_t st) {
  const int parts = select_parts(rows, vocab, k);
  if (parts > 1) {
    // part length: a multiple of 4 elements, so the parts of a 16-byte aligned row keep
    // the vector loads; ceil(vocab / seg) parts cover the row, none of them empty
    int seg = (vocab + parts - 1) / parts;
    seg = (seg + 3) & ~3;
    const int np = (vocab + seg - 1) / seg;
    const size_t n = (size_t)rows * np * k;
    float* cv = static_cast<float*>(ws);
    int32_t* ci = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + ((n * sizeof(float) + 255) & ~(size_t)255));
    const dim3 grid(np, rows);
    if (k <= 2)
      hipLaunchKernelGGL(draft_select_part_kernel<2>, grid, dim3(SCAN_THREADS), 0, st, logits, gumbel, vocab, inv_temp, k, seg, cv, ci);
    else if (k <= 6)
      hipLaunchKernelGGL(draft_select_part_kernel<6>, grid, dim3(SCAN_THREADS), 0, st, logits, gumbel, vocab, inv_temp, k, seg, cv, ci);
    else
      hipLaunchKernelGGL(draft_select_part_kernel<SEL_MAX>, grid, dim3(SCAN_THREADS), 0, st, logits, gumbel, vocab, inv_temp, k, seg, cv, ci);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(draft_select_merge_kernel, dim3(rows), dim3(64), 0, st, cv, ci, np, k, out);
    return hipGetLastError();
  }
  if (k <= 2)
    hipLaunchKernelGGL(draft_select_kernel<2>, dim3(rows), dim3(SCAN_THREADS), 0, st, logits, gumbel, vocab, inv_temp, k, out);
  else if (k <= 6)
    hipLaunchKernelGGL(draft_select_kernel<6>, dim3(rows), dim3(SCAN_THREADS), 0, st, logits, gumbel, vocab, inv_temp, k, out);
  else
    hipLaunchKernelGGL(draft_select_kernel<SEL_MAX>, dim3(rows), dim3(SCAN_THREADS), 0, st, logits, gumbel, vocab, inv_temp, k, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ acceptance walk

// One wavefront. Each step scans the nodes after `cur` 64 at a time for the first child
// of `cur` carrying the target's token; `cur` strictly increases, so the walk ends
// within T steps for any input.
__global__ __launch_bounds__(64) void tree_accept_kernel(const int32_t* __restrict__ parents,
                                                         const int32_t* __restrict__ tokens,
                                                         const int32_t* __restrict__ tgt, int T,
                                                         int32_t* __restrict__ path,
                                                         int32_t* __restrict__ len,
                                                         int32_t* __restrict__ bonus) {
  const int lane = threadIdx.x;
  int cur = 0, L = 0;
  while (true) {
    const int want = tgt[cur];
    int found = -1;
    for (int base = cur + 1; base < T; base += 64) {
      const int i = base + lane;
      const bool hit = i < T && parents[i] == cur && tokens[i] == want;
      const unsigned long long m = __ballot(hit);
      if (m) { found = base + __ffsll((long long)m) - 1; break; }
    }
    if (found < 0) break;
    if (lane == 0) path[L] = found;
    ++L;
    cur = found;
  }
  for (int i = L + lane; i < T; i += 64) path[i] = -1;
  if (lane == 0) {
    *len = L;
    *bonus = tgt[cur];
  }
}

// ------------------------------------------------------------------ stochastic verification

// Rows 0 .. T-1: the target's logits at temperature 1/inv_tt; rows T .. 2T-1: the draft's at
// 1/inv_td; y = fp32(l * inv). Part maxima of each row.
__global__ __launch_bounds__(256) void sv_max_kernel(const float* __restrict__ tl, const float* __restrict__ dl,
                                                     int T, int V, float inv_tt, float inv_td, int seg,
                                                     float* __restrict__ pmax) {
  __shared__ float red[256];
  const int row = blockIdx.y, p = blockIdx.x;
  const bool tgt = row < T;
  const float* x = (tgt ? tl : dl) + (size_t)(tgt ? row : row - T) * V;
  const float inv = tgt ? inv_tt : inv_td;
  const int lo = p * seg, hi = min(V, lo + seg);
  float m = -INFINITY;
  for (int i = lo + threadIdx.x; i < hi; i += 256) m = fmaxf(m, x[i] * inv);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) pmax[(size_t)row * gridDim.x + p] = red[0];
}

// Part sums of e = fp64(expf(fp32(y - M))), M the row maximum (the parts' maxima combined);
// each thread's elements in order, then a fixed tree.
__global__ __launch_bounds__(256) void sv_sum_kernel(const float* __restrict__ tl, const float* __restrict__ dl,
                                                     int T, int V, float inv_tt, float inv_td, int seg,
                                                     const float* __restrict__ pmax, double* __restrict__ psum) {
  __shared__ double red[256];
  const int row = blockIdx.y, p = blockIdx.x, parts = gridDim.x;
  const bool tgt = row < T;
  const float* x = (tgt ? tl : dl) + (size_t)(tgt ? row : row - T) * V;
  const float inv = tgt ? inv_tt : inv_td;
  float M = -INFINITY;
  for (int q = 0; q < parts; ++q) M = fmaxf(M, pmax[(size_t)row * parts + q]);
  const int lo = p * seg, hi = min(V, lo + seg);
  double sum = 0.0;
  for (int i = lo + threadIdx.x; i < hi; i += 256) sum += (double)expf(x[i] * inv - M);
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) psum[(size_t)row * parts + p] = red[0];
}

constexpr int SV_THREADS = 1024;
constexpr int SV_MAX_REJ = 256;   // rejections one walk can record (at most T - 1 children)

// The walk (one workgroup). At node u the current residual distribution is evaluated
// pointwise: p = e_t / Z_t, then for each recorded rejection r: p = max(p - q, 0) / Zr[r],
// q = e_d / Z_d. A rejection appends the V-wide sum of the new residual (fixed order);
// a zero sum restarts from the node's own distribution.
struct SvRow {
  float Mt, Md;
  double Zt, Zd;
};

__device__ __forceinline__ double sv_p(const float* tl_row, const float* dl_row, int v, float inv_tt, float inv_td,
                                       const SvRow& r, const double* zr, int nrej) {
  double p = (double)expf(tl_row[v] * inv_tt - r.Mt) / r.Zt;
  if (nrej) {
    const double q = (double)expf(dl_row[v] * inv_td - r.Md) / r.Zd;
    for (int k = 0; k < nrej; ++k) p = fmax(p - q, 0.0) / zr[k];
  }
  return p;
}

__device__ double sv_block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = SV_THREADS / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double s = red[0];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(SV_THREADS) void sv_walk_kernel(const int32_t* __restrict__ parents,
                                                             const int32_t* __restrict__ tokens,
                                                             const float* __restrict__ tl, const float* __restrict__ dl,
                                                             int T, int V, float inv_tt, float inv_td, int parts,
                                                             const float* __restrict__ pmax,
                                                             const double* __restrict__ psum,
                                                             const double* __restrict__ uni,
                                                             const double* __restrict__ buni,
                                                             int32_t* __restrict__ path, int32_t* __restrict__ len,
                                                             int32_t* __restrict__ bonus) {
  __shared__ int par[256];
  __shared__ double red[SV_THREADS];
  __shared__ double zr[SV_MAX_REJ];
  __shared__ SvRow row;
  __shared__ double s_total;
  __shared__ int s_x[SV_THREADS / 64];
  const int tid = threadIdx.x;
  for (int i = tid; i < T; i += SV_THREADS) {
    par[i] = parents[i];
    path[i] = -1;
  }
  __syncthreads();
  int cur = 0, L = 0, nrej = 0;
  SvRow r;
  while (true) {
    if (tid == 0) {
      SvRow w;
      w.Mt = w.Md = -INFINITY;
      for (int q = 0; q < parts; ++q) {
        w.Mt = fmaxf(w.Mt, pmax[(size_t)cur * parts + q]);
        w.Md = fmaxf(w.Md, pmax[(size_t)(T + cur) * parts + q]);
      }
      w.Zt = w.Zd = 0.0;
      for (int q = 0; q < parts; ++q) {
        w.Zt += psum[(size_t)cur * parts + q];
        w.Zd += psum[(size_t)(T + cur) * parts + q];
      }
      row = w;
    }
    __syncthreads();
    r = row;
    __syncthreads();
    const float* trow = tl + (size_t)cur * V;
    const float* drow = dl + (size_t)cur * V;
    nrej = 0;
    int next = -1;
    for (int c = cur + 1; c < T; ++c) {   // children in index order (a block-uniform loop)
      if (par[c] != cur) continue;
      // a token id outside [0, V) is never accepted (and never read)
      const int x = tokens[c];
      const bool okx = x >= 0 && x < V;
      const int xs = okx ? x : 0;
      const double px = okx ? sv_p(trow, drow, xs, inv_tt, inv_td, r, zr, nrej) : 0.0;
      const double qx = (double)expf(drow[xs] * inv_td - r.Md) / r.Zd;
      if (uni[c] * qx < px) {
        next = c;
        break;
      }
      // rejected: the next residual's normalizer, the sum of max(P - Q, 0) over V
      double part = 0.0;
      for (int v = tid; v < V; v += SV_THREADS) {
        const double pv = sv_p(trow, drow, v, inv_tt, inv_td, r, zr, nrej);
        const double qv = (double)expf(drow[v] * inv_td - r.Md) / r.Zd;
        part += fmax(pv - qv, 0.0);
      }
      const double z = sv_block_sum(part, red);
      if (z > 0.0 && nrej < SV_MAX_REJ) {
        if (tid == 0) zr[nrej] = z;
        __syncthreads();
        ++nrej;
      } else {
        nrej = 0;   // no mass left: the node's own distribution again
      }
    }
    if (next < 0) break;
    if (tid == 0) path[L] = next;
    ++L;
    cur = next;
  }
  // bonus from the residual the stopping node ended with: the lowest v whose cumulative
  // probability exceeds u * total (thread-contiguous chunks in index order, chunk totals
  // combined in thread order)
  const float* trow = tl + (size_t)cur * V;
  const float* drow = dl + (size_t)cur * V;
  const int chunk = (V + SV_THREADS - 1) / SV_THREADS;
  const int lo = min(V, tid * chunk), hi = min(V, lo + chunk);
  double own = 0.0;
  for (int v = lo; v < hi; ++v) own += sv_p(trow, drow, v, inv_tt, inv_td, r, zr, nrej);
  red[tid] = own;
  __syncthreads();
  if (tid == 0) {
    double acc = 0.0;
    for (int t = 0; t < SV_THREADS; ++t) {
      const double v = red[t];
      red[t] = acc;
      acc += v;
    }
    s_total = acc;
  }
  __syncthreads();
  const double thr = buni[cur] * s_total;
  int x = 0x7FFFFFFF;
  double cum = red[tid];
  for (int v = lo; v < hi; ++v) {
    cum += sv_p(trow, drow, v, inv_tt, inv_td, r, zr, nrej);
    if (cum > thr) {
      x = v;
      break;
    }
  }
  // block minimum of the crossing points (x increases with the thread index)
  for (int sh = 32; sh > 0; sh >>= 1) x = min(x, __shfl_xor(x, sh, 64));
  if ((tid & 63) == 0) s_x[tid >> 6] = x;
  __syncthreads();
  if (tid == 0) {
    int b = 0x7FFFFFFF;
    for (int w = 0; w < SV_THREADS / 64; ++w) b = min(b, s_x[w]);
    *len = L;
    *bonus = b == 0x7FFFFFFF ? V - 1 : b;
  }
}

int sv_parts(int V) { return std::max(1, std::min(32, V / 4096)); }

size_t sv_ws_bytes(int T, int V) {
  const size_t n = (size_t)2 * T * sv_parts(V);
  return ((n * sizeof(float) + 255) & ~(size_t)255) + n * sizeof(double);
}

hipError_t launch_stochastic_accept(const int32_t* parents, const int32_t* tokens, const float* draft_logits,
                                    const float* target_logits, int T, int V, float inv_td, float inv_tt,
                                    const double* uni, const double* buni, int32_t* path, int32_t* len,
                                    int32_t* bonus, void* ws, hipStream_t st) {
  if (T < 1 || T > 256 || V < 1) return hipErrorInvalidValue;
  const int parts = sv_parts(V);
  const int seg = (V + parts - 1) / parts;
  const size_t n = (size_t)2 * T * parts;
  float* pmax = static_cast<float*>(ws);
  double* psum = reinterpret_cast<double*>(static_cast<char*>(ws) + ((n * sizeof(float) + 255) & ~(size_t)255));
  const dim3 grid(parts, 2 * T);
  hipLaunchKernelGGL(sv_max_kernel, grid, dim3(256), 0, st, target_logits, draft_logits, T, V, inv_tt, inv_td, seg,
                     pmax);
  hipLaunchKernelGGL(sv_sum_kernel, grid, dim3(256), 0, st, target_logits, draft_logits, T, V, inv_tt, inv_td, seg,
                     pmax, psum);
  hipLaunchKernelGGL(sv_walk_kernel, dim3(1), dim3(SV_THREADS), 0, st, parents, tokens, target_logits, draft_logits, T,
                     V, inv_tt, inv_td, parts, pmax, psum, uni, buni, path, len, bonus);
  return hipGetLastError();
}

hipError_t launch_tree_accept(const int32_t* parents, const int32_t* tokens, const int32_t* tgt,
                              int T, int32_t* path, int32_t* len, int32_t* bonus, hipStream_t st) {
  hipLaunchKernelGGL(tree_accept_kernel, dim3(1), dim3(64), 0, st, parents, tokens, tgt, T, path, len, bonus);
  return hipGetLastError();
}

}  // namespace ss
