// Internal launcher interface between the C ABI layer (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace ss {

enum Epilogue { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };

// Tiled int4 layout: per (16-row tile, 128-wide K chunk) one block of 1 KB of codes in
// the GEMM's lane order followed by 16 rows x 2 groups of (scale, zero) fp16 pairs.
constexpr int TILE_BLOCK_BYTES = 1024 + 16 * 2 * 4;

// Folded RMSNorm: the sums of h^2 of a token row come in groups of 256 columns (ssq[t][g],
// g < ssq_groups(H)), written by resid_finish / row_stats.
inline int ssq_groups(int H) { return (H + 255) / 256; }

// ------------------------------------------------------------------ W4A16 GEMM (gemm_w4.hip)

// Decomposition of one int4 GEMM: units = token blocks x tile groups x K ranges; a unit is
// one workgroup's job. Split K ranges leave fp32 partials [splits][T][nout] in the
// workspace, added in range order by the consumer or by the reduce kernel.
struct W4Plan {
  int TT;          // 16-token tiles per token block (1..4)
  int tb_count;    // token blocks of 64
  int nch;         // 128-wide K chunks
  int NL;          // logical tiles: 32 rows (SwiGLU: 16 gate rows + their 16 up rows)
  int nout;        // columns of a partial slice: N, or 2 I for SwiGLU
  int n_groups, splits, units, G;
  size_t ws_bytes; // partials (0 when K is not split)
};
// reduce_launch: the GEMM adds its own K ranges (no consumer does it)
W4Plan plan_w4(int T, int N, int K, int epi, int swiglu_I, bool reduce_launch);
int w4_tpw_max(int TT, int epi);

struct W4Args {
  const uint16_t* x;   // bf16 [T][K]
  const uint8_t* qw;   // tiled blocks (tiled) or codes [N][K/2]
  const uint16_t* sc;  // fp16 [N][K/64] (plain layout)
  const uint16_t* zp;
  bool tiled;
  int T, N, K;
  int epi;
  int swiglu_I;
  float* y_f32;
  uint16_t* y_bf16;
  float* resid;
  uint16_t* u_bf16;
  bool defer_reduce;   // split K ranges: leave the partials to the consumer
  // RMSNorm folded into a consumer GEMM: x = bf16(h * gain), outputs of token row t scaled
  // by 1 / sqrt(sum(ssq_in[t][0 .. ssq_n)) / rms_H + rms_eps); ssq_n = ssq_groups(H)
  const float* ssq_in;
  int ssq_n, rms_H;
  float rms_eps;
};
hipError_t launch_w4(const W4Args& a, const W4Plan& pl, void* ws, hipStream_t st);
// Device scratch of the no-allocation linear (file-scope array in gemm_w4.hip): its bytes,
// and its address on the current device (looked up once per device).
constexpr size_t W4_SCRATCH_BYTES = (size_t)16 << 20;
hipError_t w4_scratch(void** out);

// ------------------------------------------------------------------ bf16-weight GEMM (gemm_bf16.hip)

struct GemmArgs {
  const uint16_t* x;   // bf16 [T][K]
  const uint16_t* wb;  // bf16 weights [N][K]
  int T, N, K;
  int epi;
  int swiglu_I;
  float* y_f32;
  uint16_t* y_bf16;
  float* resid;
  uint16_t* u_bf16;
  const float* ssq_in;   // folded RMSNorm, as W4Args
  int ssq_n, rms_H;
  float rms_eps;
};

// Decomposition of one bf16 GEMM call: row blocks x token blocks, each cut into 128-wide
// K chunks; whole blocks first (dp_rounds per workgroup), the rest split evenly (stream-K)
// over G_sk workgroups whose partials a reduce kernel adds in K order.
struct GemmPlan {
  int TT;
  int rb_count, tb_count, nchunks, nsteps;
  int G, dp_rounds, sk_first, sk_blocks, G_sk;
  long long sk_units;
  size_t ws_bytes;
};
GemmPlan plan_gemm(int T, int N, int K, int epi, int swiglu_I);
hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& pl, void* ws, hipStream_t st);
// the bf16 GEMM's hand-off waits give up after a bound; a set flag means that happened
// (a pipeline fault: results of that launch are invalid). Cleared by the read.
hipError_t gemm_bf16_wait_expired(int* expired);

// ------------------------------------------------------------------ layer glue (misc.hip)

// Finish a residual GEMM: with splits > 1, h32[t][n] += sum over splits of part[s][t][n]
// (range order); then, with a gain, the next RMSNorm's inputs hg = bf16(h32 * gain) and
// ssq[t][g] (sums of h^2 per 256-column group g). row_stats: the same without partials.
hipError_t launch_resid_finish(const float* part, int splits, float* h32, int T, int H, const uint16_t* gain,
                               uint16_t* hg, float* ssq, hipStream_t st);
hipError_t launch_row_stats(const float* h32, int T, int H, const uint16_t* gain, uint16_t* hg, float* ssq,
                            hipStream_t st);
// RoPE angles of one step: rope[t][i] = (cos, sin) of (C + depth[t]) theta^(-2i/hd) for
// i < hd/2, evaluated in fp64 and rounded to fp32 (all layers share them).
hipError_t launch_rope_table(const int32_t* depth, int T, int C, int hd, float theta, float2* rope,
                             hipStream_t st);
// qkv values v[t][n] = sum over splits of part[s][t][n] (splits > 1) or qkv32[t][n]; RoPE
// from the step's table on the q and k heads, scatter to q [T][nq][hd] and tree K / V
// [nkv][T][hd] (bf16).
hipError_t launch_qkv_finish(const float* part, int splits, const float* qkv32, const float2* rope, int T,
                             int nq, int nkv, int hd, uint16_t* q, uint16_t* kt, uint16_t* vt, hipStream_t st);

// quantization
hipError_t launch_quantize_g64(const uint16_t* w, int64_t n, int64_t k, uint8_t* q, uint16_t* s,
                               uint16_t* z, hipStream_t st);
hipError_t launch_dequantize_g64(const uint8_t* q, const uint16_t* s, const uint16_t* z, int64_t n,
                                 int64_t k, uint16_t* out, hipStream_t st);
hipError_t launch_w4_tile(const uint8_t* q, const uint16_t* s, const uint16_t* z, int64_t n, int64_t k,
                          uint8_t* tiled, hipStream_t st);

// KV commit: per-layer cache and tree K/V pointers (at most KVC_MAX_LAYERS per launch)
constexpr int KVC_MAX_LAYERS = 64;
struct KvCommitPtrs {
  uint16_t* kc[KVC_MAX_LAYERS];
  uint16_t* vc[KVC_MAX_LAYERS];
  const uint16_t* kt[KVC_MAX_LAYERS];
  const uint16_t* vt[KVC_MAX_LAYERS];
};
hipError_t launch_kv_commit(const KvCommitPtrs& a, int layers, int nkv, int hd, int c_stride, int C, int T,
                            const int32_t* path, const int32_t* accept_len, hipStream_t st);

// tree + attention
hipError_t launch_tree_mask(const int32_t* parents, int T, uint64_t* mask, int32_t* depth,
                            int32_t* err, hipStream_t st);

struct AttnArgs {
  const uint16_t* q;      // [T][nq][hd]
  const uint16_t* kc;     // [nkv][c_stride][hd]
  const uint16_t* vc;
  const uint16_t* kt;     // [nkv][T][hd]
  const uint16_t* vt;
  const uint64_t* mask;   // [T][W]
  uint16_t* out;          // [T][nq][hd] (nullable)
  float* out_f32;         // (nullable)
  int T, C, c_stride, nq, nkv, hd;
  float sm_scale;
};
struct AttnPlan {
  int splits;             // KV splits of the prefix (the tree part is one more split)
  int keys_per_split;
  int qblocks;            // query-row blocks per KV head
  size_t ws_bytes;
};
AttnPlan plan_attention(int T, int C, int nq, int nkv, int hd);
hipError_t launch_attention(const AttnArgs& a, const AttnPlan& pl, void* ws, hipStream_t st);

// layer glue
hipError_t launch_embed(const int32_t* tokens, const uint16_t* embed, int T, int H, int V, float* h32,
                        int32_t* err, hipStream_t st);
hipError_t launch_bf16_to_f32(const uint16_t* in, size_t n, float* out, hipStream_t st);
hipError_t launch_f32_to_bf16(const float* in, size_t n, uint16_t* out, hipStream_t st);
// R output rows; rows (nullable) selects source rows of h32 [src_rows][H]
hipError_t launch_rmsnorm(const float* h32, const uint16_t* gain, int R, int H, float eps,
                          uint16_t* out, const int32_t* rows, int src_rows, int32_t* err,
                          hipStream_t st);

// selection / acceptance
hipError_t launch_row_argmax(const float* logits, int rows, int vocab, int32_t* out, hipStream_t st);
hipError_t launch_draft_select(const float* logits, const float* gumbel, int rows, int vocab,
                               float inv_temp, int k, int32_t* out, void* ws, hipStream_t st);
// workspace bytes of launch_draft_select (0: one pass, no workspace)
size_t draft_select_ws_bytes(int rows, int vocab, int k);
// draft-tree expansion (ss_tree_expand): lse partials of the frontier rows, then one wave
// that scores, picks and appends; meta = {nodes, frontier size, step, 0}
size_t expand_ws_bytes(int R, int vocab);
hipError_t launch_expand_init(int root_token, int T, int R, int32_t* parents, int32_t* tokens, float* cum,
                              int32_t* frontier, int32_t* meta, hipStream_t st);
hipError_t launch_expand(const float* logits, const int32_t* children, int R, int vocab, float inv_temp, int k,
                         int T, int D, int32_t* parents, int32_t* tokens, float* cum, int32_t* frontier,
                         int32_t* meta, void* ws, hipStream_t st);
// stochastic tree verification (ss_tree_accept_stochastic): row statistics of the target's
// and the draft's logits, then one workgroup's multi-round speculative-sampling walk
size_t sv_ws_bytes(int T, int V);
hipError_t launch_stochastic_accept(const int32_t* parents, const int32_t* tokens, const float* draft_logits,
                                    const float* target_logits, int T, int V, float inv_td, float inv_tt,
                                    const double* uni, const double* buni, int32_t* path, int32_t* len,
                                    int32_t* bonus, void* ws, hipStream_t st);
hipError_t launch_tree_accept(const int32_t* parents, const int32_t* tokens, const int32_t* tgt,
                              int T, int32_t* path, int32_t* len, int32_t* bonus, hipStream_t st);

}  // namespace ss
