/*
 * subspec.h -- C ABI of the SubSpec substitute-draft hot path on MI355X (gfx950).
 *
 * SubSpec drafts with the target model's own layers quantized to 4 bits (the
 * "substitute" layers), sharing the target's resident layers and KV cache, and
 * verifies a deep, narrow token tree with one target pass.
 * Pages cited below, by title:
 *   [Review]   "SubSpec: Using the Target Model's Own Low-Bit Shadow as Its Draft Model"
 *   [Summary]  "Speculate Deep and Accurate: Lossless and Training-Free Acceleration for
 *              Offloaded LLMs via Substitute Speculative Decoding" (atlas.scime.ai summary)
 *   [Abstract] the arXiv abstract of the same paper (mlsanity.com page)
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless the name ends in _host. The caller owns
 *     every buffer; the library keeps no pointer after a call returns and never
 *     allocates or frees device memory. Scratch memory comes from a caller-provided
 *     workspace sized by the matching *_workspace query.
 *   - bf16 and fp16 tensors are row-major arrays of 16-bit values; int4 weights are
 *     packed two per byte, even k in the low nibble (element k of row n in byte
 *     n*K/2 + k/2).
 *   - `stream` is a hipStream_t (NULL: the default stream). Calls only enqueue work
 *     and return; outputs are valid once the stream has reached them. Calls are
 *     re-entrant; concurrent calls on different streams need distinct workspaces.
 *     With the environment variable SS_DEBUG_SYNC=1 every call synchronizes its
 *     stream and reports device-side errors.
 *   - All argument checks run on the host before anything is launched. On any
 *     error nothing is launched, outputs are untouched, and ss_last_error() says why.
 *   - Device pointers must be 16-byte aligned; int32 arrays 4-byte aligned.
 */
#ifndef SUBSPEC_H
#define SUBSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SS_OK = 0,
  SS_ERR_INVALID_ARG = -1, /* null / misaligned pointer, negative or inconsistent size */
  SS_ERR_UNSUPPORTED = -2, /* well-formed but outside the supported shapes */
  SS_ERR_BAD_TREE = -3,    /* parents[] is not a topologically ordered tree rooted at 0 */
  SS_ERR_WORKSPACE = -4,   /* workspace null or smaller than the *_workspace query */
  SS_ERR_DEVICE = -5       /* no usable gfx950 device, or a HIP launch / runtime error */
} ss_status;

/* Message of the last error on the calling thread; never NULL ("" after success). */
const char* ss_last_error(void);
/* Version of this ABI (structs and signatures); bumped on any change. */
int ss_abi_version(void);

/* ------------------------------------------------------------------------------
 * Substitute construction. [Review] §6.2 and [Summary] "Approach": the substitute
 * layers are data-free, training-free 4-bit copies of the target's layers. Reading
 * (no quantizer is given on the pages): asymmetric min-max round-to-nearest per
 * group of 64 consecutive input features with fp16 scale s and fp16 zero z:
 *   s = fp16((max - min) / 15) (+inf -> 65504, 0 -> 1), z = fp16((0 - min) / s),
 *   a group whose z overflows fp16 is widened to include 0 and recomputed,
 *   q = clamp(rint_even(w / s + z), 0, 15); every step is one fp32 operation rounded
 *   to nearest-even, no fused multiply-add. Bit-exact with the CPU oracle.
 * w_bf16 [n][k] -> qweight u8 [n][k/2], scale fp16 [n][k/64], zero fp16 [n][k/64].
 * group must be 64; k % 64 == 0; n >= 1.
 * ------------------------------------------------------------------------------ */
ss_status ss_quantize_substitute(const void* w_bf16, int64_t n, int64_t k, int32_t group,
                                 void* qweight, void* scale, void* zero, void* stream);

/* fp16 export of a substitute weight: w = fp16(fp32(fp32(q) - z) * s), bit-exact.
 * Output w_f16 [n][k]. Same shape rules as ss_quantize_substitute. */
ss_status ss_dequantize_substitute(const void* qweight, const void* scale, const void* zero,
                                   int64_t n, int64_t k, int32_t group, void* w_f16,
                                   void* stream);

/* ------------------------------------------------------------------------------
 * Substitute linear layer ([Summary] "Approach"; [Abstract]): Y = X * deq(W)^T over
 * all T tree tokens at once, bf16 X [T][k], int4 W as above, fp32 accumulation.
 * Outputs (at least one): y_bf16 [T][n] (round-to-nearest-even of the fp32 result)
 * and/or y_f32 [T][n]. 1 <= T <= 256, k % 128 == 0, n % 16 == 0.
 * The workspace holds the fp32 partial sums of K ranges split between workgroups;
 * query its size first (may be 0). Its contents need no initialisation.
 * ------------------------------------------------------------------------------ */
size_t ss_w4a16_linear_workspace(int32_t T, int64_t n, int64_t k);
ss_status ss_w4a16_linear(const void* x_bf16, int32_t T, const void* qweight, const void* scale,
                          const void* zero, int64_t n, int64_t k, void* y_bf16, float* y_f32,
                          void* workspace, size_t ws_bytes, void* stream);

/* The substitute MLP's fused input projection with SwiGLU in its epilogue:
 * u = silu(X Wg^T) * (X Wu^T), fp32 accumulation, u rounded to bf16, where the int4
 * weight [2I][k] holds the gate rows [0, I) and the up rows [I, 2I). u_bf16 [T][I].
 * 1 <= T <= 256, k % 128 == 0, I % 16 == 0. */
size_t ss_w4a16_gate_up_swiglu_workspace(int32_t T, int64_t I, int64_t k);
ss_status ss_w4a16_gate_up_swiglu(const void* x_bf16, int32_t T, const void* qweight,
                                  const void* scale, const void* zero, int64_t I, int64_t k,
                                  void* u_bf16, void* workspace, size_t ws_bytes, void* stream);

/* Tiled int4 layout (a relocation of qweight / scale / zero, values unchanged), read
 * by the GEMMs as one contiguous 1152-byte block per 16-row tile i (rows 16 i ..
 * 16 i + 15) and 128-wide K chunk c, at byte (i * k/128 + c) * 1152:
 *   bytes 16 l .. 16 l + 15 (l = 0..63): code bytes 64 c + 16 (l / 16) .. +15 of row
 *     16 i + l % 16 (its elements k = 128 c + 32 (l / 16) .. +31);
 *   bytes 1024 + 4 (2 j + h) (j = 0..15, h = 0, 1): the fp16 scale (low half) and the
 *     fp16 zero (high half) of row 16 i + j, group 2 c + h.
 * ss_w4_tiled_bytes gives the size, n/16 * k/128 * 1152 (0 for unsupported shapes).
 * n % 16 == 0, k % 128 == 0. The _tiled linears compute exactly what the untiled ones
 * compute from the same weights. */
size_t ss_w4_tiled_bytes(int64_t n, int64_t k);
ss_status ss_w4_tile(const void* qweight, const void* scale, const void* zero, int64_t n, int64_t k,
                     void* tiled, void* stream);
ss_status ss_w4a16_linear_tiled(const void* x_bf16, int32_t T, const void* tiled, int64_t n, int64_t k,
                                void* y_bf16, float* y_f32, void* workspace, size_t ws_bytes,
                                void* stream);
ss_status ss_w4a16_gate_up_swiglu_tiled(const void* x_bf16, int32_t T, const void* tiled, int64_t I,
                                        int64_t k, void* u_bf16, void* workspace, size_t ws_bytes,
                                        void* stream);

/* Stochastic tree verification ([Review] §3.6: target sampling at temperature 0.6 keeps
 * the output distribution exact by speculative sampling with correction, §6.2; §6.3: the
 * whole tree verified in one target pass). Reading (multi-round speculative sampling over
 * the tree): P_u and Q_u are the target's and the draft's distributions at node u,
 * softmax of y = fp32(l * inv_t) with e = fp32 exp of fp32(y - max y) widened to fp64,
 * everything after in fp64. From the root, node u's children are tried in index order:
 * child c (token x) is accepted iff uniforms[c] * Q_u(x) < P(x), P the current residual
 * (P_u at first), and the walk moves to c; a rejection replaces P by max(P - Q_u, 0)
 * renormalized (by P_u again if no mass is left). Without an accepted child the bonus is
 * the lowest token whose cumulative P exceeds bonus_uniforms[u] times the total.
 * parents, tokens int32 [T]; draft_logits / target_logits fp32 [T][V] (row u: the logits
 * at node u); uniforms, bonus_uniforms fp64 [T] in [0, 1) (the random numbers, inputs);
 * outputs as ss_tree_accept (path_out[0 .. L) the accepted nodes, then -1). A token id
 * outside [0, V) is never accepted. T <= 256; workspace: ss_tree_accept_stochastic_workspace. */
size_t ss_tree_accept_stochastic_workspace(int32_t T, int32_t V);
ss_status ss_tree_accept_stochastic(const int32_t* parents, const int32_t* tokens, const float* draft_logits,
                                    const float* target_logits, int32_t T, int32_t V, float inv_t_draft,
                                    float inv_t_target, const double* uniforms, const double* bonus_uniforms,
                                    int32_t* path_out, int32_t* accept_len_out, int32_t* bonus_out, void* workspace,
                                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * Draft-tree expansion ([Review] §6.3-§6.4: a static tree, k = 6 children per expanded
 * node, depth 48 (§3.7); [Summary] "Approach": draft probabilities sharpened at
 * temperature 0.2). Reading (the pages give no expansion rule): the T slots of the tree
 * are filled over D draft steps, one level per step. Step s takes the frontier (the
 * nodes the previous step added; the root before step 0), scores each frontier node's
 * k children (ss_draft_select's top-k of y = fp32(l * inv_temp) with no noise) by the
 * path's sharpened log-probability cum[parent] + y[c] - logsumexp(y), and appends the
 * B_s = ceil((T - n) / (D - s)) best (ties: lower frontier position, then lower child
 * rank) at slots n, n + 1, ... (n = nodes so far). They become the frontier.
 *
 * State (device, caller-owned, updated in place): parents int32 [T] and tokens int32 [T]
 * (the draft step's inputs), cum fp32 [T] (path scores), frontier int32 [R] (the next
 * step's logit rows: the frontier, padded with a valid slot), meta int32 [4] = {nodes,
 * frontier size, step, 0}. ss_tree_expand_init sets the root (slot 0, token root_token,
 * parent -1, score 0) and fills the other slots with parent 0 and the root's token.
 * ss_tree_expand consumes logits fp32 [R][V] of the rows frontier[0..R) (as the draft
 * step writes them with logit_rows = frontier, n_logit_rows = R) and children int32
 * [R][k] (ss_draft_select on those logits, gumbel NULL, the same inv_temp); a call at
 * step >= D changes nothing, so a captured graph may replay it freely.
 * Requires 2 <= T <= 256, 1 <= D <= T - 1, R >= ceil((T - 1) / D), R <= k, k R <= 64.
 * Scores are fp32 (the log-sum-exp in a fixed order); workspace: ss_tree_expand_workspace.
 * ------------------------------------------------------------------------------ */
ss_status ss_tree_expand_init(int32_t root_token, int32_t T, int32_t D, int32_t R, int32_t k, int32_t* parents,
                              int32_t* tokens, float* cum, int32_t* frontier, int32_t* meta, void* stream);
size_t ss_tree_expand_workspace(int32_t R, int32_t V);
ss_status ss_tree_expand(const float* logits, const int32_t* children, int32_t R, int32_t V, float inv_temp,
                         int32_t k, int32_t T, int32_t D, int32_t* parents, int32_t* tokens, float* cum,
                         int32_t* frontier, int32_t* meta, void* workspace, size_t ws_bytes, void* stream);

/* ss_w4a16_linear_tiled without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The K-range partial sums go to a device array
 * of the library (16 MiB, one per GPU, held until the process ends) instead of a caller
 * workspace; the result is the one ss_w4a16_linear_tiled computes. Shapes whose partial
 * sums exceed the array (ss_w4a16_linear_workspace(T, n, k) > 16 MiB) are rejected with
 * SS_ERR_WORKSPACE. Every call on a GPU uses that GPU's one array: calls that overlap in
 * time on one GPU (other streams, other threads) race and must be serialized by the
 * caller. Same-stream calls are ordered and safe. */
ss_status ss_w4a16_linear_tiled_noalloc(const void* x_bf16, int32_t T, const void* tiled, int64_t n,
                                        int64_t k, void* y_bf16, float* y_f32, void* stream);

/* Dense bf16-weight linear layer, for layers the draft shares with the target
 * unquantized ([Review] §2.2 step 4: layers that fit on the GPU stay shared with the
 * target; here the LM head) and for the target verify pass. W bf16 [n][k]; otherwise
 * as ss_w4a16_linear (k % 128 == 0, n % 16 == 0). */
size_t ss_bf16_linear_workspace(int32_t T, int64_t n, int64_t k);
ss_status ss_bf16_linear(const void* x_bf16, int32_t T, const void* w_bf16, int64_t n, int64_t k,
                         void* y_bf16, float* y_f32, void* workspace, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------------
 * Token tree ([Review] §6.3: a tree of draft tokens, every root path verified at
 * once; deep and narrow in SubSpec). Reading: node 0 is the root (the last
 * committed token, not yet in the KV cache), parents[0] = -1, 0 <= parents[i] < i.
 * ss_tree_mask writes the ancestor-or-self bitmask, uint64 [T][W] with
 * W = ceil(T/64), bit (j % 64) of word (j / 64) of row i set iff j is i or an
 * ancestor of i, and depth int32 [T] (nullable). 1 <= T <= 256.
 * A parents[] that is not a tree gives an unspecified mask (never an out-of-bounds
 * access); with SS_DEBUG_SYNC=1 the call then returns SS_ERR_BAD_TREE.
 * ss_tree_validate checks a host copy of parents[] on the CPU.
 * ------------------------------------------------------------------------------ */
ss_status ss_tree_validate(const int32_t* parents_host, int32_t T);
ss_status ss_tree_mask(const int32_t* parents, int32_t T, uint64_t* mask_out, int32_t* depth_out,
                       void* stream);

/* ------------------------------------------------------------------------------
 * Tree attention over the KV cache shared with the target ([Review] §4.1, [Summary]
 * "Approach": draft and target attend over the same context). Query i of head h
 * attends to all C prefix keys of KV head h / (nq / nkv) and to the tree keys of i's
 * ancestors and itself; softmax(q.k * sm_scale) v with fp32 accumulation.
 * ------------------------------------------------------------------------------ */
typedef struct {
  const void* q;          /* bf16 [T][nq][hd] */
  const void* k_cache;    /* bf16 [nkv][c_stride][hd], first C rows valid, read only */
  const void* v_cache;    /* bf16 [nkv][c_stride][hd] */
  const void* k_tree;     /* bf16 [nkv][T][hd] */
  const void* v_tree;     /* bf16 [nkv][T][hd] */
  const int32_t* parents; /* int32 [T] */
  void* out;              /* bf16 [T][nq][hd] (nullable if out_f32 is given) */
  float* out_f32;         /* fp32 [T][nq][hd] (nullable) */
  uint64_t* mask_out;     /* uint64 [T][ceil(T/64)] (nullable): the mask used */
  int32_t T, C, c_stride, nq, nkv, hd;
  float sm_scale;         /* <= 0 selects 1/sqrt(hd) */
} ss_attn_args;

/* 1 <= T <= 256, 0 <= C <= c_stride, hd in {64, 128}, nq % nkv == 0, nq/nkv <= 16. */
size_t ss_tree_attention_workspace(int32_t T, int32_t C, int32_t nq, int32_t nkv, int32_t hd);
ss_status ss_tree_attention(const ss_attn_args* args, void* workspace, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------------
 * One forward step of the substitute draft over the whole tree ([Summary]
 * "Approach"; [Abstract]): embedding gather (or hidden_in), then per layer
 *   x = RMSNorm1(h); [q k v] = x Wqkv^T; RoPE (rotate-half, theta^(-2i/hd)) on q and k
 *   at position C + depth; tree K/V of the layer written to tree_k[l] / tree_v[l];
 *   h += TreeAttention(q, K/V) Wo^T; x = RMSNorm2(h); [g u] = x Wgu^T;
 *   h += (silu(g) * u) Wdown^T
 * and, when logits are requested, RMSNorm_final(h) times the bf16 LM head.
 * The residual stream h is kept in fp32; layer outputs are rounded to bf16 at
 * kernel boundaries. Reading (the pages give no layer): the pre-norm Qwen2.5 /
 * Llama-3.1 decoder layer, no qkv bias.
 * ------------------------------------------------------------------------------ */
typedef enum { SS_W4G64 = 0, SS_BF16 = 1, SS_W4G64_TILED = 2 } ss_weight_kind;

typedef struct {
  int32_t kind;          /* ss_weight_kind */
  const void* qweight;   /* SS_W4G64: u8 [n][k/2]; SS_W4G64_TILED: the tiled layout */
  const void* scale;     /* SS_W4G64: fp16 [n][k/64] */
  const void* zero;      /* SS_W4G64: fp16 [n][k/64] */
  const void* w;         /* SS_BF16: bf16 [n][k] */
} ss_linear;

typedef struct {
  const void* norm1;     /* bf16 [H] */
  const void* norm2;     /* bf16 [H] */
  ss_linear qkv;         /* n = (nq + 2 nkv) hd, k = H; rows: q heads, then k, then v */
  ss_linear o;           /* n = H, k = nq hd */
  ss_linear gate_up;     /* n = 2 I, k = H; rows [0, I) gate, [I, 2I) up */
  ss_linear down;        /* n = H, k = I */
  const void* k_cache;   /* bf16 [nkv][c_stride][hd] (shared with the target, read only;
                            may be null when the step's prefix is empty, C == 0) */
  const void* v_cache;
} ss_layer;

typedef struct {
  int32_t H, I, nq, nkv, hd, L, V;
  float rope_theta, rms_eps;
  int32_t c_stride;
  const void* embed;       /* bf16 [V][H] (unused when hidden_in is given) */
  const void* final_norm;  /* bf16 [H] (needed for logits) */
  const void* lm_head;     /* bf16 [V][H] (needed for logits) */
  const ss_layer* layers;  /* HOST array of L layer descriptors */
} ss_model;

typedef struct {
  const int32_t* tokens;    /* int32 [T] (unused when hidden_in is given) */
  const int32_t* parents;   /* int32 [T] */
  int32_t T, C;             /* tree tokens; committed prefix length (C <= c_stride) */
  void* const* tree_k;      /* HOST array [L] of bf16 [nkv][T][hd] outputs */
  void* const* tree_v;      /* HOST array [L] of bf16 [nkv][T][hd] outputs */
  const void* hidden_in;    /* bf16 [T][H] (nullable): start from this instead of embed */
  void* hidden_out;         /* bf16 [T][H] (nullable): h after the last layer */
  float* logits;            /* fp32 [R][V] (nullable) */
  const int32_t* logit_rows;/* int32 [R] (nullable: R = T, all rows) */
  int32_t n_logit_rows;     /* R when logit_rows is given */
} ss_step_args;

/* 1 <= T <= 256; H, nq hd, I multiples of 128; H <= 8192 and (nq + 2 nkv) hd <= 8192;
 * hd in {64, 128}; nq % nkv == 0 (else SS_ERR_UNSUPPORTED). */
size_t ss_draft_tree_step_workspace(const ss_model* model, int32_t T, int32_t C);
ss_status ss_draft_tree_step(const ss_model* model, const ss_step_args* args, void* workspace,
                             size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * Greedy verification ([Review] §3.2 and [Summary] "Key results", temperature 0).
 * ss_row_argmax: out[r] = lowest index of the maximum of logits[r][0..vocab)
 * (finite inputs). ss_tree_accept: starting at the root, repeatedly accept the
 * lowest-index child whose token equals target_argmax[current]; path_out [T] gets
 * the accepted nodes (excluding the root, the rest of the array is set to -1),
 * accept_len_out the count L, bonus_out = target_argmax[last accepted node]; the
 * cycle commits L + 1 tokens. Runs as one wavefront; bit-exact with the oracle.
 * ------------------------------------------------------------------------------ */
ss_status ss_row_argmax(const float* logits, int32_t rows, int32_t vocab, int32_t* out,
                        void* stream);
ss_status ss_tree_accept(const int32_t* parents, const int32_t* tokens,
                         const int32_t* target_argmax, int32_t T, int32_t* path_out,
                         int32_t* accept_len_out, int32_t* bonus_out, void* stream);

/* ------------------------------------------------------------------------------
 * KV commit after acceptance ([Review] §4.1: draft and target share one KV cache;
 * the cycle commits the root and the L accepted nodes). Reading: for every layer and
 * KV head, the target's tree K/V rows of the root (node 0) and of path_out[0 .. L)
 * from ss_tree_accept, already roped at C + depth, are copied to cache rows C .. C + L
 * in path order; nothing else is written. k_cache / v_cache: HOST arrays [layers] of
 * bf16 [nkv][c_stride][hd]; k_tree / v_tree: HOST arrays [layers] of bf16
 * [nkv][T][hd]; path int32 [T] and accept_len int32 [1] are DEVICE pointers (read on
 * the device, so the call can follow ss_tree_accept inside a captured graph).
 * L and path entries are clamped into [0, T - 1] on the device. hd in {64, 128},
 * 1 <= T <= 256, 0 <= C, C + T <= c_stride (else SS_ERR_UNSUPPORTED / _INVALID_ARG).
 * ------------------------------------------------------------------------------ */
ss_status ss_kv_commit(void* const* k_cache, void* const* v_cache, const void* const* k_tree,
                       const void* const* v_tree, int32_t layers, int32_t nkv, int32_t hd,
                       int32_t c_stride, int32_t C, int32_t T, const int32_t* path,
                       const int32_t* accept_len, void* stream);

/* ------------------------------------------------------------------------------
 * Draft child selection with sharpening ([Summary] "Approach": draft temperature
 * 0.2; [Review] §6.3: k = 6 children). Reading: Gumbel-top-k, i.e. k tokens drawn
 * without replacement from softmax(logits / t): y = fp32(fp32(logit * inv_temp) + g),
 * two fp32 operations, no FMA; output the k largest y, larger first, equal y by
 * lower index. gumbel fp32 [rows][vocab] (nullable: g = 0, plain top-k).
 * tokens_out int32 [rows][k]. 1 <= k <= 16, vocab >= k, inv_temp > 0.
 * Long rows are split across workgroups whose per-part k best are merged by a
 * second kernel (same result bit for bit); the parts' candidates live in the
 * caller's workspace of ss_draft_select_workspace(rows, vocab, k) bytes (0: no
 * workspace needed, it may be null). A smaller workspace returns SS_ERR_WORKSPACE.
 * ------------------------------------------------------------------------------ */
size_t ss_draft_select_workspace(int32_t rows, int32_t vocab, int32_t k);
ss_status ss_draft_select(const float* logits, const float* gumbel, int32_t rows, int32_t vocab,
                          float inv_temp, int32_t k, int32_t* tokens_out, void* workspace,
                          size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SUBSPEC_H */
