// C ABI of the substitute-draft hot path: host-side validation, workspace planning and
// kernel dispatch. Every check happens here before any launch; nothing is allocated.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/subspec.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

ss_status fail(ss_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
ss_status ok() {
  g_err.clear();
  return SS_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQ_PTR(p, align)                                                                       \
  do {                                                                                          \
    if (!(p)) return fail(SS_ERR_INVALID_ARG, "%s: %s is null", __func__, #p);                  \
    if (!aligned((p), (align)))                                                                 \
      return fail(SS_ERR_INVALID_ARG, "%s: %s is not %d-byte aligned", __func__, #p, (int)(align)); \
  } while (0)
#define OPT_PTR(p, align)                                                                       \
  do {                                                                                          \
    if ((p) && !aligned((p), (align)))                                                          \
      return fail(SS_ERR_INVALID_ARG, "%s: %s is not %d-byte aligned", __func__, #p, (int)(align)); \
  } while (0)

bool debug_sync() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("SS_DEBUG_SYNC");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

// The current device must be a gfx950; the answer is cached per device id.
ss_status check_device(const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(SS_ERR_DEVICE, "%s: no HIP device available (%s)", fn, hipGetErrorString(e));
  }
  constexpr int MAX_DEV = 64;
  if (dev >= MAX_DEV) return fail(SS_ERR_DEVICE, "%s: device id %d beyond %d", fn, dev, MAX_DEV - 1);
  static std::mutex mu;
  static int state[MAX_DEV] = {};  // 0 unknown, 1 ok, 2 bad
  std::lock_guard<std::mutex> lk(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(SS_ERR_DEVICE, "%s: hipGetDeviceProperties failed", fn);
    state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (state[dev] == 2) return fail(SS_ERR_DEVICE, "%s: device %d is %s, not gfx950", fn, dev, prop.gcnArchName);
  }
  if (state[dev] == 2) return fail(SS_ERR_DEVICE, "%s: device %d is not gfx950", fn, dev);
  return SS_OK;
}

ss_status launched(const char* fn, hipError_t e, hipStream_t st) {
  if (e != hipSuccess) return fail(SS_ERR_DEVICE, "%s: launch failed: %s", fn, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(SS_ERR_DEVICE, "%s: %s", fn, hipGetErrorString(e));
  }
  return ok();
}

// error word in a workspace, read back only under SS_DEBUG_SYNC
ss_status check_err_word(const char* fn, const int32_t* dev_err, hipStream_t st) {
  if (!debug_sync() || !dev_err) return ok();
  int32_t h = 0;
  hipError_t e = hipMemcpyAsync(&h, dev_err, sizeof h, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(SS_ERR_DEVICE, "%s: %s", fn, hipGetErrorString(e));
  if (h & 1) return fail(SS_ERR_BAD_TREE, "%s: parents[] is not a topologically ordered tree", fn);
  if (h & 2) return fail(SS_ERR_INVALID_ARG, "%s: a token id is outside [0, V)", fn);
  if (h & 4) return fail(SS_ERR_INVALID_ARG, "%s: a logit row index is outside [0, T)", fn);
  return ok();
}

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Bump {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += up(count * sizeof(T));
    return p;
  }
};

bool is_int4(const ss_linear& w) { return w.kind == SS_W4G64 || w.kind == SS_W4G64_TILED; }

ss::W4Args w4_args(const void* x, int T, const ss_linear& w, int N, int K) {
  ss::W4Args a{};
  a.x = static_cast<const uint16_t*>(x);
  a.T = T; a.N = N; a.K = K;
  a.qw = static_cast<const uint8_t*>(w.qweight);
  a.tiled = w.kind == SS_W4G64_TILED;
  if (!a.tiled) {
    a.sc = static_cast<const uint16_t*>(w.scale);
    a.zp = static_cast<const uint16_t*>(w.zero);
  }
  return a;
}

ss::GemmArgs bf16_args(const void* x, int T, const void* w, int N, int K) {
  ss::GemmArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.wb = static_cast<const uint16_t*>(w);
  a.T = T; a.N = N; a.K = K;
  return a;
}

// the bf16 GEMM's bounded hand-off waits: report an expiry (checked under SS_DEBUG_SYNC)
ss_status check_bf16_waits(const char* fn) {
  if (!debug_sync()) return SS_OK;
  int expired = 0;
  hipError_t e = ss::gemm_bf16_wait_expired(&expired);
  if (e != hipSuccess) return fail(SS_ERR_DEVICE, "%s: %s", fn, hipGetErrorString(e));
  if (expired) return fail(SS_ERR_DEVICE, "%s: a bf16 GEMM hand-off wait expired (results invalid)", fn);
  return SS_OK;
}

ss_status check_linear(const char* fn, const ss_linear& w, const char* name) {
  if (w.kind == SS_W4G64) {
    if (!w.qweight || !w.scale || !w.zero)
      return fail(SS_ERR_INVALID_ARG, "%s: %s: int4 weight, scale and zero must be non-null", fn, name);
    if (!aligned(w.qweight, 16) || !aligned(w.scale, 4) || !aligned(w.zero, 4))
      return fail(SS_ERR_INVALID_ARG, "%s: %s: misaligned int4 weight, scale or zero", fn, name);
  } else if (w.kind == SS_W4G64_TILED) {
    if (!w.qweight) return fail(SS_ERR_INVALID_ARG, "%s: %s: tiled int4 weight is null", fn, name);
    if (!aligned(w.qweight, 16)) return fail(SS_ERR_INVALID_ARG, "%s: %s: tiled int4 weight is not 16-byte aligned", fn, name);
  } else if (w.kind == SS_BF16) {
    if (!w.w) return fail(SS_ERR_INVALID_ARG, "%s: %s: bf16 weight is null", fn, name);
    if (!aligned(w.w, 16)) return fail(SS_ERR_INVALID_ARG, "%s: %s: bf16 weight is not 16-byte aligned", fn, name);
  } else {
    return fail(SS_ERR_INVALID_ARG, "%s: %s: unknown weight kind %d", fn, name, w.kind);
  }
  return SS_OK;
}

// -------------------------------------------------------------- step planning

struct StepLayout {
  int32_t* err;
  float* ssq;        // [T][ssq_groups(H)] sums of h^2 per 256-column group (RMSNorm folded into GEMMs)
  uint64_t* mask;
  int32_t* depth;
  float2* rope;      // [T][hd / 2] (cos, sin) of the step's RoPE angles
  float* h32;
  uint16_t* xn;
  float* qkv32;
  uint16_t* qbuf;
  uint16_t* attn;
  uint16_t* ubuf;
  void* gemm_ws;
  void* attn_ws;
  size_t total;
};

StepLayout plan_step(const ss_model* m, int T, int C, int R, void* base) {
  Bump bp{static_cast<char*>(base)};
  StepLayout L{};
  const int W = (T + 63) / 64;
  const int qkvN = (m->nq + 2 * m->nkv) * m->hd;
  const int rows_norm = std::max(T, R);
  L.err = bp.take<int32_t>(4);
  L.ssq = bp.take<float>((size_t)T * ss::ssq_groups(m->H));
  L.mask = bp.take<uint64_t>((size_t)T * W);
  L.depth = bp.take<int32_t>(T);
  L.rope = bp.take<float2>((size_t)T * (m->hd / 2));
  L.h32 = bp.take<float>((size_t)T * m->H);
  L.xn = bp.take<uint16_t>((size_t)rows_norm * m->H);
  L.qkv32 = bp.take<float>((size_t)T * qkvN);
  L.qbuf = bp.take<uint16_t>((size_t)T * m->nq * m->hd);
  L.attn = bp.take<uint16_t>((size_t)T * m->nq * m->hd);
  L.ubuf = bp.take<uint16_t>((size_t)T * m->I);
  size_t g = 0;
  auto need = [&](size_t bytes) { g = std::max(g, bytes); };
  // both engines' plans (a model may mix int4 and bf16 linears)
  need(ss::plan_w4(T, qkvN, m->H, ss::EPI_STORE, 0, false).ws_bytes);
  need(ss::plan_w4(T, m->H, m->nq * m->hd, ss::EPI_RESID, 0, false).ws_bytes);
  need(ss::plan_w4(T, 2 * m->I, m->H, ss::EPI_SWIGLU, m->I, true).ws_bytes);
  need(ss::plan_w4(T, m->H, m->I, ss::EPI_RESID, 0, false).ws_bytes);
  need(ss::plan_gemm(T, qkvN, m->H, ss::EPI_STORE, 0).ws_bytes);
  need(ss::plan_gemm(T, m->H, m->nq * m->hd, ss::EPI_RESID, 0).ws_bytes);
  need(ss::plan_gemm(T, 2 * m->I, m->H, ss::EPI_SWIGLU, m->I).ws_bytes);
  need(ss::plan_gemm(T, m->H, m->I, ss::EPI_RESID, 0).ws_bytes);
  if (R > 0 && m->V > 0) need(ss::plan_gemm(R, m->V, m->H, ss::EPI_STORE, 0).ws_bytes);
  L.gemm_ws = bp.take<char>(g);
  L.attn_ws = bp.take<char>(ss::plan_attention(T, C, m->nq, m->nkv, m->hd).ws_bytes);
  L.total = bp.off;
  return L;
}

ss_status check_model(const char* fn, const ss_model* m) {
  if (!m) return fail(SS_ERR_INVALID_ARG, "%s: model is null", fn);
  if (m->H <= 0 || m->I <= 0 || m->nq <= 0 || m->nkv <= 0 || m->hd <= 0 || m->L <= 0)
    return fail(SS_ERR_INVALID_ARG, "%s: model sizes must be positive", fn);
  if (m->hd != 64 && m->hd != 128) return fail(SS_ERR_UNSUPPORTED, "%s: hd must be 64 or 128", fn);
  if (m->nq % m->nkv) return fail(SS_ERR_UNSUPPORTED, "%s: nq must be a multiple of nkv", fn);
  if (m->nq / m->nkv > 16) return fail(SS_ERR_UNSUPPORTED, "%s: nq / nkv must be <= 16", fn);
  if (m->H % 128 || m->I % 128 || (m->nq * m->hd) % 128)
    return fail(SS_ERR_UNSUPPORTED, "%s: H, I and nq*hd must be multiples of 128", fn);
  if (m->H > 8192 || (m->nq + 2 * m->nkv) * m->hd > 8192)
    return fail(SS_ERR_UNSUPPORTED, "%s: H and (nq + 2 nkv) * hd must be <= 8192", fn);
  if (!m->layers) return fail(SS_ERR_INVALID_ARG, "%s: layers is null", fn);
  if (m->c_stride < 0) return fail(SS_ERR_INVALID_ARG, "%s: c_stride is negative", fn);
  if (!(m->rms_eps >= 0.f) || !(m->rope_theta > 0.f))
    return fail(SS_ERR_INVALID_ARG, "%s: rms_eps must be >= 0 and rope_theta > 0", fn);
  for (int l = 0; l < m->L; ++l) {
    const ss_layer& ly = m->layers[l];
    if (!ly.norm1 || !ly.norm2) return fail(SS_ERR_INVALID_ARG, "%s: layer %d: null norm gain", fn, l);
    // a null cache is allowed with an empty prefix (C == 0, checked by the step)
    if ((ly.k_cache && !aligned(ly.k_cache, 16)) || (ly.v_cache && !aligned(ly.v_cache, 16)))
      return fail(SS_ERR_INVALID_ARG, "%s: layer %d: KV cache not 16-byte aligned", fn, l);
    ss_status s;
    if ((s = check_linear(fn, ly.qkv, "qkv")) != SS_OK) return s;
    if ((s = check_linear(fn, ly.o, "o")) != SS_OK) return s;
    if ((s = check_linear(fn, ly.gate_up, "gate_up")) != SS_OK) return s;
    if ((s = check_linear(fn, ly.down, "down")) != SS_OK) return s;
  }
  return SS_OK;
}

}  // namespace

extern "C" {

const char* ss_last_error(void) { return g_err.c_str(); }
int ss_abi_version(void) { return 2; }

// ------------------------------------------------------------------ quantization

ss_status ss_quantize_substitute(const void* w_bf16, int64_t n, int64_t k, int32_t group,
                                 void* qweight, void* scale, void* zero, void* stream) {
  const char* fn = __func__;
  if (group != 64) return fail(SS_ERR_UNSUPPORTED, "%s: group must be 64 (got %d)", fn, group);
  if (n <= 0 || k <= 0) return fail(SS_ERR_INVALID_ARG, "%s: n and k must be positive", fn);
  if (k % 64) return fail(SS_ERR_UNSUPPORTED, "%s: k must be a multiple of 64", fn);
  if (n * (k / 64) > (int64_t)4 * 0x7FFFFFFF) return fail(SS_ERR_UNSUPPORTED, "%s: too many groups", fn);
  REQ_PTR(w_bf16, 16); REQ_PTR(qweight, 16); REQ_PTR(scale, 2); REQ_PTR(zero, 2);
  ss_status s = check_device(fn);
  if (s != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_quantize_g64(static_cast<const uint16_t*>(w_bf16), n, k,
                                              static_cast<uint8_t*>(qweight), static_cast<uint16_t*>(scale),
                                              static_cast<uint16_t*>(zero), st), st);
}

ss_status ss_dequantize_substitute(const void* qweight, const void* scale, const void* zero, int64_t n,
                                   int64_t k, int32_t group, void* w_f16, void* stream) {
  const char* fn = __func__;
  if (group != 64) return fail(SS_ERR_UNSUPPORTED, "%s: group must be 64 (got %d)", fn, group);
  if (n <= 0 || k <= 0) return fail(SS_ERR_INVALID_ARG, "%s: n and k must be positive", fn);
  if (k % 64) return fail(SS_ERR_UNSUPPORTED, "%s: k must be a multiple of 64", fn);
  REQ_PTR(qweight, 16); REQ_PTR(scale, 2); REQ_PTR(zero, 2); REQ_PTR(w_f16, 16);
  ss_status s = check_device(fn);
  if (s != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_dequantize_g64(static_cast<const uint8_t*>(qweight),
                                                static_cast<const uint16_t*>(scale),
                                                static_cast<const uint16_t*>(zero), n, k,
                                                static_cast<uint16_t*>(w_f16), st), st);
}

// ------------------------------------------------------------------ linear layers

// Shape and pointer checks shared by the linear layers; need = the workspace the plan asks for.
static ss_status linear_common(const char* fn, const void* x, int32_t T, int64_t n, int64_t k,
                               void* y_bf16, float* y_f32, void* ws, size_t ws_bytes, size_t need) {
  REQ_PTR(x, 16);
  if (!y_bf16 && !y_f32) return fail(SS_ERR_INVALID_ARG, "%s: y_bf16 and y_f32 are both null", fn);
  OPT_PTR(y_bf16, 2); OPT_PTR(y_f32, 4);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(SS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
  OPT_PTR(ws, 16);
  return SS_OK;
}

static ss_status linear_sizes(const char* fn, int32_t T, int64_t n, int64_t k) {
  if (T < 1 || T > 256) return fail(SS_ERR_UNSUPPORTED, "%s: T must be in 1..256 (got %d)", fn, T);
  if (n <= 0 || k <= 0) return fail(SS_ERR_INVALID_ARG, "%s: n and k must be positive", fn);
  if (k % 128) return fail(SS_ERR_UNSUPPORTED, "%s: k must be a multiple of 128", fn);
  if (n % 16) return fail(SS_ERR_UNSUPPORTED, "%s: n must be a multiple of 16", fn);
  if (n > 0x7FFFFFFF / 256 || k > 0x7FFFFFFF / 2) return fail(SS_ERR_UNSUPPORTED, "%s: n or k too large", fn);
  return SS_OK;
}

static bool linear_shape_ok(int32_t T, int64_t n, int64_t k) {
  return T >= 1 && T <= 256 && n > 0 && k > 0 && k % 128 == 0 && n % 16 == 0 && n <= 0x7FFFFFFF / 256 &&
         k <= 0x7FFFFFFF / 2;
}

size_t ss_w4a16_linear_workspace(int32_t T, int64_t n, int64_t k) {
  if (!linear_shape_ok(T, n, k)) return 0;
  return ss::plan_w4(T, (int)n, (int)k, ss::EPI_STORE, 0, true).ws_bytes;
}
size_t ss_bf16_linear_workspace(int32_t T, int64_t n, int64_t k) {
  if (!linear_shape_ok(T, n, k)) return 0;
  return ss::plan_gemm(T, (int)n, (int)k, ss::EPI_STORE, 0).ws_bytes;
}

static ss_status w4_linear(const char* fn, const void* x, int32_t T, const ss_linear& w, int64_t n, int64_t k,
                           void* y_bf16, float* y_f32, void* ws, size_t ws_bytes, void* stream) {
  ss_status s = linear_sizes(fn, T, n, k);
  if (s != SS_OK) return s;
  const ss::W4Plan pl = ss::plan_w4(T, (int)n, (int)k, ss::EPI_STORE, 0, true);
  if ((s = linear_common(fn, x, T, n, k, y_bf16, y_f32, ws, ws_bytes, pl.ws_bytes)) != SS_OK) return s;
  if ((s = check_linear(fn, w, "weight")) != SS_OK) return s;
  if ((s = check_device(fn)) != SS_OK) return s;
  ss::W4Args a = w4_args(x, T, w, (int)n, (int)k);
  a.epi = ss::EPI_STORE;
  a.y_f32 = y_f32;
  a.y_bf16 = static_cast<uint16_t*>(y_bf16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_w4(a, pl, ws, st), st);
}

ss_status ss_w4a16_linear(const void* x_bf16, int32_t T, const void* qweight, const void* scale,
                          const void* zero, int64_t n, int64_t k, void* y_bf16, float* y_f32,
                          void* workspace, size_t ws_bytes, void* stream) {
  const ss_linear w{SS_W4G64, qweight, scale, zero, nullptr};
  return w4_linear(__func__, x_bf16, T, w, n, k, y_bf16, y_f32, workspace, ws_bytes, stream);
}

static ss_status w4_gate_up(const char* fn, const void* x, int32_t T, const ss_linear& w, int64_t I, int64_t k,
                            void* u_bf16, void* ws, size_t ws_bytes, void* stream) {
  if (T < 1 || T > 256) return fail(SS_ERR_UNSUPPORTED, "%s: T must be in 1..256 (got %d)", fn, T);
  if (I <= 0 || k <= 0) return fail(SS_ERR_INVALID_ARG, "%s: I and k must be positive", fn);
  if (k % 128) return fail(SS_ERR_UNSUPPORTED, "%s: k must be a multiple of 128", fn);
  if (I % 16) return fail(SS_ERR_UNSUPPORTED, "%s: I must be a multiple of 16", fn);
  if (2 * I > 0x7FFFFFFF / 256 || k > 0x7FFFFFFF / 2) return fail(SS_ERR_UNSUPPORTED, "%s: I or k too large", fn);
  REQ_PTR(x, 16); REQ_PTR(u_bf16, 2);
  ss_status s = check_linear(fn, w, "weight");
  if (s != SS_OK) return s;
  const ss::W4Plan pl = ss::plan_w4(T, (int)(2 * I), (int)k, ss::EPI_SWIGLU, (int)I, true);
  if (pl.ws_bytes > 0 && (!ws || ws_bytes < pl.ws_bytes))
    return fail(SS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, pl.ws_bytes, ws ? ws_bytes : 0);
  OPT_PTR(ws, 16);
  if ((s = check_device(fn)) != SS_OK) return s;
  ss::W4Args a = w4_args(x, T, w, (int)(2 * I), (int)k);
  a.epi = ss::EPI_SWIGLU;
  a.swiglu_I = (int)I;
  a.u_bf16 = static_cast<uint16_t*>(u_bf16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_w4(a, pl, ws, st), st);
}

size_t ss_w4a16_gate_up_swiglu_workspace(int32_t T, int64_t I, int64_t k) {
  if (T < 1 || T > 256 || I <= 0 || I % 16 || k < 128 || k % 128 || 2 * I > 0x7FFFFFFF / 256) return 0;
  return ss::plan_w4(T, (int)(2 * I), (int)k, ss::EPI_SWIGLU, (int)I, true).ws_bytes;
}

ss_status ss_w4a16_gate_up_swiglu(const void* x_bf16, int32_t T, const void* qweight, const void* scale,
                                  const void* zero, int64_t I, int64_t k, void* u_bf16, void* workspace,
                                  size_t ws_bytes, void* stream) {
  const ss_linear w{SS_W4G64, qweight, scale, zero, nullptr};
  return w4_gate_up(__func__, x_bf16, T, w, I, k, u_bf16, workspace, ws_bytes, stream);
}

size_t ss_w4_tiled_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || n % 16 || k % 128) return 0;
  return (size_t)(n / 16) * (size_t)(k / 128) * ss::TILE_BLOCK_BYTES;
}

ss_status ss_w4_tile(const void* qweight, const void* scale, const void* zero, int64_t n, int64_t k,
                     void* tiled, void* stream) {
  const char* fn = __func__;
  if (n <= 0 || k <= 0) return fail(SS_ERR_INVALID_ARG, "%s: n and k must be positive", fn);
  if (n % 16 || k % 128) return fail(SS_ERR_UNSUPPORTED, "%s: n must be a multiple of 16 and k of 128", fn);
  REQ_PTR(qweight, 16); REQ_PTR(scale, 2); REQ_PTR(zero, 2); REQ_PTR(tiled, 16);
  ss_status s = check_device(fn);
  if (s != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_w4_tile(static_cast<const uint8_t*>(qweight), static_cast<const uint16_t*>(scale),
                                         static_cast<const uint16_t*>(zero), n, k, static_cast<uint8_t*>(tiled), st), st);
}

ss_status ss_w4a16_linear_tiled(const void* x_bf16, int32_t T, const void* tiled, int64_t n, int64_t k,
                                void* y_bf16, float* y_f32, void* workspace, size_t ws_bytes, void* stream) {
  const ss_linear w{SS_W4G64_TILED, tiled, nullptr, nullptr, nullptr};
  return w4_linear(__func__, x_bf16, T, w, n, k, y_bf16, y_f32, workspace, ws_bytes, stream);
}

ss_status ss_w4a16_linear_tiled_noalloc(const void* x_bf16, int32_t T, const void* tiled, int64_t n, int64_t k,
                                        void* y_bf16, float* y_f32, void* stream) {
  const char* fn = __func__;
  ss_status s = linear_sizes(fn, T, n, k);
  if (s != SS_OK) return s;
  const ss::W4Plan pl = ss::plan_w4(T, (int)n, (int)k, ss::EPI_STORE, 0, true);
  if (pl.ws_bytes > ss::W4_SCRATCH_BYTES)
    return fail(SS_ERR_WORKSPACE, "%s: this shape needs %zu bytes of partial sums, beyond the %zu-byte device scratch",
                fn, pl.ws_bytes, ss::W4_SCRATCH_BYTES);
  if ((s = linear_common(fn, x_bf16, T, n, k, y_bf16, y_f32, nullptr, 0, 0)) != SS_OK) return s;
  const ss_linear w{SS_W4G64_TILED, tiled, nullptr, nullptr, nullptr};
  if ((s = check_linear(fn, w, "weight")) != SS_OK) return s;
  if ((s = check_device(fn)) != SS_OK) return s;
  void* scratch = nullptr;
  const hipError_t e = ss::w4_scratch(&scratch);
  if (e != hipSuccess) return fail(SS_ERR_DEVICE, "%s: device scratch address: %s", fn, hipGetErrorString(e));
  ss::W4Args a = w4_args(x_bf16, T, w, (int)n, (int)k);
  a.epi = ss::EPI_STORE;
  a.y_f32 = y_f32;
  a.y_bf16 = static_cast<uint16_t*>(y_bf16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_w4(a, pl, scratch, st), st);
}

ss_status ss_w4a16_gate_up_swiglu_tiled(const void* x_bf16, int32_t T, const void* tiled, int64_t I, int64_t k,
                                        void* u_bf16, void* workspace, size_t ws_bytes, void* stream) {
  const ss_linear w{SS_W4G64_TILED, tiled, nullptr, nullptr, nullptr};
  return w4_gate_up(__func__, x_bf16, T, w, I, k, u_bf16, workspace, ws_bytes, stream);
}

ss_status ss_bf16_linear(const void* x_bf16, int32_t T, const void* w_bf16, int64_t n, int64_t k,
                         void* y_bf16, float* y_f32, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = __func__;
  ss_status s = linear_sizes(fn, T, n, k);
  if (s != SS_OK) return s;
  const ss::GemmPlan pl = ss::plan_gemm(T, (int)n, (int)k, ss::EPI_STORE, 0);
  if ((s = linear_common(fn, x_bf16, T, n, k, y_bf16, y_f32, workspace, ws_bytes, pl.ws_bytes)) != SS_OK) return s;
  REQ_PTR(w_bf16, 16);
  if ((s = check_device(fn)) != SS_OK) return s;
  ss::GemmArgs a = bf16_args(x_bf16, T, w_bf16, (int)n, (int)k);
  a.epi = ss::EPI_STORE;
  a.y_f32 = y_f32;
  a.y_bf16 = static_cast<uint16_t*>(y_bf16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = launched(fn, ss::launch_gemm(a, pl, workspace, st), st);
  if (s != SS_OK) return s;
  return check_bf16_waits(fn);
}

// ------------------------------------------------------------------ tree

ss_status ss_tree_validate(const int32_t* parents_host, int32_t T) {
  const char* fn = __func__;
  if (!parents_host) return fail(SS_ERR_INVALID_ARG, "%s: parents_host is null", fn);
  if (T < 1) return fail(SS_ERR_INVALID_ARG, "%s: T must be >= 1", fn);
  if (parents_host[0] != -1) return fail(SS_ERR_BAD_TREE, "%s: parents[0] must be -1", fn);
  for (int i = 1; i < T; ++i)
    if (parents_host[i] < 0 || parents_host[i] >= i)
      return fail(SS_ERR_BAD_TREE, "%s: parents[%d] = %d is not in [0, %d)", fn, i, parents_host[i], i);
  return ok();
}

static ss_status debug_validate_parents(const char* fn, const int32_t* parents, int T, hipStream_t st) {
  if (!debug_sync()) return ok();
  std::vector<int32_t> h(T);
  hipError_t e = hipMemcpyAsync(h.data(), parents, T * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(SS_ERR_DEVICE, "%s: %s", fn, hipGetErrorString(e));
  ss_status s = ss_tree_validate(h.data(), T);
  if (s != SS_OK) return fail(s, "%s: %s", fn, g_err.c_str());
  return ok();
}

ss_status ss_tree_mask(const int32_t* parents, int32_t T, uint64_t* mask_out, int32_t* depth_out,
                       void* stream) {
  const char* fn = __func__;
  if (T < 1 || T > 256) return fail(SS_ERR_UNSUPPORTED, "%s: T must be in 1..256 (got %d)", fn, T);
  REQ_PTR(parents, 4); REQ_PTR(mask_out, 8); OPT_PTR(depth_out, 4);
  ss_status s = check_device(fn);
  if (s != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = launched(fn, ss::launch_tree_mask(parents, T, mask_out, depth_out, nullptr, st), st);
  if (s != SS_OK) return s;
  return debug_validate_parents(fn, parents, T, st);
}

// ------------------------------------------------------------------ attention

static ss_status attn_sizes(const char* fn, int T, int C, int nq, int nkv, int hd) {
  if (T < 1 || T > 256) return fail(SS_ERR_UNSUPPORTED, "%s: T must be in 1..256 (got %d)", fn, T);
  if (C < 0) return fail(SS_ERR_INVALID_ARG, "%s: C must be >= 0", fn);
  if (nq <= 0 || nkv <= 0) return fail(SS_ERR_INVALID_ARG, "%s: nq and nkv must be positive", fn);
  if (hd != 64 && hd != 128) return fail(SS_ERR_UNSUPPORTED, "%s: hd must be 64 or 128", fn);
  if (nq % nkv) return fail(SS_ERR_UNSUPPORTED, "%s: nq must be a multiple of nkv", fn);
  if (nq / nkv > 16) return fail(SS_ERR_UNSUPPORTED, "%s: nq / nkv must be <= 16", fn);
  if ((int64_t)C + T > (1 << 24)) return fail(SS_ERR_UNSUPPORTED, "%s: C + T too large", fn);
  return SS_OK;
}

static size_t attn_ws_total(int T, int C, int nq, int nkv, int hd) {
  const int W = (T + 63) / 64;
  return up(4 * sizeof(int32_t)) + up((size_t)T * W * 8) + ss::plan_attention(T, C, nq, nkv, hd).ws_bytes;
}

size_t ss_tree_attention_workspace(int32_t T, int32_t C, int32_t nq, int32_t nkv, int32_t hd) {
  if (attn_sizes("ss_tree_attention_workspace", T, C, nq, nkv, hd) != SS_OK) return 0;
  return attn_ws_total(T, C, nq, nkv, hd);
}

ss_status ss_tree_attention(const ss_attn_args* a, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = __func__;
  if (!a) return fail(SS_ERR_INVALID_ARG, "%s: args is null", fn);
  ss_status s = attn_sizes(fn, a->T, a->C, a->nq, a->nkv, a->hd);
  if (s != SS_OK) return s;
  if (a->C > a->c_stride) return fail(SS_ERR_INVALID_ARG, "%s: C > c_stride", fn);
  REQ_PTR(a->q, 16); REQ_PTR(a->k_tree, 16); REQ_PTR(a->v_tree, 16); REQ_PTR(a->parents, 4);
  if (a->C > 0) { REQ_PTR(a->k_cache, 16); REQ_PTR(a->v_cache, 16); }
  if (!a->out && !a->out_f32) return fail(SS_ERR_INVALID_ARG, "%s: out and out_f32 are both null", fn);
  OPT_PTR(a->out, 2); OPT_PTR(a->out_f32, 4); OPT_PTR(a->mask_out, 8);
  const size_t need = attn_ws_total(a->T, a->C, a->nq, a->nkv, a->hd);
  if (!workspace || ws_bytes < need)
    return fail(SS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? ws_bytes : 0);
  REQ_PTR(workspace, 16);
  if ((s = check_device(fn)) != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Bump bp{static_cast<char*>(workspace)};
  int32_t* err = bp.take<int32_t>(4);
  uint64_t* mask = bp.take<uint64_t>((size_t)a->T * ((a->T + 63) / 64));
  void* aws = bp.take<char>(ss::plan_attention(a->T, a->C, a->nq, a->nkv, a->hd).ws_bytes);
  if (a->mask_out) mask = a->mask_out;
  hipError_t e = ss::launch_tree_mask(a->parents, a->T, mask, nullptr, err, st);
  if (e != hipSuccess) return fail(SS_ERR_DEVICE, "%s: %s", fn, hipGetErrorString(e));
  ss::AttnArgs aa{};
  aa.q = static_cast<const uint16_t*>(a->q);
  aa.kc = static_cast<const uint16_t*>(a->k_cache);
  aa.vc = static_cast<const uint16_t*>(a->v_cache);
  aa.kt = static_cast<const uint16_t*>(a->k_tree);
  aa.vt = static_cast<const uint16_t*>(a->v_tree);
  aa.mask = mask;
  aa.out = static_cast<uint16_t*>(a->out);
  aa.out_f32 = a->out_f32;
  aa.T = a->T; aa.C = a->C; aa.c_stride = a->c_stride; aa.nq = a->nq; aa.nkv = a->nkv; aa.hd = a->hd;
  aa.sm_scale = (a->sm_scale > 0.f) ? a->sm_scale : 1.0f / std::sqrt((float)a->hd);
  s = launched(fn, ss::launch_attention(aa, ss::plan_attention(a->T, a->C, a->nq, a->nkv, a->hd), aws, st), st);
  if (s != SS_OK) return s;
  return check_err_word(fn, err, st);
}

// ------------------------------------------------------------------ draft step

size_t ss_draft_tree_step_workspace(const ss_model* model, int32_t T, int32_t C) {
  if (!model || T < 1 || T > 256 || C < 0 || model->H <= 0 || model->nkv <= 0 || model->hd <= 0)
    return 0;
  return plan_step(model, T, C, (model->V > 0 && model->lm_head) ? T : 0, nullptr).total;
}

ss_status ss_draft_tree_step(const ss_model* m, const ss_step_args* a, void* workspace, size_t ws_bytes,
                             void* stream) {
  const char* fn = __func__;
  ss_status s = check_model(fn, m);
  if (s != SS_OK) return s;
  if (!a) return fail(SS_ERR_INVALID_ARG, "%s: args is null", fn);
  const int T = a->T, C = a->C;
  if ((s = attn_sizes(fn, T, C, m->nq, m->nkv, m->hd)) != SS_OK) return s;
  if (C > m->c_stride) return fail(SS_ERR_INVALID_ARG, "%s: C > c_stride", fn);
  REQ_PTR(a->parents, 4);
  if (!a->tree_k || !a->tree_v) return fail(SS_ERR_INVALID_ARG, "%s: tree_k / tree_v arrays are null", fn);
  for (int l = 0; l < m->L; ++l) {
    if (C > 0 && (!m->layers[l].k_cache || !m->layers[l].v_cache))
      return fail(SS_ERR_INVALID_ARG, "%s: layer %d: null KV cache with a prefix of %d keys", fn, l, C);
    if (!a->tree_k[l] || !a->tree_v[l]) return fail(SS_ERR_INVALID_ARG, "%s: tree K/V of layer %d is null", fn, l);
    if (!aligned(a->tree_k[l], 16) || !aligned(a->tree_v[l], 16))
      return fail(SS_ERR_INVALID_ARG, "%s: tree K/V of layer %d not 16-byte aligned", fn, l);
  }
  if (a->hidden_in) {
    OPT_PTR(a->hidden_in, 16);
  } else {
    REQ_PTR(a->tokens, 4);
    if (!m->embed || m->V <= 0) return fail(SS_ERR_INVALID_ARG, "%s: embed / V needed without hidden_in", fn);
  }
  OPT_PTR(a->hidden_out, 2);
  int R = 0;
  if (a->logits) {
    OPT_PTR(a->logits, 4);
    if (!m->lm_head || !m->final_norm || m->V <= 0)
      return fail(SS_ERR_INVALID_ARG, "%s: logits need lm_head, final_norm and V > 0", fn);
    if (m->V % 16) return fail(SS_ERR_UNSUPPORTED, "%s: V must be a multiple of 16", fn);
    if (!aligned(m->lm_head, 16)) return fail(SS_ERR_INVALID_ARG, "%s: lm_head not 16-byte aligned", fn);
    if (a->logit_rows) {
      OPT_PTR(a->logit_rows, 4);
      if (a->n_logit_rows < 1 || a->n_logit_rows > 256)
        return fail(SS_ERR_UNSUPPORTED, "%s: n_logit_rows must be in 1..256", fn);
      R = a->n_logit_rows;
    } else {
      R = T;
    }
  }
  const size_t need = plan_step(m, T, C, R, nullptr).total;
  if (!workspace || ws_bytes < need)
    return fail(SS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? ws_bytes : 0);
  REQ_PTR(workspace, 16);
  if ((s = check_device(fn)) != SS_OK) return s;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const StepLayout Ly = plan_step(m, T, C, R, workspace);
  const int H = m->H, I = m->I, nq = m->nq, nkv = m->nkv, hd = m->hd;
  const int qkvN = (nq + 2 * nkv) * hd;
  hipError_t e = hipSuccess;
#define RUN(expr)                                                                   \
  do {                                                                              \
    e = (expr);                                                                     \
    if (e != hipSuccess) return fail(SS_ERR_DEVICE, "%s: %s: %s", fn, #expr, hipGetErrorString(e)); \
  } while (0)

  RUN(ss::launch_tree_mask(a->parents, T, Ly.mask, Ly.depth, Ly.err, st));
  RUN(ss::launch_rope_table(Ly.depth, T, C, hd, m->rope_theta, Ly.rope, st));
  if (a->hidden_in) RUN(ss::launch_bf16_to_f32(static_cast<const uint16_t*>(a->hidden_in), (size_t)T * H, Ly.h32, st));
  else RUN(ss::launch_embed(a->tokens, static_cast<const uint16_t*>(m->embed), T, H, m->V, Ly.h32, Ly.err, st));

  const ss::AttnPlan apl = ss::plan_attention(T, C, nq, nkv, hd);
  for (int l = 0; l < m->L; ++l) {
    const ss_layer& ly = m->layers[l];
    uint16_t* tk = static_cast<uint16_t*>(a->tree_k[l]);
    uint16_t* tv = static_cast<uint16_t*>(a->tree_v[l]);
    // RMSNorm is folded into the GEMM that consumes it: xn holds bf16(h * gain) and ssq the
    // sums of h^2 per 256-column group, written by whoever finished h (row_stats for layer
    // 0, then resid_finish after the residual GEMMs); the consumer GEMM scales its output
    // rows by 1 / rms.
    if (l == 0) RUN(ss::launch_row_stats(Ly.h32, T, H, static_cast<const uint16_t*>(ly.norm1), Ly.xn, Ly.ssq, st));
    auto consume_norm = [&](auto& g) {
      g.ssq_in = Ly.ssq;
      g.ssq_n = ss::ssq_groups(H);
      g.rms_H = H;
      g.rms_eps = m->rms_eps;
    };
    // qkv: int4 on the W4 engine (its K ranges' partials go straight to the RoPE scatter),
    // bf16 on the bf16 engine (whole output in qkv32)
    if (is_int4(ly.qkv)) {
      ss::W4Args g = w4_args(Ly.xn, T, ly.qkv, qkvN, H);
      g.epi = ss::EPI_STORE;
      g.y_f32 = Ly.qkv32;
      g.defer_reduce = true;
      consume_norm(g);
      const ss::W4Plan pl = ss::plan_w4(T, qkvN, H, g.epi, 0, false);
      RUN(ss::launch_w4(g, pl, Ly.gemm_ws, st));
      RUN(ss::launch_qkv_finish(static_cast<const float*>(Ly.gemm_ws), pl.splits, Ly.qkv32, Ly.rope, T, nq, nkv,
                                hd, Ly.qbuf, tk, tv, st));
    } else {
      ss::GemmArgs g = bf16_args(Ly.xn, T, ly.qkv.w, qkvN, H);
      g.epi = ss::EPI_STORE;
      g.y_f32 = Ly.qkv32;
      consume_norm(g);
      RUN(ss::launch_gemm(g, ss::plan_gemm(T, qkvN, H, g.epi, 0), Ly.gemm_ws, st));
      RUN(ss::launch_qkv_finish(nullptr, 1, Ly.qkv32, Ly.rope, T, nq, nkv, hd, Ly.qbuf, tk, tv, st));
    }
    {
      ss::AttnArgs aa{};
      aa.q = Ly.qbuf;
      aa.kc = static_cast<const uint16_t*>(ly.k_cache);
      aa.vc = static_cast<const uint16_t*>(ly.v_cache);
      aa.kt = tk; aa.vt = tv; aa.mask = Ly.mask; aa.out = Ly.attn;
      aa.T = T; aa.C = C; aa.c_stride = m->c_stride; aa.nq = nq; aa.nkv = nkv; aa.hd = hd;
      aa.sm_scale = 1.0f / std::sqrt((float)hd);
      RUN(ss::launch_attention(aa, apl, Ly.attn_ws, st));
    }
    // residual GEMMs: h += x W^T, then the next RMSNorm's inputs (hg = bf16(h * gain), ssq)
    // in resid_finish (which also adds the W4 engine's K ranges) or row_stats
    auto residual = [&](const ss_linear& w, const void* x, int K, const void* gain) -> hipError_t {
      hipError_t e2;
      if (is_int4(w)) {
        ss::W4Args g = w4_args(x, T, w, H, K);
        g.epi = ss::EPI_RESID;
        g.resid = Ly.h32;
        g.defer_reduce = true;
        const ss::W4Plan pl = ss::plan_w4(T, H, K, g.epi, 0, false);
        if ((e2 = ss::launch_w4(g, pl, Ly.gemm_ws, st)) != hipSuccess) return e2;
        return ss::launch_resid_finish(static_cast<const float*>(Ly.gemm_ws), pl.splits, Ly.h32, T, H,
                                       static_cast<const uint16_t*>(gain), Ly.xn, Ly.ssq, st);
      }
      ss::GemmArgs g = bf16_args(x, T, w.w, H, K);
      g.epi = ss::EPI_RESID;
      g.resid = Ly.h32;
      if ((e2 = ss::launch_gemm(g, ss::plan_gemm(T, H, K, g.epi, 0), Ly.gemm_ws, st)) != hipSuccess) return e2;
      if (!gain) return hipSuccess;
      return ss::launch_row_stats(Ly.h32, T, H, static_cast<const uint16_t*>(gain), Ly.xn, Ly.ssq, st);
    };
    RUN(residual(ly.o, Ly.attn, nq * hd, ly.norm2));
    // MLP block: gate_up with SwiGLU (rows scaled by RMSNorm-2), then down
    if (is_int4(ly.gate_up)) {
      ss::W4Args g = w4_args(Ly.xn, T, ly.gate_up, 2 * I, H);
      g.epi = ss::EPI_SWIGLU;
      g.swiglu_I = I;
      g.u_bf16 = Ly.ubuf;
      consume_norm(g);
      RUN(ss::launch_w4(g, ss::plan_w4(T, 2 * I, H, g.epi, I, true), Ly.gemm_ws, st));
    } else {
      ss::GemmArgs g = bf16_args(Ly.xn, T, ly.gate_up.w, 2 * I, H);
      g.epi = ss::EPI_SWIGLU;
      g.swiglu_I = I;
      g.u_bf16 = Ly.ubuf;
      consume_norm(g);
      RUN(ss::launch_gemm(g, ss::plan_gemm(T, 2 * I, H, g.epi, I), Ly.gemm_ws, st));
    }
    // the next layer's RMSNorm-1 inputs (none after the last layer)
    RUN(residual(ly.down, Ly.ubuf, I, (l + 1 < m->L) ? m->layers[l + 1].norm1 : nullptr));
  }
  if (a->hidden_out) RUN(ss::launch_f32_to_bf16(Ly.h32, (size_t)T * H, static_cast<uint16_t*>(a->hidden_out), st));
  if (a->logits) {
    RUN(ss::launch_rmsnorm(Ly.h32, static_cast<const uint16_t*>(m->final_norm), R, H, m->rms_eps, Ly.xn,
                           a->logit_rows, T, Ly.err, st));
    ss::GemmArgs g = bf16_args(Ly.xn, R, m->lm_head, m->V, H);
    g.epi = ss::EPI_STORE;
    g.y_f32 = a->logits;
    RUN(ss::launch_gemm(g, ss::plan_gemm(R, m->V, H, g.epi, 0), Ly.gemm_ws, st));
  }
#undef RUN
  s = launched(fn, hipSuccess, st);
  if (s != SS_OK) return s;
  if ((s = check_bf16_waits(fn)) != SS_OK) return s;
  return check_err_word(fn, Ly.err, st);
}

// ------------------------------------------------------------------ verification / selection

ss_status ss_row_argmax(const float* logits, int32_t rows, int32_t vocab, int32_t* out, void* stream) {
  const char* fn = __func__;
  if (rows < 1 || vocab < 1) return fail(SS_ERR_INVALID_ARG, "%s: rows and vocab must be positive", fn);
  if (rows > 65535) return fail(SS_ERR_UNSUPPORTED, "%s: rows must be <= 65535", fn);
  REQ_PTR(logits, 4); REQ_PTR(out, 4);
  ss_status s = check_device(fn);
  if (s != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_row_argmax(logits, rows, vocab, out, st), st);
}

ss_status ss_tree_accept(const int32_t* parents, const int32_t* tokens, const int32_t* target_argmax,
                         int32_t T, int32_t* path_out, int32_t* accept_len_out, int32_t* bonus_out,
                         void* stream) {
  const char* fn = __func__;
  if (T < 1 || T > 4096) return fail(SS_ERR_UNSUPPORTED, "%s: T must be in 1..4096 (got %d)", fn, T);
  REQ_PTR(parents, 4); REQ_PTR(tokens, 4); REQ_PTR(target_argmax, 4);
  REQ_PTR(path_out, 4); REQ_PTR(accept_len_out, 4); REQ_PTR(bonus_out, 4);
  ss_status s = check_device(fn);
  if (s != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = launched(fn, ss::launch_tree_accept(parents, tokens, target_argmax, T, path_out, accept_len_out,
                                          bonus_out, st), st);
  if (s != SS_OK) return s;
  return debug_validate_parents(fn, parents, T, st);
}

static ss_status expand_sizes(const char* fn, int32_t R, int32_t k, int32_t T, int32_t D) {
  if (T < 2 || T > 256) return fail(SS_ERR_UNSUPPORTED, "%s: T must be in 2..256 (got %d)", fn, T);
  if (D < 1 || D > T - 1) return fail(SS_ERR_INVALID_ARG, "%s: D must be in 1..T-1 (got %d)", fn, D);
  if (R < (T - 1 + D - 1) / D) return fail(SS_ERR_INVALID_ARG, "%s: R = %d rows cannot hold the %d nodes a step adds",
                                           fn, R, (T - 1 + D - 1) / D);
  if (k < R || k * R > 64) return fail(SS_ERR_UNSUPPORTED, "%s: need R <= k and k * R <= 64 (k=%d, R=%d)", fn, k, R);
  return SS_OK;
}

ss_status ss_tree_expand_init(int32_t root_token, int32_t T, int32_t D, int32_t R, int32_t k, int32_t* parents,
                              int32_t* tokens, float* cum, int32_t* frontier, int32_t* meta, void* stream) {
  const char* fn = __func__;
  ss_status s = expand_sizes(fn, R, k, T, D);
  if (s != SS_OK) return s;
  if (root_token < 0) return fail(SS_ERR_INVALID_ARG, "%s: root_token must be a token id", fn);
  REQ_PTR(parents, 4); REQ_PTR(tokens, 4); REQ_PTR(cum, 4); REQ_PTR(frontier, 4); REQ_PTR(meta, 4);
  if ((s = check_device(fn)) != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_expand_init(root_token, T, R, parents, tokens, cum, frontier, meta, st), st);
}

size_t ss_tree_expand_workspace(int32_t R, int32_t V) {
  if (R < 1 || R > 64 || V < 1) return 0;
  return ss::expand_ws_bytes(R, V);
}

ss_status ss_tree_expand(const float* logits, const int32_t* children, int32_t R, int32_t V, float inv_temp,
                         int32_t k, int32_t T, int32_t D, int32_t* parents, int32_t* tokens, float* cum,
                         int32_t* frontier, int32_t* meta, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = __func__;
  ss_status s = expand_sizes(fn, R, k, T, D);
  if (s != SS_OK) return s;
  if (V < k) return fail(SS_ERR_INVALID_ARG, "%s: vocab %d smaller than k %d", fn, V, k);
  if (!(inv_temp > 0.f) || !std::isfinite(inv_temp)) return fail(SS_ERR_INVALID_ARG, "%s: inv_temp must be > 0", fn);
  REQ_PTR(logits, 4); REQ_PTR(children, 4);
  REQ_PTR(parents, 4); REQ_PTR(tokens, 4); REQ_PTR(cum, 4); REQ_PTR(frontier, 4); REQ_PTR(meta, 4);
  const size_t need = ss::expand_ws_bytes(R, V);
  if (!workspace || ws_bytes < need)
    return fail(SS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? ws_bytes : 0);
  REQ_PTR(workspace, 16);
  if ((s = check_device(fn)) != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_expand(logits, children, R, V, inv_temp, k, T, D, parents, tokens, cum, frontier,
                                        meta, workspace, st), st);
}

size_t ss_tree_accept_stochastic_workspace(int32_t T, int32_t V) {
  if (T < 1 || T > 256 || V < 1) return 0;
  return ss::sv_ws_bytes(T, V);
}

ss_status ss_tree_accept_stochastic(const int32_t* parents, const int32_t* tokens, const float* draft_logits,
                                    const float* target_logits, int32_t T, int32_t V, float inv_t_draft,
                                    float inv_t_target, const double* uniforms, const double* bonus_uniforms,
                                    int32_t* path_out, int32_t* accept_len_out, int32_t* bonus_out, void* workspace,
                                    size_t ws_bytes, void* stream) {
  const char* fn = __func__;
  if (T < 1 || T > 256) return fail(SS_ERR_UNSUPPORTED, "%s: T must be in 1..256 (got %d)", fn, T);
  if (V < 1) return fail(SS_ERR_INVALID_ARG, "%s: V must be positive", fn);
  if (!(inv_t_draft > 0.f) || !(inv_t_target > 0.f) || !std::isfinite(inv_t_draft) || !std::isfinite(inv_t_target))
    return fail(SS_ERR_INVALID_ARG, "%s: the inverse temperatures must be finite and > 0", fn);
  REQ_PTR(parents, 4); REQ_PTR(tokens, 4); REQ_PTR(draft_logits, 4); REQ_PTR(target_logits, 4);
  REQ_PTR(uniforms, 8); REQ_PTR(bonus_uniforms, 8);
  REQ_PTR(path_out, 4); REQ_PTR(accept_len_out, 4); REQ_PTR(bonus_out, 4);
  const size_t need = ss::sv_ws_bytes(T, V);
  if (!workspace || ws_bytes < need)
    return fail(SS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? ws_bytes : 0);
  REQ_PTR(workspace, 16);
  ss_status s = check_device(fn);
  if (s != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = launched(fn, ss::launch_stochastic_accept(parents, tokens, draft_logits, target_logits, T, V, inv_t_draft,
                                                inv_t_target, uniforms, bonus_uniforms, path_out, accept_len_out,
                                                bonus_out, workspace, st), st);
  if (s != SS_OK) return s;
  return debug_validate_parents(fn, parents, T, st);
}

ss_status ss_kv_commit(void* const* k_cache, void* const* v_cache, const void* const* k_tree,
                       const void* const* v_tree, int32_t layers, int32_t nkv, int32_t hd, int32_t c_stride,
                       int32_t C, int32_t T, const int32_t* path, const int32_t* accept_len, void* stream) {
  const char* fn = __func__;
  if (!k_cache || !v_cache || !k_tree || !v_tree)
    return fail(SS_ERR_INVALID_ARG, "%s: the per-layer pointer arrays must be non-null", fn);
  if (layers < 1 || nkv < 1) return fail(SS_ERR_INVALID_ARG, "%s: layers and nkv must be positive", fn);
  if (hd != 64 && hd != 128) return fail(SS_ERR_UNSUPPORTED, "%s: hd must be 64 or 128", fn);
  if (T < 1 || T > 256) return fail(SS_ERR_UNSUPPORTED, "%s: T must be in 1..256 (got %d)", fn, T);
  if (C < 0 || (int64_t)C + T > c_stride)
    return fail(SS_ERR_INVALID_ARG, "%s: need 0 <= C and C + T <= c_stride (C=%d T=%d c_stride=%d)", fn, C, T,
                c_stride);
  REQ_PTR(path, 4); REQ_PTR(accept_len, 4);
  for (int l = 0; l < layers; ++l) {
    if (!k_cache[l] || !v_cache[l] || !k_tree[l] || !v_tree[l])
      return fail(SS_ERR_INVALID_ARG, "%s: layer %d: null cache or tree pointer", fn, l);
    if (!aligned(k_cache[l], 16) || !aligned(v_cache[l], 16) || !aligned(k_tree[l], 16) || !aligned(v_tree[l], 16))
      return fail(SS_ERR_INVALID_ARG, "%s: layer %d: pointers must be 16-byte aligned", fn, l);
  }
  ss_status s = check_device(fn);
  if (s != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int l0 = 0; l0 < layers; l0 += ss::KVC_MAX_LAYERS) {
    const int n = std::min(layers - l0, ss::KVC_MAX_LAYERS);
    ss::KvCommitPtrs a{};
    for (int i = 0; i < n; ++i) {
      a.kc[i] = static_cast<uint16_t*>(k_cache[l0 + i]);
      a.vc[i] = static_cast<uint16_t*>(v_cache[l0 + i]);
      a.kt[i] = static_cast<const uint16_t*>(k_tree[l0 + i]);
      a.vt[i] = static_cast<const uint16_t*>(v_tree[l0 + i]);
    }
    hipError_t e = ss::launch_kv_commit(a, n, nkv, hd, c_stride, C, T, path, accept_len, st);
    if (e != hipSuccess) return launched(fn, e, st);
  }
  return launched(fn, hipSuccess, st);
}

static ss_status select_sizes(const char* fn, int32_t rows, int32_t vocab, int32_t k) {
  if (rows < 1 || vocab < 1) return fail(SS_ERR_INVALID_ARG, "%s: rows and vocab must be positive", fn);
  if (rows > 65535) return fail(SS_ERR_UNSUPPORTED, "%s: rows must be <= 65535", fn);
  if (k < 1 || k > 16) return fail(SS_ERR_UNSUPPORTED, "%s: k must be in 1..16 (got %d)", fn, k);
  if (vocab < k) return fail(SS_ERR_INVALID_ARG, "%s: vocab < k", fn);
  return SS_OK;
}

size_t ss_draft_select_workspace(int32_t rows, int32_t vocab, int32_t k) {
  if (select_sizes("ss_draft_select_workspace", rows, vocab, k) != SS_OK) return 0;
  return ss::draft_select_ws_bytes(rows, vocab, k);
}

ss_status ss_draft_select(const float* logits, const float* gumbel, int32_t rows, int32_t vocab,
                          float inv_temp, int32_t k, int32_t* tokens_out, void* workspace,
                          size_t ws_bytes, void* stream) {
  const char* fn = __func__;
  ss_status s0 = select_sizes(fn, rows, vocab, k);
  if (s0 != SS_OK) return s0;
  const size_t need = ss::draft_select_ws_bytes(rows, vocab, k);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(SS_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? ws_bytes : 0);
  if (need > 0) REQ_PTR(workspace, 16);
  if (!(inv_temp > 0.f) || std::isinf(inv_temp)) return fail(SS_ERR_INVALID_ARG, "%s: inv_temp must be finite and > 0", fn);
  REQ_PTR(logits, 4); OPT_PTR(gumbel, 4); REQ_PTR(tokens_out, 4);
  ss_status s = check_device(fn);
  if (s != SS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(fn, ss::launch_draft_select(logits, gumbel, rows, vocab, inv_temp, k, tokens_out, workspace, st), st);
}

}  // extern "C"
