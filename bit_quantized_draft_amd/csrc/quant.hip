// Substitute construction: int4 group-64 quantization and the fp16 dequantized export.
//
// The substitute layers are data-free 4-bit copies of the target's own layers
// (Summary page "Speculate Deep and Accurate ...", "Approach"; Review page "SubSpec:
// Using the Target Model's Own Low-Bit Shadow as Its Draft Model", §6.2). The pages
// give no quantizer; this is asymmetric min-max round-to-nearest with fp16 scale and
// zero per 64 consecutive inputs. Every float step is a single fp32 operation rounded
// to nearest-even (the library is built with -ffp-contract=off and correctly rounded
// division), so the codes match any IEEE implementation of the same steps bit for bit.
//
// One wavefront quantizes one group: lane l holds element l, min / max come from a
// wavefront reduction, and lanes pair up to write the packed bytes (even k in the
// low nibble).
#include "common.h"
#include "kernels.h"

namespace ss {

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, SS_WAVE));
  return v;
}

// fp16 round-to-nearest-even overflows to infinity from 65520 on. The overflow rules are
// applied to the fp32 value explicitly, so they do not depend on whether the hardware
// conversion saturates or produces infinity.
constexpr float kF16Overflow = 65520.0f;

// Returns false when the zero overflows fp16 (the caller widens the range).
__device__ __forceinline__ bool scale_zero(float lo, float hi, float& s, float& z) {
  const float range = hi - lo;
  const float scale = range / 15.0f;
  float sf = (scale >= kF16Overflow) ? 65504.0f : __half2float(__float2half_rn(scale));
  if (sf == 0.0f) sf = 1.0f;
  const float zf = (0.0f - lo) / sf;
  s = sf;
  if (fabsf(zf) >= kF16Overflow) return false;
  z = __half2float(__float2half_rn(zf));
  return true;
}

__global__ __launch_bounds__(256) void quantize_g64_kernel(const uint16_t* __restrict__ w, int64_t n,
                                                           int64_t k, uint8_t* __restrict__ q,
                                                           uint16_t* __restrict__ s_out,
                                                           uint16_t* __restrict__ z_out) {
  const int lane = threadIdx.x & 63;
  const int64_t G = k >> 6;
  const int64_t grp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp >= n * G) return;  // whole wave exits together
  const int64_t row = grp / G, g = grp - row * G;
  const float x = bf16_to_f32(w[row * k + g * 64 + lane]);
  const float lo = wave_min(x);
  const float hi = wave_max(x);
  float s, z;
  if (!scale_zero(lo, hi, s, z)) scale_zero(fminf(lo, 0.0f), fmaxf(hi, 0.0f), s, z);
  const float v = (x / s) + z;
  const float r = __builtin_rintf(v);
  const int code = (int)fminf(fmaxf(r, 0.0f), 15.0f);
  const int hi_code = __shfl_down(code, 1, SS_WAVE);
  if ((lane & 1) == 0) q[row * (k >> 1) + g * 32 + (lane >> 1)] = (uint8_t)(code | (hi_code << 4));
  if (lane == 0) {
    s_out[grp] = __half_as_ushort(__float2half_rn(s));
    // the zero is (0 - lo) / s; 0 - lo is +0 for lo = +-0, but the compiler may fold
    // 0 - lo into -lo (giving -0): canonicalize the sign of a zero on the bits
    const uint16_t zb = __half_as_ushort(__float2half_rn(z));
    z_out[grp] = (zb == 0x8000u) ? (uint16_t)0 : zb;
  }
}

// one thread per 8 codes (one 32-bit word of packed weights)
__global__ __launch_bounds__(256) void dequantize_g64_kernel(const uint32_t* __restrict__ q,
                                                             const uint16_t* __restrict__ s,
                                                             const uint16_t* __restrict__ z,
                                                             int64_t n, int64_t k,
                                                             u32x4_t* __restrict__ out) {
  const int64_t words = n * k / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = (i * 8) / k, col = (i * 8) - row * k;
    const int64_t gi = row * (k >> 6) + (col >> 6);
    const float sf = fp16_bits_to_f32(s[gi]);
    const float zf = fp16_bits_to_f32(z[gi]);
    const uint32_t word = q[i];
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = ((float)((word >> (4 * e)) & 0xF) - zf) * sf;
      // overflow to +-inf as round-to-nearest-even defines it (not hardware saturation)
      h[e] = (fabsf(d) >= kF16Overflow) ? (d > 0.f ? 0x7C00u : 0xFC00u)
                                        : (uint32_t)__half_as_ushort(__float2half_rn(d));
    }
    out[i] = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
}

// Relocation into the tiled layout, block (tile i, chunk c). One thread per 16-byte
// unit: unit l < 64 holds the codes of lane l (row 16 i + l % 16, code bytes
// 64 c + 16 (l / 16) .. +15 of that row); unit 64 + w holds the (scale, zero) words
// 4 w .. 4 w + 3, word 2 j + h being scale | zero << 16 of row 16 i + j, group 2 c + h.
__global__ __launch_bounds__(256) void w4_tile_kernel(const uint8_t* __restrict__ q, const uint16_t* __restrict__ s,
                                                      const uint16_t* __restrict__ z, int64_t n, int64_t k,
                                                      uint8_t* __restrict__ tiled) {
  constexpr int UNITS = TILE_BLOCK_BYTES / 16;   // 72
  const int64_t nchunks = k >> 7, G = k >> 6;
  const int64_t total = (n >> 4) * nchunks * UNITS;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t blk = idx / UNITS;
    const int u = (int)(idx - blk * UNITS);
    const int64_t tile = blk / nchunks, c = blk - tile * nchunks;
    u32x4_t v;
    if (u < 64) {
      const int64_t row = tile * 16 + (u & 15);
      v = *reinterpret_cast<const u32x4_t*>(q + row * (k >> 1) + c * 64 + (u >> 4) * 16);
    } else {
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int word = (u - 64) * 4 + e;   // 2 j + h
        const int64_t gi = (tile * 16 + (word >> 1)) * G + 2 * c + (word & 1);
        w4[e] = (uint32_t)s[gi] | ((uint32_t)z[gi] << 16);
      }
      v = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
    }
    *reinterpret_cast<u32x4_t*>(tiled + blk * TILE_BLOCK_BYTES + u * 16) = v;
  }
}

hipError_t launch_w4_tile(const uint8_t* q, const uint16_t* s, const uint16_t* z, int64_t n, int64_t k,
                          uint8_t* tiled, hipStream_t st) {
  const int64_t units = (n >> 4) * (k >> 7) * (TILE_BLOCK_BYTES / 16);
  const int64_t blocks = std::min<int64_t>((units + 255) / 256, 65536);
  hipLaunchKernelGGL(w4_tile_kernel, dim3((unsigned)blocks), dim3(256), 0, st, q, s, z, n, k, tiled);
  return hipGetLastError();
}

hipError_t launch_quantize_g64(const uint16_t* w, int64_t n, int64_t k, uint8_t* q, uint16_t* s,
                               uint16_t* z, hipStream_t st) {
  const int64_t groups = n * (k >> 6);
  const int64_t blocks = (groups + 3) / 4;
  hipLaunchKernelGGL(quantize_g64_kernel, dim3((unsigned)blocks), dim3(256), 0, st, w, n, k, q, s, z);
  return hipGetLastError();
}

hipError_t launch_dequantize_g64(const uint8_t* q, const uint16_t* s, const uint16_t* z, int64_t n,
                                 int64_t k, uint16_t* out, hipStream_t st) {
  const int64_t words = n * k / 8;
  const int64_t blocks = std::min<int64_t>((words + 255) / 256, 65536);
  hipLaunchKernelGGL(dequantize_g64_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(q), s, z, n, k, reinterpret_cast<u32x4_t*>(out));
  return hipGetLastError();
}

}  // namespace ss
