// MXFP8 re-quantization of bf16 rows for the scaled fp8 GEMM (gemm.hip,
// gemm_mx8_kernel): every 32 consecutive K values of a row share one
// power-of-two scale 2^s (E8M0 byte s + 127), the smallest with
// max|v| <= 448 2^s, and each value v / 2^s is rounded to nearest-even OCP
// FP8 E4M3.  An all-zero block takes byte 0 (2^-127) and keeps each zero's
// sign; a block holding a NaN or an Inf takes the NaN scale (byte 255) and
// zero codes, so every product with it is NaN.  The pages' low-precision arm
// is NVFP4 with an E4M3 scale per 16 (page "port the MiniMax-H3 omni-modal
// video+audio DiT", update "NVFP4 arm grounded"); the matrix cores here take
// MX block scales natively instead.
#include "common.h"
#include "kernels.h"
#include "mx8.h"

namespace dit {

// One thread per 32-value block: four 16-byte loads of bf16, two 16-byte code
// stores, one scale byte.
__global__ __launch_bounds__(256) void quantize_mx8_kernel(int64_t n_blocks, int kb, const bf16_t* __restrict__ x,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n_blocks) return;
  (void)kb;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = src[q];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = __uint_as_float(ww[i] << 16);
      v[8 * q + 2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = nan_max(amax, fabsf(v[i]));
  int div;
  const uint32_t sbyte = mx_scale(amax, &div);
  uint32_t packed[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) packed[w] = mx_code4(v[4 * w], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3], sbyte, div);
  uint4* dst = reinterpret_cast<uint4*>(codes + t * 32);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  scales[t] = static_cast<uint8_t>(sbyte);
}

// MXFP4 (the weight format of the MXFP4 GEMMs): every 32 consecutive K values
// share one power-of-two scale 2^s, the smallest with max|v| <= 6 2^s, and each
// value v / 2^s goes to the nearest OCP FP4 E2M1 value (magnitudes 0, 0.5, 1,
// 1.5, 2, 3, 4, 6), ties to the even mantissa bit; two codes per byte, the one
// at even K in the low nibble.  Zero and non-finite blocks as for MXFP8.
__device__ __forceinline__ uint32_t mx4_scale(float amax, int* div) {
  if (!(amax <= 3.40282347e38f)) {
    *div = 0;
    return 255u;
  }
  if (amax == 0.0f) {
    *div = 0;
    return 0u;
  }
  int ef;
  const float f = frexpf(amax, &ef);  // amax = f 2^ef, f in [0.5, 1)
  int s = ef - 1 - 2 + (f > 0.75f ? 1 : 0);  // leading digits above 1.5 would not fit 6 2^(ef-3)
  s = s < -127 ? -127 : (s > 127 ? 127 : s);
  *div = s;
  return static_cast<uint32_t>(s + 127);
}

// E2M1 code of y (|y| <= 6 by the scale; larger clamps to 6): the magnitude
// code counts the rounding thresholds at or below |y| -- the midpoints
// between neighbouring values, each tie going to the neighbour whose mantissa
// bit is 0 (0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4,
// 5 -> 4) -- and the sign bit is y's, -0 included.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return (__float_as_uint(y) >> 31) << 3 | m;
}

// One thread per 32-value block: four 16-byte loads of bf16, one 16-byte code
// store, one scale byte.
__global__ __launch_bounds__(256) void quantize_mx4_kernel(int64_t n_blocks, const bf16_t* __restrict__ x,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n_blocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = src[q];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = __uint_as_float(ww[i] << 16);
      v[8 * q + 2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = nan_max(amax, fabsf(v[i]));
  int div;
  const uint32_t sbyte = mx4_scale(amax, &div);
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
  if (sbyte != 255u) {
#pragma unroll
    for (int i = 0; i < 32; ++i) packed[i / 8] |= e2m1_code(ldexpf(v[i], -div)) << (4 * (i % 8));
  }
  *reinterpret_cast<uint4*>(codes + t * 16) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  scales[t] = static_cast<uint8_t>(sbyte);
}

hipError_t quantize_mx4(int R, int K, const uint16_t* x, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t n_blocks = static_cast<int64_t>(R) * (K / 32);
  if (n_blocks == 0) return hipSuccess;
  LaunchScope scope_(kCntQuantMx4, s);
  hipLaunchKernelGGL(quantize_mx4_kernel, dim3(static_cast<unsigned>((n_blocks + 255) / 256)), dim3(256), 0, s,
                     n_blocks, x, codes, scales);
  return hipGetLastError();
}

hipError_t quantize_mx8(int R, int K, const uint16_t* x, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t n_blocks = static_cast<int64_t>(R) * (K / 32);
  if (n_blocks == 0) return hipSuccess;
  LaunchScope scope_(kCntQuantMx8, s);
  hipLaunchKernelGGL(quantize_mx8_kernel, dim3(static_cast<unsigned>((n_blocks + 255) / 256)), dim3(256), 0, s,
                     n_blocks, K / 32, x, codes, scales);
  return hipGetLastError();
}

}  // namespace dit
