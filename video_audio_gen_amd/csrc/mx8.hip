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

namespace dit {

// Nearest-even E4M3 of a finite y, clamped to +-448 (0x7E), sign kept.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t sgn = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal steps of 2^-9 (8 steps give code 0x08 = 2^-6)
    mag = static_cast<uint32_t>(rintf(a * 512.0f));
  } else {
    const uint32_t ua = __float_as_uint(a);
    int e = static_cast<int>(ua >> 23) - 127;
    uint32_t keep = (ua >> 20) & 7u;
    const uint32_t rem = ua & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
    if (keep == 8u) {
      keep = 0;
      ++e;
    }
    mag = (static_cast<uint32_t>(e + 7) << 3) | keep;
  }
  return sgn | mag;
}

// The block's scale exponent s (byte s + 127), or 255 / 0 for a non-finite
// / all-zero block; `div` receives the exponent the values are divided by.
__device__ __forceinline__ uint32_t mx_scale(float amax, int* div) {
  if (!(amax <= 3.40282347e38f)) {  // NaN or Inf
    *div = 0;
    return 255u;
  }
  if (amax == 0.0f) {
    *div = 0;
    return 0u;
  }
  int ef;
  const float f = frexpf(amax, &ef);  // amax = f 2^ef, f in [0.5, 1): floor(log2 amax) = ef - 1
  int s = ef - 1 - 8 + (f > 0.875f ? 1 : 0);  // leading digits above 1.75 would not fit 448 2^(ef-9)
  s = s < -127 ? -127 : (s > 127 ? 127 : s);
  *div = s;
  return static_cast<uint32_t>(s + 127);
}

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
  for (int w = 0; w < 8; ++w) {
    uint32_t p = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = sbyte == 255u ? 0u : e4m3_rne(ldexpf(v[4 * w + i], -div));
      p |= c << (8 * i);
    }
    packed[w] = p;
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + t * 32);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  scales[t] = static_cast<uint8_t>(sbyte);
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
