// int8 slices of fp32 rows for the fp32 GEMM (gemm.hip): a row x is scaled by
// 2^-e with max|x| < 2^e and cut into five truncating 7-bit digits,
// x 2^-e = sum_s a_s 2^-7(s+1) + r, |r| < 2^-35; every step is exact in fp32.
// A row holding a NaN or an Inf gets the exponent kSliceNonFinite and zero
// digits.
// Layout: five planes of [Kp/32][R][32] int8 (K-step-major: the 32 rows of one
// 32-wide K step are 1 KB of consecutive bytes), then R int32 exponents 256
// bytes further aligned.  Kp = K rounded up to 32; slices past K are zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

constexpr int kSlices = 5;
constexpr int kSliceK = 32;

__host__ __device__ inline int slice_kp(int K) { return (K + kSliceK - 1) / kSliceK * kSliceK; }
__host__ __device__ inline size_t slice_plane_bytes(int R, int K) { return static_cast<size_t>(R) * slice_kp(K); }
__host__ __device__ inline size_t slice_exp_offset(int R, int K) {
  return (kSlices * slice_plane_bytes(R, K) + 255) & ~size_t(255);
}

// Exponent stored for a row holding a NaN or an Inf: its digits are written
// as zero and every product with the row comes out NaN (the GEMM epilogue
// checks both operands' exponents), so a diverged activation stays visible.
constexpr int kSliceNonFinite = 0x40000000;

// Exponent e with |m| < 2^e for m = max|x| of a row (0 for an all-zero row,
// kSliceNonFinite when the max is NaN or Inf).
__device__ __forceinline__ int slice_exponent(float mx) {
  if (!(mx <= 3.40282347e38f)) return kSliceNonFinite;
  int e = 0;
  if (mx > 0.f) frexpf(mx, &e);
  return e;
}

// Writes the five slices of the four values x[0..3] at K positions k..k+3 of
// row `row` (k a multiple of 4).
__device__ __forceinline__ void slice_store4(const float* x, int e, int row, int k, int R, int Kp, int8_t* P) {
  float f[4];
  const bool finite = e != kSliceNonFinite;
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = finite ? ldexpf(x[j], -e) : 0.f;
  const size_t plane = static_cast<size_t>(R) * Kp;
  int8_t* dst = P + (static_cast<size_t>(k / kSliceK) * R + row) * kSliceK + (k % kSliceK);
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] *= 128.f;
      const float d = truncf(f[j]);
      f[j] -= d;
      w |= (static_cast<uint32_t>(static_cast<int>(d)) & 0xFFu) << (8 * j);
    }
    *reinterpret_cast<uint32_t*>(dst + sl * plane) = w;
  }
}

}  // namespace dit
