// MXFP8 quantization arithmetic shared by the quantizer kernel and the
// producers that write their output straight in MXFP8 (the modulated norms,
// the attention output, the SiLU-gated MLP input): every 32 consecutive K
// values share one power-of-two scale 2^s (E8M0 byte s + 127), the smallest
// with max|v| <= 448 2^s, and each value v / 2^s is rounded to nearest-even
// OCP FP8 E4M3.  An all-zero block takes byte 0 (2^-127) and keeps each
// zero's sign; a block holding a NaN or an Inf takes the NaN scale (byte 255)
// and zero codes.
#pragma once
#include "common.h"

namespace dit {

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

// NaN-propagating max over each aligned group of 8 lanes, by DPP moves
// (quad swaps xor 1 and xor 2, then the half-row mirror i <-> 7 - i, which
// pairs the group's two quads): no LDS traffic.
__device__ __forceinline__ float mx_group8_max(float v) {
  v = nan_max(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = nan_max(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = nan_max(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  return v;
}

// Codes of four values of a block with scale byte `sbyte` and exponent
// `div`, packed little-endian: v / 2^div by v_ldexp (exact: |v / 2^div| <=
// 448 by the choice of the scale, and anything below E4M3's smallest step
// becomes a signed zero either way), then v_cvt_pk_fp8_f32, which on this GPU
// rounds to nearest even into OCP E4M3 -- checked on every finite bf16 value
// of magnitude <= 448 against a bitwise encoder, and against the reference
// quantizer on all bf16 bit patterns by the tests.
__device__ __forceinline__ uint32_t mx_code4(float v0, float v1, float v2, float v3, uint32_t sbyte, int div) {
  if (sbyte == 255u) return 0u;
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v0, -div), ldexpf(v1, -div), 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v2, -div), ldexpf(v3, -div), p, true);
  return static_cast<uint32_t>(p);
}

}  // namespace dit
