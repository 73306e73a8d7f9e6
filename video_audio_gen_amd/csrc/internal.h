// Internal helpers shared by the host translation units of the library.
#pragma once

#include <stdarg.h>

#include <stdint.h>

namespace dit {
// Record a thread-local error message and return `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// int8 slices of an fp32 weight matrix [R, K] for the f32 GEMM (host_builders.cpp).
// Returns -1, or the first row holding a NaN or an Inf (the output is then
// incomplete and must not be used).
int64_t host_slice_rows(int64_t R, int64_t K, int64_t Kp, const float* X, int8_t* out);
// MXFP8 codes [R, K] and E8M0 scales [R, K/32] of a weight matrix (K a
// multiple of 32), the same arithmetic as the device quantizer; returns -1, or
// the first row holding a NaN or an Inf (output then incomplete).
int64_t host_quantize_mx8(int64_t R, int64_t K, const float* X, uint8_t* codes, uint8_t* scales);
// MXFP4 (E2M1 codes [R, K/2], two per byte, even K low; E8M0 scales [R, K/32]); the first non-finite row, or -1
int64_t host_quantize_mx4(int64_t R, int64_t K, const float* X, uint8_t* codes, uint8_t* scales);
}  // namespace dit
