// Host-side launch helpers of the gfx950 DiT kernels.  Each returns the
// hipError_t of its launch; shapes are validated by the caller (dit_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dit {

enum Counter {
  kCntGemmBf16 = 0, kCntGemmF32, kCntAttnBf16, kCntAttnF32, kCntModnorm, kCntRopeSplit,
  kCntSiluGate, kCntGatedResidual, kCntAdaln, kCntPatchIn, kCntPatchOut, kCntEuler,
  kCntGemmF32Reduce, kCntConvert, kCntResidNormSlice, kCntSiluSlice, kCntCfgEuler, kCntResidModnorm,
  kCntGemmMx8, kCntQuantMx8, kCntGemmMx4, kCntQuantMx4, kCntNum
};
void count_launch(Counter c);

// Counts one launch of family `c` and, while profiling is on, records a HIP
// event pair around it on the launch stream.  Construct it immediately before
// the kernel launch; it records the end event when it goes out of scope.
class LaunchScope {
 public:
  LaunchScope(Counter c, hipStream_t s);
  ~LaunchScope();
 private:
  int slot_;
  hipStream_t s_;
};

// ---- GEMM: C[M,N] = A[M,K] . B[N,K]^T (+ bias)
size_t gemm_bf16_ws_bytes(int M, int N, int K);
// What the bf16 GEMM does with v = A.B^T + bias:
//   kEpiBf16 / kEpiF32: store C[M,N] as bf16 / fp32;
//   kEpiSiluGate: B's rows come in 64-row groups [32 gate | 32 up] of the same
//     32 features; C is m[M, N/2] bf16, m = silu(bf16(g)) * bf16(u) in fp32, rounded
//     to bf16 (N a multiple of 64).
enum GemmEpiMode { kEpiBf16 = 0, kEpiF32 = 1, kEpiSiluGate = 2 };
struct GemmEpilogue {
  int mode;
};
hipError_t gemm_bf16(int M, int N, int K, const uint16_t* A, const uint16_t* B, const float* bias,
                     void* C, const GemmEpilogue& ep, hipStream_t s);
// MXFP8: A [M,K] and B [N,K] as E4M3 bytes, each with E8M0 scales [rows][K/32]
// (quantize_mx8); K a multiple of 128; epilogues as gemm_bf16.
hipError_t gemm_mx8(int M, int N, int K, const uint8_t* A, const uint8_t* Asc, const uint8_t* B, const uint8_t* Bsc,
                    const float* bias, void* C, const GemmEpilogue& ep, hipStream_t s);
bool gemm_mx8_supported(int M, int N, int K);
// MXFP4 weights: A as for gemm_mx8; B [N, K/2] two OCP E2M1 codes per byte
// (the value at even K in the low nibble) with E8M0 scales [N][K/32]
// (quantize_mx4); K a multiple of 128; epilogues as gemm_bf16.
hipError_t gemm_mx4(int M, int N, int K, const uint8_t* A, const uint8_t* Asc, const uint8_t* B, const uint8_t* Bsc,
                    const float* bias, void* C, const GemmEpilogue& ep, hipStream_t s);
// bf16 rows [R, K] (K a multiple of 32) -> E2M1 codes [R, K/2] + E8M0 scales [R, K/32]
hipError_t quantize_mx4(int R, int K, const uint16_t* x, uint8_t* codes, uint8_t* scales, hipStream_t s);
// bf16 rows [R, K] (K a multiple of 32) -> E4M3 codes [R, K] + E8M0 scales [R, K/32]
hipError_t quantize_mx8(int R, int K, const uint16_t* x, uint8_t* codes, uint8_t* scales, hipStream_t s);
// f32: B is given as its int8 slices (slice_rows layout: 5 planes of
// [Kp/32][N][32] int8, Kp = K rounded up to 32, then N int32 exponents, each
// part 256-byte aligned); A is sliced into ws on the way.
size_t gemm_f32_slices_bytes(int R, int K);
hipError_t slice_rows(int R, int K, const float* X, void* slices, hipStream_t s);
size_t gemm_f32_ws_bytes(int M, int N, int K);
hipError_t gemm_f32(int M, int N, int K, const float* A, const void* B_slices, const float* bias,
                    float* C, void* ws, hipStream_t s);
// A also given as slices; the product goes to fp64 split-K partials
// part[slot][M][N] (no bias) that the consumer sums in split order: columns
// below col_split have s_lo partials, the others s_hi; gemm_f32_splits is the
// layout's slot count, max(s_lo, s_hi).  A group of one split is stored
// finished instead: float(value + bias[col]) at float index col of the
// doubles part[0][row][0 .. N) (row stride 2N floats), which the consumer
// reads as is.
struct F32Splits {
  int s_lo, s_hi, col_split;
};
int gemm_f32_splits(int N, int K);
F32Splits gemm_f32_split_groups(int N, int K);
size_t gemm_f32_part_bytes(int M, int N, int K);
hipError_t gemm_f32_sliced(int M, int N, int K, const void* A_slices, const void* B_slices, const float* bias,
                           double* part, hipStream_t s);
// Which K, N the GEMMs accept (checked by the ABI layer before launching).
bool gemm_bf16_supported(int M, int N, int K);
bool gemm_f32_supported(int M, int N, int K);

// ---- attention (q, k, v head-major [H, N, hd]; o [N, H*hd])
// o8 / o8s non-null: o is written in MXFP8 instead (codes [N][H*hd], scales
// [N][H*hd/32]; the bf16 values quantized as quantize_mx8 does) and `o` is unused.
hipError_t attention_bf16(int N, int H, int hd, int n_docs, const int32_t* cu, int max_seqlen,
                          const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                          hipStream_t s, uint8_t* o8 = nullptr, uint8_t* o8s = nullptr);
hipError_t attention_f32(int N, int H, int hd, int n_docs, const int32_t* cu, int max_seqlen,
                         const float* q, const float* k, const float* v, float* o, hipStream_t s);
bool attention_supported(bool bf16, int hd);

// ---- bandwidth-bound kernels
// x is float32, or float64 when x_f64 (the fp32 stream's residual; output then float32)
hipError_t modnorm(bool bf16_out, int norm, float eps, int N, int D, bool x_f64, const void* x,
                   const float* mod, int which, const int32_t* cond_idx, void* h, hipStream_t s);
bool modnorm_supported(int D);
hipError_t rope_split(bool bf16, int N, int H, int hd, int rot, const void* qkv, const float* cos,
                      const float* sin, void* q, void* k, void* v, hipStream_t s);
bool rope_split_supported(bool bf16, int hd, int rot);
hipError_t silu_gate(bool bf16, int N, int F, const void* u, void* m, hipStream_t s);
// bf16 stream: x = fma(gate[c], a, x) with gmod's gate (gate_which: 0 gate_msa,
// 1 gate_mlp), as gated_residual stores it, then h = modnorm(x) with nmod's
// shift/scale (norm_which), in one pass.
hipError_t resid_modnorm(int norm, float eps, int N, int D, float* x, const float* a, const float* gmod,
                         int gate_which, const float* nmod, int norm_which, const int32_t* cond_idx, uint16_t* h,
                         hipStream_t s);
// MXFP8 model: the two kernels above with h written as E4M3 codes [N][D] and
// E8M0 scales [N][D/32] (D a multiple of 32), bit-identical to quantize_mx8 of
// the bf16 h they would store.
hipError_t modnorm_mx8(int norm, float eps, int N, int D, const float* x, const float* mod, int which,
                       const int32_t* cond_idx, uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t resid_modnorm_mx8(int norm, float eps, int N, int D, float* x, const float* a, const float* gmod,
                             int gate_which, const float* nmod, int norm_which, const int32_t* cond_idx,
                             uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t gated_residual(int N, int D, bool x_f64, void* x, const float* a, const float* mod, int which,
                          const int32_t* cond_idx, hipStream_t s);
// ---- fused row kernels of the fp32 stream (fused_f32.hip); part: fp64 split-K
// partials [S][N][cols] of the preceding gemm_f32_sliced, bias (required with
// part) added after them; a one-split group's columns are read finished.
// resid_norm_slice: with part, x += gate(gmod, which) * a; then the norm of x,
// modulated from nmod (which) unless nmod is null, sliced into `slices` (rows
// N, K = D) or stored to y, or neither when both are null.
bool fused_f32_supported(int D, int F);
hipError_t resid_norm_slice(int N, int D, F32Splits sg, const double* part, const float* bias, const float* gmod, int gate_which,
                            const float* nmod, int norm_which, int norm, float eps, const int32_t* cond_idx, double* x,
                            void* slices, float* y, hipStream_t s);
hipError_t silu_slice(int N, int F, F32Splits sg, const double* part, const float* bias, void* slices, hipStream_t s);
// qk_norm: q and k RMS-normalised over each head (eps, no weight) before the rotation
hipError_t rope_part(int N, int H, int hd, int rot, F32Splits sg, const double* part, const float* bias, const float* cos,
                     const float* sin, float* q, float* k, float* v, int qk_norm, float eps, hipStream_t s);
hipError_t widen_f32(int64_t n, const float* src, double* dst, hipStream_t s);
hipError_t narrow_f64(int64_t n, const double* src, float* dst, hipStream_t s);
// mod[b][c][j] = W[b][modality(c)][j] . e[c] + bias[b][modality(c)][j]
struct AdalnBlockPtrs {
  const void* w[4];      // per modality [6D, d], stream dtype
  const float* bias[4];  // per modality [6D]
};
hipError_t adaln(bool w_bf16, int n_blocks, const AdalnBlockPtrs* blocks_host, int n_cond,
                 const int* cond_modality_host, int six_d, int cond_dim, const float* e,
                 float* mod, hipStream_t s);
// latent segment -> tokens [n, C*pt*ph*pw] (io: 1 patch3d, 2 channel-major)
hipError_t patch_in(int io, int C, const int* patch, const int* grid, const float* latent,
                    float* tokens, hipStream_t s);
hipError_t patch_out(int io, int C, const int* patch, const int* grid, const float* tokens,
                     float* latent, hipStream_t s);
hipError_t euler(int64_t n, float* x, const float* v, const float* dt, hipStream_t s);
// x += dt * (vu + w * (vc - vu)), each operation rounded to fp32
hipError_t cfg_euler(int64_t n, float* x, const float* vc, const float* vu, float w, const float* dt,
                     hipStream_t s);

}  // namespace dit
