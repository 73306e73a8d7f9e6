// Row kernels that join the fp32 stream's GEMMs.  An fp32 GEMM of the block
// leaves fp64 split-K partials; the kernel after it sums them in split order,
// adds the bias and rounds once to fp32 (the value a stand-alone reduction
// would store), applies its own operation and, where the next GEMM reads the
// result, cuts that GEMM's int8 slices directly (slices.h).  Columns the
// GEMM's split plan gives one split arrive already finished (the same
// rounding, done by the GEMM) as 4-byte floats.  A block then runs 11
// launches instead of 17, and the modulated norms and the SiLU product never
// make a round trip through HBM as fp32.
//
//   resid_norm_slice  x += gate * a (fp64 residual), then the AdaLN-modulated
//                     norm of the next sub-layer, sliced; or the plain final
//                     norm as fp32; or the residual update alone
//   rope_part         RoPE + QKV split of the QKV projection
//   silu_slice        SiLU gate of the MLP input projection, sliced
//
// Pages: "port the MiniMax-H3 omni-modal video+audio DiT", section "The
// device-resident forward (W2b)" (indexed AdaLN modulate, NeoX rotate_half
// from a per-row cos/sin cache, gated Add); "the 2.4B fp32 DiT onto the
// device", section "What moved" (LayerNorm, partial rotary, SiluAndMul).
#include "common.h"
#include "kernels.h"
#include "slices.h"

namespace dit {

// Columns col..col+3 of row `row` of a GEMM result [M, ncol] held as S fp64
// split-K partials [S][M][ncol]: summed in split order from zero, bias (never
// null here) added last, rounded once.  Up to eight splits are loaded before
// any is added, so their latencies overlap.
template <int NS>
__device__ __forceinline__ void add_parts4(const double* __restrict__ p, size_t MN, double* v) {
  double2 a[NS], b[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    a[u] = reinterpret_cast<const double2*>(p + u * MN)[0];
    b[u] = reinterpret_cast<const double2*>(p + u * MN)[1];
  }
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    v[0] += a[u].x; v[1] += a[u].y; v[2] += b[u].x; v[3] += b[u].y;
  }
}

// SF > 0: the split count is the compile-time SF (no branch, so a thread's
// loads for all its columns can be in flight together); SF = 0: S at run time.
template <int SF>
__device__ __forceinline__ void sum_parts4(const double* __restrict__ part, int S, size_t MN, size_t off,
                                           const float* __restrict__ bias, int col, float* out) {
  // the bias first, so its load is in flight with the partials'
  const float4 bb = *reinterpret_cast<const float4*>(bias + col);
  double v[4] = {0.0, 0.0, 0.0, 0.0};
  const double* p = part + off;
  if constexpr (SF > 0) {
#pragma unroll
    for (int s = 0; s + 8 <= SF; s += 8) add_parts4<8>(p + s * MN, MN, v);
    if constexpr (SF % 8 > 0) add_parts4<SF % 8>(p + (SF / 8 * 8) * MN, MN, v);
  } else {
    int s = 0;
    for (; s + 8 <= S; s += 8) add_parts4<8>(p + s * MN, MN, v);
    switch (S - s) {  // uniform
      case 1: add_parts4<1>(p + s * MN, MN, v); break;
      case 2: add_parts4<2>(p + s * MN, MN, v); break;
      case 3: add_parts4<3>(p + s * MN, MN, v); break;
      case 4: add_parts4<4>(p + s * MN, MN, v); break;
      case 5: add_parts4<5>(p + s * MN, MN, v); break;
      case 6: add_parts4<6>(p + s * MN, MN, v); break;
      case 7: add_parts4<7>(p + s * MN, MN, v); break;
      default: break;
    }
  }
  v[0] += static_cast<double>(bb.x); v[1] += static_cast<double>(bb.y);
  v[2] += static_cast<double>(bb.z); v[3] += static_cast<double>(bb.w);
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = static_cast<float>(v[e]);
}

// Columns col..col+3 of a one-split group: the GEMM stored them finished
// (bias added, rounded once) as floats at the start of the row's slot-0
// doubles.
__device__ __forceinline__ void own_parts4(const double* __restrict__ part, size_t off, int col, float* out) {
  const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(part + (off - col)) + col);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}

// Columns below cb carry s_lo partials, the others s_hi (the GEMM's split
// groups); SF is the compile-time form of s_lo.
template <int SF>
__device__ __forceinline__ void sum_parts4g(const double* __restrict__ part, int s_lo, int s_hi, int cb, size_t MN,
                                            size_t off, const float* __restrict__ bias, int col, float* out) {
  if (col < cb) {
    if (SF == 1 || (SF == 0 && s_lo == 1))
      own_parts4(part, off, col, out);
    else
      sum_parts4<SF>(part, s_lo, MN, off, bias, col, out);
  } else if (s_hi == 1) {
    own_parts4(part, off, col, out);
  } else {
    sum_parts4<0>(part, s_hi, MN, off, bias, col, out);
  }
}

// Workgroup barrier for LDS only: waits for this wave's LDS operations, not
// for its global stores (__syncthreads() would also wait for the residual
// row just stored).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Row reductions over the workgroup (blockDim.x a multiple of 64, <= 1024).
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum_f64(v);
  const int nw = blockDim.x >> 6;
  if (nw == 1) return v;
  lds_barrier();  // red may still be read by the previous reduction
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  double t = 0.0;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int nw = blockDim.x >> 6;
  if (nw == 1) return v;
  lds_barrier();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t = nan_max(t, red[i]);
  return t;
}

// Row max of the four-float chunks a thread holds, then the row's exponent
// and its slices; chunks between the row's width and the 32-padded width are
// written as zero slices.
template <int NCH>
__device__ __forceinline__ void slice_row(float (*y)[4], int C4, int row, int R, int K, float* redf, int8_t* sl) {
  const int t = threadIdx.x, NT = blockDim.x;
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
    if (t + NT * i < C4)
      mx = nan_max(mx, nan_max(nan_max(fabsf(y[i][0]), fabsf(y[i][1])), nan_max(fabsf(y[i][2]), fabsf(y[i][3]))));
  mx = block_max(mx, redf);
  const int e = slice_exponent(mx);
  const int Kp = slice_kp(K);
  if (t == 0) reinterpret_cast<int32_t*>(sl + slice_exp_offset(R, K))[row] = e;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = t + NT * i;
    if (c < C4) slice_store4(y[i], e, row, 4 * c, R, Kp, sl);
  }
  const float z[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c = C4 + t; c < Kp / 4; c += NT) slice_store4(z, e, row, 4 * c, R, Kp, sl);
}

// ============================================================================ residual + norm + slices
// One workgroup per token row.  With `part`: a = the GEMM result (partials +
// bias), x += gate[cond(row)] * a in fp64 (the product of two floats is exact,
// so the update rounds once).  Then, unless both sl and y are null, the row's
// norm in fp64 (LayerNorm when norm == 1, else RmsNorm), modulated by
// (1 + scale) and shift from nmod when nmod is non-null, rounded to fp32 and
// either sliced into sl (rows N, K = D) or stored to y.
template <int NCH, int SF>
__global__ __launch_bounds__(1024) void resid_norm_slice_kernel(
    int N, int D, int S, int S_hi, int cb, const double* __restrict__ part, const float* __restrict__ bias,
    const float* __restrict__ gmod, int gate_k, const float* __restrict__ nmod, int shift_k, int scale_k,
    int norm, float eps, const int32_t* __restrict__ cond_idx, double* __restrict__ x, int8_t* __restrict__ sl,
    float* __restrict__ y) {
  __shared__ double red[16];
  __shared__ float redf[16];
  const int row = blockIdx.x, t = threadIdx.x, NT = blockDim.x;
  const int D4 = D >> 2;
  const int cr = cond_idx != nullptr ? cond_idx[row] : 0;
  double* xr = x + static_cast<size_t>(row) * D;
  double v[NCH][4];
  double s = 0.0;
  // the modulation of the norm, loaded with the row so its latency overlaps
  const bool modulate = nmod != nullptr && (sl != nullptr || y != nullptr);
  const float4* sh = nullptr;
  const float4* sc = nullptr;
  if (modulate) {
    sh = reinterpret_cast<const float4*>(nmod + (static_cast<size_t>(cr) * 6 + shift_k) * D);
    sc = reinterpret_cast<const float4*>(nmod + (static_cast<size_t>(cr) * 6 + scale_k) * D);
  }
  float4 msc[NCH], msh[NCH];
  // Every load is issued without a branch (a thread past the row's end reads
  // its last chunk and drops it), so all of them are in flight at once.
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = t + NT * i;
    const int cc = c < D4 ? c : D4 - 1;
    if (modulate) {  // uniform
      msc[i] = sc[cc];
      msh[i] = sh[cc];
    }
    const double2 x0 = reinterpret_cast<const double2*>(xr + 4 * cc)[0];
    const double2 x1 = reinterpret_cast<const double2*>(xr + 4 * cc)[1];
    v[i][0] = x0.x; v[i][1] = x0.y; v[i][2] = x1.x; v[i][3] = x1.y;
    if (part != nullptr) {  // uniform
      const float4 g = reinterpret_cast<const float4*>(gmod + (static_cast<size_t>(cr) * 6 + gate_k) * D)[cc];
      float a[4];
      sum_parts4g<SF>(part, S, S_hi, cb, static_cast<size_t>(N) * D, static_cast<size_t>(row) * D + 4 * cc, bias, 4 * cc,
                      a);
      v[i][0] += static_cast<double>(g.x) * static_cast<double>(a[0]);
      v[i][1] += static_cast<double>(g.y) * static_cast<double>(a[1]);
      v[i][2] += static_cast<double>(g.z) * static_cast<double>(a[2]);
      v[i][3] += static_cast<double>(g.w) * static_cast<double>(a[3]);
    }
    if (c >= D4) v[i][0] = v[i][1] = v[i][2] = v[i][3] = 0.0;
    s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  }
  if (part != nullptr) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = t + NT * i;
      if (c < D4) {
        reinterpret_cast<double2*>(xr + 4 * c)[0] = make_double2(v[i][0], v[i][1]);
        reinterpret_cast<double2*>(xr + 4 * c)[1] = make_double2(v[i][2], v[i][3]);
      }
    }
  }
  if (sl == nullptr && y == nullptr) return;
  const double inv_d = 1.0 / static_cast<double>(D);
  const double mean = norm == 1 ? block_sum(s, red) * inv_d : 0.0;
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (t + NT * i < D4) {
      const double a = v[i][0] - mean, b = v[i][1] - mean, c = v[i][2] - mean, d = v[i][3] - mean;
      ss += (a * a + b * b) + (c * c + d * d);
    }
  }
  ss = block_sum(ss, red);
  const double rstd = 1.0 / sqrt(ss * inv_d + static_cast<double>(eps));
  float yv[NCH][4];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = t + NT * i;
    if (c < D4) {
      double z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = (v[i][e] - mean) * rstd;
      if (modulate) {
        const float4 a = msc[i], b = msh[i];
        z[0] = z[0] * (1.0 + static_cast<double>(a.x)) + static_cast<double>(b.x);
        z[1] = z[1] * (1.0 + static_cast<double>(a.y)) + static_cast<double>(b.y);
        z[2] = z[2] * (1.0 + static_cast<double>(a.z)) + static_cast<double>(b.z);
        z[3] = z[3] * (1.0 + static_cast<double>(a.w)) + static_cast<double>(b.w);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) yv[i][e] = static_cast<float>(z[e]);
    } else {
      yv[i][0] = yv[i][1] = yv[i][2] = yv[i][3] = 0.f;
    }
  }
  if (y != nullptr) {
    float* yr = y + static_cast<size_t>(row) * D;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = t + NT * i;
      if (c < D4) reinterpret_cast<float4*>(yr)[c] = make_float4(yv[i][0], yv[i][1], yv[i][2], yv[i][3]);
    }
    return;
  }
  slice_row<NCH>(yv, D4, row, N, D, redf, sl);
}

// ============================================================================ SiLU gate + slices
// One workgroup per token row of the [gate | up] projection (2F columns):
// m = silu(g) * u evaluated in fp64 and rounded once, then sliced (rows N,
// K = F).
template <int NCH, int SF>
__global__ __launch_bounds__(1024) void silu_slice_kernel(int N, int F, int S, int S_hi, int cb,
                                                        const double* __restrict__ part,
                                                       const float* __restrict__ bias, int8_t* __restrict__ sl) {
  __shared__ float redf[16];
  const int row = blockIdx.x, t = threadIdx.x, NT = blockDim.x;
  const int F4 = F >> 2;
  const size_t MN = static_cast<size_t>(N) * 2 * F;
  const size_t base = static_cast<size_t>(row) * 2 * F;
  float m[NCH][4];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = t + NT * i;
    const int cc = c < F4 ? c : F4 - 1;  // branch-free loads, as in resid_norm_slice
    float g[4], u[4];
    sum_parts4g<SF>(part, S, S_hi, cb, MN, base + 4 * cc, bias, 4 * cc, g);
    sum_parts4g<SF>(part, S, S_hi, cb, MN, base + F + 4 * cc, bias, F + 4 * cc, u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double gd = g[e];
      m[i][e] = c < F4 ? static_cast<float>(gd / (1.0 + exp(-gd)) * static_cast<double>(u[e])) : 0.f;
    }
  }
  slice_row<NCH>(m, F4, row, N, F, redf, sl);
}

// ============================================================================ RoPE + QKV split
// The QKV projection [N, 3D] (columns q | k | v, head h at h*hd) from its
// partials to head-major q, k, v [H, N, hd]; NeoX rotate_half on the first
// `rot` dims of q and k with cos/sin by token row, evaluated in fp64 (each
// output is one rounding of its exact value).  Thread (n, h, which, j), j
// fastest: for q and k, vector pair j of the rotated half (columns 4j and
// rot/2 + 4j) or two pass-through vectors; for v, columns 8j .. 8j+7.
template <int SF>
// qk_norm: q and k are first divided by the RMS of their head's hd values
// (sqrt(mean + eps), fp64; page "port the MiniMax-H3 omni-modal video+audio
// DiT", update "video-VAE decoder block ported": per-head RMS q/k norm without
// weight).  A head's hd/8 threads are consecutive lanes of one wavefront and
// reduce by butterfly shuffles; RoPE preserves the RMS, so norm-then-rotate
// equals rotate-then-norm.
__global__ __launch_bounds__(256) void rope_part_kernel(int N, int H, int hd, int rot, int S, int S_hi, int cb,
                                                       const double* __restrict__ part,
                                                       const float* __restrict__ bias,
                                                       const float* __restrict__ cosb,
                                                       const float* __restrict__ sinb, float* __restrict__ q,
                                                       float* __restrict__ k, float* __restrict__ v, int qk_norm,
                                                       float eps) {
  const int tph = hd / 8;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  // whole heads are in or out of range (the total is a multiple of tph), so
  // the shuffles below never read an exited lane of the thread's head
  if (t >= static_cast<int64_t>(N) * H * 3 * tph) return;
  const int j = static_cast<int>(t % tph);
  const int which = static_cast<int>((t / tph) % 3);
  const int h = static_cast<int>((t / (3 * tph)) % H);
  const int n = static_cast<int>(t / (static_cast<int64_t>(3 * tph) * H));
  const int D = H * hd;
  const int half = rot / 2;
  const size_t MN = static_cast<size_t>(N) * 3 * D;
  const int col0 = which * D + h * hd;
  const size_t src = static_cast<size_t>(n) * 3 * D + col0;
  float* d = (which == 0 ? q : which == 1 ? k : v) + (static_cast<size_t>(h) * N + n) * hd;
  const bool rotary = which < 2 && j < half / 4;
  // this thread's 8 values: dims i0..i0+3 and i1..i1+3 (a rotary pair), or
  // i0..i0+7 (v, or q/k dims past rot)
  const int i0 = rotary ? j * 4 : (which == 2 ? 8 * j : rot + 8 * (j - half / 4));
  const int i1 = rotary ? half + j * 4 : i0 + 4;
  // the rotation's cos/sin first, so their loads overlap the partials'
  float4 c = make_float4(0.f, 0.f, 0.f, 0.f), sn = c;
  if (rotary) {
    c = *reinterpret_cast<const float4*>(cosb + static_cast<size_t>(n) * half + i0);
    sn = *reinterpret_cast<const float4*>(sinb + static_cast<size_t>(n) * half + i0);
  }
  float x1[4], x2[4];
  sum_parts4g<SF>(part, S, S_hi, cb, MN, src + i0, bias, col0 + i0, x1);
  sum_parts4g<SF>(part, S, S_hi, cb, MN, src + i1, bias, col0 + i1, x2);
  double sc = 1.0;
  if (qk_norm) {  // uniform
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += double(x1[e]) * double(x1[e]) + double(x2[e]) * double(x2[e]);
    for (int o = 1; o < tph; o <<= 1) ss += xor_lane_rt(ss, o);
    if (which < 2) sc = 1.0 / sqrt(ss / hd + static_cast<double>(eps));
  }
  if (rotary) {
    const float cc[4] = {c.x, c.y, c.z, c.w}, ssn[4] = {sn.x, sn.y, sn.z, sn.w};
    float o1[4], o2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double a = double(x1[e]) * sc, b = double(x2[e]) * sc;
      o1[e] = static_cast<float>(a * double(cc[e]) - b * double(ssn[e]));
      o2[e] = static_cast<float>(b * double(cc[e]) + a * double(ssn[e]));
    }
    vec16<float>::store(d + i0, o1);
    vec16<float>::store(d + i1, o2);
  } else {
    // v, or the pass-through dims of q and k: copied (normalised for q, k)
    if (sc != 1.0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x1[e] = static_cast<float>(double(x1[e]) * sc);
        x2[e] = static_cast<float>(double(x2[e]) * sc);
      }
    }
    vec16<float>::store(d + i0, x1);
    vec16<float>::store(d + i1, x2);
  }
}

// ============================================================================ host side
// Row kernels: one workgroup per row, NCH four-float chunks per thread with
// NCH the least of 1, 2, 3, 4, 6, 8 that keeps the workgroup within 1024
// threads, and as many wavefronts as the row then needs: every load of a row
// is issued at once, by as many wavefronts as possible.
// One workgroup per row, NCH four-float chunks per thread with NCH the least
// of 1, 2, 3, 4, 6, 8 that keeps the workgroup within 1024 threads, and as
// many wavefronts as the row then needs.  Split counts 1, 2, 4, 6 and 8 are
// compile-time template arguments (every load of a thread in flight at once);
// other counts are read at run time.
static void row_shape(int c4, int* nch, int* nt) {
  *nch = c4 <= 1024 ? 1 : c4 <= 2048 ? 2 : c4 <= 3072 ? 3 : c4 <= 4096 ? 4 : c4 <= 6144 ? 6 : 8;
  *nt = ((c4 + *nch - 1) / *nch + 63) / 64 * 64;
}

#define DIT_SF_CASES(LAUNCH)                                   \
  switch (S) {                                                 \
    case 1: LAUNCH(1); break;                                  \
    case 2: LAUNCH(2); break;                                  \
    case 4: LAUNCH(4); break;                                  \
    case 6: LAUNCH(6); break;                                  \
    case 8: LAUNCH(8); break;                                  \
    default: LAUNCH(0); break;                                 \
  }

template <int NCH>
static void launch_rns(int nt, int N, int D, int S, int S_hi, int cb, const double* part, const float* bias, const float* gmod,
                       int gate_k, const float* nmod, int shift_k, int scale_k, int norm, float eps,
                       const int32_t* ci, double* x, int8_t* sl, float* y, hipStream_t s) {
#define DIT_L(SF_)                                                                                     \
  hipLaunchKernelGGL((resid_norm_slice_kernel<NCH, SF_>), dim3(N), dim3(nt), 0, s, N, D, S, S_hi, cb, part, bias, gmod, \
                     gate_k, nmod, shift_k, scale_k, norm, eps, ci, x, sl, y)
  DIT_SF_CASES(DIT_L)
#undef DIT_L
}

template <int NCH>
static void launch_silu(int nt, int N, int F, int S, int S_hi, int cb, const double* part, const float* bias,
                        int8_t* sl, hipStream_t s) {
#define DIT_L(SF_) \
  hipLaunchKernelGGL((silu_slice_kernel<NCH, SF_>), dim3(N), dim3(nt), 0, s, N, F, S, S_hi, cb, part, bias, sl)
  DIT_SF_CASES(DIT_L)
#undef DIT_L
}

bool fused_f32_supported(int D, int F) {
  return D > 0 && F > 0 && D % 4 == 0 && F % 4 == 0 && D <= 8192 && F <= 24576;
}

hipError_t resid_norm_slice(int N, int D, F32Splits sg, const double* part, const float* bias, const float* gmod, int gate_which,
                            const float* nmod, int norm_which, int norm, float eps, const int32_t* cond_idx, double* x,
                            void* slices, float* y, hipStream_t s) {
  if (N == 0) return hipSuccess;
  // D <= 8192: at most two chunks per thread (the fp64 row stays in registers)
  if (D % 4 || D > 8192 || (slices != nullptr && y != nullptr) || (part != nullptr && bias == nullptr))
    return hipErrorInvalidValue;
  LaunchScope scope_(kCntResidNormSlice, s);
  const int gate_k = gate_which == 0 ? 2 : 5;
  const int shift_k = norm_which == 0 ? 0 : 3, scale_k = norm_which == 0 ? 1 : 4;
  int nch, nt;
  row_shape(D / 4, &nch, &nt);
  int8_t* sl = static_cast<int8_t*>(slices);
  const int S = sg.s_lo;
#define DIT_R(NCH_)                                                                                          \
  launch_rns<NCH_>(nt, N, D, S, sg.s_hi, sg.col_split, part, bias, gmod, gate_k, nmod, shift_k, scale_k, norm, eps, cond_idx, x, sl, y, s)
  if (nch == 1)
    DIT_R(1);
  else
    DIT_R(2);
#undef DIT_R
  return hipGetLastError();
}

hipError_t silu_slice(int N, int F, F32Splits sg, const double* part, const float* bias, void* slices, hipStream_t s) {
  if (N == 0) return hipSuccess;
  // F <= 24576: at most six chunks per thread
  if (F % 4 || F > 24576 || bias == nullptr) return hipErrorInvalidValue;
  LaunchScope scope_(kCntSiluSlice, s);
  int nch, nt;
  row_shape(F / 4, &nch, &nt);
  int8_t* sl = static_cast<int8_t*>(slices);
  switch (nch) {
    case 1: launch_silu<1>(nt, N, F, sg.s_lo, sg.s_hi, sg.col_split, part, bias, sl, s); break;
    case 2: launch_silu<2>(nt, N, F, sg.s_lo, sg.s_hi, sg.col_split, part, bias, sl, s); break;
    case 3: launch_silu<3>(nt, N, F, sg.s_lo, sg.s_hi, sg.col_split, part, bias, sl, s); break;
    case 4: launch_silu<4>(nt, N, F, sg.s_lo, sg.s_hi, sg.col_split, part, bias, sl, s); break;
    default: launch_silu<6>(nt, N, F, sg.s_lo, sg.s_hi, sg.col_split, part, bias, sl, s); break;
  }
  return hipGetLastError();
}

hipError_t rope_part(int N, int H, int hd, int rot, F32Splits sg, const double* part, const float* bias, const float* cos,
                     const float* sin, float* q, float* k, float* v, int qk_norm, float eps, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (!rope_split_supported(false, hd, rot) || bias == nullptr) return hipErrorInvalidValue;
  if (qk_norm && (hd / 8) & (hd / 8 - 1)) return hipErrorInvalidValue;  // a head's lanes: a power of two
  LaunchScope scope_(kCntRopeSplit, s);
  const int64_t total = static_cast<int64_t>(N) * H * 3 * (hd / 8);
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
#define DIT_L(SF_) \
  hipLaunchKernelGGL((rope_part_kernel<SF_>), grid, dim3(256), 0, s, N, H, hd, rot, S, sg.s_hi, sg.col_split, part, \
                     bias, cos, sin, q, k, v, qk_norm, eps)
  const int S = sg.s_lo;
  DIT_SF_CASES(DIT_L)
#undef DIT_L
  return hipGetLastError();
}
#undef DIT_SF_CASES

}  // namespace dit
