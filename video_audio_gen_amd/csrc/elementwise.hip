// Bandwidth-bound kernels of the DiT block: AdaLN modulate+norm, RoPE-from-cache
// with the QKV split, SiLU gate, gated residual, the AdaLN table, patch in/out
// and the Euler update.  Every kernel reads and writes each byte once with
// 16-byte (or 8-byte for bf16 quads) coalesced accesses.  Row reductions run
// as wavefront butterfly shuffles; where a row spans several wavefronts (the
// norms at width 6144: 64-512 threads per row) the partial sums meet in LDS
// behind a workgroup barrier.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mx8.h"

namespace dit {

// ============================================================================ modulate + norm
// Page "port the MiniMax-H3 omni-modal video+audio DiT", section "The
// device-resident forward (W2b)": RmsNorm reduces in f32, then an indexed AdaLN
// modulate; page "the 2.4B fp32 DiT onto the device", section "What moved":
// LayerNorm for the music model.

template <typename TO> struct store4;
template <> struct store4<float> {
  static __device__ __forceinline__ void st(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};
template <> struct store4<bf16_t> {
  static __device__ __forceinline__ void st(bf16_t* p, float4 v) {
    uint2 t;
    t.x = pack_bf16x2(v.x, v.y);
    t.y = pack_bf16x2(v.z, v.w);
    *reinterpret_cast<uint2*>(p) = t;
  }
};

// fp32 output (an fp32 stream or the final norm): the row sums run in fp64,
// so the normalised row is the fp32 rounding of its exact value in practice.
// bf16 output: fp32 sums (the bf16 rounding dominates).  The residual x is
// float32 (bf16 stream) or float64 (fp32 stream).
template <typename TO> struct norm_acc { typedef float T; };
template <> struct norm_acc<float> { typedef double T; };

// TPR threads (TPR/64 wavefronts) per row, 256/TPR rows per block; thread t of
// a row holds float4 chunks t, t+TPR, ... (at most NCH) in registers, so x is
// read once.  Sums: butterfly inside the wavefront, then across the row's
// wavefronts through LDS.
template <typename A, int WPR>
__device__ __forceinline__ A row_sum(A v, A* red, int wrow, int wsub, int lane) {
  v += xor_lane<32>(v); v += xor_lane<16>(v); v += xor_lane<8>(v);
  v += xor_lane<4>(v); v += xor_lane<2>(v); v += xor_lane<1>(v);
  if (WPR == 1) return v;
  __syncthreads();
  if (lane == 0) red[wrow * WPR + wsub] = v;
  __syncthreads();
  A t = 0;
#pragma unroll
  for (int i = 0; i < WPR; ++i) t += red[wrow * WPR + i];
  return t;
}

// Four consecutive residual values as the accumulation type.
template <typename TX> struct load4;
template <> struct load4<float> {
  template <typename A>
  static __device__ __forceinline__ void ld(const float* p, A* v) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = A(t.x); v[1] = A(t.y); v[2] = A(t.z); v[3] = A(t.w);
  }
};
template <> struct load4<double> {
  template <typename A>
  static __device__ __forceinline__ void ld(const double* p, A* v) {
    const double2 t0 = reinterpret_cast<const double2*>(p)[0], t1 = reinterpret_cast<const double2*>(p)[1];
    v[0] = A(t0.x); v[1] = A(t0.y); v[2] = A(t1.x); v[3] = A(t1.y);
  }
};

// TPR threads per row (TPR/64 wavefronts; 256/TPR rows per workgroup below
// 256 threads, one above).  ROWS consecutive rows per workgroup, one after
// the other: the row PF ahead is in flight while the current row reduces, and
// the shift/scale rows stay in registers while consecutive rows share their
// modulation row (a packed segment is contiguous), so they come from L2 once
// per workgroup instead of once per row.  Every row's arithmetic is the same
// as with ROWS = 1.
//
// RES (bf16 stream): the gated residual of the sub-layer before runs first,
// x = fma(gate[c], a, x) per element -- the value the separate gated-residual
// kernel stores -- x is written back and the row normalised from it.
template <typename TX, typename TO, int TPR, int NCH, int ROWS, int PF = 1, bool RES = false>
__global__ __launch_bounds__(TPR > 256 ? TPR : 256) void modnorm_kernel(int N, int D, int norm, float eps,
                                                     const TX* __restrict__ x,
                                                     const float* __restrict__ mod, int shift_k,
                                                     int scale_k, const int32_t* __restrict__ cond_idx,
                                                     TO* __restrict__ h, float* xw, const float* __restrict__ a,
                                                     const float* __restrict__ gmod, int gate_k,
                                                     uint8_t* __restrict__ hs) {
  typedef typename norm_acc<TO>::T A;
  constexpr int WPR = TPR / 64, RPB = (TPR > 256 ? TPR : 256) / TPR;
  __shared__ A red[2][RPB * WPR];
  const int lane = threadIdx.x & 63;
  const int wrow = threadIdx.x / TPR;             // row within the block
  const int wsub = (threadIdx.x % TPR) >> 6;      // wavefront within the row
  const int t = threadIdx.x % TPR;
  const int D4 = D >> 2;
  const A inv_d = A(1) / A(D);
  A v[PF + 1][NCH][4];
  float4 shv[NCH], scv[NCH];
  int cur_cond = -1;
  auto row_of = [&](int it) { return (blockIdx.x * ROWS + it) * RPB + wrow; };
  // A dead row (past N) reads row N-1 so every barrier stays reachable, and
  // stores nothing.
  auto load_row = [&](int r_raw, A (*dst)[4]) {
    const bool row_live = r_raw < N;
    const int r = row_live ? r_raw : N - 1;
    if constexpr (RES) {
      float* xr = xw + static_cast<size_t>(r) * D;
      const float* ar = a + static_cast<size_t>(r) * D;
      const float* gr = gmod + (static_cast<size_t>(cond_idx[r]) * 6 + gate_k) * D;
      float4 xv[NCH], av[NCH], gv[NCH];
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = t + TPR * i;
        if (c < D4) {
          xv[i] = reinterpret_cast<const float4*>(xr)[c];
          av[i] = reinterpret_cast<const float4*>(ar)[c];
          gv[i] = reinterpret_cast<const float4*>(gr)[c];
        }
      }
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = t + TPR * i;
        if (c < D4) {
          const float4 y = make_float4(__builtin_fmaf(gv[i].x, av[i].x, xv[i].x), __builtin_fmaf(gv[i].y, av[i].y, xv[i].y),
                                       __builtin_fmaf(gv[i].z, av[i].z, xv[i].z), __builtin_fmaf(gv[i].w, av[i].w, xv[i].w));
          if (row_live) reinterpret_cast<float4*>(xr)[c] = y;
          dst[i][0] = A(y.x); dst[i][1] = A(y.y); dst[i][2] = A(y.z); dst[i][3] = A(y.w);
        } else {
          dst[i][0] = dst[i][1] = dst[i][2] = dst[i][3] = A(0);
        }
      }
    } else {
      const TX* xr = x + static_cast<size_t>(r) * D;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = t + TPR * i;
        if (c < D4) {
          load4<TX>::ld(xr + 4 * c, dst[i]);
        } else {
          dst[i][0] = dst[i][1] = dst[i][2] = dst[i][3] = A(0);
        }
      }
    }
  };
#pragma unroll
  for (int p = 0; p < PF && p < ROWS; ++p) load_row(row_of(p), v[p]);
#pragma unroll
  for (int it = 0; it < ROWS; ++it) {
    const int row_raw = (blockIdx.x * ROWS + it) * RPB + wrow;
    if ((blockIdx.x * ROWS + it) * RPB >= N) break;  // uniform: no live row left in the block
    const bool live = row_raw < N;
    const int row = live ? row_raw : N - 1;
    A (*vc)[4] = v[it % (PF + 1)];
    if (it + PF < ROWS) load_row(row_of(it + PF), v[(it + PF) % (PF + 1)]);
    if (mod != nullptr) {
      const int cr = cond_idx[row];
      if (cr != cur_cond) {
        cur_cond = cr;
        const float4* sh = reinterpret_cast<const float4*>(mod + (static_cast<size_t>(cr) * 6 + shift_k) * D);
        const float4* sc = reinterpret_cast<const float4*>(mod + (static_cast<size_t>(cr) * 6 + scale_k) * D);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int c = t + TPR * i;
          if (c < D4) {
            shv[i] = sh[c];
            scv[i] = sc[c];
          }
        }
      }
    }
    A s = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (t + TPR * i < D4) s += (vc[i][0] + vc[i][1]) + (vc[i][2] + vc[i][3]);
    A mean = 0;
    if (norm == 1) mean = row_sum<A, WPR>(s, red[0], wrow, wsub, lane) * inv_d;
    A ss = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = t + TPR * i;
      if (c < D4) {
        const A a = vc[i][0] - mean, b = vc[i][1] - mean, cc = vc[i][2] - mean, d = vc[i][3] - mean;
        ss += (a * a + b * b) + (cc * cc + d * d);
      }
    }
    ss = row_sum<A, WPR>(ss, red[1], wrow, wsub, lane);
    if (live) {
      const A rstd = A(1) / sqrt(ss * inv_d + A(eps));
      TO* hr = h + static_cast<size_t>(row) * D;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = t + TPR * i;
        if (c < D4) {
          A y0 = (vc[i][0] - mean) * rstd, y1 = (vc[i][1] - mean) * rstd;
          A y2 = (vc[i][2] - mean) * rstd, y3 = (vc[i][3] - mean) * rstd;
          if (mod != nullptr) {
            const float4 a = scv[i], b = shv[i];
            y0 = y0 * (A(1) + A(a.x)) + A(b.x);
            y1 = y1 * (A(1) + A(a.y)) + A(b.y);
            y2 = y2 * (A(1) + A(a.z)) + A(b.z);
            y3 = y3 * (A(1) + A(a.w)) + A(b.w);
          }
          if constexpr (std::is_same<TO, uint8_t>::value) {
            // MXFP8 output (codes [N][D], scales [N][D/32]): the bf16 value of
            // each output, as a stored bf16 h, quantized per 32 consecutive
            // columns, which are this thread's 4 and those of the 7 threads
            // beside it (chunks 8q .. 8q+7 of the row; D is a multiple of 32).
            const float f[4] = {bf16_to_f32(f32_to_bf16(float(y0))), bf16_to_f32(f32_to_bf16(float(y1))),
                                bf16_to_f32(f32_to_bf16(float(y2))), bf16_to_f32(f32_to_bf16(float(y3)))};
            float am = nan_max(nan_max(fabsf(f[0]), fabsf(f[1])), nan_max(fabsf(f[2]), fabsf(f[3])));
            am = mx_group8_max(am);
            int div;
            const uint32_t sb = mx_scale(am, &div);
            *reinterpret_cast<uint32_t*>(hr + 4 * c) = mx_code4(f[0], f[1], f[2], f[3], sb, div);
            if ((c & 7) == 0) hs[static_cast<size_t>(row) * (D / 32) + (c >> 3)] = static_cast<uint8_t>(sb);
          } else {
            store4<TO>::st(hr + 4 * c, make_float4(float(y0), float(y1), float(y2), float(y3)));
          }
        }
      }
    }
  }
}

bool modnorm_supported(int D) { return D > 0 && D % 4 == 0 && D <= 8192; }

template <typename TX, typename TO, bool RES = false>
static hipError_t modnorm_t(int norm, float eps, int N, int D, const TX* x, const float* mod,
                            int which, const int32_t* ci, TO* h, hipStream_t s, float* xw = nullptr,
                            const float* a = nullptr, const float* gmod = nullptr, int gate_k = 0,
                            uint8_t* hs = nullptr) {
  if (std::is_same<TO, uint8_t>::value && D % 32 != 0) return hipErrorInvalidValue;
  const int d4 = D / 4;
  const int shift_k = which == 0 ? 0 : 3, scale_k = which == 0 ? 1 : 4;
  // two rows per workgroup once there are enough rows to fill the chip
  constexpr int R = sizeof(TX) == 4 ? 2 : 1;
#define DIT_MN(TPR, K)                                                                                \
  if ((d4 + TPR - 1) / TPR <= K) {                                                                   \
    constexpr int NTH = TPR > 256 ? TPR : 256, RPB = NTH / TPR;                                       \
    if (N >= 4096 * RPB) {                                                                            \
      const int nb = (N + RPB * R - 1) / (RPB * R);                                                   \
      hipLaunchKernelGGL((modnorm_kernel<TX, TO, TPR, K, R, 1, RES>), dim3(nb), dim3(NTH), 0, s, N, D, norm, \
                         eps, x, mod, shift_k, scale_k, ci, h, xw, a, gmod, gate_k, hs);                        \
    } else {                                                                                          \
      hipLaunchKernelGGL((modnorm_kernel<TX, TO, TPR, K, 1, 1, RES>), dim3((N + RPB - 1) / RPB), dim3(NTH), 0, \
                         s, N, D, norm, eps, x, mod, shift_k, scale_k, ci, h, xw, a, gmod, gate_k, hs);         \
    }                                                                                                 \
    return hipGetLastError();                                                                         \
  }
  if (d4 <= 256) {
    DIT_MN(64, 1) DIT_MN(64, 2) DIT_MN(64, 4)
  } else if (d4 <= 1024) {
    DIT_MN(128, 4) DIT_MN(128, 8)
  } else {
    // wide rows: 512 threads per row up to 6144 (fewer registers per thread,
    // more waves in flight: 6144-wide rows 65 -> 69 % of HBM against 256).
    // The thread count depends on D only, so a row's sums run in the same
    // order whatever N is (a document alone equals it packed, bit for bit).
    DIT_MN(512, 3) DIT_MN(256, 8)
  }
#undef DIT_MN
  return hipErrorInvalidValue;
}

hipError_t modnorm(bool bf16_out, int norm, float eps, int N, int D, bool x_f64, const void* x,
                   const float* mod, int which, const int32_t* cond_idx, void* h, hipStream_t s) {
  if (N == 0) return hipSuccess;
  LaunchScope scope_(kCntModnorm, s);
  if (x_f64) {
    if (bf16_out) return hipErrorInvalidValue;  // an fp64 residual belongs to the fp32 stream
    return modnorm_t<double, float>(norm, eps, N, D, static_cast<const double*>(x), mod, which, cond_idx,
                                    static_cast<float*>(h), s);
  }
  if (bf16_out)
    return modnorm_t<float, bf16_t>(norm, eps, N, D, static_cast<const float*>(x), mod, which, cond_idx,
                                    static_cast<bf16_t*>(h), s);
  return modnorm_t<float, float>(norm, eps, N, D, static_cast<const float*>(x), mod, which, cond_idx,
                                 static_cast<float*>(h), s);
}

// Gated residual of the sub-layer before (gmod's gate_which row: 0 gate_msa,
// 1 gate_mlp) then modulate + norm of the next one (nmod's norm_which rows),
// one pass over x.
hipError_t resid_modnorm(int norm, float eps, int N, int D, float* x, const float* a, const float* gmod,
                         int gate_which, const float* nmod, int norm_which, const int32_t* cond_idx, bf16_t* h,
                         hipStream_t s) {
  if (N == 0) return hipSuccess;
  LaunchScope scope_(kCntResidModnorm, s);
  // x is read and written through xw only (the read-only pointer stays null)
  return modnorm_t<float, bf16_t, true>(norm, eps, N, D, static_cast<const float*>(nullptr), nmod, norm_which,
                                        cond_idx, h, s, x, a, gmod, gate_which == 0 ? 2 : 5);
}

// The same two kernels with h written in MXFP8 (codes [N][D], scales
// [N][D/32]): the bf16 values a stored h would hold, quantized as
// quantize_mx8 does, so the MXFP8 GEMM after them reads what it would read
// from a separate quantization of h.
hipError_t modnorm_mx8(int norm, float eps, int N, int D, const float* x, const float* mod, int which,
                       const int32_t* cond_idx, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (N == 0) return hipSuccess;
  LaunchScope scope_(kCntModnorm, s);
  return modnorm_t<float, uint8_t>(norm, eps, N, D, x, mod, which, cond_idx, codes, s, nullptr, nullptr, nullptr, 0,
                                   scales);
}
hipError_t resid_modnorm_mx8(int norm, float eps, int N, int D, float* x, const float* a, const float* gmod,
                             int gate_which, const float* nmod, int norm_which, const int32_t* cond_idx,
                             uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (N == 0) return hipSuccess;
  LaunchScope scope_(kCntResidModnorm, s);
  return modnorm_t<float, uint8_t, true>(norm, eps, N, D, static_cast<const float*>(nullptr), nmod, norm_which,
                                         cond_idx, codes, s, x, a, gmod, gate_which == 0 ? 2 : 5, scales);
}

// ============================================================================ RoPE + QKV split
// qkv [N, 3D] token-major with columns [q_all | k_all | v_all] -> q, k, v
// head-major [H, N, hd].  NeoX rotate_half on the first `rot` dims of each head,
// cos/sin looked up by token row (page "port the MiniMax-H3 omni-modal
// video+audio DiT", section "The device-resident forward (W2b)": plain NeoX
// rotate_half fed by a per-row cos/sin cache; page "the 2.4B fp32 DiT onto the
// device", section "What moved": partial rotary).  Thread (n, h, j) handles the
// 16-byte vectors j and rot/2/V + j of the rotated half (or two pass-through
// vectors), and two vectors of v.  Consecutive threads walk j then h, so a
// wavefront reads and writes contiguous runs.
template <typename T>
__global__ __launch_bounds__(256) void rope_split_kernel(int N, int H, int hd, int rot,
                                                        const T* __restrict__ qkv,
                                                        const float* __restrict__ cosb,
                                                        const float* __restrict__ sinb,
                                                        T* __restrict__ q, T* __restrict__ k,
                                                        T* __restrict__ v) {
  constexpr int V = vec16<T>::N;
  const int tph = hd / (2 * V);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= static_cast<int64_t>(N) * H * tph) return;
  const int j = static_cast<int>(t % tph);
  const int h = static_cast<int>((t / tph) % H);
  const int n = static_cast<int>(t / (static_cast<int64_t>(tph) * H));
  const int D = H * hd;
  const int half = rot / 2;
  const T* src = qkv + static_cast<size_t>(n) * 3 * D + static_cast<size_t>(h) * hd;
  const size_t dst_off = (static_cast<size_t>(h) * N + n) * hd;
  if (j < half / V) {
    const int i0 = j * V, i1 = half + j * V;
    float c[V], sn[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      c[e] = cosb[static_cast<size_t>(n) * half + i0 + e];
      sn[e] = sinb[static_cast<size_t>(n) * half + i0 + e];
    }
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const T* s = src + which * D;
      T* d = (which == 0 ? q : k) + dst_off;
      float x1[V], x2[V], o1[V], o2[V];
      vec16<T>::load(s + i0, x1);
      vec16<T>::load(s + i1, x2);
      // products of floats are exact in fp64: each output is one rounding of
      // its exact value (fp32 stream); the bf16 rounding dominates otherwise
#pragma unroll
      for (int e = 0; e < V; ++e) {
        o1[e] = static_cast<float>(double(x1[e]) * double(c[e]) - double(x2[e]) * double(sn[e]));
        o2[e] = static_cast<float>(double(x2[e]) * double(c[e]) + double(x1[e]) * double(sn[e]));
      }
      vec16<T>::store(d + i0, o1);
      vec16<T>::store(d + i1, o2);
    }
  } else {
    const int jj = j - half / V;
    const int i0 = rot + 2 * jj * V, i1 = i0 + V;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const T* s = src + which * D;
      T* d = (which == 0 ? q : k) + dst_off;
      *reinterpret_cast<uint4*>(d + i0) = *reinterpret_cast<const uint4*>(s + i0);
      *reinterpret_cast<uint4*>(d + i1) = *reinterpret_cast<const uint4*>(s + i1);
    }
  }
  const T* sv = src + 2 * D;
  T* dv = v + dst_off;
  *reinterpret_cast<uint4*>(dv + 2 * j * V) = *reinterpret_cast<const uint4*>(sv + 2 * j * V);
  *reinterpret_cast<uint4*>(dv + (2 * j + 1) * V) =
      *reinterpret_cast<const uint4*>(sv + (2 * j + 1) * V);
}

bool rope_split_supported(bool bf16, int hd, int rot) {
  const int V = bf16 ? 8 : 4;
  return hd > 0 && rot > 0 && rot <= hd && rot % 2 == 0 && (rot / 2) % V == 0 && hd % (2 * V) == 0 &&
         (hd - rot) % (2 * V) == 0;
}

hipError_t rope_split(bool bf16, int N, int H, int hd, int rot, const void* qkv, const float* cos,
                      const float* sin, void* q, void* k, void* v, hipStream_t s) {
  if (N == 0) return hipSuccess;
  LaunchScope scope_(kCntRopeSplit, s);
  const int V = bf16 ? 8 : 4;
  const int64_t total = static_cast<int64_t>(N) * H * (hd / (2 * V));
  dim3 grid(static_cast<unsigned>((total + 255) / 256)), block(256);
  if (bf16)
    hipLaunchKernelGGL(rope_split_kernel<bf16_t>, grid, block, 0, s, N, H, hd, rot,
                       static_cast<const bf16_t*>(qkv), cos, sin, static_cast<bf16_t*>(q),
                       static_cast<bf16_t*>(k), static_cast<bf16_t*>(v));
  else
    hipLaunchKernelGGL(rope_split_kernel<float>, grid, block, 0, s, N, H, hd, rot,
                       static_cast<const float*>(qkv), cos, sin, static_cast<float*>(q),
                       static_cast<float*>(k), static_cast<float*>(v));
  return hipGetLastError();
}

// ============================================================================ SiLU gate
// m[n, j] = silu(u[n, j]) * u[n, F + j]; silu(z) = z / (1 + e^-z).  The music
// model's [value | gate] projection is half-swapped at stage time, so one
// kernel serves both (page "the 2.4B fp32 DiT onto the device", section "What
// moved": SiluAndMul over a stage-time half swap).
template <typename T>
__global__ __launch_bounds__(256) void silu_gate_kernel(int N, int F, const T* __restrict__ u,
                                                       T* __restrict__ m) {
  constexpr int V = vec16<T>::N;
  const int fv = F / V;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= static_cast<int64_t>(N) * fv) return;
  const int n = static_cast<int>(t / fv);
  const int j = static_cast<int>(t % fv) * V;
  const T* ur = u + static_cast<size_t>(n) * 2 * F;
  float g[V], up[V], o[V];
  vec16<T>::load(ur + j, g);
  vec16<T>::load(ur + F + j, up);
  // fp32 stream: evaluated in fp64 and rounded once; bf16: fp32 arithmetic
#pragma unroll
  for (int e = 0; e < V; ++e) {
    if (sizeof(T) == 4) {
      const double gd = g[e];
      o[e] = static_cast<float>(gd / (1.0 + exp(-gd)) * double(up[e]));
    } else {
      o[e] = g[e] / (1.0f + expf(-g[e])) * up[e];
    }
  }
  vec16<T>::store(m + static_cast<size_t>(n) * F + j, o);
}

hipError_t silu_gate(bool bf16, int N, int F, const void* u, void* m, hipStream_t s) {
  if (N == 0) return hipSuccess;
  LaunchScope scope_(kCntSiluGate, s);
  const int V = bf16 ? 8 : 4;
  if (F % V) return hipErrorInvalidValue;
  const int64_t total = static_cast<int64_t>(N) * (F / V);
  dim3 grid(static_cast<unsigned>((total + 255) / 256)), block(256);
  if (bf16)
    hipLaunchKernelGGL(silu_gate_kernel<bf16_t>, grid, block, 0, s, N, F,
                       static_cast<const bf16_t*>(u), static_cast<bf16_t*>(m));
  else
    hipLaunchKernelGGL(silu_gate_kernel<float>, grid, block, 0, s, N, F,
                       static_cast<const float*>(u), static_cast<float*>(m));
  return hipGetLastError();
}

// ============================================================================ gated residual
// x[n, j] += gate[cond_idx[n]][j] * a[n, j] (page "port the MiniMax-H3
// omni-modal video+audio DiT", section "The device-resident forward (W2b)":
// Add with an indexed AdaLN gate).  x is float32 (bf16 stream: one fused
// multiply-add) or float64 (fp32 stream: the product of two floats is exact in
// fp64, so the update is one fp64 rounding).
template <typename TX>
__global__ __launch_bounds__(256) void gated_residual_kernel(int N, int D, TX* __restrict__ x,
                                                            const float* __restrict__ a,
                                                            const float* __restrict__ mod, int gate_k,
                                                            const int32_t* __restrict__ cond_idx) {
  const int d4 = D / 4;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= static_cast<int64_t>(N) * d4) return;
  const int n = static_cast<int>(t / d4);
  const int c = static_cast<int>(t % d4);
  const float4 g = reinterpret_cast<const float4*>(
      mod + (static_cast<size_t>(cond_idx[n]) * 6 + gate_k) * D)[c];
  const float4 av = reinterpret_cast<const float4*>(a)[t];
  TX* xp = x + 4 * t;
  // one rounding per element: fma (for a float64 x the product of two floats
  // is exact, so this is x + g a rounded once either way)
  xp[0] = fma(TX(g.x), TX(av.x), xp[0]);
  xp[1] = fma(TX(g.y), TX(av.y), xp[1]);
  xp[2] = fma(TX(g.z), TX(av.z), xp[2]);
  xp[3] = fma(TX(g.w), TX(av.w), xp[3]);
}

hipError_t gated_residual(int N, int D, bool x_f64, void* x, const float* a, const float* mod, int which,
                          const int32_t* cond_idx, hipStream_t s) {
  if (N == 0) return hipSuccess;
  LaunchScope scope_(kCntGatedResidual, s);
  const int64_t total = static_cast<int64_t>(N) * (D / 4);
  dim3 grid(static_cast<unsigned>((total + 255) / 256)), block(256);
  if (x_f64)
    hipLaunchKernelGGL(gated_residual_kernel<double>, grid, block, 0, s, N, D, static_cast<double*>(x), a, mod,
                       which == 0 ? 2 : 5, cond_idx);
  else
    hipLaunchKernelGGL(gated_residual_kernel<float>, grid, block, 0, s, N, D, static_cast<float*>(x), a, mod,
                       which == 0 ? 2 : 5, cond_idx);
  return hipGetLastError();
}

// ============================================================================ residual widen / narrow
// The fp32 stream carries its residual in float64: tokens enter by exact
// widening and leave rounded to nearest float32.
__global__ __launch_bounds__(256) void widen_kernel(int64_t n, const float* __restrict__ src, double* __restrict__ dst) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < n) dst[t] = static_cast<double>(src[t]);
}
__global__ __launch_bounds__(256) void narrow_kernel(int64_t n, const double* __restrict__ src, float* __restrict__ dst) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < n) dst[t] = static_cast<float>(src[t]);
}

hipError_t widen_f32(int64_t n, const float* src, double* dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  LaunchScope scope_(kCntConvert, s);
  hipLaunchKernelGGL(widen_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, n, src, dst);
  return hipGetLastError();
}
hipError_t narrow_f64(int64_t n, const double* src, float* dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  LaunchScope scope_(kCntConvert, s);
  hipLaunchKernelGGL(narrow_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, n, src, dst);
  return hipGetLastError();
}

// ============================================================================ AdaLN table
// mod[c][j] = W[m(c)][j, :] . e[c, :] + bias[m(c)][j]; sums in fp64 so the
// table is the correctly rounded fp32 of the dot product in practice.
struct CondMap {
  int n_cond;
  int modality[64];
};

// Four consecutive weights as floats.
template <typename TW> struct wload4;
template <> struct wload4<float> {
  static __device__ __forceinline__ float4 ld(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <> struct wload4<bf16_t> {
  static __device__ __forceinline__ float4 ld(const bf16_t* p) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(t.x << 16), __uint_as_float(t.x & 0xFFFF0000u), __uint_as_float(t.y << 16),
                       __uint_as_float(t.y & 0xFFFF0000u));
  }
};

// blockIdx.z: the block (weights at p + z * stride bytes, output rows at
// mod + z * n_cond * six_d).  Eight lanes per output row, eight rows per
// wavefront, 32 per workgroup: lane k of a row reads four consecutive weights
// at k, k + 8, ... (in float4 steps), so the eight lanes of a row read 128
// contiguous bytes per step, and the row's sum closes in three shuffle steps.
constexpr int ADA_LPR = 8, ADA_ROWS = 256 / ADA_LPR, ADA_U = 8;
template <typename TW>
__global__ __launch_bounds__(256) void adaln_kernel(int six_d, int cond_dim, AdalnBlockPtrs p, int64_t w_stride,
                                                   int64_t b_stride, CondMap cm, const float* __restrict__ e,
                                                   float* __restrict__ mod) {
  const int kp = threadIdx.x % ADA_LPR;
  const int j_raw = blockIdx.x * ADA_ROWS + threadIdx.x / ADA_LPR;
  const int m = blockIdx.y;
  if (p.w[m] == nullptr) return;
  const bool live = j_raw < six_d;
  const int j = live ? j_raw : six_d - 1;  // dead rows still take part in the shuffles
  const TW* w = reinterpret_cast<const TW*>(static_cast<const char*>(p.w[m]) + blockIdx.z * w_stride) +
                static_cast<size_t>(j) * cond_dim;
  const float* bias = reinterpret_cast<const float*>(reinterpret_cast<const char*>(p.bias[m]) + blockIdx.z * b_stride);
  float* out = mod + static_cast<size_t>(blockIdx.z) * cm.n_cond * six_d;
  auto dot4 = [](float4 wv, float4 ev) {
    return static_cast<double>(wv.x) * static_cast<double>(ev.x) + static_cast<double>(wv.y) * static_cast<double>(ev.y) +
           static_cast<double>(wv.z) * static_cast<double>(ev.z) + static_cast<double>(wv.w) * static_cast<double>(ev.w);
  };
  // Up to ADA_U float4 per lane (cond_dim <= 4 * 8 * ADA_U): the row's weights
  // are loaded once, all in flight together, and reused for every
  // conditioning row; longer rows stream per conditioning row.
  const bool in_regs = cond_dim <= 4 * ADA_LPR * ADA_U;
  float4 wr[ADA_U];
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < ADA_U; ++u) {
      const int kk = 4 * kp + 4 * ADA_LPR * u;
      wr[u] = kk < cond_dim ? wload4<TW>::ld(w + kk) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  for (int c = 0; c < cm.n_cond; ++c) {
    if (cm.modality[c] != m) continue;
    const float* ec = e + static_cast<size_t>(c) * cond_dim;
    double acc = 0.0;
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < ADA_U; ++u) {
        const int kk = 4 * kp + 4 * ADA_LPR * u;
        if (kk < cond_dim) acc += dot4(wr[u], *reinterpret_cast<const float4*>(ec + kk));
      }
    } else {
      for (int kk = 4 * kp; kk < cond_dim; kk += 4 * ADA_LPR)
        acc += dot4(wload4<TW>::ld(w + kk), *reinterpret_cast<const float4*>(ec + kk));
    }
    static_assert(ADA_LPR == 8, "three butterfly steps");
    acc += xor_lane<4>(acc); acc += xor_lane<2>(acc); acc += xor_lane<1>(acc);
    if (kp == 0 && live) out[static_cast<size_t>(c) * six_d + j] = static_cast<float>(acc + static_cast<double>(bias[j]));
  }
}

hipError_t adaln(bool w_bf16, int n_blocks, const AdalnBlockPtrs* blocks_host, int n_cond,
                 const int* cond_modality_host, int six_d, int cond_dim, const float* e,
                 float* mod, hipStream_t s) {
  if (n_cond > 64 || cond_dim % 4) return hipErrorInvalidValue;
  if (n_blocks == 0) return hipSuccess;
  CondMap cm;
  cm.n_cond = n_cond;
  int n_mod = 0;
  for (int c = 0; c < n_cond; ++c) {
    cm.modality[c] = cond_modality_host[c];
    if (cond_modality_host[c] + 1 > n_mod) n_mod = cond_modality_host[c] + 1;
  }
  // One launch for all blocks when their weights sit at one stride from
  // block to block (the staged slab's layout), else one launch per block.
  auto byte = [](const void* q) { return static_cast<int64_t>(reinterpret_cast<intptr_t>(q)); };
  int64_t ws = 0, bs = 0;
  bool uniform = false;
  for (int mm = 0; mm < n_mod && n_blocks > 1; ++mm) {
    if (blocks_host[0].w[mm] == nullptr) continue;
    if (!uniform) {
      ws = byte(blocks_host[1].w[mm]) - byte(blocks_host[0].w[mm]);
      bs = byte(blocks_host[1].bias[mm]) - byte(blocks_host[0].bias[mm]);
      uniform = true;
    }
    for (int b = 1; b < n_blocks; ++b)
      if (byte(blocks_host[b].w[mm]) - byte(blocks_host[0].w[mm]) != b * ws ||
          byte(blocks_host[b].bias[mm]) - byte(blocks_host[0].bias[mm]) != b * bs)
        uniform = false, mm = n_mod, b = n_blocks;  // stop: per-block launches
  }
  const int launches = uniform ? 1 : n_blocks;
  for (int b = 0; b < launches; ++b) {
    dim3 grid((six_d + ADA_ROWS - 1) / ADA_ROWS, n_mod, uniform ? n_blocks : 1), block(256);
    LaunchScope scope_(kCntAdaln, s);
    float* out = mod + static_cast<size_t>(b) * n_cond * six_d;
    if (w_bf16)
      hipLaunchKernelGGL(adaln_kernel<bf16_t>, grid, block, 0, s, six_d, cond_dim, blocks_host[b], ws, bs, cm, e, out);
    else
      hipLaunchKernelGGL(adaln_kernel<float>, grid, block, 0, s, six_d, cond_dim, blocks_host[b], ws, bs, cm, e, out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// ============================================================================ patch in / out
// io 1 (patch3d): latent [C, T*pt, H*ph, W*pw] <-> tokens [T*H*W, pt*ph*pw*C],
// tokens in raster (t, h, w) order, vector order (pt, ph, pw, c) with c
// fastest (a convolution with kernel == stride is a linear map of the flattened
// patch; page "port the MiniMax-H3 omni-modal video+audio DiT", update "Encoder
// complete").  io 2 (channel-major): latent [C, L] <-> tokens [L, C], the
// frame-major view under which a 1x1 convolution is a GEMM (page "the 2.4B fp32
// DiT onto the device", section "What moved").  Pure index work: bit-exact.
struct PatchGeom {
  int io, C, pt, ph, pw, T, H, W;
};

__device__ __forceinline__ int64_t patch_latent_index(const PatchGeom& g, int64_t t) {
  const int cv = g.pt * g.ph * g.pw * g.C;
  const int64_t tok = t / cv;
  int e = static_cast<int>(t % cv);
  if (g.io == 2) return static_cast<int64_t>(e) * g.T + tok;  // T holds L
  const int c = e % g.C;
  e /= g.C;
  const int ipw = e % g.pw;
  e /= g.pw;
  const int iph = e % g.ph;
  const int ipt = e / g.ph;
  const int w = static_cast<int>(tok % g.W);
  const int h = static_cast<int>((tok / g.W) % g.H);
  const int tt = static_cast<int>(tok / (static_cast<int64_t>(g.W) * g.H));
  const int64_t Tp = static_cast<int64_t>(g.T) * g.pt, Hp = static_cast<int64_t>(g.H) * g.ph,
                Wp = static_cast<int64_t>(g.W) * g.pw;
  return ((static_cast<int64_t>(c) * Tp + (tt * g.pt + ipt)) * Hp + (h * g.ph + iph)) * Wp +
         (w * g.pw + ipw);
}

__global__ __launch_bounds__(256) void patch_in_kernel(PatchGeom g, int64_t total,
                                                      const float* __restrict__ latent,
                                                      float* __restrict__ tokens) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < total) tokens[t] = latent[patch_latent_index(g, t)];
}
__global__ __launch_bounds__(256) void patch_out_kernel(PatchGeom g, int64_t total,
                                                       const float* __restrict__ tokens,
                                                       float* __restrict__ latent) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < total) latent[patch_latent_index(g, t)] = tokens[t];
}

static PatchGeom make_geom(int io, int C, const int* patch, const int* grid, int64_t* total) {
  PatchGeom g;
  g.io = io;
  g.C = C;
  if (io == 1) {
    g.pt = patch[0]; g.ph = patch[1]; g.pw = patch[2];
    g.T = grid[0]; g.H = grid[1]; g.W = grid[2];
    *total = static_cast<int64_t>(g.T) * g.H * g.W * g.pt * g.ph * g.pw * C;
  } else {
    g.pt = g.ph = g.pw = 1;
    g.T = grid[0]; g.H = g.W = 1;
    *total = static_cast<int64_t>(g.T) * C;
  }
  return g;
}

hipError_t patch_in(int io, int C, const int* patch, const int* grid, const float* latent,
                    float* tokens, hipStream_t s) {
  int64_t total;
  PatchGeom g = make_geom(io, C, patch, grid, &total);
  if (total == 0) return hipSuccess;
  LaunchScope scope_(kCntPatchIn, s);
  hipLaunchKernelGGL(patch_in_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0,
                     s, g, total, latent, tokens);
  return hipGetLastError();
}

hipError_t patch_out(int io, int C, const int* patch, const int* grid, const float* tokens,
                     float* latent, hipStream_t s) {
  int64_t total;
  PatchGeom g = make_geom(io, C, patch, grid, &total);
  if (total == 0) return hipSuccess;
  LaunchScope scope_(kCntPatchOut, s);
  hipLaunchKernelGGL(patch_out_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                     0, s, g, total, tokens, latent);
  return hipGetLastError();
}

// ============================================================================ Euler step
// x += dt * v in fp32 with the product rounded before the sum (no contraction),
// the euler eta=0 update with rf_v_to_x0 folded in.
__global__ __launch_bounds__(256) void euler_kernel(int64_t n, float* __restrict__ x,
                                                   const float* __restrict__ v,
                                                   const float* __restrict__ dt) {
#pragma clang fp contract(off)
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) {
    const float p = dt[0] * v[i];
    x[i] = x[i] + p;
  }
}

hipError_t euler(int64_t n, float* x, const float* v, const float* dt, hipStream_t s) {
  if (n == 0) return hipSuccess;
  LaunchScope scope_(kCntEuler, s);
  hipLaunchKernelGGL(euler_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, n,
                     x, v, dt);
  return hipGetLastError();
}

// ============================================================================ guided Euler step
// Classifier-free guidance then the Euler update, each operation rounded to
// fp32 in turn (no contraction): g = vu + w (vc - vu); x += dt g.
__global__ __launch_bounds__(256) void cfg_euler_kernel(int64_t n, float* __restrict__ x,
                                                       const float* __restrict__ vc,
                                                       const float* __restrict__ vu, float w,
                                                       const float* __restrict__ dt) {
#pragma clang fp contract(off)
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) {
    const float u = vu[i];
    const float d = vc[i] - u;
    const float g = u + w * d;
    const float p = dt[0] * g;
    x[i] = x[i] + p;
  }
}

hipError_t cfg_euler(int64_t n, float* x, const float* vc, const float* vu, float w, const float* dt,
                     hipStream_t s) {
  if (n == 0) return hipSuccess;
  LaunchScope scope_(kCntCfgEuler, s);
  hipLaunchKernelGGL(cfg_euler_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     n, x, vc, vu, w, dt);
  return hipGetLastError();
}

}  // namespace dit
