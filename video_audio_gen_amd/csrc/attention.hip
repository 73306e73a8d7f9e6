// Packed varlen non-causal attention: inside each document [cu[d], cu[d+1]),
// o = softmax(q k^T / sqrt(hd)) v, no term across documents (page "port the
// MiniMax-H3 omni-modal video+audio DiT", section "Correctness gates": the
// shared block attention run non-causal over packed varlen; page "the 2.4B fp32
// DiT onto the device", section "What moved": non-causal attention without
// bias).  Flash-style: key/value tiles stream through LDS, the softmax runs
// online in registers, and the score matrix never reaches HBM.  Key tiles start
// at each document's first token, so a document's result is the same alone
// and packed.
//
// q, k, v are head-major [H, N, hd]; o is token-major [N, H*hd] (the layout the
// output projection reads).
#include "common.h"
#include "kernels.h"

namespace dit {

// ============================================================================ bf16, MFMA
// Workgroup = one (head, document, 128-query tile); four wavefronts of 32
// queries.  Scores are computed transposed, S^T = K Q^T, on
// v_mfma_f32_32x32x16_bf16 so each lane owns one query and 16 of its keys per
// 32-key block: the row max and row sum stay in the lane plus one partner lane.
// The probabilities, rounded to bf16, are already in the B-operand layout of
// the next MFMA, O^T = V^T P^T, given V^T in LDS with the key order inside
// each 16-key group permuted to match (bits 2 and 3 of the key swapped).
namespace ab {
constexpr int HD = 128, QT = 128, KT = 64, NT = 256;
constexpr int VT_STRIDE = KT + 8;  // bf16 elements per V^T row (144 bytes)
}  // namespace ab

__device__ __forceinline__ int ab_kswz(int r, int c) { return r * 16 + (c ^ (r & 15)); }
__device__ __forceinline__ int ab_vperm(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__global__ __launch_bounds__(ab::NT) void attention_bf16_kernel(int N, int H,
                                                                   const int32_t* __restrict__ cu,
                                                                   const bf16_t* __restrict__ q,
                                                                   const bf16_t* __restrict__ k,
                                                                   const bf16_t* __restrict__ v,
                                                                   bf16_t* __restrict__ o,
                                                                   float scale_log2) {
  using namespace ab;
  // One LDS block: K tile (16 KB, swizzled rows of 16 chunks) then V^T (18 KB);
  // reused whole for the output transpose at the end (4 x 32 x 136 bf16 = 34 KB).
  __shared__ uint4 smem[(KT * HD + HD * VT_STRIDE) / 8];
  uint4* Ks = smem;
  bf16_t* Vt = reinterpret_cast<bf16_t*>(smem + KT * HD / 8);

  const int qt = blockIdx.x, h = blockIdx.y, d = blockIdx.z;
  const int s0 = cu[d], len = cu[d + 1] - s0;
  const int q0 = qt * QT;
  if (q0 >= len) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;

  const size_t head_off = static_cast<size_t>(h) * N * HD;
  const int qi = q0 + wave * 32 + lr;  // this lane's query (document-relative)
  bf16x8_t qf[HD / 16];
  {
    const bool ok = qi < len;
    const bf16_t* qp = q + head_off + static_cast<size_t>(s0 + (ok ? qi : 0)) * HD;
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) {
      const uint4 t = ok ? *reinterpret_cast<const uint4*>(qp + 16 * c + 8 * lg) : make_uint4(0, 0, 0, 0);
      qf[c] = __builtin_bit_cast(bf16x8_t, t);
    }
  }

  f32x16_t acc_o[HD / 32];
#pragma unroll
  for (int i = 0; i < HD / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc_o[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int n_kt = (len + KT - 1) / KT;
  for (int t = 0; t < n_kt; ++t) {
    const int k0 = t * KT;
    __syncthreads();  // previous tile fully consumed
    // K tile: 64 keys x 16 chunks; V tile transposed into V^T.
#pragma unroll
    for (int i = 0; i < (KT * HD / 8) / NT; ++i) {
      const int id = tid + NT * i, r = id >> 4, c = id & 15;
      const int kk = k0 + r;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (kk < len) {
        const size_t off = head_off + static_cast<size_t>(s0 + kk) * HD + c * 8;
        kv = *reinterpret_cast<const uint4*>(k + off);
        vv = *reinterpret_cast<const uint4*>(v + off);
      }
      Ks[ab_kswz(r, c)] = kv;
      const int pc = ab_vperm(r);
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Vt[(c * 8 + e) * VT_STRIDE + pc] = static_cast<bf16_t>((e & 1) ? (vw[e >> 1] >> 16) : (vw[e >> 1] & 0xFFFFu));
    }
    __syncthreads();

    // S^T for keys [k0, k0+64): two 32x32 tiles, K = hd.
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int c = 0; c < HD / 16; ++c) {
        const bf16x8_t ta = __builtin_bit_cast(bf16x8_t, Ks[ab_kswz(kb * 32 + lr, 2 * c + lg)]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, qf[c], s[kb], 0, 0, 0);
      }
    }
    // Online softmax (base 2, scale folded in).  Lane holds keys
    // k0 + 32*kb + 8*(e/4) + 4*lg + e%4 of its query.
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
        const float x = key < len ? s[kb][e] * scale_log2 : -INFINITY;
        s[kb][e] = x;
        mt = fmaxf(mt, x);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(s[kb][e] - m_new);
        s[kb][e] = p;
        ps += p;
      }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int i = 0; i < HD / 32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[i][e] *= alpha;

    // O^T += V^T P^T over four 16-key groups.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int kb = g >> 1, base = (g & 1) * 8;
      const uint4 pw = make_uint4(pack_bf16x2(s[kb][base + 0], s[kb][base + 1]),
                                  pack_bf16x2(s[kb][base + 2], s[kb][base + 3]),
                                  pack_bf16x2(s[kb][base + 4], s[kb][base + 5]),
                                  pack_bf16x2(s[kb][base + 6], s[kb][base + 7]));
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int i = 0; i < HD / 32; ++i) {
        const bf16x8_t tv = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(&Vt[(i * 32 + lr) * VT_STRIDE + g * 16 + 8 * lg]));
        acc_o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tv, pf, acc_o[i], 0, 0, 0);
      }
    }
  }

  // Normalise and write through LDS so each query row leaves as 16-byte chunks.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  __syncthreads();
  bf16_t* Os = reinterpret_cast<bf16_t*>(smem) + wave * 32 * (HD + 8);  // 32 rows x 136 per wave
#pragma unroll
  for (int i = 0; i < HD / 32; ++i)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int dd = i * 32 + 8 * e4 + 4 * lg;
      uint2 w;
      w.x = pack_bf16x2(acc_o[i][4 * e4] * inv, acc_o[i][4 * e4 + 1] * inv);
      w.y = pack_bf16x2(acc_o[i][4 * e4 + 2] * inv, acc_o[i][4 * e4 + 3] * inv);
      *reinterpret_cast<uint2*>(&Os[lr * (HD + 8) + dd]) = w;
    }
  __syncthreads();
  const int D = H * HD;
#pragma unroll
  for (int i = 0; i < (32 * HD / 8) / 64; ++i) {
    const int id = lane + 64 * i, r = id >> 4, c = id & 15;
    const int qq = q0 + wave * 32 + r;
    if (qq < len)
      *reinterpret_cast<uint4*>(o + static_cast<size_t>(s0 + qq) * D + h * HD + c * 8) =
          *reinterpret_cast<const uint4*>(&Os[r * (HD + 8) + c * 8]);
  }
}

// ============================================================================ f32 stream
// Workgroup = one (head, document, 16-query tile); each wavefront owns 4
// queries and walks them one at a time: lane j scores key j of the 64-key tile,
// the wavefront reduces max and sum, and lane d accumulates output dims d,
// d + 64 with the probabilities broadcast by readlane.  Scores, softmax and
// the weighted sum run in fp64 and the output is rounded once to fp32: the
// fp32 stream is held to rel 1e-5 / abs 1e-6, which fp32 sums over 24 blocks
// do not meet.
namespace af {
constexpr int QT = 16, QW = 4, KT = 64, NT = 256;
}

template <int HD>
__global__ __launch_bounds__(af::NT) void attention_f32_kernel(int N, int H, const int32_t* __restrict__ cu,
                                                              const float* __restrict__ q,
                                                              const float* __restrict__ k,
                                                              const float* __restrict__ v,
                                                              float* __restrict__ o, double scale) {
  using namespace af;
  constexpr int KS = HD + 1;
  __shared__ float Ks[KT * KS];
  __shared__ float Vs[KT * HD];
  __shared__ float Qs[QT * HD];
  const int qt = blockIdx.x, h = blockIdx.y, d = blockIdx.z;
  const int s0 = cu[d], len = cu[d + 1] - s0;
  const int q0 = qt * QT;
  if (q0 >= len) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t head_off = static_cast<size_t>(h) * N * HD;

  for (int i = tid; i < QT * HD; i += NT) {
    const int r = i / HD, c = i % HD;
    Qs[i] = (q0 + r < len) ? q[head_off + static_cast<size_t>(s0 + q0 + r) * HD + c] : 0.f;
  }

  constexpr int DPL = (HD + 63) / 64;  // output dims per lane
  double acc[QW][DPL];
  double m_run[QW], l_run[QW];
#pragma unroll
  for (int qq = 0; qq < QW; ++qq) {
    m_run[qq] = -INFINITY;
    l_run[qq] = 0.0;
#pragma unroll
    for (int u = 0; u < DPL; ++u) acc[qq][u] = 0.0;
  }

  const int n_kt = (len + KT - 1) / KT;
  for (int t = 0; t < n_kt; ++t) {
    const int k0 = t * KT;
    __syncthreads();
    for (int i = tid; i < KT * HD; i += NT) {
      const int r = i / HD, c = i % HD;
      const bool ok = k0 + r < len;
      const size_t off = head_off + static_cast<size_t>(s0 + k0 + r) * HD + c;
      Ks[r * KS + c] = ok ? k[off] : 0.f;
      Vs[r * HD + c] = ok ? v[off] : 0.f;
    }
    __syncthreads();
    const bool key_ok = k0 + lane < len;
#pragma unroll
    for (int qq = 0; qq < QW; ++qq) {
      const float* qr = Qs + (wave * QW + qq) * HD;
      double sc = 0.0;
#pragma unroll 8
      for (int c = 0; c < HD; ++c) sc += double(qr[c]) * double(Ks[lane * KS + c]);
      sc = key_ok ? sc * scale : -INFINITY;
      double mt = sc;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mt = fmax(mt, __shfl_xor(mt, off, 64));
      const double m_new = fmax(m_run[qq], mt);
      const double alpha = exp(m_run[qq] - m_new);
      const double p = key_ok ? exp(sc - m_new) : 0.0;
      double ps = p;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off, 64);
      l_run[qq] = l_run[qq] * alpha + ps;
      m_run[qq] = m_new;
#pragma unroll
      for (int u = 0; u < DPL; ++u) acc[qq][u] *= alpha;
      const int64_t pbits = __double_as_longlong(p);
      const int plo = static_cast<int>(pbits & 0xFFFFFFFF), phi = static_cast<int>(pbits >> 32);
      for (int j = 0; j < KT; ++j) {
        const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(plo, j));
        const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(phi, j));
        const double pj = __longlong_as_double(static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo));
#pragma unroll
        for (int u = 0; u < DPL; ++u) {
          const int dd = lane + 64 * u;
          if (dd < HD) acc[qq][u] += pj * double(Vs[j * HD + dd]);
        }
      }
    }
  }
  const int D = H * HD;
#pragma unroll
  for (int qq = 0; qq < QW; ++qq) {
    const int qi = q0 + wave * QW + qq;
    if (qi >= len) continue;
    const double inv = 1.0 / l_run[qq];
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      const int dd = lane + 64 * u;
      if (dd < HD) o[static_cast<size_t>(s0 + qi) * D + h * HD + dd] = static_cast<float>(acc[qq][u] * inv);
    }
  }
}

bool attention_supported(bool bf16, int hd) {
  if (bf16) return hd == ab::HD;
  return hd == 32 || hd == 64 || hd == 128;
}

hipError_t attention_bf16(int N, int H, int hd, int n_docs, const int32_t* cu, int max_seqlen,
                          const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                          hipStream_t s) {
  if (N == 0 || n_docs == 0 || max_seqlen == 0) return hipSuccess;
  LaunchScope scope_(kCntAttnBf16, s);
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(hd));
  dim3 grid((max_seqlen + ab::QT - 1) / ab::QT, H, n_docs);
  hipLaunchKernelGGL(attention_bf16_kernel, grid, dim3(ab::NT), 0, s, N, H, cu, q, k, v, o, scale_log2);
  return hipGetLastError();
}

hipError_t attention_f32(int N, int H, int hd, int n_docs, const int32_t* cu, int max_seqlen,
                         const float* q, const float* k, const float* v, float* o, hipStream_t s) {
  if (N == 0 || n_docs == 0 || max_seqlen == 0) return hipSuccess;
  LaunchScope scope_(kCntAttnF32, s);
  const double scale = 1.0 / sqrt(static_cast<double>(hd));
  dim3 grid((max_seqlen + af::QT - 1) / af::QT, H, n_docs);
  switch (hd) {
    case 32: hipLaunchKernelGGL(attention_f32_kernel<32>, grid, dim3(af::NT), 0, s, N, H, cu, q, k, v, o, scale); break;
    case 64: hipLaunchKernelGGL(attention_f32_kernel<64>, grid, dim3(af::NT), 0, s, N, H, cu, q, k, v, o, scale); break;
    case 128: hipLaunchKernelGGL(attention_f32_kernel<128>, grid, dim3(af::NT), 0, s, N, H, cu, q, k, v, o, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dit
