// Dense contractions of the DiT block: C[M,N] = A[M,K] . B[N,K]^T + bias[N].
// A is the activation (row-major, K contiguous), B the weight in nn.Linear
// layout [out, in] (K contiguous) -- the MatmulBT of page "the 2.4B fp32 DiT
// onto the device, staged once", section "What moved, and onto what".
//
// bf16: v_mfma_f32_32x32x16_bf16, fp32 accumulation, 256x256x64 workgroup
//   tiles, four wavefronts of 128x128, A/B tiles double-buffered in LDS with an
//   XOR swizzle of the 16-byte chunks so the MFMA operand reads are
//   bank-conflict free.
// f32: exact products and fp64 sums on v_mfma_f64_16x16x4_f64 (fp32 operands
//   widened on the way in), 64x64x16 tiles and a deterministic split-K whose
//   partition depends only on (N, K): each partial is reduced in a fixed order
//   and rounded to fp32 once.  fp32 accumulation over K = 2560..10240 breaks
//   the fp32 parity bound of rel 1e-5 / abs 1e-6 on ~9% of the music model's
//   outputs, so the f32 path accumulates in fp64.
//
// In both, the value of C[i][j] depends only on row i of A, row j of B and K --
// never on M or on where row i sits in a tile -- so a document computed alone
// and the same document inside a packed batch give bit-identical results.
#include "common.h"
#include "kernels.h"

namespace dit {

// ============================================================================ bf16 GEMM
namespace gb {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WM = 128, WN = 128;            // per-wave tile
constexpr int NWAVE = (BM / WM) * (BN / WN);  // 4
constexpr int NT = NWAVE * 64;                // 256 threads
constexpr int TM = WM / 32, TN = WN / 32;     // 32x32 MFMA tiles per wave: 4 x 4
constexpr int CHUNKS_A = BM * (BK / 8) / NT;  // 16-byte chunks per thread per tile: 8
constexpr int CHUNKS_B = BN * (BK / 8) / NT;  // 8
}  // namespace gb

// 16-byte chunk c (0..7) of row r of a BK=64 bf16 tile row lives at physical
// chunk c ^ ((r >> 1) & 7): the 16 rows read by one 16-lane LDS pass then hit
// 16 distinct 4-bank groups.
__device__ __forceinline__ int gb_swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

__global__ __launch_bounds__(gb::NT, 1) void gemm_bf16_kernel(int M, int N, int K,
                                                              const bf16_t* __restrict__ A,
                                                              const bf16_t* __restrict__ B,
                                                              const float* __restrict__ bias,
                                                              void* __restrict__ Cv, int c_f32,
                                                              int tiles_m, int tiles_n) {
  using namespace gb;
  __shared__ uint4 smem[2 * (BM + BN) * (BK / 8)];  // 2 stages x (A + B) x 16-byte chunks = 128 KB
  uint4* As = smem;
  uint4* Bs = smem + 2 * BM * (BK / 8);

  // Tile order: walk M fastest inside a column of tiles so consecutive
  // workgroups reuse the same weight tile.
  const int bid = blockIdx.x;
  const int tm = bid % tiles_m;
  const int tn = bid / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = (wave / (BN / WN)) * WM, wc = (wave % (BN / WN)) * WN;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Prefetch registers: eight 16-byte chunks of A and of B per thread, held in
  // named variables (an array here is demoted to LDS/scratch by the compiler).
  static_assert(CHUNKS_A == 8 && CHUNKS_B == 8, "prefetch registers are unrolled for 8 chunks");
  uint4 ra0, ra1, ra2, ra3, ra4, ra5, ra6, ra7, rb0, rb1, rb2, rb3, rb4, rb5, rb6, rb7;
#define GB_REP8(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7)
#define GB_LD(i)                                                                              \
  {                                                                                           \
    const int id = tid + NT * (i), r = id >> 3, c = id & 7;                                   \
    const int gm = m0 + r, gn = n0 + r;                                                       \
    ra##i = gm < M ? *reinterpret_cast<const uint4*>(A + static_cast<size_t>(gm) * K + kload + c * 8) \
                   : make_uint4(0, 0, 0, 0);                                                  \
    rb##i = gn < N ? *reinterpret_cast<const uint4*>(B + static_cast<size_t>(gn) * K + kload + c * 8) \
                   : make_uint4(0, 0, 0, 0);                                                  \
  }
#define GB_ST(i)                                                                              \
  {                                                                                           \
    const int id = tid + NT * (i);                                                            \
    As[sstage * BM * 8 + gb_swz(id >> 3, id & 7)] = ra##i;                                    \
    Bs[sstage * BN * 8 + gb_swz(id >> 3, id & 7)] = rb##i;                                    \
  }
#define GB_GLOAD(k0)         \
  {                          \
    const int kload = (k0);  \
    GB_REP8(GB_LD)           \
  }
#define GB_SSTORE(st)        \
  {                          \
    const int sstage = (st); \
    GB_REP8(GB_ST)           \
  }

  const int KT = K / BK;
  GB_GLOAD(0)
  GB_SSTORE(0)
  __syncthreads();

  const int lr = lane & 31, lg = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) {
      GB_GLOAD((kt + 1) * BK)
    }
    const uint4* a = As + st * BM * 8;
    const uint4* b = Bs + st * BN * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t fa[TM], fb[TN];
      const int c = ks * 2 + lg;
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = __builtin_bit_cast(bf16x8_t, a[gb_swz(wr + i * 32 + lr, c)]);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = __builtin_bit_cast(bf16x8_t, b[gb_swz(wc + j * 32 + lr, c)]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      GB_SSTORE(st ^ 1)
    }
    __syncthreads();
  }
#undef GB_GLOAD
#undef GB_SSTORE
#undef GB_LD
#undef GB_ST
#undef GB_REP8

  // Epilogue: lane l of a 32x32 tile holds column l%32, rows 8*(e/4) + 4*(l/32) + e%4.
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int gn = n0 + wc + j * 32 + lr;
    if (gn >= N) continue;
    const float bv = bias != nullptr ? bias[gn] : 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int gm = m0 + wr + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
        if (gm < M) {
          const float v = acc[i][j][e] + bv;
          if (c_f32)
            static_cast<float*>(Cv)[static_cast<size_t>(gm) * N + gn] = v;
          else
            static_cast<bf16_t*>(Cv)[static_cast<size_t>(gm) * N + gn] = f32_to_bf16(v);
        }
      }
    }
  }
}

bool gemm_bf16_supported(int M, int N, int K) { return M >= 0 && N > 0 && K > 0 && K % gb::BK == 0; }
size_t gemm_bf16_ws_bytes(int, int, int) { return 0; }

hipError_t gemm_bf16(int M, int N, int K, const uint16_t* A, const uint16_t* B, const float* bias,
                     void* C, bool c_f32, void*, hipStream_t s) {
  if (M == 0) return hipSuccess;
  LaunchScope scope_(kCntGemmBf16, s);
  const int tiles_m = (M + gb::BM - 1) / gb::BM, tiles_n = (N + gb::BN - 1) / gb::BN;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3(tiles_m * tiles_n), dim3(gb::NT), 0, s, M, N, K, A, B,
                     bias, C, c_f32 ? 1 : 0, tiles_m, tiles_n);
  return hipGetLastError();
}

// ============================================================================ f32 GEMM, fp64 accumulation
namespace gf {
constexpr int BM = 64, BN = 64, BK = 16, PAD = 20;  // LDS rows padded to 20 floats
constexpr int NT = 256;
}  // namespace gf

// Split count from (N, K) only, so a row's result never depends on M.
static int gf_splits(int N, int K) {
  const int tiles_n = (N + gf::BN - 1) / gf::BN;
  const int chunks = (K + gf::BK - 1) / gf::BK;
  int s = (1536 + tiles_n - 1) / tiles_n;
  int cap = chunks / 16;
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return s;
}

// MFMA 16x16x4 f64: lane l supplies A[l%16][k = l/16] and B[k = l/16][l%16];
// the result lane l holds D[4*i + l/16][l%16], i = 0..3.  Over four
// consecutive MFMAs, lane group g = l/16 feeds k = 4g + j (j = MFMA index), so
// each lane reads one float4 per row per 16-wide K chunk.
__global__ __launch_bounds__(gf::NT) void gemm_f32_kernel(int M, int N, int K,
                                                         const float* __restrict__ A,
                                                         const float* __restrict__ B,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ C,
                                                         double* __restrict__ part, int splits,
                                                         int chunks_per_split, int tiles_m) {
  using namespace gf;
  __shared__ float As[2][BM][PAD];
  __shared__ float Bs[2][BN][PAD];
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int sp = blockIdx.y;
  const int m0 = tm * BM, n0 = tn * BN;
  const int chunks = (K + BK - 1) / BK;
  const int c_begin = sp * chunks_per_split;
  int c_end = c_begin + chunks_per_split;
  if (c_end > chunks) c_end = chunks;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
  const int lrow = tid >> 2, lcol = (tid & 3) * 4;  // loader: one float4 of A and of B

  f64x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};

  float4 ra, rb;
#define GF_GLOAD(ch)                                                                                    \
  {                                                                                                     \
    const int k = (ch) * BK + lcol;                                                                     \
    const int gm = m0 + lrow, gn = n0 + lrow;                                                           \
    ra = (gm < M && k < K) ? *reinterpret_cast<const float4*>(A + static_cast<size_t>(gm) * K + k)  \
                           : make_float4(0.f, 0.f, 0.f, 0.f);                                       \
    rb = (gn < N && k < K) ? *reinterpret_cast<const float4*>(B + static_cast<size_t>(gn) * K + k)  \
                           : make_float4(0.f, 0.f, 0.f, 0.f);                                       \
  }
#define GF_SSTORE(st)                                          \
  {                                                            \
    *reinterpret_cast<float4*>(&As[st][lrow][lcol]) = ra;      \
    *reinterpret_cast<float4*>(&Bs[st][lrow][lcol]) = rb;      \
  }

  if (c_begin < c_end) {
    GF_GLOAD(c_begin)
    GF_SSTORE(0)
  }
  __syncthreads();
  const int r16 = lane & 15, g = lane >> 4;
  for (int ch = c_begin; ch < c_end; ++ch) {
    const int st = (ch - c_begin) & 1;
    if (ch + 1 < c_end) GF_GLOAD(ch + 1)
    float4 fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = *reinterpret_cast<const float4*>(&As[st][wr + i * 16 + r16][4 * g]);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const float4*>(&Bs[st][wc + j * 16 + r16][4 * g]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)fa[i].x, (double)fb[j].x, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)fa[i].y, (double)fb[j].y, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)fa[i].z, (double)fb[j].z, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)fa[i].w, (double)fb[j].w, acc[i][j], 0, 0, 0);
      }
    if (ch + 1 < c_end) GF_SSTORE(st ^ 1)
    __syncthreads();
  }
#undef GF_GLOAD
#undef GF_SSTORE

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + wc + j * 16 + r16;
      if (gn >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gm = m0 + wr + i * 16 + 4 * e + g;
        if (gm >= M) continue;
        if (splits == 1) {
          const double v = acc[i][j][e] + (bias != nullptr ? static_cast<double>(bias[gn]) : 0.0);
          C[static_cast<size_t>(gm) * N + gn] = static_cast<float>(v);
        } else {
          part[(static_cast<size_t>(sp) * M + gm) * N + gn] = acc[i][j][e];
        }
      }
    }
}

// Fixed-order reduction of the split-K partials, bias added in fp64, one rounding.
__global__ __launch_bounds__(256) void gemm_f32_reduce_kernel(int M, int N, int splits,
                                                             const double* __restrict__ part,
                                                             const float* __restrict__ bias,
                                                             float* __restrict__ C) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t MN = static_cast<int64_t>(M) * N;
  if (t >= MN) return;
  double v = 0.0;
  for (int s = 0; s < splits; ++s) v += part[s * MN + t];
  if (bias != nullptr) v += static_cast<double>(bias[t % N]);
  C[t] = static_cast<float>(v);
}

bool gemm_f32_supported(int M, int N, int K) { return M >= 0 && N > 0 && K > 0 && K % 4 == 0; }

size_t gemm_f32_ws_bytes(int M, int N, int K) {
  const int s = gf_splits(N, K);
  return s > 1 ? static_cast<size_t>(s) * M * N * sizeof(double) : 0;
}

hipError_t gemm_f32(int M, int N, int K, const float* A, const float* B, const float* bias,
                    float* C, void* ws, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int splits = gf_splits(N, K);
  const int chunks = (K + gf::BK - 1) / gf::BK;
  const int cps = (chunks + splits - 1) / splits;
  const int tiles_m = (M + gf::BM - 1) / gf::BM, tiles_n = (N + gf::BN - 1) / gf::BN;
  {
    LaunchScope scope_(kCntGemmF32, s);
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(tiles_m * tiles_n, splits), dim3(gf::NT), 0, s, M, N, K,
                       A, B, bias, C, static_cast<double*>(ws), splits, cps, tiles_m);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t MN = static_cast<int64_t>(M) * N;
  {
    LaunchScope scope_(kCntGemmF32Reduce, s);
    hipLaunchKernelGGL(gemm_f32_reduce_kernel, dim3(static_cast<unsigned>((MN + 255) / 256)), dim3(256),
                       0, s, M, N, splits, static_cast<const double*>(ws), bias, C);
  }
  return hipGetLastError();
}

}  // namespace dit
