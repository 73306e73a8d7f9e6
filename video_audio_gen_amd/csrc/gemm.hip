// Dense contractions of the DiT block: C[M,N] = A[M,K] . B[N,K]^T + bias[N].
// A is the activation (row-major, K contiguous), B the weight in nn.Linear
// layout [out, in] (K contiguous) -- the MatmulBT of page "the 2.4B fp32 DiT
// onto the device, staged once", section "What moved, and onto what".
//
// bf16: v_mfma_f32_32x32x16_bf16, fp32 accumulation, 256x256x64 workgroup
//   tiles, eight wavefronts of 128x64; A/B tiles stream HBM -> LDS by direct
//   buffer loads (double-buffered, 128 KB) into an XOR-swizzled layout so the
//   MFMA operand reads are bank-conflict free, and the next k-step's operands
//   are read while the current MFMAs run.
// f32: exact products and fp64 sums on v_mfma_f64_16x16x4_f64 (fp32 operands
//   widened on the way in), 64x64x16 tiles and a deterministic split-K whose
//   partition depends only on (N, K): each partial is reduced in a fixed order
//   and rounded to fp32 once.  The fp32 parity bound (rel 1e-5 / abs 1e-6)
//   after the music model's 24 blocks leaves room for about one rounding per
//   stored value: fp32 accumulation, and even six-term bf16 splitting of the
//   operands with fp64 sums of each MFMA (whose 16-product sums truncate),
//   break it; correctly rounded GEMMs keep it.
//
// In both, the value of C[i][j] depends only on row i of A, row j of B and K --
// never on M or on where row i sits in a tile -- so a document computed alone
// and the same document inside a packed batch give bit-identical results.
#include "common.h"
#include "kernels.h"

namespace dit {

// ============================================================================ bf16 GEMM
#ifndef DIT_GEMM_BK
#define DIT_GEMM_BK 64
#endif
#ifndef DIT_GEMM_STAGES
#define DIT_GEMM_STAGES 2
#endif
namespace gb {
constexpr int BM = 256, BN = 256, BK = DIT_GEMM_BK;
constexpr int STAGES = DIT_GEMM_STAGES;       // LDS ring: tiles k+1 .. k+STAGES-1 load while k computes
#ifndef DIT_GEMM_WAVES
#define DIT_GEMM_WAVES 8
#endif
// 8 wavefronts of 128x64 (two per SIMD: one can issue MFMAs while the other
// waits; measured 42-46% of peak against 37-40% for 4 of 128x128) or 4 of 128x128.
constexpr int WM = 128, WN = DIT_GEMM_WAVES == 8 ? 64 : 128;  // per-wave tile
constexpr int NWAVE = (BM / WM) * (BN / WN);
constexpr int NT = NWAVE * 64;                // 256 threads
constexpr int TM = WM / 32, TN = WN / 32;     // 32x32 MFMA tiles per wave
constexpr int CPR = BK / 8;                   // 16-byte chunks per tile row: 4
constexpr int DMA_PER_WAVE = BM * CPR / 64 / NWAVE;  // buffer_load...lds per operand per wave per stage: 4
}  // namespace gb

// Chunk c of row r of a tile row of CPR 16-byte chunks lives at physical chunk
// c ^ ((r / (16 / CPR)) % CPR): the 16 rows read at one logical chunk by a
// 16-lane LDS pass then cover all 16 four-bank groups once.
constexpr int gb_log2(int v) { return v <= 1 ? 0 : 1 + gb_log2(v / 2); }
__device__ __forceinline__ int gb_swz(int r, int c) {
  constexpr int sh = gb_log2(16 / gb::CPR);
  return r * gb::CPR + (c ^ ((r >> sh) & (gb::CPR - 1)));
}
static_assert(gb::CPR == 4 || gb::CPR == 8, "tile rows of 4 or 8 16-byte chunks");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Tiles move HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging, no
// ds_write): lane l of one instruction writes its 16 bytes at LDS base + 16*l,
// and a read past the buffer's num_records returns zero, which pads the M and N
// tails.  A 256x32 tile is 16 such instructions; wave w issues 4w .. 4w+3.
// Instruction i covers LDS chunks 64i .. 64i+63 = rows 16i .. 16i+15, so lane l
// fetches row 16i + l/4 at the logical chunk whose swizzled position is l%4.
__global__ __launch_bounds__(gb::NT) void gemm_bf16_kernel(int M, int N, int K,
                                                              const bf16_t* __restrict__ A,
                                                              const bf16_t* __restrict__ B,
                                                              const float* __restrict__ bias,
                                                              void* __restrict__ Cv, int c_f32,
                                                              int tiles_m, int tiles_n) {
  using namespace gb;
  __shared__ uint4 smem[STAGES * (BM + BN) * CPR];  // STAGES x (A + B): 128 KB at 2 x 64 or 4 x 32
  uint4* As = smem;
  uint4* Bs = smem + STAGES * BM * CPR;

  // Walk M fastest inside a column of tiles so consecutive workgroups share
  // the weight tile.
  const int bid = blockIdx.x;
  const int tm = bid % tiles_m;
  const int tn = bid / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = (wave / (BN / WN)) * WM, wc = (wave % (BN / WN)) * WN;

  const int a_rows = M - m0 < BM ? M - m0 : BM;
  const int b_rows = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(A + static_cast<size_t>(m0) * K), 0, a_rows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(B + static_cast<size_t>(n0) * K), 0, b_rows * K * 2, 0x00020000);
  // Byte offset of this lane's chunk for instruction j of its wave: instruction
  // i covers rows (64/CPR) i .. (64/CPR) i + 64/CPR - 1.
  uint32_t voff[DMA_PER_WAVE];
#pragma unroll
  for (int j = 0; j < DMA_PER_WAVE; ++j) {
    const int i = wave * DMA_PER_WAVE + j;
    const int row = (64 / CPR) * i + lane / CPR;
    const int c = gb_swz(row, lane % CPR) - row * CPR;  // logical chunk stored at position lane % CPR
    voff[j] = static_cast<uint32_t>(row * K + c * 8) * 2u;
  }

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

#define GB_DMA(stage, k0)                                                                               \
  {                                                                                                     \
    const int soff = (k0) * 2;                                                                          \
    _Pragma("unroll") for (int j = 0; j < DMA_PER_WAVE; ++j) {                                         \
      const int i = wave * DMA_PER_WAVE + j;                                                            \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(As + (stage) * BM * CPR + i * 64), 16,  \
                                               voff[j], soff, 0, 0);                                   \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + (stage) * BN * CPR + i * 64), 16,  \
                                               voff[j], soff, 0, 0);                                   \
    }                                                                                                   \
  }

  const int KT = K / BK;
  const int lr = lane & 31, lg = lane >> 5;

// One BK tile of MFMAs from LDS stage `st`: the operands of k-step s+1 are
// read while the 16 MFMAs of k-step s run.
#define GB_COMPUTE(st)                                                                                  \
  {                                                                                                     \
    const uint4* a_ = As + (st) * BM * CPR;                                                             \
    const uint4* b_ = Bs + (st) * BN * CPR;                                                             \
    bf16x8_t fa[2][TM], fb[2][TN];                                                                      \
    _Pragma("unroll") for (int i = 0; i < TM; ++i) fa[0][i] =                                          \
        __builtin_bit_cast(bf16x8_t, a_[gb_swz(wr + i * 32 + lr, lg)]);                                 \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[0][j] =                                          \
        __builtin_bit_cast(bf16x8_t, b_[gb_swz(wc + j * 32 + lr, lg)]);                                 \
    _Pragma("unroll") for (int ks = 0; ks < BK / 16; ++ks) {                                           \
      const int cur = ks & 1;                                                                           \
      if (ks + 1 < BK / 16) {                                                                           \
        const int c_ = (ks + 1) * 2 + lg;                                                               \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) fa[cur ^ 1][i] =                                \
            __builtin_bit_cast(bf16x8_t, a_[gb_swz(wr + i * 32 + lr, c_)]);                             \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[cur ^ 1][j] =                                \
            __builtin_bit_cast(bf16x8_t, b_[gb_swz(wc + j * 32 + lr, c_)]);                             \
      }                                                                                                 \
      _Pragma("unroll") for (int i = 0; i < TM; ++i)                                                   \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                 \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0); \
    }                                                                                                   \
  }

  // Prologue: tiles 0 .. STAGES-2 in flight.
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < KT) GB_DMA(p, p * BK)

  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % STAGES;
    // Tile kt must have landed: the younger in-flight tiles (2*DMA_PER_WAVE
    // loads each per wave) may stay outstanding.
    const int younger = KT - 1 - kt < STAGES - 2 ? KT - 1 - kt : STAGES - 2;
    constexpr int PER = 2 * DMA_PER_WAVE;
#define GB_VMCNT(n) (0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
    if (STAGES >= 4 && younger >= 2)
      __builtin_amdgcn_s_waitcnt(GB_VMCNT(2 * PER < 63 ? 2 * PER : 63));
    else if (STAGES >= 3 && younger >= 1)
      __builtin_amdgcn_s_waitcnt(GB_VMCNT(PER));
    else
      __builtin_amdgcn_s_waitcnt(GB_VMCNT(0));
#undef GB_VMCNT
    __syncthreads();  // every wave's part of tile kt is in LDS; stage (kt-1) is free
    if (kt + STAGES - 1 < KT) GB_DMA((kt + STAGES - 1) % STAGES, (kt + STAGES - 1) * BK)
    GB_COMPUTE(st)
    // Inside the block: the operand reads of k-step 0, then in each k-step the
    // MFMAs, the first TM+TN of them each followed by one operand read of the
    // next k-step.
    __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int t = 0; t < TM * TN; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (ks + 1 < BK / 16 && t < TM + TN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  }
#undef GB_COMPUTE
#undef GB_DMA

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

// K a multiple of 32; a 256-row tile of either operand must fit 32-bit buffer offsets.
bool gemm_bf16_supported(int M, int N, int K) {
  return M >= 0 && N > 0 && K > 0 && K % gb::BK == 0 && static_cast<int64_t>(gb::BM) * K * 2 < (int64_t(1) << 31);
}
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
// Exact products (fp32 operands widened to fp64) and fp64 sums on
// v_mfma_f64_16x16x4_f64, one rounding to fp32 at the end: the result is the
// correctly rounded value of the dot product except at fp64 near-ties.
// Within a 16-wide K chunk the MFMAs run k-step-outer, so consecutive MFMAs of
// a wavefront write different accumulators.  Split-K partials are fp64,
// reduced in a fixed order.
// Tile shape: 2 x 2 wavefronts of 32 x 32 (2 x 2 MFMA tiles), 64 x 64 x 16
// workgroup tiles, ~1024 workgroups per GEMM.  Measured on the music model's
// shapes, 48x64 and 48x32 wavefront tiles with 96- and 192-row workgroups, and
// 512..2048 workgroups, all land within 10%: v_mfma_f64_16x16x4_f64 alone
// sustains ~43 TFLOP/s on gfx950 (55% of the 78.6 TFLOP/s the datasheet
// gives), and this kernel runs at 42-44 on the large shapes.
#ifndef DIT_GF_WAVES_M
#define DIT_GF_WAVES_M 2
#endif
#ifndef DIT_GF_WAVES_N
#define DIT_GF_WAVES_N 2
#endif
#ifndef DIT_GF_TI
#define DIT_GF_TI 2
#endif
#ifndef DIT_GF_TJ
#define DIT_GF_TJ 2
#endif
#ifndef DIT_GF_TARGET
#define DIT_GF_TARGET 1024
#endif
namespace gf {
constexpr int TI = DIT_GF_TI, TJ = DIT_GF_TJ;          // 16x16 MFMA tiles per wave
constexpr int WM = 16 * TI, WN = 16 * TJ;              // per-wave tile
constexpr int BM = DIT_GF_WAVES_M * WM, BN = DIT_GF_WAVES_N * WN, BK = 16;
constexpr int PAD = 20;                                // LDS rows padded to 20 floats: conflict-free float4 reads
constexpr int NT = 64 * DIT_GF_WAVES_M * DIT_GF_WAVES_N;
constexpr int A_LD = (BM * 4 + NT - 1) / NT, B_LD = (BN * 4 + NT - 1) / NT;  // float4 loads per thread
}  // namespace gf

// Split count from (N, K) only, so a row's result never depends on M: about
// DIT_GF_TARGET workgroups when the rows fit one tile, each split >= 256 of K.
static int gf_splits(int N, int K) {
  const int tiles_n = (N + gf::BN - 1) / gf::BN;
  const int chunks = (K + gf::BK - 1) / gf::BK;
  int s = (DIT_GF_TARGET + tiles_n - 1) / tiles_n;
  int cap = chunks / 16;
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  return s < 1 ? 1 : s;
}

// MFMA 16x16x4 f64: lane l supplies A[l%16][k = l/16] and B[k = l/16][l%16];
// the result lane l holds D[4*i + l/16][l%16], i = 0..3.  Over four
// consecutive k-steps, lane group g = l/16 feeds k = 4g + j (j = step), so each
// lane reads one float4 per row per 16-wide K chunk.
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
  const int c_end = c_begin + chunks_per_split < chunks ? c_begin + chunks_per_split : chunks;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = (wave / DIT_GF_WAVES_N) * WM, wc = (wave % DIT_GF_WAVES_N) * WN;

  f64x4_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};

  // Loader: float4 q of this thread is row (tid + NT q) / 4, k 4 ((tid + NT q) % 4).
  float4 ra[A_LD], rb[B_LD];
  auto gload = [&](int ch) {
#pragma unroll
    for (int q = 0; q < A_LD; ++q) {
      const int id = tid + NT * q, r = id >> 2, k = ch * BK + 4 * (id & 3);
      const int gm = m0 + r;
      ra[q] = (r < BM && gm < M && k < K) ? *reinterpret_cast<const float4*>(A + static_cast<size_t>(gm) * K + k)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < B_LD; ++q) {
      const int id = tid + NT * q, r = id >> 2, k = ch * BK + 4 * (id & 3);
      const int gn = n0 + r;
      rb[q] = (r < BN && gn < N && k < K) ? *reinterpret_cast<const float4*>(B + static_cast<size_t>(gn) * K + k)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int q = 0; q < A_LD; ++q) {
      const int id = tid + NT * q;
      if ((id >> 2) < BM) *reinterpret_cast<float4*>(&As[st][id >> 2][4 * (id & 3)]) = ra[q];
    }
#pragma unroll
    for (int q = 0; q < B_LD; ++q) {
      const int id = tid + NT * q;
      if ((id >> 2) < BN) *reinterpret_cast<float4*>(&Bs[st][id >> 2][4 * (id & 3)]) = rb[q];
    }
  };

  if (c_begin < c_end) {
    gload(c_begin);
    sstore(0);
  }
  __syncthreads();
  const int r16 = lane & 15, g = lane >> 4;
  for (int ch = c_begin; ch < c_end; ++ch) {
    const int st = (ch - c_begin) & 1;
    if (ch + 1 < c_end) gload(ch + 1);
    float4 fa[TI], fb[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) fa[i] = *reinterpret_cast<const float4*>(&As[st][wr + i * 16 + r16][4 * g]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb[j] = *reinterpret_cast<const float4*>(&Bs[st][wc + j * 16 + r16][4 * g]);
    const float* fa_ = reinterpret_cast<const float*>(fa);
    const float* fb_ = reinterpret_cast<const float*>(fb);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const double av = static_cast<double>(fa_[4 * i + kk]);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, static_cast<double>(fb_[4 * j + kk]), acc[i][j], 0, 0, 0);
      }
    if (ch + 1 < c_end) sstore(st ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int gn = n0 + wc + j * 16 + r16;
    if (gn >= N) continue;
    const double bv = (splits == 1 && bias != nullptr) ? static_cast<double>(bias[gn]) : 0.0;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gm = m0 + wr + i * 16 + 4 * e + g;
        if (gm >= M) continue;
        if (splits == 1)
          C[static_cast<size_t>(gm) * N + gn] = static_cast<float>(acc[i][j][e] + bv);
        else
          part[(static_cast<size_t>(sp) * M + gm) * N + gn] = acc[i][j][e];
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
