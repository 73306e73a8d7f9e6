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
// f32: each row of A and B scaled by a power of two and cut into five 7-bit
//   integer slices; the slice products run exactly on v_mfma_i32_32x32x32_i8
//   and are combined in fp64, rounded to fp32 once (details below).  The fp32
//   parity bound (rel 1e-5 / abs 1e-6) after the music model's 24 blocks
//   leaves room for about one rounding per stored value: fp32 accumulation,
//   and even six-term bf16 splitting of the operands with fp32 MFMA sums
//   (whose 16-product sums truncate), break it; nearly correctly rounded
//   GEMMs keep it.
//
// In both, the value of C[i][j] depends only on row i of A, row j of B, K and
// the device's compute-unit count (the fp32 GEMM's split-K plan) -- never on M
// or on where row i sits in a tile -- so a document computed alone and the
// same document inside a packed batch give bit-identical results.
#include "common.h"
#include "kernels.h"
#include "slices.h"

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
static_assert(gb::WN == 64 && gb::BN % 64 == 0, "the SiLU-gate epilogue pairs a wave's two 32-column tiles");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier without the memory fence of __syncthreads(): LDS written
// by direct loads is covered by explicit vmcnt waits before it (the fence
// would add vmcnt(0), i.e. also wait for the copies just issued for later
// tiles), and the "memory" clobber keeps the compiler from moving LDS reads
// across it.
__device__ __forceinline__ void go_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Tiles move HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging, no
// ds_write): lane l of one instruction writes its 16 bytes at LDS base + 16*l,
// and a read past the buffer's num_records returns zero, which pads the M and N
// tails.  A 256x32 tile is 16 such instructions; wave w issues 4w .. 4w+3.
// Instruction i covers LDS chunks 64i .. 64i+63 = rows 16i .. 16i+15, so lane l
// fetches row 16i + l/4 at the logical chunk whose swizzled position is l%4.
//
// MX (MXFP8) instantiation: A and B are OCP E4M3 bytes with one E8M0 scale per
// 32 consecutive K values (Asc [M][K/32], Bsc [N][K/32]); a 128-byte tile row
// is 128 K values, two k-steps of v_mfma_scale_f32_32x32x64_f8f6f4.  In that
// instruction lane (r, g) (row r = lane % 32, g = lane / 32) supplies bytes
// 0-15 from the step's first 32-value block and bytes 16-31 from its second
// (any assignment inside a block works if A and B share it: lane g takes
// values 16g .. 16g+15 of each block), and the scale of block g of row r.
// The four scales of a row in a tile are one dword, staged through LDS with
// the tile (one direct dword load per wave).
template <bool MX>
__device__ __forceinline__ void gemm_tile_body(int M, int N, int K, const void* __restrict__ Av,
                                               const void* __restrict__ Bv, const uint8_t* __restrict__ Asc,
                                               const uint8_t* __restrict__ Bsc, const float* __restrict__ bias,
                                               void* __restrict__ Cv, GemmEpilogue ep, int tiles_m, int tiles_n,
                                               int banded) {
  using namespace gb;
  // bytes of one operand row; a tile row is always BK * 2 = 128 bytes
  const int rowb = MX ? K : 2 * K;
  // STAGES x (A + B): 128 KB at 2 x 64 or 4 x 32; MX adds each stage's scale
  // dwords of the A and B rows (STAGES x 2 KB)
  constexpr int SC_CHUNKS = MX ? STAGES * (BM + BN) / 4 : 0;
  __shared__ uint4 smem[STAGES * (BM + BN) * CPR + SC_CHUNKS];
  uint4* As = smem;
  uint4* Bs = smem + STAGES * BM * CPR;
  uint32_t* Ss = reinterpret_cast<uint32_t*>(smem + STAGES * (BM + BN) * CPR);  // [stage][A rows | B rows]

  const int bid = blockIdx.x;
  int tm, tn;
  if (banded) {
    // Bands of 4 tile rows, walked column by column with the rows fastest, so
    // a band's four A tiles are reused across every column of B.  Workgroups
    // go to the 8 XCDs round-robin; in each run of 128, XCD x takes 16
    // consecutive tiles of that order (four columns of one band), so the CUs
    // sharing an L2 share their A and B tiles.  The grid is padded to whole
    // runs; the padding exits here.
    constexpr int XG = 16, G = 4;
    const int t = (bid / (8 * XG)) * (8 * XG) + (bid % 8) * XG + (bid / 8) % XG;
    if (t >= tiles_m * tiles_n) return;
    const int band = t / (G * tiles_n);
    const int gr = tiles_m - band * G < G ? tiles_m - band * G : G;  // rows in this band
    const int rr = t - band * G * tiles_n;
    tm = band * G + rr % gr;
    tn = rr / gr;
  } else {
    // Column-major: M fastest inside a column of tiles, so consecutive
    // workgroups share the weight tile while A streams from the last-level cache.
    tm = bid % tiles_m;
    tn = bid / tiles_m;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = (wave / (BN / WN)) * WM, wc = (wave % (BN / WN)) * WN;

  const int a_rows = M - m0 < BM ? M - m0 : BM;
  const int b_rows = N - n0 < BN ? N - n0 : BN;
  const char* A = static_cast<const char*>(Av);
  const char* B = static_cast<const char*>(Bv);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(A + static_cast<size_t>(m0) * rowb), 0, a_rows * rowb, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(B + static_cast<size_t>(n0) * rowb), 0, b_rows * rowb, 0x00020000);
  // Byte offset of this lane's chunk for instruction j of its wave: instruction
  // i covers rows (64/CPR) i .. (64/CPR) i + 64/CPR - 1.
  uint32_t voff[DMA_PER_WAVE];
#pragma unroll
  for (int j = 0; j < DMA_PER_WAVE; ++j) {
    const int i = wave * DMA_PER_WAVE + j;
    const int row = (64 / CPR) * i + lane / CPR;
    const int c = gb_swz(row, lane % CPR) - row * CPR;  // logical chunk stored at position lane % CPR
    voff[j] = static_cast<uint32_t>(row * rowb + c * 16);
  }

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

// MX: wave w also copies the scale dwords of tile kt_ of 64 rows -- A rows
// 64w.. for w < 4, B rows 64(w-4).. otherwise -- to Ss[stage][row] (lane l's
// dword lands at the instruction's LDS base + 4l).
#define GB_DMA(stage, kt_)                                                                              \
  {                                                                                                     \
    const int soff = (kt_) * (BK * 2);                                                                  \
    _Pragma("unroll") for (int j = 0; j < DMA_PER_WAVE; ++j) {                                         \
      const int i = wave * DMA_PER_WAVE + j;                                                            \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(As + (stage) * BM * CPR + i * 64), 16,  \
                                               voff[j], soff, 0, 0);                                   \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + (stage) * BN * CPR + i * 64), 16,  \
                                               voff[j], soff, 0, 0);                                   \
    }                                                                                                   \
    if constexpr (MX)                                                                                   \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wave < 4 ? rsa : rsb,                                   \
                                               (lds_ptr_t)(Ss + (stage) * (BM + BN) + 64 * wave), 4,   \
                                               s_voff, 4 * (kt_), 0, 0);                               \
  }

  const int KT = MX ? K / (2 * BK) : K / BK;
  const int lr = lane & 31, lg = lane >> 5;
  // MX: scale rows [M][K/32] bytes; a tile's four scales of a row are one
  // dword.  Rows past M or N read as zero (their outputs are not stored).
  const int kb = K / 32;  // scale bytes per row
  __amdgpu_buffer_rsrc_t rsa = ra, rsb = rb;
  uint32_t s_voff = 0;
  if constexpr (MX) {
    rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Asc + static_cast<size_t>(m0) * kb), 0, a_rows * kb,
                                            0x00020000);
    rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Bsc + static_cast<size_t>(n0) * kb), 0, b_rows * kb,
                                            0x00020000);
    s_voff = static_cast<uint32_t>((64 * (wave & 3) + lane) * kb);
  }
  uint32_t sa[TM], sb[TN];

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

// MX: one tile is two k-steps of 64; a lane's 32-byte operand is logical
// chunks 4s + g and 4s + 2 + g of its row (bytes 16g.. of each 32-value block).
// Byte 2s + g of the scale dword is this lane's block of step s.
typedef int mx_v4i __attribute__((ext_vector_type(4)));
typedef int mx_v8i __attribute__((ext_vector_type(8)));
#define GB_MX_OPER(base, row, s_)                                                                       \
  __builtin_shufflevector(__builtin_bit_cast(mx_v4i, (base)[gb_swz((row), 4 * (s_) + lg)]),            \
                          __builtin_bit_cast(mx_v4i, (base)[gb_swz((row), 4 * (s_) + 2 + lg)]), 0, 1, 2,  \
                          3, 4, 5, 6, 7)
#define GB_MX_MFMA(s_)                                                                                  \
  _Pragma("unroll") for (int i = 0; i < TM; ++i)                                                       \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                     \
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                                     \
          xa[s_][i], xb[s_][j], acc[i][j], 0, 0, 0,                                                    \
          static_cast<int>((sa[i] >> (8 * (2 * (s_) + lg))) & 0xFFu), 0,                               \
          static_cast<int>((sb[j] >> (8 * (2 * (s_) + lg))) & 0xFFu));
#define GB_COMPUTE_MX(st)                                                                               \
  {                                                                                                     \
    const uint4* a_ = As + (st) * BM * CPR;                                                             \
    const uint4* b_ = Bs + (st) * BN * CPR;                                                             \
    mx_v8i xa[2][TM], xb[2][TN];                                                                        \
    _Pragma("unroll") for (int i = 0; i < TM; ++i) xa[0][i] = GB_MX_OPER(a_, wr + i * 32 + lr, 0);     \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) xb[0][j] = GB_MX_OPER(b_, wc + j * 32 + lr, 0);     \
    _Pragma("unroll") for (int i = 0; i < TM; ++i) xa[1][i] = GB_MX_OPER(a_, wr + i * 32 + lr, 1);     \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) xb[1][j] = GB_MX_OPER(b_, wc + j * 32 + lr, 1);     \
    GB_MX_MFMA(0)                                                                                       \
    GB_MX_MFMA(1)                                                                                       \
  }

  // Prologue: tiles 0 .. STAGES-2 in flight.
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < KT) GB_DMA(p, p)

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
    go_barrier();  // every wave's part of tile kt is in LDS; stage (kt-1) is free
    if (kt + STAGES - 1 < KT) GB_DMA((kt + STAGES - 1) % STAGES, kt + STAGES - 1)
    if constexpr (MX) {
      // tile kt's scale dwords: staged with its operands
      const uint32_t* ss = Ss + st * (BM + BN);
#pragma unroll
      for (int i = 0; i < TM; ++i) sa[i] = ss[wr + i * 32 + lr];
#pragma unroll
      for (int j = 0; j < TN; ++j) sb[j] = ss[BM + wc + j * 32 + lr];
      GB_COMPUTE_MX(st)
      // The scale and step 0's operand reads, then step 0's MFMAs each
      // followed by two reads of step 1's operands, then step 1's MFMAs.
      __builtin_amdgcn_sched_group_barrier(0x100, TM + TN + 2 * (TM + TN), 0);
#pragma unroll
      for (int t = 0; t < TM * TN; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (t < TM + TN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int t = 0; t < TM * TN; ++t) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      continue;
    }
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
#undef GB_COMPUTE_MX
#undef GB_MX_MFMA
#undef GB_MX_OPER
#undef GB_DMA

  // Epilogue: lane l of a 32x32 tile holds column l%32, rows 8*(e/4) + 4*(l/32) + e%4.
  // Rows e and e+1 are adjacent, so lane pairs (2c, 2c+1) swap one value and
  // store two adjacent columns each (measured: 1.7-2.9% off the four block
  // GEMMs against one 2- or 4-byte store per element).
  if (ep.mode == kEpiSiluGate) {
    // Columns come in 64-wide groups [32 gate | 32 up] of the same 32 MLP
    // features (the staged row order), so a wave's two 32-column tiles hold
    // the gate and the up value of one output: both rounded to bf16 as a
    // stored u would be, then silu(g) * up in fp32, rounded to bf16.
    const int gn = n0 + wc + lr;  // gate column; its up column is gn + 32
    if (gn < N) {
      const int F = N >> 1;
      const int f = ((n0 + wc) >> 1) + lr;
      const float bg = bias != nullptr ? bias[gn] : 0.f;
      const float bu = bias != nullptr ? bias[gn + 32] : 0.f;
      bf16_t* Mo = static_cast<bf16_t*>(Cv);
      // feature pairs (F is a multiple of 32): lanes 2c and 2c+1 trade one
      // value so each stores two adjacent outputs of its row in 4 bytes
      const bool odd = lane & 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const int gm = m0 + wr + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
          float mv[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float g = bf16_to_f32(f32_to_bf16(acc[i][0][e + h] + bg));
            const float u = bf16_to_f32(f32_to_bf16(acc[i][1][e + h] + bu));
            mv[h] = g / (1.0f + expf(-g)) * u;
          }
          const float recv = __shfl_xor(odd ? mv[0] : mv[1], 1, 64);
          const int row = odd ? gm + 1 : gm;
          if (row < M)
            *reinterpret_cast<uint32_t*>(Mo + static_cast<size_t>(row) * F + (odd ? f - 1 : f)) =
                odd ? pack_bf16x2(recv, mv[1]) : pack_bf16x2(mv[0], recv);
        }
      }
    }
    return;
  }
  if ((N & 1) == 0 && (reinterpret_cast<uintptr_t>(Cv) & 7) == 0) {
    // Column pairs: lanes 2c and 2c+1 trade one value so the even lane stores
    // columns (2c, 2c+1) of row r and the odd lane those of row r+1, one
    // 4-byte (bf16) or 8-byte (fp32) store each.  (Odd N or a C not 8-byte
    // aligned: one store per element below.)
    const bool odd = lane & 1;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int gn = n0 + wc + j * 32 + lr;
      const float bv = bias != nullptr && gn < N ? bias[gn] : 0.f;
      const int col = odd ? gn - 1 : gn;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const int gm = m0 + wr + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
          const float v0 = acc[i][j][e] + bv, v1 = acc[i][j][e + 1] + bv;
          const float recv = __shfl_xor(odd ? v0 : v1, 1, 64);
          const int row = odd ? gm + 1 : gm;
          if (row < M && col < N) {
            const float lo = odd ? recv : v0, hi = odd ? v1 : recv;
            const size_t o = static_cast<size_t>(row) * N + col;
            if (ep.mode == kEpiF32)
              *reinterpret_cast<float2*>(static_cast<float*>(Cv) + o) = make_float2(lo, hi);
            else
              *reinterpret_cast<uint32_t*>(static_cast<bf16_t*>(Cv) + o) = pack_bf16x2(lo, hi);
          }
        }
      }
    }
    return;
  }
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
          const size_t o = static_cast<size_t>(gm) * N + gn;
          if (ep.mode == kEpiF32) {
            static_cast<float*>(Cv)[o] = v;
          } else {
            static_cast<bf16_t*>(Cv)[o] = f32_to_bf16(v);
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(gb::NT) void gemm_bf16_kernel(int M, int N, int K, const bf16_t* __restrict__ A,
                                                              const bf16_t* __restrict__ B,
                                                              const float* __restrict__ bias,
                                                              void* __restrict__ Cv, GemmEpilogue ep, int tiles_m,
                                                              int tiles_n, int banded) {
  gemm_tile_body<false>(M, N, K, A, B, nullptr, nullptr, bias, Cv, ep, tiles_m, tiles_n, banded);
}

__global__ __launch_bounds__(gb::NT) void gemm_mx8_kernel(int M, int N, int K, const uint8_t* __restrict__ A,
                                                             const uint8_t* __restrict__ Asc,
                                                             const uint8_t* __restrict__ B,
                                                             const uint8_t* __restrict__ Bsc,
                                                             const float* __restrict__ bias, void* __restrict__ Cv,
                                                             GemmEpilogue ep, int tiles_m, int tiles_n, int banded) {
  gemm_tile_body<true>(M, N, K, A, B, Asc, Bsc, bias, Cv, ep, tiles_m, tiles_n, banded);
}

// K a multiple of the 64-wide K tile; a 256-row tile of either operand must fit 32-bit buffer offsets.
bool gemm_bf16_supported(int M, int N, int K) {
  return M >= 0 && N > 0 && K > 0 && K % gb::BK == 0 && static_cast<int64_t>(gb::BM) * K * 2 < (int64_t(1) << 31);
}
size_t gemm_bf16_ws_bytes(int, int, int) { return 0; }

hipError_t gemm_bf16(int M, int N, int K, const uint16_t* A, const uint16_t* B, const float* bias,
                     void* C, const GemmEpilogue& ep, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (ep.mode == kEpiSiluGate && N % 64 != 0) return hipErrorInvalidValue;
  LaunchScope scope_(kCntGemmBf16, s);
  const int tiles_m = (M + gb::BM - 1) / gb::BM, tiles_n = (N + gb::BN - 1) / gb::BN;
  // Tile order from the shapes (measured on the 6144-wide block's GEMMs at
  // 18,432 and 26,624 rows): banded when B has few column tiles, or when A
  // outgrows the 256 MB last-level cache (column-major order then re-streams
  // it from HBM for every few columns) and B is not too wide; column-major
  // otherwise.
  const double a_bytes = 2.0 * M * K;
  const int banded = tiles_n <= 32 || (a_bytes > 256.0 * (1 << 20) && tiles_n <= 96);
  const int nblk = banded ? (tiles_m * tiles_n + 127) / 128 * 128 : tiles_m * tiles_n;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3(nblk), dim3(gb::NT), 0, s, M, N, K, A, B,
                     bias, C, ep, tiles_m, tiles_n, banded);
  return hipGetLastError();
}

bool gemm_mx8_supported(int M, int N, int K) {
  return M >= 0 && N > 0 && K > 0 && K % (2 * gb::BK) == 0 && static_cast<int64_t>(gb::BM) * K < (int64_t(1) << 31);
}

hipError_t gemm_mx8(int M, int N, int K, const uint8_t* A, const uint8_t* Asc, const uint8_t* B, const uint8_t* Bsc,
                    const float* bias, void* C, const GemmEpilogue& ep, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (ep.mode == kEpiSiluGate && N % 64 != 0) return hipErrorInvalidValue;
  LaunchScope scope_(kCntGemmMx8, s);
  const int tiles_m = (M + gb::BM - 1) / gb::BM, tiles_n = (N + gb::BN - 1) / gb::BN;
  // tile order as the bf16 GEMM's, with A's bytes at one per value
  const double a_bytes = 1.0 * M * K;
  const int banded = tiles_n <= 32 || (a_bytes > 256.0 * (1 << 20) && tiles_n <= 96);
  const int nblk = banded ? (tiles_m * tiles_n + 127) / 128 * 128 : tiles_m * tiles_n;
  hipLaunchKernelGGL(gemm_mx8_kernel, dim3(nblk), dim3(gb::NT), 0, s, M, N, K, A, Asc, B, Bsc, bias, C, ep, tiles_m,
                     tiles_n, banded);
  return hipGetLastError();
}

// ============================================================================ f32 GEMM, int8 slices
// Error-free splitting onto the integer matrix cores (the Ozaki scheme on
// int8 units).  Each row x of A (and of B) is scaled by the power of two 2^-e
// that brings it inside (-1, 1), and the scaled row is cut into S = 5 signed
// 7-bit integer slices: x 2^-e = sum_s a_s 2^-7s + r with a_s in [-127, 127] and
// |r| < 2^-35.  The product of two rows is then
//   2^(e_i + f_j) sum_{s,t} 2^-7(s+t) (a_s . b_t)
// where every a_s . b_t is an exact int32 dot product on
// v_mfma_i32_32x32x32_i8.  Slice pairs with s + t <= S + 1 are kept (15 of
// 25); the rest, with r, weigh below 2^-32 of the scaled product per term, so
// the sum before its one rounding to fp32 is within ~0.02 fp32 ulps (rms, of
// the output's rms) of the exact dot product, against 0.24 for the rounding
// itself.  Pairs with equal s + t share one int32 accumulator (5 of them):
// 5 pairs x 127^2 x K stays below 2^31 for K <= 26630, and splits never exceed
// 16384 of K.  The integer sums are exact; each partial's five levels are
// combined in fp64 (one rounding), and the split-K partials are summed in a
// fixed order.  The split plan depends on (N, K) and the compute-unit count,
// so results are bit-reproducible on devices with the same number of CUs (a
// device with another count may round a different set of partials).
//
// Workgroup tile 192 x 64 (a few hundred rows of activations are covered by
// one or two tiles, so each weight slice is read once per row tile), K step
// 32, twelve wavefronts of 32 x 32 (three per SIMD); slices of A and B stream
// HBM -> LDS by direct buffer loads into a three-stage ring (120 KB).
namespace go {
constexpr int S = 5;                      // slices per operand
constexpr int BM = 192, BN = 64, BK = 32, NW = 12, NT = 64 * NW, STAGES = 3;
constexpr int APLANE = BM * BK / 16;      // 16-byte chunks of one A slice tile: 384
constexpr int BPLANE = BN * BK / 16;      // ... of one B slice tile: 128
constexpr int AOPER = S * APLANE, BOPER = S * BPLANE;
constexpr int STAGE = AOPER + BOPER;      // 2560 chunks = 40 KB
constexpr int NDMA = STAGE / 64;          // 1 KB direct loads per stage: 40
constexpr int AQ = AOPER / 64;            // the first 30 of them fill A
constexpr int DMA_MAX = (NDMA + NW - 1) / NW;  // per wave: 4 (waves 0-3) or 3
constexpr int KSPLIT_MAX = 16384;
}  // namespace go


// s_waitcnt vmcnt(n) for a run-time n (larger n waits for the n = 7 case).
__device__ __forceinline__ void go_wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F77); break;
  }
}

// Padded K of the slice planes (a multiple of the K step; pad slices are zero).
static inline int go_kp(int K) { return (K + go::BK - 1) / go::BK * go::BK; }

// Chunk c (0/1) of row r of a slice tile sits at r*2 + (c ^ ((r / 8) % 2)):
// the 16 rows a 16-lane ds_read_b128 pass reads cover all 64 banks.
__device__ __forceinline__ int go_swz(int r, int c) { return r * 2 + (c ^ ((r >> 3) & 1)); }

// ---------------------------------------------------------------- slicing
// One workgroup per row: the row's max, then its slices (slices.h).
__global__ __launch_bounds__(256) void slice_rows_kernel(int R, int K, int Kp, const float* __restrict__ X,
                                                        int8_t* __restrict__ P, int32_t* __restrict__ E) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* x = X + static_cast<size_t>(row) * K;
  float mx = 0.f;
  for (int k = 4 * tid; k < K; k += 4 * 256) {
    const float4 v = *reinterpret_cast<const float4*>(x + k);
    mx = nan_max(mx, nan_max(nan_max(fabsf(v.x), fabsf(v.y)), nan_max(fabsf(v.z), fabsf(v.w))));
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = nan_max(nan_max(red[0], red[1]), nan_max(red[2], red[3]));
  const int e = slice_exponent(mx);
  if (tid == 0) E[row] = e;
  for (int k = 4 * tid; k < Kp; k += 4 * 256) {
    const float4 v = k < K ? *reinterpret_cast<const float4*>(x + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float f[4] = {v.x, v.y, v.z, v.w};
    slice_store4(f, e, row, k, R, Kp, P);
  }
}

// ---------------------------------------------------------------- GEMM

__global__ __launch_bounds__(go::NT) void gemm_f32_kernel(int M, int N, int Kp,
                                                         const int8_t* __restrict__ Ap, const int32_t* __restrict__ Ae,
                                                         const int8_t* __restrict__ Bp, const int32_t* __restrict__ Be,
                                                         const float* __restrict__ bias, float* __restrict__ C,
                                                         double* __restrict__ part, int s1, int s2, int n1, int sps1,
                                                         int sps2, int tiles_m, int tiles_n) {
  using namespace go;
  __shared__ uint4 smem[STAGES * STAGE];  // 120 KB
  // Work items: N tiles 0 .. n1-1 in s1 splits of sps1 K steps, then the other
  // N tiles in s2 splits of sps2 (the longer items first).  Workgroups go to
  // the 8 XCDs round-robin; each run of 256 gives XCD x the 32 consecutive
  // items 32x .. 32x+31 (row tile fastest, then N tile, then split), so the
  // row tiles sharing a weight tile share an L2.
  const int w = (blockIdx.x / 256) * 256 + (blockIdx.x % 8) * 32 + (blockIdx.x / 8) % 32;
  const int items1 = n1 * s1, items2 = (tiles_n - n1) * s2;
  if (w >= tiles_m * (items1 + items2)) return;
  const int tm = w % tiles_m, it = w / tiles_m;
  const bool first = it < items1;
  const int tn = first ? it % n1 : n1 + (it - items1) % (tiles_n - n1);
  const int sp = first ? it / n1 : (it - items1) / (tiles_n - n1);
  const int steps_per_split = first ? sps1 : sps2;
  const int m0 = tm * BM, n0 = tn * BN;
  const int ksteps = Kp / BK;
  const int t_begin = sp * steps_per_split;
  const int t_end = t_begin + steps_per_split < ksteps ? t_begin + steps_per_split : ksteps;
  const int nsteps = t_end > t_begin ? t_end - t_begin : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches and buffer descriptors
  const int lr = lane & 31, lg = lane >> 5;
  const int wr = (wave % 6) * 32, wc = (wave / 6) * 32;

  // Direct loads: instruction q = wave + 12 j fills 1 KB = 32 rows of one
  // slice plane: q < 30 row block q%6 of A plane q/6, else row block (q-30)%2
  // of B plane (q-30)/2; lane l fetches row 32 (block) + l/2 at the logical
  // chunk the swizzle stores at position l%2.  Rows past M or N get an offset
  // past the buffer, which reads as zero.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(Ap), 0, static_cast<uint32_t>(S * static_cast<int64_t>(M) * Kp), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(Bp), 0, static_cast<uint32_t>(S * static_cast<int64_t>(N) * Kp), 0x00020000);
  const int ndma = wave < NDMA - NW * (DMA_MAX - 1) ? DMA_MAX : DMA_MAX - 1;
  uint32_t voff[DMA_MAX];
#pragma unroll
  for (int j = 0; j < DMA_MAX; ++j) {
    const int q = wave + NW * j;
    const bool a_op = q < AQ;
    const int plane = a_op ? q / 6 : (q - AQ) / 2;
    const int r = 32 * (a_op ? q % 6 : (q - AQ) % 2) + (lane >> 1);
    const int c = (lane & 1) ^ ((r >> 3) & 1);
    const int grow = (a_op ? m0 : n0) + r;
    const int rows = a_op ? M : N;
    // slice layout [plane][K step][row][32 bytes]: one instruction reads 1 KB in a row
    voff[j] = (q < NDMA && grow < rows)
                  ? static_cast<uint32_t>((static_cast<int64_t>(plane) * (Kp / BK) * rows + grow) * BK + 16 * c)
                  : 0xFFFFFFF0u;
  }
  const uint32_t a_step = static_cast<uint32_t>(M) * BK, b_step = static_cast<uint32_t>(N) * BK;  // bytes per K step
  auto dma = [&](int t, int st) {
#pragma unroll
    for (int j = 0; j < DMA_MAX; ++j) {
      const int q = wave + NW * j;
      if (j < ndma) {
        const uint32_t off = voff[j] == 0xFFFFFFF0u ? voff[j] : voff[j] + static_cast<uint32_t>(t) * (q < AQ ? a_step : b_step);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(q < AQ ? ra : rb, (lds_ptr_t)(smem + st * STAGE + q * 64), 16, off, 0,
                                                 0, 0);
      }
    }
  };

  typedef int v4i __attribute__((ext_vector_type(4)));
  typedef int v16i __attribute__((ext_vector_type(16)));
  v16i acc[S];
#pragma unroll
  for (int d = 0; d < S; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[d][e] = 0;

  static_assert(STAGES == 3, "the wait counts below assume two copies in flight");
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < nsteps) dma(t_begin + p, p);
  for (int i = 0; i < nsteps; ++i) {
    const int st = i % STAGES;
    // Step i's copy landed once only the next step's copy (this wave's 3 or 4
    // loads) is outstanding: loads complete in issue order.
    go_wait_vm(i + 1 < nsteps ? ndma : 0);
    // Every wave's share of step i is in LDS and stage (i-1) is free.  A bare
    // s_barrier: __syncthreads() would also wait for the copy just issued
    // for step i+1 (vmcnt(0)), which serialises the ring.
    go_barrier();
    if (i + STAGES - 1 < nsteps) dma(t_begin + i + STAGES - 1, (i + STAGES - 1) % STAGES);
    const uint4* sa = smem + st * STAGE;
    const uint4* sb = sa + AOPER;
    v4i fa[S], fb[S];
#pragma unroll
    for (int p = 0; p < S; ++p) {
      fa[p] = __builtin_bit_cast(v4i, sa[p * APLANE + go_swz(wr + lr, lg)]);
      fb[p] = __builtin_bit_cast(v4i, sb[p * BPLANE + go_swz(wc + lr, lg)]);
    }
    // pair (s, t) accumulates in acc[s + t]; the order keeps two MFMAs on one
    // accumulator at least two instructions apart (levels 4 3 2 4 3 2 4 3 2 4 3 1 4 0 1)
#define GO_MFMA(s_, t_) acc[(s_) + (t_)] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[s_], fb[t_], acc[(s_) + (t_)], 0, 0, 0);
    GO_MFMA(4, 0) GO_MFMA(3, 0) GO_MFMA(2, 0) GO_MFMA(3, 1) GO_MFMA(2, 1) GO_MFMA(1, 1) GO_MFMA(2, 2)
    GO_MFMA(1, 2) GO_MFMA(0, 2) GO_MFMA(1, 3) GO_MFMA(0, 3) GO_MFMA(1, 0) GO_MFMA(0, 4) GO_MFMA(0, 0)
    GO_MFMA(0, 1)
#undef GO_MFMA
  }

  // Lane holds column wc + lr, rows wr + 8 (e/4) + 4 lg + e%4 of each level.
  const int gn = n0 + wc + lr;
  // C null: fp64 partials for a consumer that sums them itself (any split count)
  const bool direct = s1 == 1 && s2 == 1 && C != nullptr;
  if ((N & 1) == 0 && (reinterpret_cast<uintptr_t>(C) & 7) == 0) {
    // Rows e and e+1 are adjacent: lanes 2c and 2c+1 swap one value, and each
    // stores two adjacent columns of its row (16-byte partials, 8-byte C).
    const bool odd = lr & 1;
    const int gnc = gn < N ? gn : N - 1;
    const int fe = Be[gnc];
    const bool bad_col = fe == kSliceNonFinite;
    const double bv = (direct && bias != nullptr) ? static_cast<double>(bias[gnc]) : 0.0;
    const double bv_pair = __shfl_xor(bv, 1, 64);  // the partner column's bias
    const int col = odd ? gn - 1 : gn;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const int gm = m0 + wr + 8 * (e >> 2) + 4 * lg + (e & 3);
      double v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = gm + h < M ? gm + h : M - 1;
        // sum_d acc_d 2^-7(d+2): each term exact in fp64, five terms
        double x = 0.0;
#pragma unroll
        for (int d = S - 1; d >= 0; --d) x += ldexp(static_cast<double>(acc[d][e + h]), -7 * (d + 2));
        const int ae = Ae[r];
        v[h] = (bad_col || ae == kSliceNonFinite) ? __builtin_nan("") : ldexp(x, ae + fe);
      }
      const double recv = __shfl_xor(odd ? v[0] : v[1], 1, 64);
      const int row = odd ? gm + 1 : gm;
      if (row < M && col < N) {
        const double lo = odd ? recv : v[0], hi = odd ? v[1] : recv;
        if (direct) {
          const double b_lo = odd ? bv_pair : bv, b_hi = odd ? bv : bv_pair;  // columns col, col + 1
          *reinterpret_cast<float2*>(C + static_cast<size_t>(row) * N + col) =
              make_float2(static_cast<float>(lo + b_lo), static_cast<float>(hi + b_hi));
        } else {
          *reinterpret_cast<double2*>(part + (static_cast<size_t>(sp) * M + row) * N + col) = make_double2(lo, hi);
        }
      }
    }
    return;
  }
  if (gn >= N) return;
  const int fe = Be[gn];
  const double bv = (direct && bias != nullptr) ? static_cast<double>(bias[gn]) : 0.0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int gm = m0 + wr + 8 * (e >> 2) + 4 * lg + (e & 3);
    if (gm >= M) continue;
    // sum_d acc_d 2^-7(d+2): each term exact in fp64, five terms
    double v = 0.0;
#pragma unroll
    for (int d = S - 1; d >= 0; --d) v += ldexp(static_cast<double>(acc[d][e]), -7 * (d + 2));
    const int ae = Ae[gm];
    v = (fe == kSliceNonFinite || ae == kSliceNonFinite) ? __builtin_nan("") : ldexp(v, ae + fe);
    if (direct)
      C[static_cast<size_t>(gm) * N + gn] = static_cast<float>(v + bv);
    else
      part[(static_cast<size_t>(sp) * M + gm) * N + gn] = v;
  }
}

// Split plan from (N, K) and the device alone, so a row's result never
// depends on M.  One workgroup fits a CU (120 KB of LDS).  Measured on MI355X:
// a K step takes ~1.1 us, a round of workgroups adds ~5 steps of fixed cost
// (first copies in flight, epilogue), and each split adds an fp64 partial of
// the row tile that is written and read back once (192 N 16 bytes at
// ~4.5 TB/s, i.e. N / 1600 steps per slot).  Plans: every N tile in s splits
// (ceil(tiles_n s / CUs) rounds of ceil(steps / s) steps), or the first n1
// tiles in s1 splits filling k whole rounds and the rest in s2 = 2..4 s1
// splits after them, which evens out a last, partial round.  Splits have
// >= 8 steps and <= 16384 of K; the cheapest plan wins.
static int go_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  return cus;
}
struct GoSplit {
  int s1, s2, n1;  // N tiles [0, n1) in s1 splits, the rest in s2
};
static GoSplit go_split(int N, int K) {
  const int tiles_n = (N + go::BN - 1) / go::BN;
  const int steps = go_kp(K) / go::BK;
  const int cus = go_cus();
  int lo = (steps * go::BK + go::KSPLIT_MAX - 1) / go::KSPLIT_MAX;  // int32 headroom
  int hi = steps / 8;
  if (hi > 64) hi = 64;
  if (hi < lo) hi = lo;
  if (lo < 1) lo = 1;
  const double part_steps = N / 1600.0;
  GoSplit best{lo, lo, tiles_n};
  double best_cost = 1e30;
  for (int sp = lo; sp <= hi; ++sp) {
    const int rounds = (tiles_n * sp + cus - 1) / cus;
    const double cost = static_cast<double>(rounds) * ((steps + sp - 1) / sp + 5) + part_steps * sp;
    if (cost < best_cost) best_cost = cost, best = GoSplit{sp, sp, tiles_n};
  }
  for (int a = lo; a <= hi; ++a) {
    for (int k = 1; k <= 2; ++k) {
      if (cus * k % a) continue;
      const int n1 = cus * k / a;  // k whole rounds of s1 = a splits
      if (n1 <= 0 || n1 >= tiles_n) continue;
      for (int m = 2; m <= 4; ++m) {
        const int b = a * m;
        if (b > hi) break;
        const int r = tiles_n - n1;
        const int rounds2 = (r * b + cus - 1) / cus;
        const double cost = k * ((steps + a - 1) / a + 5.0) + rounds2 * ((steps + b - 1) / b + 5.0) +
                            part_steps * (static_cast<double>(n1) * a + static_cast<double>(r) * b) / tiles_n;
        if (cost < best_cost) best_cost = cost, best = GoSplit{a, b, n1};
      }
    }
  }
  return best;
}

// Fixed-order reduction of the split-K partials, bias added in fp64, one rounding.
__global__ __launch_bounds__(256) void gemm_f32_reduce_kernel(int M, int N, int s1, int s2, int cb,
                                                             const double* __restrict__ part,
                                                             const float* __restrict__ bias,
                                                             float* __restrict__ C) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t MN = static_cast<int64_t>(M) * N;
  if (t >= MN) return;
  double v = 0.0;
  const int splits = t % N < cb ? s1 : s2;  // partials of this column
  for (int s = 0; s < splits; ++s) v += part[s * MN + t];
  if (bias != nullptr) v += static_cast<double>(bias[t % N]);
  C[t] = static_cast<float>(v);
}

// K a multiple of 4; every slice buffer must fit 32-bit buffer offsets.
bool gemm_f32_supported(int M, int N, int K) {
  const int64_t kp = go_kp(K);
  return M >= 0 && N > 0 && K > 0 && K % 4 == 0 && go::S * kp * (M > N ? M : N) < (int64_t(1) << 31) - 256;
}

static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
size_t gemm_f32_slices_bytes(int R, int K) {
  return al256(static_cast<size_t>(go::S) * R * go_kp(K)) + al256(sizeof(int32_t) * R);
}
static int go_slots(const GoSplit& g) { return g.s1 > g.s2 ? g.s1 : g.s2; }
size_t gemm_f32_ws_bytes(int M, int N, int K) {
  const int s = go_slots(go_split(N, K));
  return gemm_f32_slices_bytes(M, K) + (s > 1 ? al256(static_cast<size_t>(s) * M * N * sizeof(double)) : 0);
}

hipError_t slice_rows(int R, int K, const float* X, void* slices, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int kp = go_kp(K);
  int8_t* P = static_cast<int8_t*>(slices);
  int32_t* E = reinterpret_cast<int32_t*>(P + al256(static_cast<size_t>(go::S) * R * kp));
  LaunchScope scope_(kCntConvert, s);
  hipLaunchKernelGGL(slice_rows_kernel, dim3(R), dim3(256), 0, s, R, K, kp, X, P, E);
  return hipGetLastError();
}

int gemm_f32_splits(int N, int K) { return go_slots(go_split(N, K)); }
F32Splits gemm_f32_split_groups(int N, int K) {
  const GoSplit g = go_split(N, K);
  return F32Splits{g.s1, g.s2, g.n1 * go::BN < N ? g.n1 * go::BN : N};
}
size_t gemm_f32_part_bytes(int M, int N, int K) {
  return al256(static_cast<size_t>(gemm_f32_splits(N, K)) * M * N * sizeof(double));
}

static hipError_t launch_gemm_f32(int M, int N, int kp, const int8_t* Ap, const int32_t* Ae, const int8_t* Bp,
                                  const int32_t* Be, const float* bias, float* C, double* part, const GoSplit& g,
                                  hipStream_t s) {
  const int steps = kp / go::BK;
  const int sps1 = (steps + g.s1 - 1) / g.s1, sps2 = (steps + g.s2 - 1) / g.s2;
  const int tiles_m = (M + go::BM - 1) / go::BM, tiles_n = (N + go::BN - 1) / go::BN;
  const int64_t work = static_cast<int64_t>(tiles_m) * (static_cast<int64_t>(g.n1) * g.s1 +
                                                        static_cast<int64_t>(tiles_n - g.n1) * g.s2);
  if (work >= (int64_t(1) << 31) - 256) return hipErrorInvalidValue;
  const unsigned blocks = static_cast<unsigned>((work + 255) / 256 * 256);
  LaunchScope scope_(kCntGemmF32, s);
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(blocks), dim3(go::NT), 0, s, M, N, kp, Ap, Ae, Bp, Be, bias, C, part,
                     g.s1, g.s2, g.n1, sps1, sps2, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t gemm_f32_sliced(int M, int N, int K, const void* As, const void* Bs, double* part, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int kp = go_kp(K);
  const int8_t* Ap = static_cast<const int8_t*>(As);
  const int32_t* Ae = reinterpret_cast<const int32_t*>(Ap + al256(static_cast<size_t>(go::S) * M * kp));
  const int8_t* Bp = static_cast<const int8_t*>(Bs);
  const int32_t* Be = reinterpret_cast<const int32_t*>(Bp + al256(static_cast<size_t>(go::S) * N * kp));
  return launch_gemm_f32(M, N, kp, Ap, Ae, Bp, Be, nullptr, nullptr, part, go_split(N, K), s);
}

hipError_t gemm_f32(int M, int N, int K, const float* A, const void* Bs, const float* bias, float* C,
                    void* ws, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int kp = go_kp(K);
  char* w = static_cast<char*>(ws);
  hipError_t e = slice_rows(M, K, A, w, s);
  if (e != hipSuccess) return e;
  const int8_t* Ap = reinterpret_cast<const int8_t*>(w);
  const int32_t* Ae = reinterpret_cast<const int32_t*>(w + al256(static_cast<size_t>(go::S) * M * kp));
  const int8_t* Bp = static_cast<const int8_t*>(Bs);
  const int32_t* Be = reinterpret_cast<const int32_t*>(Bp + al256(static_cast<size_t>(go::S) * N * kp));
  double* part = reinterpret_cast<double*>(w + gemm_f32_slices_bytes(M, K));
  const GoSplit g = go_split(N, K);
  e = launch_gemm_f32(M, N, kp, Ap, Ae, Bp, Be, bias, C, part, g, s);
  if (e != hipSuccess || (g.s1 == 1 && g.s2 == 1)) return e;  // one split writes C itself
  const int64_t MN = static_cast<int64_t>(M) * N;
  const int cb = g.n1 * go::BN < N ? g.n1 * go::BN : N;
  {
    LaunchScope scope_(kCntGemmF32Reduce, s);
    hipLaunchKernelGGL(gemm_f32_reduce_kernel, dim3(static_cast<unsigned>((MN + 255) / 256)), dim3(256),
                       0, s, M, N, g.s1, g.s2, cb, part, bias, C);
  }
  return hipGetLastError();
}

}  // namespace dit
