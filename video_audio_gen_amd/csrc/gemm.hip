// Dense contractions of the DiT block's bf16 stream: C[M,N] = A[M,K] . B[N,K]^T
// + bias[N].  A is the activation (row-major, K contiguous), B the weight in
// nn.Linear layout [out, in] (K contiguous) -- the MatmulBT of page "the 2.4B
// fp32 DiT onto the device, staged once", section "What moved, and onto what".
//
// bf16: v_mfma_f32_32x32x16_bf16, fp32 accumulation, 256x256x64 workgroup
//   tiles, eight wavefronts of 128x64 in two groups that alternate between
//   reading a K tile's operands from LDS into registers and running that
//   tile's MFMAs from registers (one group of each per SIMD); A/B tiles
//   stream HBM -> LDS by direct buffer loads (double-buffered, 128 KB) into an
//   XOR-swizzled layout so the operand reads are bank-conflict free.
// MXFP8: the same tiles of E4M3 bytes (128 K values per 128-byte tile row) on
//   v_mfma_scale_f32_32x32x64_f8f6f4, with each row's E8M0 block scales.
// MXFP4 weights: A in MXFP8 as above, B as OCP E2M1 nibbles (128 K values per
//   64-byte tile row) on the same instruction with B's format set to FP4.
// (The fp32 stream's GEMM on int8 slices is in gemm_slices.hip.)
//
// The value of C[i][j] depends only on row i of A, row j of B and K -- never
// on M or on where row i sits in a tile -- so a document computed alone and
// the same document inside a packed batch give bit-identical results.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dit {

// ============================================================================ bf16 GEMM
namespace gb {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGES = 2;                     // LDS ring: tile k+1 (and the copy of k+2) while k is read
constexpr int WM = 128, WN = 64;              // per-wave tile: 8 wavefronts, two per SIMD
constexpr int NWAVE = (BM / WM) * (BN / WN);
constexpr int NT = NWAVE * 64;                // 512 threads
constexpr int TM = WM / 32, TN = WN / 32;     // 32x32 MFMA tiles per wave
constexpr int CPR = BK / 8;                   // 16-byte chunks per 128-byte tile row: 8
}  // namespace gb

// Chunk c of row r of a tile row of CPR 16-byte chunks lives at physical chunk
// c ^ ((r / (16 / CPR)) % CPR): the 16 rows read at one logical chunk by a
// 16-lane LDS pass then cover all 16 four-bank groups once.
constexpr int gb_log2(int v) { return v <= 1 ? 0 : 1 + gb_log2(v / 2); }
__device__ __forceinline__ int gb_swz(int r, int c) {
  constexpr int sh = gb_log2(16 / gb::CPR);
  return r * gb::CPR + (c ^ ((r >> sh) & (gb::CPR - 1)));
}
static_assert(gb::WN == 64 && gb::BN % 64 == 0, "the SiLU-gate epilogue pairs a wave's two 32-column tiles");
// FP4 B tile rows of four chunks: chunk c of row r at r*4 + (c ^ ((r / 4) % 4)).
__device__ __forceinline__ int gb_swz4(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }
enum GemmFormat { kGemmBf16 = 0, kGemmMx8 = 1, kGemmMx4 = 2 };
// bf16 results staged through LDS before their 16-byte stores: 16-byte chunk
// c of tile row r at c ^ (4 * ((r & 1) | ((r >> 1) & 2))).  One write
// instruction of the MFMA layout covers rows r, r+1, r+4, r+5 (r = 0 or 2 mod
// 8) at four consecutive chunks 4k .. 4k+3 each; the xor sends the four rows
// to four different 64-byte bank groups.
__device__ __forceinline__ int gb_stage_chunk(int r, int c) { return c ^ (4 * ((r & 1) | ((r >> 1) & 2))); }


// Tiles move HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging, no
// ds_write): lane l of one instruction writes its 16 bytes at LDS base + 16*l,
// and a read past the buffer's num_records returns zero, which pads the M and N
// tails.  A 256-row tile of 128-byte rows is 32 such instructions, each
// covering LDS chunks 64i .. 64i+63 = rows 8i .. 8i+7 (lane l: row 8i + l/8 at
// the logical chunk whose swizzled position is l%8).
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
//
// MXFP4-weight (B4) instantiation: B holds two E2M1 values per byte, the value
// at even K in the low nibble, so a tile row is 64 bytes (four 16-byte chunks,
// one per 32-value block).  The instruction takes an FP4 operand as 32
// consecutive values of K per lane (lane half g: the k-step's K 32g ..
// 32g+31) and an FP8 operand as two runs of 16 (bytes 0-15: K 16g .. 16g+15,
// bytes 16-31: K 32+16g ..; measured with identity operands), so with A's
// bytes placed as above (block 2s then block 2s+1, values 16g .. of each)
// lane (r, g) passes B's whole block 2s + g -- one 16-byte chunk -- and each
// FP4 value meets the FP8 value of the same K; the block scales stay as for
// MXFP8 (lane g: block 2s + g).
template <int FMT>  // kGemmBf16, kGemmMx8, kGemmMx4
__device__ __forceinline__ void gemm_tile_body(int M, int N, int K, const void* __restrict__ Av,
                                               const void* __restrict__ Bv, const uint8_t* __restrict__ Asc,
                                               const uint8_t* __restrict__ Bsc, const float* __restrict__ bias,
                                               void* __restrict__ Cv, GemmEpilogue ep, int tiles_m, int tiles_n,
                                               int banded) {
  using namespace gb;
  constexpr bool MX = FMT != kGemmBf16;
  constexpr bool B4 = FMT == kGemmMx4;
  constexpr int CPR_B = B4 ? CPR / 2 : CPR;  // 16-byte chunks per B tile row
  // bytes of one operand row; an A tile row is always BK * 2 = 128 bytes, a B
  // tile row too except for FP4 B (64 bytes)
  const int rowb = MX ? K : 2 * K;
  const int rowb_b = B4 ? K / 2 : rowb;
  // STAGES x (A + B): 128 KB (96 KB with FP4 B); MX adds each stage's scale
  // dwords of the A and B rows (STAGES x 2 KB)
  constexpr int SC_CHUNKS = MX ? STAGES * (BM + BN) / 4 : 0;
  __shared__ uint4 smem[STAGES * (BM * CPR + BN * CPR_B) + SC_CHUNKS];
  uint4* As = smem;
  uint4* Bs = smem + STAGES * BM * CPR;
  uint32_t* Ss = reinterpret_cast<uint32_t*>(smem + STAGES * (BM * CPR + BN * CPR_B));  // [stage][A rows | B rows]

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
      const_cast<char*>(B + static_cast<size_t>(n0) * rowb_b), 0, b_rows * rowb_b, 0x00020000);
  // Copy instruction j of a wave covers tile rows 64 (wave % 4) + 8 j ..
  // + 7, lane l fetching row 64 (wave % 4) + 8 j + l / 8 at the logical chunk
  // that the swizzle stores at position l % 8.  The swizzle of row r + 8 j
  // depends on j only through j % 2, so two lane offsets serve all eight
  // instructions; the 8 j rows go into the scalar offset.
  constexpr int DMA_G = BM * CPR / 64 / 4;  // per operand per wave of a group: 8
  static_assert(CPR == 8, "the copy offsets below assume 128-byte tile rows of eight chunks");
  uint32_t voff2[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int row = 64 * (wave & 3) + 8 * par + lane / CPR;
    const int c = gb_swz(row, lane % CPR) - row * CPR;
    voff2[par] = static_cast<uint32_t>((row - 8 * par) * rowb + c * 16);
  }
  // FP4 B: instruction j of a group-0 wave covers B tile rows 64 (wave % 4) +
  // 16 j .. + 15, lane l row 64 (wave % 4) + 16 j + l / 4 at the logical chunk
  // that the four-chunk swizzle stores at position l % 4; the swizzle of those
  // rows does not depend on j, so one lane offset serves all four.
  constexpr int DMA_B4 = BN * CPR_B / 64 / 4;  // per wave of group 0: 4
  uint32_t voff_b4 = 0;
  if constexpr (B4) {
    const int row = 64 * (wave & 3) + lane / CPR_B;
    const int c = gb_swz4(row, lane % CPR_B) - row * CPR_B;
    voff_b4 = static_cast<uint32_t>(row * rowb_b + c * 16);
  }

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

// Half a tile per group: group 1 copies the A tile (and the A scales), group 0
// the B tile (and the B scales); wave w of a group moves rows 64 (w % 4) ..
#define GB_DMA_HALF(stage, kt_)                                                                         \
  {                                                                                                     \
    const int soff = (kt_) * (BK * 2);                                                                  \
    if (grp == 1) {                                                                                     \
      _Pragma("unroll") for (int j = 0; j < DMA_G; ++j) {                                              \
        const int i = (wave & 3) * DMA_G + j;                                                           \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(As + (stage) * BM * CPR + i * 64), 16,\
                                                 voff2[j & 1], soff + 8 * j * rowb, 0, 0);             \
      }                                                                                                 \
      if constexpr (MX)                                                                                 \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(Ss + (stage) * (BM + BN) + 64 * (wave & 3)), \
                                                 4, s_voff, 4 * (kt_), 0, 0);                          \
    } else if constexpr (B4) {                                                                          \
      _Pragma("unroll") for (int j = 0; j < DMA_B4; ++j) {                                             \
        const int i = (wave & 3) * DMA_B4 + j;                                                          \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + (stage) * BN * CPR_B + i * 64),  \
                                                 16, voff_b4, (kt_) * BK + 16 * j * rowb_b, 0, 0);     \
      }                                                                                                 \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                         \
          rsb, (lds_ptr_t)(Ss + (stage) * (BM + BN) + BM + 64 * (wave & 3)), 4, s_voff, 4 * (kt_), 0, 0); \
    } else {                                                                                            \
      _Pragma("unroll") for (int j = 0; j < DMA_G; ++j) {                                              \
        const int i = (wave & 3) * DMA_G + j;                                                           \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(Bs + (stage) * BN * CPR + i * 64), 16,\
                                                 voff2[j & 1], soff + 8 * j * rowb, 0, 0);             \
      }                                                                                                 \
      if constexpr (MX)                                                                                 \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                       \
            rsb, (lds_ptr_t)(Ss + (stage) * (BM + BN) + BM + 64 * (wave & 3)), 4, s_voff, 4 * (kt_), 0, 0); \
    }                                                                                                   \
  }
  const int KT = MX ? K / (2 * BK) : K / BK;
  const int lr = lane & 31, lg = lane >> 5;
  const int kb = K / 32;
  __amdgpu_buffer_rsrc_t rsa = ra, rsb = rb;
  uint32_t s_voff = 0;
  if constexpr (MX) {
    rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Asc + static_cast<size_t>(m0) * kb), 0, a_rows * kb,
                                            0x00020000);
    rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Bsc + static_cast<size_t>(n0) * kb), 0, b_rows * kb,
                                            0x00020000);
    s_voff = static_cast<uint32_t>((64 * (wave & 3) + lane) * kb);
  }
  const int grp = wave >> 2;
  typedef int mx_v4i __attribute__((ext_vector_type(4)));
  typedef int mx_v8i __attribute__((ext_vector_type(8)));
  constexpr int KS = MX ? 2 : BK / 16;
  typedef typename std::conditional<MX, mx_v8i, bf16x8_t>::type frag_t;
  frag_t fa[KS][TM], fb[KS][TN];
  uint32_t sa[TM / 2], sb[TN / 2];
  auto read_tile = [&](int st) {
    const uint4* a_ = As + st * BM * CPR;
    const uint4* b_ = Bs + st * BN * CPR_B;
    if constexpr (MX) {
      // A row's tile scale dword holds its blocks 0-3; this lane's blocks for
      // k-steps 0 and 1 are g and 2 + g.  Two rows (2r', 2r'+1) share one
      // register: byte 2 (row % 2) + k-step, picked by the MFMAs' op_sel.
      const uint32_t* ss = Ss + st * (BM + BN);
      const uint32_t sel = lg ? 0x07050301u : 0x06040200u;
#pragma unroll
      for (int i = 0; i < TM / 2; ++i)
        sa[i] = __builtin_amdgcn_perm(ss[wr + (2 * i + 1) * 32 + lr], ss[wr + 2 * i * 32 + lr], sel);
#pragma unroll
      for (int j = 0; j < TN / 2; ++j)
        sb[j] = __builtin_amdgcn_perm(ss[BM + wc + (2 * j + 1) * 32 + lr], ss[BM + wc + 2 * j * 32 + lr], sel);
#pragma unroll
      for (int s_ = 0; s_ < 2; ++s_) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fa[s_][i] = __builtin_shufflevector(__builtin_bit_cast(mx_v4i, a_[gb_swz(wr + i * 32 + lr, 4 * s_ + lg)]),
                                              __builtin_bit_cast(mx_v4i, a_[gb_swz(wr + i * 32 + lr, 4 * s_ + 2 + lg)]),
                                              0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (B4) {
            // the whole 32-value block 2s + g of the row (chunk 2s + g)
            const mx_v4i z = {0, 0, 0, 0};
            fb[s_][j] = __builtin_shufflevector(__builtin_bit_cast(mx_v4i, b_[gb_swz4(wc + j * 32 + lr, 2 * s_ + lg)]), z,
                                                0, 1, 2, 3, 4, 5, 6, 7);
          } else {
            fb[s_][j] = __builtin_shufflevector(__builtin_bit_cast(mx_v4i, b_[gb_swz(wc + j * 32 + lr, 4 * s_ + lg)]),
                                                __builtin_bit_cast(mx_v4i, b_[gb_swz(wc + j * 32 + lr, 4 * s_ + 2 + lg)]),
                                                0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[ks][i] = __builtin_bit_cast(bf16x8_t, a_[gb_swz(wr + i * 32 + lr, ks * 2 + lg)]);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[ks][j] = __builtin_bit_cast(bf16x8_t, b_[gb_swz(wc + j * 32 + lr, ks * 2 + lg)]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < TM; ++i) asm volatile("" : "+v"(fa[ks][i]));
#pragma unroll
      for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(fb[ks][j]));
    }
    if constexpr (MX) {
#pragma unroll
      for (int i = 0; i < TM / 2; ++i) asm volatile("" : "+v"(sa[i]));
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) asm volatile("" : "+v"(sb[j]));
    }
  };
  auto mfma_tile = [&]() {
    if constexpr (MX) {
#define GB_MX_MFMA(ks_, i_, j_)                                                                         \
  acc[i_][j_] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                                       \
      fa[ks_][i_], fb[ks_][j_], acc[i_][j_], 0, B4 ? 4 : 0, 2 * ((i_) & 1) + (ks_), static_cast<int>(sa[(i_) / 2]), \
      2 * ((j_) & 1) + (ks_), static_cast<int>(sb[(j_) / 2]));
#define GB_MX_STEP(ks_)                                                                                 \
  GB_MX_MFMA(ks_, 0, 0) GB_MX_MFMA(ks_, 0, 1) GB_MX_MFMA(ks_, 1, 0) GB_MX_MFMA(ks_, 1, 1)              \
  GB_MX_MFMA(ks_, 2, 0) GB_MX_MFMA(ks_, 2, 1) GB_MX_MFMA(ks_, 3, 0) GB_MX_MFMA(ks_, 3, 1)
      static_assert(TM == 4 && TN == 2, "the unrolled MX k-steps");
      GB_MX_STEP(0)
      GB_MX_STEP(1)
#undef GB_MX_STEP
#undef GB_MX_MFMA
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(acc[i][j]));
  };
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    go_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The K loop in phases one workgroup barrier apart.  Group 0 (waves 0-3)
  // reads tile k's operands into registers in phase 2k and runs its MFMAs on
  // them in phase 2k+1; group 1 (waves 4-7) does the same one phase later, so
  // on every SIMD one wave streams MFMAs from registers while the other reads
  // LDS (an MFMA wave alone keeps the matrix core busy).  Group 1 takes one
  // extra barrier first and group 0 one after its last MFMAs, so every wave
  // executes the same number.  Measured per 64-deep K tile: ~1,100 clocks of
  // reads (and copy issue) against ~1,030 of MFMAs per group, where one
  // barrier per tile with all eight waves reading and multiplying took
  // ~3,500.
  //
  // Copies: tile t+2 goes into tile t's stage.  Group 1 issues its A half
  // right after its own reads of tile t (group 0 read it a phase earlier),
  // group 0 its B half after its reads of tile t+1 (a phase later) -- each
  // after the reads of its phase, since the compiler makes any LDS read wait
  // for the direct-to-LDS copies in flight.  Each group waits for its copies
  // before the barrier ahead of the other group's first read of them: group 1
  // at the end of its next MFMA phase, group 0 before its reads of tile t+1.
  GB_DMA_HALF(0, 0)
  if (KT > 1) GB_DMA_HALF(1, 1)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (grp == 1) phase_barrier();
  for (int kt = 0; kt < KT; ++kt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's copies into tile kt's stage are done
    read_tile(kt & 1);
    if (grp == 1 && kt + 2 < KT) GB_DMA_HALF(kt & 1, kt + 2)
    if (grp == 0 && kt >= 1 && kt + 1 < KT) GB_DMA_HALF((kt + 1) & 1, kt + 1)
    phase_barrier();
    mfma_tile();
    if (grp == 1) __builtin_amdgcn_s_waitcnt(0x0F70);  // its A half of tile kt+2 has landed
    phase_barrier();
  }
  if (grp == 0) phase_barrier();
#undef GB_DMA_HALF

  // Epilogue: lane l of a 32x32 tile holds column l%32, rows 8*(e/4) + 4*(l/32) + e%4.
  // Rows e and e+1 are adjacent, so lane pairs (2c, 2c+1) swap one value and
  // store two adjacent columns each (measured: 1.7-2.9% off the four block
  // GEMMs against one 2- or 4-byte store per element).
  // bf16 results go through LDS (free: every wave is past its last read of
  // the ring) so that each lane stores 16 bytes and each store instruction
  // writes whole rows of the tile: from the MFMA layout a lane could store
  // only 4 bytes, and an instruction wrote 64-byte pieces of four rows (the
  // epilogue took ~7 us of a 256 x 256 tile's ~150).
  char* const st_lds = reinterpret_cast<char*>(smem);
  auto stage_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
  };
  static_assert(sizeof(smem) >= BM * (BN / 2) * 2, "the SiLU-gate epilogue stages 256 rows x 128 bf16 features");
  if (ep.mode == kEpiSiluGate) {
    // Columns come in 64-wide groups [32 gate | 32 up] of the same 32 MLP
    // features (the staged row order), so a wave's two 32-column tiles hold
    // the gate and the up value of one output: both rounded to bf16 as a
    // stored u would be, then silu(g) * up in fp32, rounded to bf16.  The
    // tile's 128 features of a row (256 bytes, 16 chunks) are staged, then
    // stored by rows.
    const int F = N >> 1;
    const int gn = n0 + wc + lr;  // gate column; its up column is gn + 32
    const float bg = bias != nullptr && gn < N ? bias[gn] : 0.f;
    const float bu = bias != nullptr && gn < N ? bias[gn + 32] : 0.f;
    const int fl = (wc >> 1) + lr;  // feature within the tile
    // feature pairs: lanes 2c and 2c+1 trade one value so each writes two
    // adjacent outputs of its row in 4 bytes
    const bool odd = lane & 1;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int r = wr + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
        float mv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float g = bf16_to_f32(f32_to_bf16(acc[i][0][e + h] + bg));
          const float u = bf16_to_f32(f32_to_bf16(acc[i][1][e + h] + bu));
          mv[h] = g / (1.0f + expf(-g)) * u;
        }
        const float recv = xor_lane<1>(odd ? mv[0] : mv[1]);
        const int row = odd ? r + 1 : r;
        const int f = odd ? fl - 1 : fl;
        *reinterpret_cast<uint32_t*>(st_lds + row * 256 + gb_stage_chunk(row, f >> 3) * 16 + (f & 7) * 2) =
            odd ? pack_bf16x2(recv, mv[1]) : pack_bf16x2(mv[0], recv);
      }
    }
    stage_barrier();
    bf16_t* Mo = static_cast<bf16_t*>(Cv);
    const int f0 = n0 >> 1;
#pragma unroll
    for (int p = 0; p < BM * 16 / NT; ++p) {
      const int row = p * (NT / 16) + (tid >> 4), k = tid & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(st_lds + row * 256 + gb_stage_chunk(row, k) * 16);
      if (m0 + row < M && f0 + 8 * k < F)
        *reinterpret_cast<uint4*>(Mo + static_cast<size_t>(m0 + row) * F + f0 + 8 * k) = v;
    }
    return;
  }
  // The tile goes through LDS in passes of RP rows: the whole tile (128 KB)
  // in the bf16 and MXFP8 forms' rings, halves in the MXFP4 form's 98 KB one.
  constexpr int RP = sizeof(smem) >= BM * BN * 2 ? BM : BM / 2;
  static_assert(RP % WM == 0 || WM % RP == 0, "a pass holds whole row blocks of the waves");
  if (ep.mode == kEpiBf16 && (N & 7) == 0 && (reinterpret_cast<uintptr_t>(Cv) & 15) == 0) {
    // The tile's 256 columns of a row (512 bytes, 32 chunks) staged, then
    // stored by rows; lanes 2c and 2c+1 trade one value as below.
    const bool odd = lane & 1;
    bf16_t* Co = static_cast<bf16_t*>(Cv);
#pragma unroll
    for (int pass = 0; pass < BM / RP; ++pass) {
      if (pass > 0) stage_barrier();  // the previous pass's rows have been read
      if (wr / RP == pass) {          // uniform: this wave's rows are in the pass
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int gn = n0 + wc + j * 32 + lr;
          const float bv = bias != nullptr && gn < N ? bias[gn] : 0.f;
          const int col = wc + j * 32 + (odd ? lr - 1 : lr);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
              const int r = wr - pass * RP + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
              const float v0 = acc[i][j][e] + bv, v1 = acc[i][j][e + 1] + bv;
              const float recv = xor_lane<1>(odd ? v0 : v1);
              const int row = odd ? r + 1 : r;
              const float lo = odd ? recv : v0, hi = odd ? v1 : recv;
              *reinterpret_cast<uint32_t*>(st_lds + row * 512 + gb_stage_chunk(row, col >> 3) * 16 + (col & 7) * 2) =
                  pack_bf16x2(lo, hi);
            }
          }
        }
      }
      stage_barrier();
#pragma unroll
      for (int p = 0; p < RP * 32 / NT; ++p) {
        const int row = p * (NT / 32) + (tid >> 5), k = tid & 31;
        const uint4 v = *reinterpret_cast<const uint4*>(st_lds + row * 512 + gb_stage_chunk(row, k) * 16);
        const int grow = m0 + pass * RP + row;
        if (grow < M && n0 + 8 * k < N)
          *reinterpret_cast<uint4*>(Co + static_cast<size_t>(grow) * N + n0 + 8 * k) = v;
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
          const float recv = xor_lane<1>(odd ? v0 : v1);
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
  gemm_tile_body<kGemmBf16>(M, N, K, A, B, nullptr, nullptr, bias, Cv, ep, tiles_m, tiles_n, banded);
}

__global__ __launch_bounds__(gb::NT) void gemm_mx8_kernel(int M, int N, int K, const uint8_t* __restrict__ A,
                                                             const uint8_t* __restrict__ Asc,
                                                             const uint8_t* __restrict__ B,
                                                             const uint8_t* __restrict__ Bsc,
                                                             const float* __restrict__ bias, void* __restrict__ Cv,
                                                             GemmEpilogue ep, int tiles_m, int tiles_n, int banded) {
  gemm_tile_body<kGemmMx8>(M, N, K, A, B, Asc, Bsc, bias, Cv, ep, tiles_m, tiles_n, banded);
}

__global__ __launch_bounds__(gb::NT) void gemm_mx4_kernel(int M, int N, int K, const uint8_t* __restrict__ A,
                                                             const uint8_t* __restrict__ Asc,
                                                             const uint8_t* __restrict__ B,
                                                             const uint8_t* __restrict__ Bsc,
                                                             const float* __restrict__ bias, void* __restrict__ Cv,
                                                             GemmEpilogue ep, int tiles_m, int tiles_n, int banded) {
  gemm_tile_body<kGemmMx4>(M, N, K, A, B, Asc, Bsc, bias, Cv, ep, tiles_m, tiles_n, banded);
}

// K a multiple of the 64-wide K tile; a 256-row tile of either operand must fit 32-bit buffer offsets.
bool gemm_bf16_supported(int M, int N, int K) {
  return M >= 0 && N > 0 && K > 0 && K % gb::BK == 0 && static_cast<int64_t>(gb::BM) * K * 2 < (int64_t(1) << 31);
}
size_t gemm_bf16_ws_bytes(int, int, int) { return 0; }

hipError_t gemm_bf16(int M, int N, int K, const uint16_t* A, const uint16_t* B, const float* bias,
                     void* C, const GemmEpilogue& ep, hipStream_t s) {
  if (M == 0) return hipSuccess;
  // SiLU-gate output rows are stored in 16-byte pieces
  if (ep.mode == kEpiSiluGate && (N % 64 != 0 || (reinterpret_cast<uintptr_t>(C) & 15) != 0)) return hipErrorInvalidValue;
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
  // SiLU-gate output rows are stored in 16-byte pieces
  if (ep.mode == kEpiSiluGate && (N % 64 != 0 || (reinterpret_cast<uintptr_t>(C) & 15) != 0)) return hipErrorInvalidValue;
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

// MXFP4 weights: A as for gemm_mx8, B [N, K/2] two E2M1 codes per byte (even K
// in the low nibble) with E8M0 scales [N][K/32].
hipError_t gemm_mx4(int M, int N, int K, const uint8_t* A, const uint8_t* Asc, const uint8_t* B, const uint8_t* Bsc,
                    const float* bias, void* C, const GemmEpilogue& ep, hipStream_t s) {
  if (M == 0) return hipSuccess;
  // SiLU-gate output rows are stored in 16-byte pieces
  if (ep.mode == kEpiSiluGate && (N % 64 != 0 || (reinterpret_cast<uintptr_t>(C) & 15) != 0)) return hipErrorInvalidValue;
  LaunchScope scope_(kCntGemmMx4, s);
  const int tiles_m = (M + gb::BM - 1) / gb::BM, tiles_n = (N + gb::BN - 1) / gb::BN;
  const double a_bytes = 1.0 * M * K;
  const int banded = tiles_n <= 32 || (a_bytes > 256.0 * (1 << 20) && tiles_n <= 96);
  const int nblk = banded ? (tiles_m * tiles_n + 127) / 128 * 128 : tiles_m * tiles_n;
  hipLaunchKernelGGL(gemm_mx4_kernel, dim3(nblk), dim3(gb::NT), 0, s, M, N, K, A, Asc, B, Bsc, bias, C, ep, tiles_m,
                     tiles_n, banded);
  return hipGetLastError();
}

}  // namespace dit
