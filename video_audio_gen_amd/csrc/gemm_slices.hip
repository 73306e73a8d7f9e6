// The fp32 stream's GEMM: C[M,N] = A[M,K] . B[N,K]^T + bias[N] in fp32 with
// near-correct rounding, on the int8 matrix cores.  Each row of A and B is
// scaled by a power of two and cut into five 7-bit integer slices (slices.h);
// the slice products run exactly on v_mfma_i32_32x32x32_i8 and are combined in
// fp64, rounded to fp32 once.  The fp32 parity bound (rel 1e-5 / abs 1e-6)
// after the music model's 24 blocks leaves room for about one rounding per
// stored value: fp32 accumulation, and even six-term bf16 splitting of the
// operands with fp32 MFMA sums (whose 16-product sums truncate), break it;
// nearly correctly rounded GEMMs keep it.  (Page "the 2.4B fp32 DiT onto the
// device, staged once", section "What moved, and onto what": MatmulBT, fp32
// stays fp32.)
//
// The value of C[i][j] depends only on row i of A, row j of B, K and the
// device's compute-unit count (the split-K plan) -- never on M or on where row
// i sits in a tile -- so a document computed alone and the same document
// inside a packed batch give bit-identical results.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "slices.h"

namespace dit {

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
// Workgroup tile 176 x 64 (a few hundred rows of activations are covered by
// one or two tiles, so each weight slice is read once per row tile), K step
// 32, eight wavefronts in two groups that alternate between reading a step's
// slice fragments into registers and multiplying (below); slices of A and B
// stream HBM -> LDS by direct buffer loads into a four-stage ring (160 KB).
namespace go {
constexpr int S = 5;                      // slices per operand
constexpr int BM = 192, BN = 64, BK = 32, NW = 8, NT = 64 * NW, STAGES = 4;  // BM: rows of an A slice tile in LDS
constexpr int BMT = 176;                  // rows a tile computes: 5 blocks of 32, one of 16 (LDS rows 176.. read zero)
constexpr int APLANE = BM * BK / 16;      // 16-byte chunks of one A slice tile: 384
constexpr int BPLANE = BN * BK / 16;      // ... of one B slice tile: 128
constexpr int AOPER = S * APLANE, BOPER = S * BPLANE;
constexpr int STAGE = AOPER + BOPER;      // 2560 chunks = 40 KB
constexpr int NDMA = STAGE / 64;          // 1 KB direct loads per stage: 40
constexpr int AQ = AOPER / 64;            // the first 30 of them fill A
constexpr int DMA_W = NDMA / 4;          // per wave of the copying group: 10
constexpr int KSPLIT_MAX = 16384;
}  // namespace go


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
  __shared__ uint4 smem[STAGES * STAGE];  // 160 KB
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
  const int m0 = tm * BMT, n0 = tn * BN;
  const int ksteps = Kp / BK;
  const int t_begin = sp * steps_per_split;
  const int t_end = t_begin + steps_per_split < ksteps ? t_begin + steps_per_split : ksteps;
  const int nsteps = t_end > t_begin ? t_end - t_begin : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches and buffer descriptors
  const int lr = lane & 31, lg = lane >> 5;
  // Two groups of four wavefronts, one of each per SIMD (wave w runs on SIMD
  // w % 4), alternate between reading a K step's slice fragments from LDS
  // into registers and running that step's MFMAs from registers, one
  // workgroup barrier per phase.  The tile's rows are five blocks of 32 and
  // one of 16 (rows 160-175).  Of column block k % 2, the wave of group 0 on
  // SIMD k takes row blocks 3 (k / 2) and 3 (k / 2) + 1 (30 MFMAs per step);
  // of group 1, the wave on SIMD 0 or 1 (role 1) takes the slice pairs of
  // levels 2-4 of row block 2 (12 MFMAs), the wave on SIMD 2 or 3 (role 2) the
  // 16-row block (9) and the pairs of levels 0-1 of row block 2 (3), which it
  // hands to role 1 through LDS at the end.  While group 0 multiplies, group
  // 1 reads its fragments and issues the copies, and while group 1
  // multiplies, group 0 reads: each SIMD's matrix core runs 42 MFMAs per step
  // with no phase in which it waits on LDS.
  //
  // The 16-row block: A's rows 0-15 are the tile's rows 160-175 of slice s and
  // its rows 16-31 the same rows of slice s + 1, so one MFMA against slice t
  // of B adds pair (s, t) to rows 0-15 (accumulator elements 0-7) and pair
  // (s + 1, t) to rows 16-31 (elements 8-15) of accumulator set s + t: its
  // lower half sums level s + t, its upper half level s + t + 1.  With s in
  // {0, 2, 4} and s + t <= 4, nine MFMAs cover the 15 kept pairs; level d is
  // the lower half of set d plus the upper half of set d - 1 (set 4's upper
  // half, level 5, is never read).
  const int grp = wave >> 2, sk = wave & 3;
  const int role = grp == 0 ? 0 : 1 + (sk >> 1);
  const int wc = (sk & 1) * 32;
  const int nb = grp == 0 ? 2 : 1;                                     // row blocks this wave stores
  const int wr0 = grp == 0 ? (sk >> 1) * 96 : (role == 1 ? 64 : 160);  // its first row
  // The epilogue's scale exponents, loaded now so their latency hides under
  // the K loop: column wc + lr, and rows wr0 + lr and wr0 + 32 + lr (lane
  // l's value serves the other lanes of its row block through a shuffle).
  const int gn = n0 + wc + lr;
  const int gnc = gn < N ? gn : N - 1;
  const int fe = Be[gnc];
  // A one-split item rounds its own result: C (every item one split), or,
  // with C null and a bias, the fp32 values in the partial buffer that a
  // consumer of the partials reads in their place.
  const bool direct = s1 == 1 && s2 == 1 && C != nullptr;
  const bool own32 = direct || (C == nullptr && bias != nullptr && (first ? s1 : s2) == 1);
  const float bias_v = (own32 && bias != nullptr) ? bias[gnc] : 0.f;
  int ae_row[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int gm = m0 + wr0 + 32 * b + lr;
    ae_row[b] = b < nb ? Ae[gm < M ? gm : M - 1] : 0;
  }

  // Copies (group 1 only): instruction q = 10 (wave % 4) + j fills 1 KB = 32
  // rows of one slice plane: q < 30 row block q%6 of A plane q/6, else row
  // block (q-30)%2 of B plane (q-30)/2; lane l fetches row 32 (block) + l/2
  // at the logical chunk the swizzle stores at position l%2.  Rows past M or
  // N get an offset past the buffer, which reads as zero.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(Ap), 0, static_cast<uint32_t>(S * static_cast<int64_t>(M) * Kp), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(Bp), 0, static_cast<uint32_t>(S * static_cast<int64_t>(N) * Kp), 0x00020000);
  // Lane l's part of every copy's offset: row l/2 of the 32-row block, at the
  // chunk the swizzle stores at position l%2 (rows 32 blk + l/2 share bit 3
  // with l/2, so the swizzle is the same for every block).  The rest of an
  // offset is uniform and formed at issue, so the ten copies share one VGPR.
  const uint32_t lane_off = static_cast<uint32_t>((lane >> 1) * BK + 16 * ((lane & 1) ^ ((lane >> 4) & 1)));
  const uint32_t a_step = static_cast<uint32_t>(M) * BK, b_step = static_cast<uint32_t>(N) * BK;  // bytes per K step
  auto dma = [&](int t, int st) {
#pragma unroll
    for (int j = 0; j < DMA_W; ++j) {
      const int q = sk * DMA_W + j;
      const bool a_op = q < AQ;
      const int plane = a_op ? q / 6 : (q - AQ) / 2;
      const int blk = a_op ? q % 6 : (q - AQ) % 2;
      const int rows = a_op ? M : N;
      const int row0 = (a_op ? m0 : n0) + 32 * blk;
      // rows of this block that exist (A rows past the tile's 176 read zero)
      int valid = rows - row0;
      if (a_op && BMT - 32 * blk < valid) valid = BMT - 32 * blk;
      // slice layout [plane][K step][row][32 bytes]: one instruction reads 1 KB in a row
      const uint32_t sbase = static_cast<uint32_t>((static_cast<int64_t>(plane) * (Kp / BK) * rows + row0) * BK) +
                             static_cast<uint32_t>(t) * (a_op ? a_step : b_step);
      const uint32_t off = (lane >> 1) < valid ? sbase + lane_off : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_op ? ra : rb, (lds_ptr_t)(smem + st * STAGE + q * 64), 16, off, 0,
                                               0, 0);
    }
  };
  // s_waitcnt vmcnt(n) for n = 0, 10 or 20 of this wave's copies still in flight
  auto wait_copies = [&](int n) {
    if (n >= 20)
      __builtin_amdgcn_s_waitcnt(0x4F74);  // vmcnt(20): low bits 4, high bits 1
    else if (n >= 10)
      __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };

  typedef int v4i __attribute__((ext_vector_type(4)));
  typedef int v16i __attribute__((ext_vector_type(16)));
  v16i acc[2][S];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int d = 0; d < S; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[b][d][e] = 0;
  v4i fa[2][S], fb[S];
  // LDS chunk bases of this lane's A reads (+ p APLANE for slice p): role 0
  // rows wr0 + lr and wr0 + 32 + lr; role 1 row 64 + lr; role 2 the 16-row
  // block's dual rows (lanes 16-31 of a half one slice further on: plane 5,
  // read for the never-used upper half of set 4, is the start of the B
  // planes) and row block 2's row 64 + lr.
  const int abase0 = role == 2 ? go_swz(160 + (lr & 15), lg) + ((lr >> 4) & 1) * APLANE : go_swz(wr0 + lr, lg);
  const int abase1 = role == 2 ? go_swz(64 + lr, lg) : abase0 + 64;
  // The role is a compile-time constant of each K loop below (one loop per
  // role), so a loop holds only that role's fragments and accumulators.
  auto read_step = [&](int st, auto role_c) {
    constexpr int R = decltype(role_c)::value;
    const uint4* sa = smem + st * STAGE;
    const uint4* sb = sa + AOPER;
#pragma unroll
    for (int p = 0; p < S; ++p) fb[p] = __builtin_bit_cast(v4i, sb[p * BPLANE + go_swz(wc + lr, lg)]);
    if constexpr (R != 2) {
#pragma unroll
      for (int p = 0; p < S; ++p) fa[0][p] = __builtin_bit_cast(v4i, sa[abase0 + p * APLANE]);
      if constexpr (R == 0) {
#pragma unroll
        for (int p = 0; p < S; ++p) fa[1][p] = __builtin_bit_cast(v4i, sa[abase1 + p * APLANE]);
      }
    } else {
      // the 16-row block as slice pairs (0, 1), (2, 3), (4, -), then row
      // block 2's slices 0 and 1
#pragma unroll
      for (int j = 0; j < 3; ++j) fa[0][j] = __builtin_bit_cast(v4i, sa[abase0 + 2 * j * APLANE]);
      fa[0][3] = __builtin_bit_cast(v4i, sa[abase1]);
      fa[0][4] = __builtin_bit_cast(v4i, sa[abase1 + APLANE]);
    }
    // the reads complete inside the phase: the asm takes every fragment
#pragma unroll
    for (int p = 0; p < S; ++p) {
      asm volatile("" : "+v"(fb[p]), "+v"(fa[0][p]));
      if constexpr (R == 0) asm volatile("" : "+v"(fa[1][p]));
    }
  };
  // pair (s, t) accumulates in level s + t; the order keeps two MFMAs on one
  // accumulator at least two instructions apart (levels 4 3 2 4 3 2 4 3 2 4 3
  // 1 4 0 1)
  auto mfma_block = [&](v16i (&a)[S], const v4i (&A)[S]) {
#define GO_MFMA(s_, t_) a[(s_) + (t_)] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[s_], fb[t_], a[(s_) + (t_)], 0, 0, 0);
    GO_MFMA(4, 0) GO_MFMA(3, 0) GO_MFMA(2, 0) GO_MFMA(3, 1) GO_MFMA(2, 1) GO_MFMA(1, 1) GO_MFMA(2, 2)
    GO_MFMA(1, 2) GO_MFMA(0, 2) GO_MFMA(1, 3) GO_MFMA(0, 3) GO_MFMA(1, 0) GO_MFMA(0, 4) GO_MFMA(0, 0)
    GO_MFMA(0, 1)
#undef GO_MFMA
  };
  // role 1: row block 2's pairs of levels 2-4 (levels 4 3 2 4 3 2 4 3 2 4 3 4)
  auto mfma_upper = [&](v16i (&a)[S], const v4i (&A)[S]) {
#define GO_MFMA(s_, t_) a[(s_) + (t_)] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[s_], fb[t_], a[(s_) + (t_)], 0, 0, 0);
    GO_MFMA(4, 0) GO_MFMA(3, 0) GO_MFMA(2, 0) GO_MFMA(3, 1) GO_MFMA(2, 1) GO_MFMA(1, 1) GO_MFMA(2, 2)
    GO_MFMA(1, 2) GO_MFMA(0, 2) GO_MFMA(1, 3) GO_MFMA(0, 3) GO_MFMA(0, 4)
#undef GO_MFMA
  };
  // role 2: the 16-row block's sets (pair (2j, t) and (2j+1, t) into set
  // 2j + t of a) and row block 2's pairs (0,0), (1,0), (0,1) into levels of b
  // (sets 0 2 4 1 3 b0 2 4 b1 3 b1 4)
  auto mfma_tail = [&](v16i (&a)[S], v16i (&b)[S], const v4i (&A)[S]) {
#define GO_T(j_, t_) a[2 * (j_) + (t_)] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[j_], fb[t_], a[2 * (j_) + (t_)], 0, 0, 0);
#define GO_B(s_, t_) b[(s_) + (t_)] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[3 + (s_)], fb[t_], b[(s_) + (t_)], 0, 0, 0);
    GO_T(0, 0) GO_T(1, 0) GO_T(2, 0) GO_T(0, 1) GO_T(1, 1) GO_B(0, 0) GO_T(0, 2) GO_T(1, 2) GO_B(1, 0) GO_T(0, 3)
    GO_B(0, 1) GO_T(0, 4)
#undef GO_T
#undef GO_B
  };
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    go_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Phases: group 0 reads step i in phase 2i and multiplies in 2i+1; group 1
  // one phase later (an extra barrier first; group 0 takes one after its last
  // MFMAs, so both execute the same number).  Group 1 issues the copies of
  // step i+3 (into the stage of step i-1, which both groups finished reading
  // by the barrier opening phase 2i) at the start of its read phase 2i+1,
  // and at its end waits until only the copies of steps i+2 and i+3 are in
  // flight: step i+1 has landed before the barrier ahead of group 0's read of
  // it.  Loads complete in issue order.
  static_assert(STAGES == 4 && DMA_W * 4 == NDMA, "the copy schedule and wait counts below");
  if (grp == 1) {
#pragma unroll
    for (int p = 0; p < 3; ++p)
      if (p < nsteps) dma(t_begin + p, p);
    wait_copies(10 * ((nsteps > 1) + (nsteps > 2)));  // step 0 has landed
  }
  go_barrier();
  if (grp == 1) phase_barrier();
  auto k_loop = [&](auto role_c) {
    constexpr int R = decltype(role_c)::value;
    for (int i = 0; i < nsteps; ++i) {
      if (R != 0 && i + 3 < nsteps) dma(t_begin + i + 3, (i + 3) % STAGES);
      read_step(i % STAGES, role_c);
      if (R != 0) wait_copies(10 * ((i + 2 < nsteps) + (i + 3 < nsteps)));
      phase_barrier();
      if constexpr (R == 0) {
        mfma_block(acc[0], fa[0]);
        mfma_block(acc[1], fa[1]);
      } else if constexpr (R == 1) {
        mfma_upper(acc[0], fa[0]);
      } else {
        mfma_tail(acc[0], acc[1], fa[0]);
      }
      // the MFMAs complete inside the phase: the asm takes every accumulator
#pragma unroll
      for (int d = 0; d < S; ++d) {
        if (R != 1 || d >= 2) asm volatile("" : "+v"(acc[0][d]));
        if (R == 0 || (R == 2 && d < 2)) asm volatile("" : "+v"(acc[1][d]));
      }
      phase_barrier();
    }
  };
  if (role == 0)
    k_loop(std::integral_constant<int, 0>{});
  else if (role == 1)
    k_loop(std::integral_constant<int, 1>{});
  else
    k_loop(std::integral_constant<int, 2>{});
  if (grp == 0) phase_barrier();

  // Row block 2's levels 0 and 1 go from the role-2 wave to the role-1 wave
  // of the same column block through LDS, free now (every wave is past its
  // last read); the role-2 wave turns its 16-row block's sets into levels.
  int32_t* const xch = reinterpret_cast<int32_t*>(smem) + (sk & 1) * (2 * 16 * 64);
  if (role == 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) xch[(d * 16 + e) * 64 + lane] = acc[1][d][e];
#pragma unroll
    for (int d = S - 1; d >= 1; --d)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[0][d][e] += acc[0][d - 1][e + 8];
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS writes are done
  go_barrier();
  if (role == 1) {
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[0][d][e] = xch[(d * 16 + e) * 64 + lane];
  }

  // Epilogue, per row block of the wave: lane holds column wc + lr, rows
  // wr + 8 (e/4) + 4 lg + e%4 of each level (the 16-row block: e < 8 only).
  // C null: fp64 partials for a consumer that sums them itself (any split
  // count); a one-split item given a bias stores float(value + bias) instead,
  // packed at the start of the row's first partial row (row r's columns at
  // float index c of the doubles r N .. r N + N - 1 of slot 0, which no item
  // of a multi-split group writes).
  const bool paired = (N & 1) == 0 && (reinterpret_cast<uintptr_t>(C) & 7) == 0;
  const double bv = static_cast<double>(bias_v);
  float* const own = direct ? C : reinterpret_cast<float*>(part);
  const size_t own_ld = direct ? static_cast<size_t>(N) : 2 * static_cast<size_t>(N);  // floats per row
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b >= nb) break;  // uniform; b stays a constant so acc stays in registers
    const int wr = wr0 + 32 * b;
    const int ne = role == 2 ? 8 : 16;  // uniform
    const v16i (&ac)[S] = acc[b];
    // the exponents of this lane's 16 rows, from the lanes that loaded them
    int aex[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) aex[e] = __shfl(ae_row[b], 8 * (e >> 2) + 4 * lg + (e & 3), 32);
    // sum_d acc_d 2^-7(d+2), the smallest level first, times 2^(row + column
    // exponent): every product by a power of two is exact, so each fma
    // rounds as the addition of that term would
    auto value = [&](int e) -> double {
      double x = static_cast<double>(ac[4][e]) * 0x1p-42;
      x = fma(static_cast<double>(ac[3][e]), 0x1p-35, x);
      x = fma(static_cast<double>(ac[2][e]), 0x1p-28, x);
      x = fma(static_cast<double>(ac[1][e]), 0x1p-21, x);
      x = fma(static_cast<double>(ac[0][e]), 0x1p-14, x);
      return (fe == kSliceNonFinite || aex[e] == kSliceNonFinite) ? __builtin_nan("") : ldexp(x, aex[e] + fe);
    };
    if (paired) {
      // Rows e and e+1 are adjacent: lanes 2c and 2c+1 swap one value, and each
      // stores two adjacent columns of its row (16-byte partials, 8-byte C).
      const bool odd = lr & 1;
      const double bv_pair = xor_lane<1>(bv);  // the partner column's bias
      const int col = odd ? gn - 1 : gn;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        if (e >= ne) continue;  // uniform; e stays a constant
        const int gm = m0 + wr + 8 * (e >> 2) + 4 * lg + (e & 3);
        const double v0 = value(e), v1 = value(e + 1);
        const double recv = xor_lane<1>(odd ? v0 : v1);
        const int row = odd ? gm + 1 : gm;
        if (row < M && col < N) {
          const double lo = odd ? recv : v0, hi = odd ? v1 : recv;
          if (own32) {
            const double b_lo = odd ? bv_pair : bv, b_hi = odd ? bv : bv_pair;  // columns col, col + 1
            *reinterpret_cast<float2*>(own + static_cast<size_t>(row) * own_ld + col) =
                make_float2(static_cast<float>(lo + b_lo), static_cast<float>(hi + b_hi));
          } else {
            *reinterpret_cast<double2*>(part + (static_cast<size_t>(sp) * M + row) * N + col) = make_double2(lo, hi);
          }
        }
      }
      continue;
    }
    if (gn >= N) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (e >= ne) continue;  // uniform; e stays a constant
      const int gm = m0 + wr + 8 * (e >> 2) + 4 * lg + (e & 3);
      if (gm >= M) continue;
      const double v = value(e);
      if (own32)
        own[static_cast<size_t>(gm) * own_ld + gn] = static_cast<float>(v + bv);
      else
        part[(static_cast<size_t>(sp) * M + gm) * N + gn] = v;
    }
  }
}

// Split plan from (N, K) and the device alone, so a row's result never
// depends on M.  One workgroup fits a CU (160 KB of LDS).  The cost model
// was measured on MI355X with a one-barrier-per-step form of this kernel: a
// K step took ~1.1 us (~0.85 us in the two-group form), a round of
// workgroups adds ~5 steps of fixed cost (first copies in flight,
// epilogue), and each split adds an fp64 partial of the row tile that is
// written and read back once (192 N 16 bytes at ~4.5 TB/s, i.e. N / 1600
// steps per slot; costed with 192-row tiles and kept for the 176-row ones,
// so the plans, and with them the results, did not change).  Plans: every N tile in s splits
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
  const int tiles_m = (M + go::BMT - 1) / go::BMT, tiles_n = (N + go::BN - 1) / go::BN;
  const int64_t work = static_cast<int64_t>(tiles_m) * (static_cast<int64_t>(g.n1) * g.s1 +
                                                        static_cast<int64_t>(tiles_n - g.n1) * g.s2);
  if (work >= (int64_t(1) << 31) - 256) return hipErrorInvalidValue;
  const unsigned blocks = static_cast<unsigned>((work + 255) / 256 * 256);
  LaunchScope scope_(kCntGemmF32, s);
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(blocks), dim3(go::NT), 0, s, M, N, kp, Ap, Ae, Bp, Be, bias, C, part,
                     g.s1, g.s2, g.n1, sps1, sps2, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t gemm_f32_sliced(int M, int N, int K, const void* As, const void* Bs, const float* bias, double* part,
                           hipStream_t s) {
  if (bias == nullptr) return hipErrorInvalidValue;  // one-split groups store finished values
  if (M == 0) return hipSuccess;
  const int kp = go_kp(K);
  const int8_t* Ap = static_cast<const int8_t*>(As);
  const int32_t* Ae = reinterpret_cast<const int32_t*>(Ap + al256(static_cast<size_t>(go::S) * M * kp));
  const int8_t* Bp = static_cast<const int8_t*>(Bs);
  const int32_t* Be = reinterpret_cast<const int32_t*>(Bp + al256(static_cast<size_t>(go::S) * N * kp));
  return launch_gemm_f32(M, N, kp, Ap, Ae, Bp, Be, bias, nullptr, part, go_split(N, K), s);
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
