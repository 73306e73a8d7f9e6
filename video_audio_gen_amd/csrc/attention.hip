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
#include "mx8.h"

namespace dit {

// ============================================================================ bf16, MFMA
// Workgroup = one (document, head, 256-query tile); eight wavefronts of 32
// queries, two per SIMD.  Scores are computed transposed, S^T = K Q^T, on
// v_mfma_f32_32x32x16_bf16, so each lane owns one query (per 32-query block)
// and 16 of its keys per 32-key block: the row max and row sum stay in the
// lane plus its partner lane l^32.
//
// The probabilities, rounded to bf16, are already the B operand of the next
// MFMA, O^T = V^T P^T, if the contraction runs over keys in the order the
// score accumulator holds them (within each 16-key group, keys 4g'..4g'+3 then
// 8+4g'..8+4g'+3 for lane half g').  V stays key-major in LDS; its transposed
// fragments come from ds_read_b64_tr_b16, which hands each lane 4 consecutive
// keys of one dimension.
//
// K and V tiles of 64 keys move HBM -> LDS by direct buffer loads, double
// buffered: while tile t's probabilities are formed, the scores of tile t+1
// are computed from LDS, and the loads of K(t+2) and V(t+1) are in flight.
// Reads past the document end return zero and those keys are masked.  The
// accumulator rescale of the online softmax is skipped (wavefront-uniform
// branch) for tiles where no row's max grows, which after the first few tiles
// is most of them.  The max is always exact, so each row's largest probability
// is 1 and is exact in bf16.
namespace ab {
constexpr int HD = 128;                    // head dim
constexpr int KT = 64;                     // keys per tile
#ifndef DIT_ATTN_QB
#define DIT_ATTN_QB 1
#endif
constexpr int QB = DIT_ATTN_QB;            // 32-query blocks per wavefront
constexpr int QW = 32 * QB;                // queries per wavefront
constexpr int NW = 8 / QB;                 // wavefronts per workgroup
constexpr int QT = QW * NW;                // queries per workgroup
constexpr int NT = NW * 64;
constexpr int TILE = KT * HD / 8;          // 16-byte chunks of one K or V tile
constexpr int DMA = TILE / 64 / NW;        // direct loads per wavefront per tile
}  // namespace ab

// K rows: chunk c of key r at r*16 + (c ^ (r % 16)), conflict-free for the
// 16-lane passes of ds_read_b128 that fetch 16 keys at one chunk.
__device__ __forceinline__ int ab_kpos(int key, int cc) { return key * 16 + (cc ^ (key & 15)); }
// V rows: the transposing read fetches 4 consecutive keys x 32 dims per 32
// lanes; XOR-ing the chunk's block-of-4 index with key % 4 spreads the four keys
// over all 64 banks.
__device__ __forceinline__ int ab_vswz(int key) { return ((key & 3) << 2) | ((key >> 2) & 3); }
__device__ __forceinline__ int ab_vpos(int key, int cc) { return key * 16 + (cc ^ ab_vswz(key)); }

typedef __attribute__((address_space(3))) void* ab_lds_t;
typedef __bf16 ab_bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 ab_bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) ab_bf16x4* ab_lds4_t;

__device__ __forceinline__ uint32_t ab_pack(float lo, float hi) {
  const ab_bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // v_cvt_pk_bf16_f32, RNE
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float ab_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float ab_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(ab::NT, 1) void attention_bf16_kernel(int N, int H, int n_docs, int qtiles,
                                                                      int work, const int32_t* __restrict__ cu,
                                                                      const bf16_t* __restrict__ q,
                                                                      const bf16_t* __restrict__ k,
                                                                      const bf16_t* __restrict__ v,
                                                                      bf16_t* __restrict__ o,
                                                                      float scale_log2, uint8_t* __restrict__ o8,
                                                                      uint8_t* __restrict__ o8s) {
  using namespace ab;
  __shared__ uint4 smem[4 * TILE];  // K[2] then V[2]: 64 KB
  uint4* const Kb = smem;
  uint4* const Vb = smem + 2 * TILE;

  // Workgroups go to the 8 XCDs round-robin.  Within each run of 256
  // consecutive workgroups (one per CU), XCD x takes 32 consecutive
  // (document, head, query tile) items, so the CUs sharing an L2 stream the
  // same head's keys at the same time, and every XCD sees every document.
  const int w = (blockIdx.x / 256) * 256 + (blockIdx.x % 8) * 32 + (blockIdx.x / 8) % 32;
  if (w >= work) return;
  const int qt = w % qtiles, h = (w / qtiles) % H, d = w / (qtiles * H);
  const int s0 = cu[d], len = cu[d + 1] - s0;
  const int q0 = qt * QT;
  if (q0 >= len) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const size_t base = (static_cast<size_t>(h) * N + s0) * HD;  // this head's document start

  // Q fragments (B operand of S^T): lane holds query lr of block qb, dims
  // 16c + 8lg .. +7.  Rows past the document end repeat its last row.
  bf16x8_t qf[QB][HD / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    int qi = q0 + wave * QW + qb * 32 + lr;
    qi = qi < len ? qi : len - 1;
    const bf16_t* qp = q + base + static_cast<size_t>(qi) * HD + 8 * lg;
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) qf[qb][c] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + 16 * c));
  }

  // Direct loads: instruction j of this wavefront fills LDS chunks
  // (4 wave + j) * 64 + lane = key * 16 + position; the lane fetches the
  // logical chunk that the swizzle stores at that position.
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(k + base), 0, len * HD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(v + base), 0, len * HD * 2, 0x00020000);
  uint32_t vok[DMA], vov[DMA];
#pragma unroll
  for (int j = 0; j < DMA; ++j) {
    const int ch = (wave * DMA + j) * 64 + lane, key = ch >> 4, pos = ch & 15;
    vok[j] = static_cast<uint32_t>(key * HD + (pos ^ (key & 15)) * 8) * 2u;
    vov[j] = static_cast<uint32_t>(key * HD + (pos ^ ab_vswz(key)) * 8) * 2u;
  }
  auto dma_k = [&](int t, int buf) {
#pragma unroll
    for (int j = 0; j < DMA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (ab_lds_t)(Kb + buf * TILE + (wave * DMA + j) * 64), 16,
                                               vok[j] + static_cast<uint32_t>(t * KT * HD * 2), 0, 0, 0);
  };
  auto dma_v = [&](int t, int buf) {
#pragma unroll
    for (int j = 0; j < DMA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (ab_lds_t)(Vb + buf * TILE + (wave * DMA + j) * 64), 16,
                                               vov[j] + static_cast<uint32_t>(t * KT * HD * 2), 0, 0, 0);
  };

  // Per-lane LDS offsets (bytes) of the K fragments (key 32kb + lr, chunk
  // 2c + lg) and of the transposing V reads (4 keys from 16g + 8r + 4(lane/32)
  // at dims 32i + 16((lane/16)%2) + 4(lane%4)).
  // The V swizzle of key 16g + 8r + vkey0 does not depend on g, so the lane
  // part of each (r, i) read offset is fixed and g adds a constant.
  const int vG = lane >> 4, ve = (lane >> 2) & 3, vc4 = lane & 3;
  const int vkey0 = 4 * (vG >> 1) + ve;
  const int vcc = 2 * (vG & 1) + (vc4 >> 1);
  int voff_lane[2][HD / 32];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < HD / 32; ++i) voff_lane[r][i] = ab_vpos(8 * r + vkey0, 4 * i + vcc) * 16 + 8 * (vc4 & 1);
  int koff_lane[HD / 16];
#pragma unroll
  for (int c = 0; c < HD / 16; ++c) koff_lane[c] = ab_kpos(lr, 2 * c + lg) * 16;

  f32x16_t acc[QB][HD / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < HD / 32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[qb][i][e] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_run[qb] = -INFINITY, l_run[qb] = 0.f;

  auto scores = [&](f32x16_t (&s)[QB][2], const uint4* kt) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[qb][kb][e] = 0.f;
#pragma unroll
    for (int c = 0; c < HD / 16; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // key 32kb + lr has the same swizzle as key lr
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const char*>(kt) + kb * 32 * 256 + koff_lane[c]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][c], s[qb][kb], 0, 0, 0);
      }
  };

  // One key tile: probabilities of tile t from its scores s, then the scores
  // of tile t+1 into sn (independent MFMAs the exp work can hide behind), then
  // O += V(t)^T P^T.
  const int n_kt = (len + KT - 1) / KT;
  auto step = [&](int t, int buf, f32x16_t(&s)[QB][2], f32x16_t(&sn)[QB][2]) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wavefront's loads of K(t+1), V(t) are done
    __syncthreads();                     // ... and everyone's; tile t-1's buffers are free
    if (t + 2 < n_kt) dma_k(t + 2, buf);
    if (t + 1 < n_kt) dma_v(t + 1, buf ^ 1);

    // Keys past the document end (last tile only).  Lane holds keys
    // 32kb + 8(e/4) + 4lg + e%4 of the tile.
    const int k0 = t * KT;
    if (k0 + KT > len) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (k0 + kb * 32 + 8 * (e >> 2) + 4 * lg + (e & 3) >= len) s[qb][kb][e] = -INFINITY;
    }
    float mt[QB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, s[qb][kb][e]);
      mt[qb] = ab_pair_max(m);
      grow |= mt[qb] > m_run[qb];
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = fmaxf(m_run[qb], mt[qb]);
        const float alpha = __builtin_amdgcn_exp2f((m_run[qb] - m_new) * scale_log2);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < HD / 32; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[qb][i][e] *= alpha;
      }
    }
    // P = 2^(s c - m c), rounded to bf16 in the B-operand layout; the row sum
    // adds the rounded values (v_dot2 with 1.0), so the weights the output is
    // normalised by are exactly the ones it was summed with.
    bf16x8_t pf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mc = m_run[qb] * scale_log2;
      float ps = 0.f;
      const ab_bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][g >> 1][8 * (g & 1) + j], scale_log2, -mc));
        }
        const uint4 pw = make_uint4(ab_pack(p[0], p[1]), ab_pack(p[2], p[3]), ab_pack(p[4], p[5]), ab_pack(p[6], p[7]));
        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(ab_bf16x2, pw.x), one2, ps, false);
        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(ab_bf16x2, pw.y), one2, ps, false);
        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(ab_bf16x2, pw.z), one2, ps, false);
        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(ab_bf16x2, pw.w), one2, ps, false);
        pf[qb][g] = __builtin_bit_cast(bf16x8_t, pw);
      }
      l_run[qb] += ps;
    }
    if (t + 1 < n_kt) scores(sn, Kb + (buf ^ 1) * TILE);
    // O^T += V^T P^T.
    const char* vt = reinterpret_cast<const char*>(Vb + buf * TILE);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < HD / 32; ++i) {
        ab_bf16x4 half_[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          half_[r] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ab_lds4_t)(vt + 16 * g * 256 + voff_lane[r][i]));
        }
        const bf16x8_t vf = __builtin_shufflevector(half_[0], half_[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][g], acc[qb][i], 0, 0, 0);
      }
  };

  dma_k(0, 0);
  if (n_kt > 1) dma_k(1, 1);
  dma_v(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  f32x16_t sa[QB][2], sb[QB][2];
  scores(sa, Kb);
  for (int t = 0; t < n_kt; t += 2) {
    step(t, 0, sa, sb);
    if (t + 1 < n_kt) step(t + 1, 1, sb, sa);
  }

  // Normalise; lane writes dims 32i + 8(e/4) + 4lg .. +3 of its query as 8 bytes.
  const int D = H * HD;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.0f / ab_pair_sum(l_run[qb]);
    const int qi = q0 + wave * QW + qb * 32 + lr;
    if (qi < len && o8 != nullptr) {
      // MXFP8 output (codes [N][D], scales [N][D/32]): the bf16 values a
      // stored o would hold, quantized per 32 dims; the lane holds 16 of the
      // block's values and its partner lane l^32 the other 16.
      uint8_t* op = o8 + static_cast<size_t>(s0 + qi) * D + h * HD + 4 * lg;
#pragma unroll
      for (int i = 0; i < HD / 32; ++i) {
        float f[16];
        float am = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          f[e] = static_cast<float>(static_cast<__bf16>(acc[qb][i][e] * inv));  // as ab_pack rounds
          am = nan_max(am, fabsf(f[e]));
        }
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(am), __float_as_uint(am), false, false);
        am = nan_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
        int div;
        const uint32_t sb = mx_scale(am, &div);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          *reinterpret_cast<uint32_t*>(op + i * 32 + 8 * e4) =
              mx_code4(f[4 * e4], f[4 * e4 + 1], f[4 * e4 + 2], f[4 * e4 + 3], sb, div);
        }
        if (lg == 0) o8s[static_cast<size_t>(s0 + qi) * (D / 32) + (h * HD) / 32 + i] = static_cast<uint8_t>(sb);
      }
    } else if (qi < len) {
      bf16_t* op = o + static_cast<size_t>(s0 + qi) * D + h * HD + 4 * lg;
#pragma unroll
      for (int i = 0; i < HD / 32; ++i)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const uint2 wv = make_uint2(ab_pack(acc[qb][i][4 * e4] * inv, acc[qb][i][4 * e4 + 1] * inv),
                                      ab_pack(acc[qb][i][4 * e4 + 2] * inv, acc[qb][i][4 * e4 + 3] * inv));
          *reinterpret_cast<uint2*>(op + i * 32 + 8 * e4) = wv;
        }
    }
  }
}

// ============================================================================ f32 stream
// Scores, softmax and the weighted sum in fp64 with one rounding of the output
// to fp32: the fp32 stream is held to rel 1e-5 / abs 1e-6 after 24 blocks,
// which fp32 dot products over the head dim do not meet.  The products run on
// v_mfma_f64_16x16x4_f64 (fp32 operands are exact in fp64).
//
// Workgroup = one (document, head, 16-query tile); its four wavefronts split
// every 64-key K/V tile (fp32 in LDS, rows padded so the operand reads are
// bank-conflict free) into 16-key blocks, one each, and keep their own online
// softmax; the four partial results are merged through LDS at the end.
// Scores are formed transposed, S^T = K Q^T: lane l then holds 4 keys
// (4i + l/16 of the block) of query l%16, which is exactly the B operand
// layout of O^T += V^T P^T, so the probabilities never leave registers; the
// row max and sum reduce over i in the lane and over the lanes l%16 + 16g.
namespace af {
constexpr int QT = 16, NW = 4, KT = 16 * NW, NT = NW * 64;
}

template <int HD>
__global__ __launch_bounds__(af::NT) void attention_f32_kernel(int N, int H, const int32_t* __restrict__ cu,
                                                              const float* __restrict__ q,
                                                              const float* __restrict__ k,
                                                              const float* __restrict__ v,
                                                              float* __restrict__ o, double scale) {
  using namespace af;
  constexpr int KS = HD + 4;    // Q/K row stride (floats): 16 rows x 4 columns hit 64 distinct banks
  constexpr int VS = HD + 16;   // V row stride: 4 rows x 16 columns hit 64 distinct banks
  constexpr int NDB = HD / 16;  // 16-dim output blocks
  constexpr int F4 = HD / 4;    // float4 per row
  constexpr int KV_FLOATS = KT * (KS + VS);
  static_assert(KV_FLOATS >= (NW * QT * (HD + 3) + QT) * 2, "the merge reuses the K/V tile space");
  __shared__ float Qs[QT * KS];
  __shared__ __align__(16) float KVs[KV_FLOATS];
  float* Ks = KVs;
  float* Vs = KVs + KT * KS;
  const int qt = blockIdx.x, h = blockIdx.y, d = blockIdx.z;
  const int s0 = cu[d], len = cu[d + 1] - s0;
  const int q0 = qt * QT;
  if (q0 >= len) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const size_t base = (static_cast<size_t>(h) * N + s0) * HD;

  // K/V tiles pass through registers: the loads of tile t+1 are issued before
  // tile t's MFMAs and land in LDS after them.  Thread tid holds the float4s
  // tid + NT j of the tile (row r = i / F4, column chunk i % F4).
  constexpr int PT = KT * F4 / NT;  // float4 per thread per operand
  static_assert(KT * F4 % NT == 0, "whole float4s per thread");
  float4 kreg[PT], vreg[PT];
  auto load_kv = [&](int k0) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int i = tid + NT * j, r = i / F4, c = i % F4;
      kreg[j] = vreg[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k0 + r < len) {
        const size_t off = base + static_cast<size_t>(k0 + r) * HD + 4 * c;
        kreg[j] = *reinterpret_cast<const float4*>(k + off);
        vreg[j] = *reinterpret_cast<const float4*>(v + off);
      }
    }
  };
  auto store_kv = [&]() {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int i = tid + NT * j, r = i / F4, c = i % F4;
      *reinterpret_cast<float4*>(&Ks[r * KS + 4 * c]) = kreg[j];
      *reinterpret_cast<float4*>(&Vs[r * VS + 4 * c]) = vreg[j];
    }
  };
  load_kv(0);
  for (int i = tid; i < QT * F4; i += NT) {
    const int r = i / F4, c = i % F4;
    const float4 t = q0 + r < len ? *reinterpret_cast<const float4*>(q + base + static_cast<size_t>(q0 + r) * HD + 4 * c)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(&Qs[r * KS + 4 * c]) = t;
  }
  store_kv();
  __syncthreads();
  // Q^T operand: lane holds Q[query r16][dim 4 ks + g]
  double qf[HD / 4];
#pragma unroll
  for (int ks = 0; ks < HD / 4; ++ks) qf[ks] = static_cast<double>(Qs[r16 * KS + 4 * ks + g]);

  f64x4_t acc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) acc[b] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  double m_run = -INFINITY, l_run = 0.0;

  const int n_kt = (len + KT - 1) / KT;
  for (int t = 0; t < n_kt; ++t) {
    const int k0 = t * KT;
    if (t > 0) {
      __syncthreads();  // previous tile consumed
      store_kv();
      __syncthreads();
    }
    if (t + 1 < n_kt) load_kv(k0 + KT);
    const int kb0 = wave * 16;  // this wavefront's key block
    if (k0 + kb0 >= len) continue;
    // S^T block: lane holds keys kb0 + 4i + g of query r16
    f64x4_t sb = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < HD / 4; ++ks)
      sb = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(Ks[(kb0 + r16) * KS + 4 * ks + g]), qf[ks], sb, 0,
                                                0, 0);
    double mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double sc = k0 + kb0 + 4 * i + g < len ? sb[i] * scale : -INFINITY;
      sb[i] = sc;
      mt = fmax(mt, sc);
    }
    mt = fmax(mt, xor_lane<16>(mt));
    mt = fmax(mt, xor_lane<32>(mt));
    const double m_new = fmax(m_run, mt);
    const double alpha = exp(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][i] *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double p = exp(sb[i] - m_new);  // exp(-inf) = 0 for keys past the end
      sb[i] = p;
      l_run += p;
    }
    // O^T += V^T P^T over the block's keys 4ks + g: B operand = p of slot ks
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int b = 0; b < NDB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(Vs[(kb0 + 4 * ks + g) * VS + b * 16 + r16]),
                                                      sb[ks], acc[b], 0, 0, 0);
  }

  // Merge the four wavefronts: m, l per query and O^T per (dim, query) go to
  // LDS; then thread t writes outputs (query, dim) = t + 256 j, dims fastest.
  double l_w = l_run + xor_lane<16>(l_run);
  l_w += xor_lane<32>(l_w);
  __syncthreads();  // K/V space free
  double* mw = reinterpret_cast<double*>(KVs);       // [NW][QT]
  double* lw = mw + NW * QT;                          // [NW][QT]
  // [NW][HD][QT], query slot qq of dim d at qq ^ (d % 16): the merge below
  // reads 64 consecutive dims of one query, which would otherwise all fall 128
  // bytes apart on the same banks
  double* ow = lw + NW * QT;
  if (g == 0) {
    mw[wave * QT + r16] = m_run;
    lw[wave * QT + r16] = l_w;
  }
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) ow[(wave * HD + b * 16 + 4 * i + g) * QT + (r16 ^ (4 * i + g))] = acc[b][i];
  __syncthreads();
  // Per query: each wavefront's factor exp(m_w - m) (0 for a wavefront that saw
  // no key of the document) and the merged denominator, once per query.
  double* fw = ow + NW * HD * QT;  // [NW][QT]
  double* dw = fw + NW * QT;       // [QT]
  if (tid < QT) {
    const int qq = tid;
    double m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmax(m, mw[w * QT + qq]);
    double den = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const double mwq = mw[w * QT + qq];
      const double f = mwq == -INFINITY ? 0.0 : exp(mwq - m);
      fw[w * QT + qq] = f;
      if (mwq != -INFINITY) den += f * lw[w * QT + qq];
    }
    dw[qq] = den;
  }
  __syncthreads();
  for (int idx = tid; idx < QT * HD; idx += NT) {
    const int qq = idx / HD, dim = idx % HD;
    if (q0 + qq >= len) continue;
    double num = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (mw[w * QT + qq] == -INFINITY) continue;
      num += fw[w * QT + qq] * ow[(w * HD + dim) * QT + (qq ^ (dim & 15))];
    }
    o[static_cast<size_t>(s0 + q0 + qq) * H * HD + static_cast<size_t>(h) * HD + dim] = static_cast<float>(num / dw[qq]);
  }
}

bool attention_supported(bool bf16, int hd) {
  if (bf16) return hd == ab::HD;
  return hd == 32 || hd == 64 || hd == 128;
}

hipError_t attention_bf16(int N, int H, int hd, int n_docs, const int32_t* cu, int max_seqlen,
                          const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                          hipStream_t s, uint8_t* o8, uint8_t* o8s) {
  if (N == 0 || n_docs == 0 || max_seqlen == 0) return hipSuccess;
  LaunchScope scope_(kCntAttnBf16, s);
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(hd));
  const int qtiles = (max_seqlen + ab::QT - 1) / ab::QT;
  const int64_t work = static_cast<int64_t>(qtiles) * H * n_docs;
  if (work > (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int blocks = static_cast<int>((work + 255) / 256 * 256);  // whole runs of 8 XCDs x 32 CUs
  hipLaunchKernelGGL(attention_bf16_kernel, dim3(blocks), dim3(ab::NT), 0, s, N, H, n_docs, qtiles,
                     static_cast<int>(work), cu, q, k, v, o, scale_log2, o8, o8s);
  return hipGetLastError();
}

hipError_t attention_f32(int N, int H, int hd, int n_docs, const int32_t* cu, int max_seqlen,
                         const float* q, const float* k, const float* v, float* o, hipStream_t s) {
  if (N == 0 || n_docs == 0 || max_seqlen == 0) return hipSuccess;
  LaunchScope scope_(kCntAttnF32, s);
  const double scale = 1.0 / sqrt(static_cast<double>(hd));
  dim3 grid((max_seqlen + af::QT - 1) / af::QT, H, n_docs);
  if (grid.y > 65535 || grid.z > 65535) return hipErrorInvalidValue;
  switch (hd) {
    case 32: hipLaunchKernelGGL(attention_f32_kernel<32>, grid, dim3(af::NT), 0, s, N, H, cu, q, k, v, o, scale); break;
    case 64: hipLaunchKernelGGL(attention_f32_kernel<64>, grid, dim3(af::NT), 0, s, N, H, cu, q, k, v, o, scale); break;
    case 128: hipLaunchKernelGGL(attention_f32_kernel<128>, grid, dim3(af::NT), 0, s, N, H, cu, q, k, v, o, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dit
