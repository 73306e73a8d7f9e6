// Shared device helpers for the gfx950 DiT kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef uint16_t bf16_t;  // raw bf16 bits

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Element traits so a kernel can be written once for float and bf16 storage.
template <typename T> struct elem;
template <> struct elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// 16-byte vector of T as floats: 4 floats or 8 bf16.
template <typename T> struct vec16;
template <> struct vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float* v) {
    float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    uint4 t = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    uint4 t;
    t.x = pack_bf16x2(v[0], v[1]);
    t.y = pack_bf16x2(v[2], v[3]);
    t.z = pack_bf16x2(v[4], v[5]);
    t.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = t;
  }
};

// The value that lane (lane ^ M) of the wavefront holds, M a power of two up
// to 32, moved without the LDS permute path: DPP quad permutations (M = 1,
// 2), DPP rotations within rows of 16 lanes (M = 8; M = 4: a lane with bit 2
// set takes the rotation that brings lane - 4, the others the one that brings
// lane + 4), and the lane-half swaps v_permlane16_swap / v_permlane32_swap
// (M = 16, 32: each returns both halves; the lane keeps its partner's).
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (M == 4) {
    const uint32_t down = __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false);  // row_ror 4: lane - 4 (mod 16)
    const uint32_t up = __builtin_amdgcn_mov_dpp(v, 0x12C, 0xF, 0xF, false);    // row_ror 12: lane + 4 (mod 16)
    return (__lane_id() & 4) ? down : up;
  } else if constexpr (M == 8) {
    return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);  // row_ror 8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows {0,0,2,2}, {1,1,3,3}
    return (__lane_id() & 16) ? r[0] : r[1];
  } else {
    static_assert(M == 32, "lane masks 1 .. 32");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // halves {0,0}, {1,1}
    return (__lane_id() & 32) ? r[0] : r[1];
  }
}
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  return __uint_as_float(xor_lane<M>(__float_as_uint(v)));
}
template <int M>
__device__ __forceinline__ double xor_lane(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = xor_lane<M>(static_cast<uint32_t>(u)), hi = xor_lane<M>(static_cast<uint32_t>(u >> 32));
  return __builtin_bit_cast(double, static_cast<uint64_t>(hi) << 32 | lo);
}
// the same for a mask known only at run time (uniform over the wavefront)
template <typename T>
__device__ __forceinline__ T xor_lane_rt(T v, int m) {
  switch (m) {
    case 1: return xor_lane<1>(v);
    case 2: return xor_lane<2>(v);
    case 4: return xor_lane<4>(v);
    case 8: return xor_lane<8>(v);
    case 16: return xor_lane<16>(v);
    default: return xor_lane<32>(v);
  }
}

// Butterfly sums: every lane adds its partner's partial at distance 32, 16,
// .., 1, so all lanes end with the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lane<32>(v); v += xor_lane<16>(v); v += xor_lane<8>(v);
  v += xor_lane<4>(v); v += xor_lane<2>(v); v += xor_lane<1>(v);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += xor_lane<32>(v); v += xor_lane<16>(v); v += xor_lane<8>(v);
  v += xor_lane<4>(v); v += xor_lane<2>(v); v += xor_lane<1>(v);
  return v;
}
// max that keeps a NaN from either side (fmaxf drops it), so a row max over
// |x| reports a non-finite row as NaN or Inf
__device__ __forceinline__ float nan_max(float a, float b) { return (a > b || a != a) ? a : b; }
__device__ __forceinline__ float wave_max(float v) {
  v = nan_max(v, xor_lane<32>(v)); v = nan_max(v, xor_lane<16>(v)); v = nan_max(v, xor_lane<8>(v));
  v = nan_max(v, xor_lane<4>(v)); v = nan_max(v, xor_lane<2>(v)); v = nan_max(v, xor_lane<1>(v));
  return v;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier without the memory fence of __syncthreads(): LDS written
// by direct loads is covered by explicit vmcnt waits before it (the fence
// would add vmcnt(0), i.e. also wait for the copies just issued for later
// tiles), and the "memory" clobber keeps the compiler from moving LDS reads
// across it.
__device__ __forceinline__ void go_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace dit
