// The fp32 GEMM of dit_gemm for callers that cannot allocate device memory or
// hand in a workspace: code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation.  Its scratch -- the int8 slices of A and B
// and the fp64 split-K partials -- lives in one file-scope device array that
// the code object carries, so the call allocates nothing.
//
// Each device holds its own copy of the array at its own address; host code
// never uses the array's name as an address (on the host it only stands in
// for the symbol): the address comes from hipGetSymbolAddress, once per
// device, with that device current.  Every call on a device shares that
// device's array and leaves its contents behind; nothing in it needs to start
// at zero (the slicing kernel writes every byte the GEMM reads, every split
// writes every partial element its reduction reads).  Calls that overlap on
// one device -- on different streams, or from different host threads without
// ordering -- race on the array.
#include <mutex>

#include "common.h"
#include "dit.h"
#include "internal.h"
#include "kernels.h"

namespace dit {

constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kNoAllocMaxDevices = 64;

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[kNoAllocMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device.
static int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(DIT_E_HIP, "dit_gemm_f32_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return set_error(DIT_E_UNSUPPORTED, "dit_gemm_f32_noalloc: device %d beyond the %d the library tracks", dev,
                     kNoAllocMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_error(DIT_E_HIP, "dit_gemm_f32_noalloc: scratch address on device %d: %s", dev,
                       hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DIT_OK;
}

}  // namespace dit

extern "C" size_t dit_gemm_f32_noalloc_limit(void) { return dit::kNoAllocScratchBytes; }

extern "C" int dit_gemm_f32_noalloc(int M, int N, int K, const float* A, const float* B, const float* bias, float* C,
                                    dit_stream_t stream) {
  using namespace dit;
  if (M < 0 || N <= 0 || K <= 0) return set_error(DIT_E_INVALID, "dit_gemm_f32_noalloc: M=%d N=%d K=%d", M, N, K);
  if (M > 0 && (A == nullptr || B == nullptr || C == nullptr))
    return set_error(DIT_E_INVALID, "dit_gemm_f32_noalloc: null operand");
  if (!gemm_f32_supported(M, N, K))
    return set_error(DIT_E_UNSUPPORTED, "dit_gemm_f32_noalloc: K=%d must be a multiple of 4 (and slices within 2 GB)", K);
  // the same layout as dit_gemm's workspace: B's slices, then A's slices and the partials
  const size_t bsl = gemm_f32_slices_bytes(N, K);
  const size_t need = bsl + gemm_f32_ws_bytes(M, N, K);
  if (need > kNoAllocScratchBytes)
    return set_error(DIT_E_WORKSPACE, "dit_gemm_f32_noalloc: [%d x %d] x [%d x %d]^T needs %zu bytes of scratch, beyond the %zu it has",
                     M, K, N, K, need, kNoAllocScratchBytes);
  if (M == 0) return DIT_OK;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != DIT_OK) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = slice_rows(N, K, B, ws, s);
  if (e == hipSuccess) e = gemm_f32(M, N, K, A, ws, bias, C, static_cast<char*>(ws) + bsl, s);
  if (e != hipSuccess) return set_error(DIT_E_HIP, "dit_gemm_f32_noalloc: %s", hipGetErrorString(e));
  return DIT_OK;
}
