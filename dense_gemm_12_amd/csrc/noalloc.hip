// gemm_ex_noalloc: the split-K / operand-repacking entry point (gemm_ex) for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  Its scratch memory
// is a fixed array in the library's device code instead of a caller-provided
// workspace.
//
// `scratch` below is a host-side stand-in in host code, not a device address:
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that pointer is ever handed to kernels
// or copies.  Every call on a device shares that device's array; gemm_ex
// never needs the workspace to start zeroed (repacked operands and split
// partials are written in full before they are read), so nothing is cleared.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mgemm.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch` per device (null until looked up)

// The device address of this device's `scratch`, looked up on first use with
// `dev` current (the calling thread's current device is restored after).
hipError_t scratch_for(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

mg_status gemm_ex_noalloc(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                          int64_t K, float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                          float beta, void *C, int64_t ldc, int config, int splits, void *stream) {
  // a forced split count whose partials do not fit the fixed scratch
  if (splits >= 2 && M > 0 && N > 0 && K > 0 &&
      (uint64_t)splits * (uint64_t)M * (uint64_t)N * 4u > (uint64_t)MG_NOALLOC_SCRATCH_BYTES)
    return MG_ESCRATCH;
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  void *ws = nullptr;
  if (e == hipSuccess) e = scratch_for(dev, &ws);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MG_EHIP;
  }
  return gemm_ex(in_type, c_type, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws,
                 (size_t)MG_NOALLOC_SCRATCH_BYTES, config, splits, stream);
}

}  // extern "C"
