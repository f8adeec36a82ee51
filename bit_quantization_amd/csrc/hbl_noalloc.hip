// hbl_forward_noalloc: hbl_forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its workspace (the codes, scales and row sums of the
// quantiser, and the partial sums of a K split) is the file-scope device
// array `scratch` below instead of a caller buffer; the kernels are those
// of hbl_forward.
//
// `scratch` names a host-side stand-in in host code.  Its device address is
// looked up with hipGetSymbolAddress once per device, on that device's first
// call, and only that address is passed on.
#include "../../include/hbl.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "hbl_internal.h"

namespace {

// One copy per GPU the library runs on, held until the process ends.
static __device__ __align__(256) unsigned char scratch[HBL_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char text[256];
    snprintf(text, sizeof text, "hipGetDevice: %s", hipGetErrorString(e));
    return hbl::set_error(HBL_ERR_HIP, text);
  }
  if (dev < 0 || dev >= kMaxDevices) return hbl::set_error(HBL_ERR_HIP, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char text[256];
      snprintf(text, sizeof text, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return hbl::set_error(HBL_ERR_HIP, text);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HBL_OK;
}

}  // namespace

extern "C" int hbl_forward_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int64_t N,
                                   int flags, int bits, const uint32_t* w_packed, const float* alpha, void* y,
                                   int64_t ldy, void* stream) {
  const size_t need = hbl_forward_workspace_size(M, N, K, bits);
  if (need > (size_t)HBL_NOALLOC_WORKSPACE_BYTES) {
    char text[256];
    snprintf(text, sizeof text,
             "M = %lld, N = %lld, K = %lld, bits = %d needs %zu bytes of workspace; the static workspace of "
             "hbl_forward_noalloc holds %d",
             (long long)M, (long long)N, (long long)K, bits, need, HBL_NOALLOC_WORKSPACE_BYTES);
    return hbl::set_error(HBL_ERR_WORKSPACE, text);
  }
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != HBL_OK) return rc;
  // every byte of the workspace a call reads is written earlier in the same
  // call (codes, scales and row sums by the quantiser, each partial-sum slab
  // by its K slice), so nothing needs clearing between calls
  return hbl_forward(x, x_dtype, M, K, ldx, N, flags, bits, w_packed, alpha, y, ldy, ws,
                     (size_t)HBL_NOALLOC_WORKSPACE_BYTES, stream);
}
