// C ABI of libhbl: argument validation, workspace carving and dispatch to the
// HIP kernels.  Every check runs on the host before anything is enqueued.
#include "../../include/hbl.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <climits>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "hbl_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HBL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

int elem_size(int dtype) { return dtype == HBL_DTYPE_BF16 ? 2 : 4; }

int check_x(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, bool hadamard) {
  if (x_dtype != HBL_DTYPE_F32 && x_dtype != HBL_DTYPE_BF16)
    return fail(HBL_ERR_MODE, "x_dtype %d is neither HBL_DTYPE_F32 nor HBL_DTYPE_BF16", x_dtype);
  if (M < 0 || M > (int64_t)INT_MAX) return fail(HBL_ERR_SHAPE, "M = %lld is out of range", (long long)M);
  if (hadamard) {
    if (!is_pow2(K) || K < 16 || K > HBL_MAX_K)
      return fail(HBL_ERR_SHAPE, "K = %lld must be a power of two in [16, %d] with HBL_HADAMARD",
                  (long long)K, HBL_MAX_K);
  } else {
    if (K < 64 || K % 64 != 0 || K > HBL_MAX_K)
      return fail(HBL_ERR_SHAPE, "K = %lld must be a multiple of 64 in [64, %d]", (long long)K,
                  HBL_MAX_K);
  }
  if (ldx < K) return fail(HBL_ERR_SHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if ((ldx * elem_size(x_dtype)) % 16 != 0)
    return fail(HBL_ERR_ALIGN, "ldx * element size = %lld bytes is not a multiple of 16",
                (long long)(ldx * elem_size(x_dtype)));
  if (M > 0 && x == nullptr) return fail(HBL_ERR_NULL, "x is NULL");
  if (!aligned16(x)) return fail(HBL_ERR_ALIGN, "x is not 16-byte aligned");
  return HBL_OK;
}

int check_bits(int bits) {
  if (bits != 8 && bits != 4) return fail(HBL_ERR_MODE, "bits = %d is neither 8 nor 4", bits);
  return HBL_OK;
}

int check_flags(int flags) {
  if (flags & ~HBL_HADAMARD) return fail(HBL_ERR_MODE, "unknown flag bits 0x%x", flags & ~HBL_HADAMARD);
  return HBL_OK;
}

int check_gemm_shape(int64_t M, int64_t N, int64_t K, int64_t ldo) {
  if (M < 0) return fail(HBL_ERR_SHAPE, "M = %lld is negative", (long long)M);
  if (N < 16 || N % 16 != 0) return fail(HBL_ERR_SHAPE, "N = %lld must be a positive multiple of 16", (long long)N);
  if (K < 64 || K % 64 != 0 || K > HBL_MAX_GEMM_K)
    return fail(HBL_ERR_SHAPE, "K = %lld must be a multiple of 64 in [64, %d]", (long long)K, HBL_MAX_GEMM_K);
  if (ldo < N) return fail(HBL_ERR_SHAPE, "ldo = %lld < N = %lld", (long long)ldo, (long long)N);
  if (ldo % 4 != 0) return fail(HBL_ERR_ALIGN, "ldo = %lld is not a multiple of 4", (long long)ldo);
  if (ldo > HBL_MAX_LDO) return fail(HBL_ERR_SHAPE, "ldo = %lld exceeds %d", (long long)ldo, HBL_MAX_LDO);
  // token rows are addressed with 64-bit offsets; the grid size is the limit
  if ((M + 127) / 128 * ((N + 127) / 128) > (int64_t)INT_MAX)
    return fail(HBL_ERR_SHAPE, "M x N is too large for one launch");
  return HBL_OK;
}

int cu_count_cached() {
  static std::mutex mu;
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (counts[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    counts[dev] = c;
  }
  return counts[dev];
}

size_t codes_bytes(int64_t M, int64_t K, int bits) {
  return bits == 8 ? (size_t)(M * K) : (size_t)(M * (K / 2));
}

// codes, then scales, then row sums, each on a 256-byte boundary
size_t codes_region(int64_t M, int64_t K, int bits) {
  return round256(codes_bytes(M, K, bits)) + 2 * round256(sizeof(float) * (size_t)M);
}

// the FP6 x FP4 path: MX6 codes come from the rotation/quantisation kernel
// for rows of 1024 .. HBL_MAX_K elements, a power of two
int check_mx_k(int64_t K) {
  if (!is_pow2(K) || K < 1024 || K > HBL_MAX_K)
    return fail(HBL_ERR_SHAPE, "K = %lld must be a power of two in [1024, %d] on the FP6 x FP4 path", (long long)K,
                HBL_MAX_K);
  return HBL_OK;
}

int check_gain(const float* gain) {
  if (!aligned16(gain)) return fail(HBL_ERR_ALIGN, "gain is not 16-byte aligned");
  return HBL_OK;
}

int quant_impl(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, bool norm, const float* gain,
               int flags, int bits, void* codes, float* scales, int32_t* rowsum, void* stream) {
  g_last_error.clear();
  int rc = check_flags(flags);
  if (!rc) rc = check_bits(bits);
  if (!rc) rc = check_x(x, x_dtype, M, K, ldx, (flags & HBL_HADAMARD) != 0);
  if (!rc && norm) rc = check_gain(gain);
  if (rc) return rc;
  if (M > 0 && (!codes || !scales)) return fail(HBL_ERR_NULL, "codes and scales must be non-NULL");
  if (!aligned16(codes) || !aligned4(scales) || !aligned4(rowsum))
    return fail(HBL_ERR_ALIGN, "codes must be 16-byte aligned, scales and rowsum 4-byte aligned");
  hipError_t e = hbl::launch_hadamard_quant(x, x_dtype == HBL_DTYPE_BF16, M, (int)K, ldx,
                                            (flags & HBL_HADAMARD) != 0, bits, codes, scales, rowsum, norm,
                                            gain, cu_count_cached(), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantise launch");
  return HBL_OK;
}

int forward_impl(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, bool norm, const float* gain,
                 int64_t N, int flags, int bits, const uint32_t* w_packed, const float* alpha, void* y,
                 int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_flags(flags);
  if (!rc) rc = check_bits(bits);
  if (!rc) rc = check_x(x, x_dtype, M, K, ldx, (flags & HBL_HADAMARD) != 0);
  if (!rc) rc = check_gemm_shape(M, N, K, ldy);
  if (!rc && norm) rc = check_gain(gain);
  if (rc) return rc;
  if (M == 0) return HBL_OK;
  if (!w_packed || !alpha || !y) return fail(HBL_ERR_NULL, "w_packed, alpha and y must be non-NULL");
  if (!aligned16(w_packed) || !aligned16(y) || !aligned4(alpha))
    return fail(HBL_ERR_ALIGN, "w_packed and y must be 16-byte aligned");
  const size_t need = codes_region(M, K, bits) + round256(hbl::gemm_partial_bytes(M, N, K));
  if (!ws || ws_bytes < need)
    return fail(HBL_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0, need);
  if (!aligned16(ws)) return fail(HBL_ERR_ALIGN, "workspace is not 16-byte aligned");
  char* base = static_cast<char*>(ws);
  void* codes = base;
  float* scales = reinterpret_cast<float*>(base + round256(codes_bytes(M, K, bits)));
  int32_t* rowsum = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(scales) + round256(sizeof(float) * (size_t)M));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hbl::decode_token_applies(x_dtype == HBL_DTYPE_BF16, M, N, K, (flags & HBL_HADAMARD) != 0, norm, bits)) {
    // a few tokens: rotation (if asked), quantisation and matmul in one
    // launch (the workspace is not used)
    hipError_t e = hbl::launch_decode_token(x, ldx, M, (int)K, bits, (flags & HBL_HADAMARD) != 0, w_packed, alpha,
                                            N, y, ldy, s);
    if (e != hipSuccess) return hip_fail(e, "few-token decode launch");
    return HBL_OK;
  }
  hipError_t e = hbl::launch_hadamard_quant(x, x_dtype == HBL_DTYPE_BF16, M, (int)K, ldx,
                                            (flags & HBL_HADAMARD) != 0, bits, codes, scales, rowsum, norm, gain,
                                            cu_count_cached(), s);
  if (e != hipSuccess) return hip_fail(e, "quantise launch");
  const size_t part_bytes = hbl::gemm_partial_bytes(M, N, K);
  void* part = part_bytes ? base + codes_region(M, K, bits) : nullptr;
  e = hbl::launch_ternary_gemm(codes, bits, scales, rowsum, w_packed, alpha, M, N, K, HBL_OUT_BF16, y, ldy, part,
                               part_bytes, cu_count_cached(), s);
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return HBL_OK;
}

}  // namespace

int hbl::set_error(int status, const char* text) { return fail(status, "%s", text); }

extern "C" {

int hbl_version(void) { return 100; }

const char* hbl_status_string(int status) {
  switch (status) {
    case HBL_OK: return "success";
    case HBL_ERR_NULL: return "a required pointer is NULL";
    case HBL_ERR_SHAPE: return "a size or leading dimension is out of range";
    case HBL_ERR_ALIGN: return "a pointer or leading dimension is misaligned";
    case HBL_ERR_MODE: return "unknown dtype, bits or flag value";
    case HBL_ERR_WORKSPACE: return "workspace missing or too small";
    case HBL_ERR_HIP: return "a HIP runtime call failed";
    default: return "unknown status";
  }
}

const char* hbl_last_error(void) { return g_last_error.c_str(); }

int hbl_device_cu_count(void) {
  int dev = 0, c = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return c;
}

size_t hbl_ternarize_workspace_size(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return round256(sizeof(double) * (size_t)hbl::ternarize_partials(N, K));
}

int hbl_ternarize_weights(const void* w, int w_dtype, int64_t N, int64_t K, uint32_t* w_packed,
                          float* alpha, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (w_dtype != HBL_DTYPE_F32 && w_dtype != HBL_DTYPE_BF16)
    return fail(HBL_ERR_MODE, "w_dtype %d is neither HBL_DTYPE_F32 nor HBL_DTYPE_BF16", w_dtype);
  if (N < 1 || K < 16 || K % 16 != 0)
    return fail(HBL_ERR_SHAPE, "need N >= 1 and K a positive multiple of 16 (N = %lld, K = %lld)",
                (long long)N, (long long)K);
  if (!w || !w_packed || !alpha) return fail(HBL_ERR_NULL, "w, w_packed and alpha must be non-NULL");
  if (!aligned16(w) || !aligned16(w_packed) || !aligned4(alpha))
    return fail(HBL_ERR_ALIGN, "w and w_packed must be 16-byte aligned, alpha 4-byte aligned");
  const size_t need = hbl_ternarize_workspace_size(N, K);
  if (!ws || ws_bytes < need)
    return fail(HBL_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0, need);
  if (!aligned16(ws)) return fail(HBL_ERR_ALIGN, "workspace is not 16-byte aligned");
  hipError_t e = hbl::launch_ternarize(w, w_dtype == HBL_DTYPE_BF16, N, K, w_packed, alpha,
                                       static_cast<double*>(ws), hbl::ternarize_partials(N, K),
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ternarize launch");
  return HBL_OK;
}

int hbl_hadamard_f32(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, float* y,
                     void* stream) {
  g_last_error.clear();
  int rc = check_x(x, x_dtype, M, K, ldx, true);
  if (rc) return rc;
  if (M > 0 && !y) return fail(HBL_ERR_NULL, "y is NULL");
  if (!aligned16(y)) return fail(HBL_ERR_ALIGN, "y is not 16-byte aligned");
  hipError_t e = hbl::launch_hadamard_f32(x, x_dtype == HBL_DTYPE_BF16, M, (int)K, ldx, y, cu_count_cached(),
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hadamard launch");
  return HBL_OK;
}

int hbl_hadamard_quant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int flags,
                       int bits, void* codes, float* scales, int32_t* rowsum, void* stream) {
  return quant_impl(x, x_dtype, M, K, ldx, false, nullptr, flags, bits, codes, scales, rowsum, stream);
}

int hbl_norm_hadamard_quant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                            const float* gain, int flags, int bits, void* codes, float* scales,
                            int32_t* rowsum, void* stream) {
  return quant_impl(x, x_dtype, M, K, ldx, true, gain, flags, bits, codes, scales, rowsum, stream);
}

int hbl_hadamard_backward_f32(const void* dy, int dy_dtype, int64_t M, int64_t K, int64_t lddy, float* dx,
                              void* stream) {
  // H is symmetric and orthogonal: the backward is the forward transform
  return hbl_hadamard_f32(dy, dy_dtype, M, K, lddy, dx, stream);
}

int hbl_ternary_gemm(const void* codes, int bits, const float* scales, const int32_t* rowsum,
                     const uint32_t* w_packed, const float* alpha, int64_t M, int64_t N, int64_t K,
                     int out_dtype, void* out, int64_t ldo, void* stream) {
  g_last_error.clear();
  int rc = check_bits(bits);
  if (!rc) rc = check_gemm_shape(M, N, K, ldo);
  if (rc) return rc;
  if (out_dtype != HBL_OUT_BF16 && out_dtype != HBL_OUT_F32 && out_dtype != HBL_OUT_I32)
    return fail(HBL_ERR_MODE, "out_dtype %d is not an HBL_OUT_* value", out_dtype);
  if (M == 0) return HBL_OK;
  if (!codes || !scales || !rowsum || !w_packed || !alpha || !out)
    return fail(HBL_ERR_NULL, "codes, scales, rowsum, w_packed, alpha and out must be non-NULL");
  if (!aligned16(codes) || !aligned16(w_packed) || !aligned16(out) || !aligned4(scales) ||
      !aligned4(rowsum) || !aligned4(alpha))
    return fail(HBL_ERR_ALIGN, "codes, w_packed and out must be 16-byte aligned");
  hipError_t e = hbl::launch_ternary_gemm(codes, bits, scales, rowsum, w_packed, alpha, M, N, K,
                                          out_dtype, out, ldo, nullptr, 0, cu_count_cached(),
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return HBL_OK;
}

size_t hbl_forward_workspace_size(int64_t M, int64_t N, int64_t K, int bits) {
  if (M < 0 || N < 0 || K <= 0 || (bits != 8 && bits != 4)) return 0;
  return codes_region(M, K, bits) + round256(hbl::gemm_partial_bytes(M, N, K));
}

int hbl_forward(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int64_t N, int flags,
                int bits, const uint32_t* w_packed, const float* alpha, void* y, int64_t ldy, void* ws,
                size_t ws_bytes, void* stream) {
  return forward_impl(x, x_dtype, M, K, ldx, false, nullptr, N, flags, bits, w_packed, alpha, y, ldy, ws,
                      ws_bytes, stream);
}

int hbl_norm_forward(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, const float* gain,
                     int64_t N, int flags, int bits, const uint32_t* w_packed, const float* alpha, void* y,
                     int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(x, x_dtype, M, K, ldx, true, gain, N, flags, bits, w_packed, alpha, y, ldy, ws, ws_bytes,
                      stream);
}

size_t hbl_mx_codes_bytes(int64_t M, int64_t K) {
  if (M < 0 || K <= 0) return 0;
  return (size_t)((M + 255) / 256 * 256) * (size_t)(K / 4 * 3);
}

size_t hbl_mx_weights_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return (size_t)((N + 127) / 128 * 128) * (size_t)(K / 4);
}

int hbl_prepare_weights_mx(const uint32_t* w_packed, int64_t N, int64_t K, uint32_t* w_mx, void* stream) {
  g_last_error.clear();
  if (N < 1 || K < 128 || K % 128 != 0)
    return fail(HBL_ERR_SHAPE, "need N >= 1 and K a positive multiple of 128 (N = %lld, K = %lld)", (long long)N,
                (long long)K);
  if (!w_packed || !w_mx) return fail(HBL_ERR_NULL, "w_packed and w_mx must be non-NULL");
  if (!aligned16(w_packed) || !aligned16(w_mx)) return fail(HBL_ERR_ALIGN, "w_packed and w_mx must be 16-byte aligned");
  hipError_t e = hbl::launch_prepare_mx4(w_packed, N, K, w_mx, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prepare launch");
  return HBL_OK;
}

int hbl_hadamard_quant_mx(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int flags, void* codes_mx,
                          float* scales, void* stream) {
  g_last_error.clear();
  int rc = check_flags(flags);
  if (!rc) rc = check_x(x, x_dtype, M, K, ldx, (flags & HBL_HADAMARD) != 0);
  if (!rc) rc = check_mx_k(K);
  if (rc) return rc;
  if (M > 0 && (!codes_mx || !scales)) return fail(HBL_ERR_NULL, "codes_mx and scales must be non-NULL");
  if (!aligned16(codes_mx) || !aligned4(scales))
    return fail(HBL_ERR_ALIGN, "codes_mx must be 16-byte aligned, scales 4-byte aligned");
  hipError_t e = hbl::launch_hadamard_quant(x, x_dtype == HBL_DTYPE_BF16, M, (int)K, ldx, (flags & HBL_HADAMARD) != 0,
                                            6, codes_mx, scales, nullptr, false, nullptr, cu_count_cached(),
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantise launch");
  return HBL_OK;
}

int hbl_ternary_gemm_mx(const void* codes_mx, const float* scales, const uint32_t* w_mx, const float* alpha,
                        int64_t M, int64_t N, int64_t K, int out_dtype, void* out, int64_t ldo, void* stream) {
  g_last_error.clear();
  int rc = check_gemm_shape(M, N, K, ldo);
  if (rc) return rc;
  if (K % 512 != 0) return fail(HBL_ERR_SHAPE, "K = %lld must be a multiple of 512 on the FP6 x FP4 path", (long long)K);
  if (out_dtype != HBL_OUT_BF16 && out_dtype != HBL_OUT_F32 && out_dtype != HBL_OUT_I32)
    return fail(HBL_ERR_MODE, "out_dtype %d is not an HBL_OUT_* value", out_dtype);
  if (M == 0) return HBL_OK;
  if (!codes_mx || !scales || !w_mx || !alpha || !out)
    return fail(HBL_ERR_NULL, "codes_mx, scales, w_mx, alpha and out must be non-NULL");
  if (!aligned16(codes_mx) || !aligned16(w_mx) || !aligned16(out) || !aligned4(scales) || !aligned4(alpha))
    return fail(HBL_ERR_ALIGN, "codes_mx, w_mx and out must be 16-byte aligned");
  hipError_t e = hbl::launch_gemm_mx(codes_mx, scales, w_mx, alpha, M, N, K, out_dtype, out, ldo, nullptr, 0,
                                     cu_count_cached(), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return HBL_OK;
}

size_t hbl_forward_mx_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0) return 0;
  return round256(hbl_mx_codes_bytes(M, K)) + round256(sizeof(float) * (size_t)M) +
         round256(hbl::gemm_mx_partial_bytes(M, N, K));
}

int hbl_forward_mx(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int64_t N, int flags,
                   const uint32_t* w_mx, const float* alpha, void* y, int64_t ldy, void* ws, size_t ws_bytes,
                   void* stream) {
  g_last_error.clear();
  int rc = check_flags(flags);
  if (!rc) rc = check_x(x, x_dtype, M, K, ldx, (flags & HBL_HADAMARD) != 0);
  if (!rc) rc = check_mx_k(K);
  if (!rc) rc = check_gemm_shape(M, N, K, ldy);
  if (rc) return rc;
  if (M == 0) return HBL_OK;
  if (!w_mx || !alpha || !y) return fail(HBL_ERR_NULL, "w_mx, alpha and y must be non-NULL");
  if (!aligned16(w_mx) || !aligned16(y) || !aligned4(alpha))
    return fail(HBL_ERR_ALIGN, "w_mx and y must be 16-byte aligned");
  const size_t need = hbl_forward_mx_workspace_size(M, N, K);
  if (!ws || ws_bytes < need)
    return fail(HBL_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0, need);
  if (!aligned16(ws)) return fail(HBL_ERR_ALIGN, "workspace is not 16-byte aligned");
  void* codes = ws;
  const size_t codes_end = round256(hbl_mx_codes_bytes(M, K));
  float* scales = reinterpret_cast<float*>(static_cast<char*>(ws) + codes_end);
  void* part = static_cast<char*>(ws) + codes_end + round256(sizeof(float) * (size_t)M);
  const size_t part_bytes = hbl::gemm_mx_partial_bytes(M, N, K);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hbl::launch_hadamard_quant(x, x_dtype == HBL_DTYPE_BF16, M, (int)K, ldx, (flags & HBL_HADAMARD) != 0,
                                            6, codes, scales, nullptr, false, nullptr, cu_count_cached(), s);
  if (e != hipSuccess) return hip_fail(e, "quantise launch");
  e = hbl::launch_gemm_mx(codes, scales, w_mx, alpha, M, N, K, HBL_OUT_BF16, y, ldy, part_bytes ? part : nullptr,
                          part_bytes, cu_count_cached(), s);
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return HBL_OK;
}

int hbl_kv_quant(const void* x, int x_dtype, int64_t B, int64_t S, int64_t H, int64_t D, int bits, int keep_bos8,
                 void* codes, float* scales, void* bos_codes, float* bos_scales, void* stream) {
  g_last_error.clear();
  if (x_dtype != HBL_DTYPE_F32 && x_dtype != HBL_DTYPE_BF16)
    return fail(HBL_ERR_MODE, "x_dtype %d is neither HBL_DTYPE_F32 nor HBL_DTYPE_BF16", x_dtype);
  if (bits != 3 && bits != 4 && bits != 8) return fail(HBL_ERR_MODE, "bits = %d is not 3, 4 or 8", bits);
  if (B < 0 || S < 1 || H < 1) return fail(HBL_ERR_SHAPE, "need B >= 0, S >= 1, H >= 1");
  if (!is_pow2(D) || D < 32 || D > 2048)
    return fail(HBL_ERR_SHAPE, "D = %lld must be a power of two in [32, 2048]", (long long)D);
  if (B * S * H > ((int64_t)1 << 40)) return fail(HBL_ERR_SHAPE, "B x S x H is too large");
  if (B == 0) return HBL_OK;
  if (!x || !codes || !scales) return fail(HBL_ERR_NULL, "x, codes and scales must be non-NULL");
  if (keep_bos8 && (!bos_codes || !bos_scales))
    return fail(HBL_ERR_NULL, "keep_bos8 needs bos_codes and bos_scales");
  if (!aligned16(x) || !aligned16(codes) || !aligned4(scales) || !aligned16(bos_codes) || !aligned4(bos_scales))
    return fail(HBL_ERR_ALIGN, "x, codes and bos_codes must be 16-byte aligned, scales 4-byte aligned");
  hipError_t e = hbl::launch_kv_quant(x, x_dtype == HBL_DTYPE_BF16, B, S, H, (int)D, bits, keep_bos8 != 0, codes,
                                      scales, bos_codes, bos_scales, cu_count_cached(),
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv quantise launch");
  return HBL_OK;
}

size_t hbl_ternarize_rotated_workspace_size(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return round256(sizeof(float) * (size_t)N * (size_t)K) + hbl_ternarize_workspace_size(N, K);
}

int hbl_ternarize_weights_rotated(const void* w, int w_dtype, int64_t N, int64_t K, uint32_t* w_packed,
                                  float* alpha, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (w_dtype != HBL_DTYPE_F32 && w_dtype != HBL_DTYPE_BF16)
    return fail(HBL_ERR_MODE, "w_dtype %d is neither HBL_DTYPE_F32 nor HBL_DTYPE_BF16", w_dtype);
  if (N < 1 || N > (int64_t)INT_MAX || !is_pow2(K) || K < 16 || K > HBL_MAX_K)
    return fail(HBL_ERR_SHAPE, "need N >= 1 and K a power of two in [16, %d] (N = %lld, K = %lld)", HBL_MAX_K,
                (long long)N, (long long)K);
  if (!w || !w_packed || !alpha) return fail(HBL_ERR_NULL, "w, w_packed and alpha must be non-NULL");
  if (!aligned16(w) || !aligned16(w_packed) || !aligned4(alpha))
    return fail(HBL_ERR_ALIGN, "w and w_packed must be 16-byte aligned, alpha 4-byte aligned");
  const size_t need = hbl_ternarize_rotated_workspace_size(N, K);
  if (!ws || ws_bytes < need)
    return fail(HBL_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0, need);
  if (!aligned16(ws)) return fail(HBL_ERR_ALIGN, "workspace is not 16-byte aligned");
  float* wr = static_cast<float*>(ws);
  double* partials = reinterpret_cast<double*>(static_cast<char*>(ws) + round256(sizeof(float) * (size_t)N * (size_t)K));
  hipStream_t s = static_cast<hipStream_t>(stream);
  // rows of W H^T are the rows of W rotated (H is symmetric)
  hipError_t e = hbl::launch_hadamard_f32(w, w_dtype == HBL_DTYPE_BF16, N, (int)K, K, wr, cu_count_cached(), s);
  if (e != hipSuccess) return hip_fail(e, "hadamard launch");
  e = hbl::launch_ternarize(wr, false, N, K, w_packed, alpha, partials, hbl::ternarize_partials(N, K), s);
  if (e != hipSuccess) return hip_fail(e, "ternarize launch");
  return HBL_OK;
}

}  // extern "C"
