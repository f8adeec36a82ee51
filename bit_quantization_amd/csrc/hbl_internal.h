// Internal declarations shared by the HIP kernel files and the C-ABI layer
// of libhbl.  Nothing here is part of the public interface (include/hbl.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hbl {

// Launchers.  Each validates nothing (the C-ABI layer has done that) and
// returns the hipError_t of the launch.
// cu_count: compute units of the device (sizes persistent grids).
// norm: RMSNorm of each row (per-channel gain, nullable) before the rotation.
// bits: 8 or 4 (codes in the public layouts), or 6: INT4 codes written as
// MX6 operands of the FP6 x FP4 matmul (K a power of two >= 1024).
hipError_t launch_hadamard_quant(const void* x, bool x_bf16, int64_t M, int K,
                                 int64_t ldx, bool hadamard, int bits,
                                 void* codes, float* scales, int32_t* rowsum,
                                 bool norm, const float* gain,
                                 int cu_count, hipStream_t s);
hipError_t launch_hadamard_f32(const void* x, bool x_bf16, int64_t M, int K,
                               int64_t ldx, float* y, int cu_count, hipStream_t s);
hipError_t launch_ternarize(const void* w, bool w_bf16, int64_t N, int64_t K,
                            uint32_t* packed, float* alpha, double* partials,
                            int n_partials, hipStream_t s);
int ternarize_partials(int64_t N, int64_t K);

// out_kind: 0 bf16, 1 f32, 2 i32 (the HBL_OUT_* values)
hipError_t launch_ternary_gemm(const void* codes, int bits, const float* scales,
                               const int32_t* rowsum, const uint32_t* wp,
                               const float* alpha, int64_t M, int64_t N,
                               int64_t K, int out_kind, void* out, int64_t ldo,
                               int cu_count, hipStream_t s);

// FP6 x FP4 matmul of MX6 codes and MX4 weights (k_gemm_mx.hip); K % 512 == 0.
hipError_t launch_gemm_mx(const void* codes, const float* scales, const uint32_t* wq,
                          const float* alpha, int64_t M, int64_t N, int64_t K,
                          int out_kind, void* out, int64_t ldo, int cu_count,
                          hipStream_t s);
// ternary layout -> MX4 layout (same size)
hipError_t launch_prepare_mx4(const uint32_t* wp, int64_t N, int64_t K, uint32_t* wq,
                              hipStream_t s);

// post-RoPE QKV / KV-cache quantiser (k_kvquant.hip); D a power of two in [32, 2048]
hipError_t launch_kv_quant(const void* x, bool x_bf16, int64_t B, int64_t S, int64_t H, int D,
                           int bits, int keep_bos8, void* codes, float* scales, void* bos_codes,
                           float* bos_scales, int cu_count, hipStream_t s);

// Token counts up to this take the weight-streaming kernel.
constexpr int kGemvMaxM = 128;

}  // namespace hbl
