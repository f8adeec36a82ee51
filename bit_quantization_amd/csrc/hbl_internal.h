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

// Tiles and K split of the persistent matmuls (k_gemm_pt, k_gemm_mx):
// 256 x 256 tiles when they alone fill the chip (cu_count of them), else
// 256 x 128; below kSplitItems tiles the K range (nk stages of 128) is
// halved while the items (tile, K slice) fit kSplitItems and each keeps at
// least 16 stages (32 when the tiles alone already fill half the chip), and
// once more (to 8 stages) while they fit half of them.  Measured on MI355X
// at N = 4096 (both layers, every split bit-identical): K = 4096, M <= 256
// best at 4 slices, M = 1024 unsplit; K = 16384, M <= 256 at 8, M = 512 at
// 4, M = 1024 at 2; from 256 tiles on, none.
struct SplitPlan {
  int bm = 256, bn, tm, tn, ksplit;
  // M-group of the item walk (split_item): an XCD's 32 consecutive items
  // cover 2 row blocks x 16 column blocks, whose codes and weights it then
  // fetches once into its L2 (measured on MI355X at M = 2048, N = K =
  // 4096: 27.0 against 27.9 us (FP6 x FP4) and 35.4 against 38.1 us (int8)
  // for groups of 8; at M = N = 4096, K = 16384: 136.7 against 140.2 us)
  int gm = 2;
  int64_t items() const { return (int64_t)tm * tn * ksplit; }
};
constexpr int kSplitItems = 256;
// wide_narrow: the narrow tiles are 128 x 256 instead of 256 x 128 (the
// FP6 x FP4 matmul, split or not)
inline SplitPlan split_plan(int64_t M, int64_t N, int64_t K, int cu_count, bool may_split,
                            bool wide_narrow = false) {
  SplitPlan p;
  const int64_t g256 = ((M + 255) / 256) * ((N + 255) / 256);
  const bool narrow = g256 < cu_count;
  p.bm = narrow && wide_narrow ? 128 : 256;
  p.bn = narrow && !wide_narrow ? 128 : 256;
  p.tm = (int)((M + p.bm - 1) / p.bm);
  p.tn = (int)((N + p.bn - 1) / p.bn);
  p.ksplit = 1;
  const int64_t G = (int64_t)p.tm * p.tn, nk = K / 128;
  auto ok = [&](int S, int64_t items, int64_t min_stages) {
    return may_split && narrow && G * S <= items && (nk / 4) % S == 0 && nk / S >= min_stages;
  };
  while (ok(p.ksplit * 2, kSplitItems, G >= kSplitItems / 2 ? 32 : 16)) p.ksplit *= 2;
  if (ok(p.ksplit * 2, kSplitItems / 2, 8)) p.ksplit *= 2;
  return p;
}

#if defined(__HIPCC__)
// Work item L of a split plan: K slice L / (tilesM tilesN), tile
// L % (tilesM tilesN); tiles walked in M-groups of gm so that the items an
// XCD runs together (consecutive L) share code rows and weight rows in its
// L2: gm row blocks by (items / gm) column blocks.
template <int BM, int BN>
__device__ __forceinline__ void split_item(int L, int tilesM, int tilesN, int gm, int64_t& m0, int64_t& n0,
                                           int& ks) {
  const int G = tilesM * tilesN;
  ks = L / G;
  const int T = L - ks * G;
  const int per_group = gm * tilesN;
  const int first_m = (T / per_group) * gm;
  const int gsz = gm < tilesM - first_m ? gm : tilesM - first_m;
  m0 = (int64_t)(first_m + (T % per_group) % gsz) * BM;
  n0 = (int64_t)((T % per_group) / gsz) * BN;
}
#endif

// out_kind: 0 bf16, 1 f32, 2 i32 (the HBL_OUT_* values).
// part: scratch for int32 partial sums of a K split of the persistent
// matmul (part_bytes of it; NULL: no split, and token counts up to
// kGemvMaxM stream the weights)
hipError_t launch_ternary_gemm(const void* codes, int bits, const float* scales,
                               const int32_t* rowsum, const uint32_t* wp,
                               const float* alpha, int64_t M, int64_t N,
                               int64_t K, int out_kind, void* out, int64_t ldo,
                               void* part, size_t part_bytes, int cu_count,
                               hipStream_t s);
// bytes of partial sums launch_ternary_gemm uses for a K split (0: none)
size_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K);

// FP6 x FP4 matmul of MX6 codes and MX4 weights (k_gemm_mx.hip); K % 512 == 0.
// part: scratch for the exact partial sums of a K split (part_bytes of
// it); NULL or too small runs the matmul unsplit
hipError_t launch_gemm_mx(const void* codes, const float* scales, const uint32_t* wq,
                          const float* alpha, int64_t M, int64_t N, int64_t K,
                          int out_kind, void* out, int64_t ldo, void* part,
                          size_t part_bytes, int cu_count, hipStream_t s);
// bytes of partial sums launch_gemm_mx uses for a K split (0: no split)
size_t gemm_mx_partial_bytes(int64_t M, int64_t N, int64_t K);
// ternary layout -> MX4 layout (same size)
hipError_t launch_prepare_mx4(const uint32_t* wp, int64_t N, int64_t K, uint32_t* wq,
                              hipStream_t s);

// post-RoPE QKV / KV-cache quantiser (k_kvquant.hip); D a power of two in [32, 2048]
hipError_t launch_kv_quant(const void* x, bool x_bf16, int64_t B, int64_t S, int64_t H, int D,
                           int bits, int keep_bos8, void* codes, float* scales, void* bos_codes,
                           float* bos_scales, int cu_count, hipStream_t s);

// Few-token decode layer (k_quant.hip): the rotation + INT8 or INT4
// quantisation of M bf16 token rows (M <= 2 up to K = 4096, else 1) and the
// dot-product matmul with the rescale of Eq. 9 in one launch, bf16 output
// [M][ldo]; the codes never leave the chip.
bool decode_token_applies(bool x_bf16, int64_t M, int64_t N, int64_t K, bool hadamard, bool norm, int bits);
hipError_t launch_decode_token(const void* x, int64_t ldx, int64_t M, int K, int bits, bool hadamard,
                               const uint32_t* wp, const float* alpha, int64_t N, void* out, int64_t ldo,
                               hipStream_t s);

// Token counts up to this take the weight-streaming kernel.
constexpr int kGemvMaxM = 128;

// Records the detail text hbl_last_error() returns on the calling thread and
// returns status (for entry points defined outside hbl_api.cpp).
int set_error(int status, const char* text);

}  // namespace hbl
