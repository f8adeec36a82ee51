// Ternary-weight integer matmul with the rescale of Eq. 9 (architecture
// write-up of "BitNet v2", §3.4 "H-BitLinear"), for gfx950:
//   acc[m][n] = sum_k q_x[m][k] q_w[n][k],  out = (scale_m * alpha) * acc.
//
// Two kernels:
//   k_gemm -- large token counts.  Block tile BM x BN, K staged through LDS
//     128 bytes at a time, double-buffered, 4 waves in a 2 x 2 grid, each
//     wave a (BM/2) x (BN/2) tile of 16x16x64 int8 MFMAs with int32
//     accumulators.  Activation codes are widened to int8 and weights are
//     decoded from two bits to the unsigned byte c = q + 1 in {0, 1, 2} on
//     their way from global memory into LDS.  The MFMA therefore sums
//     q_x * c; the epilogue subtracts sum_k q_x (the token's row sum of
//     codes) to obtain sum_k q_x * q_w exactly.
//   k_gemv -- token counts up to 16 (decode).  Bandwidth-bound: each block
//     owns 16 output features and streams their packed weights once with
//     16-byte loads; the 4 waves of a block split K and are reduced through
//     LDS.  The tokens are the 16 columns of the MFMA's second operand
//     (columns beyond M are zero).
//
// In both kernels the MFMA's first operand is the weight fragment and its
// second the activation fragment, so each lane ends with four consecutive
// output features of one token: one 8-byte bf16 store.
#include "hbl_internal.h"

namespace hbl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Streaming 16-byte load (data used once: do not keep it in the caches).
__device__ __forceinline__ uint4 load_stream(const uint32_t* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Two's-complement nibbles (bytes 0..15) to signed bytes, bytewise:
// ((u ^ 8) + 0x78) ^ 0x80 never carries between bytes.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t u) {
  return ((u ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int OUT>
__device__ __forceinline__ void store4(void* out, int64_t idx, v4i a, int32_t R, float sc) {
  const int t0 = a[0] - R, t1 = a[1] - R, t2 = a[2] - R, t3 = a[3] - R;
  if constexpr (OUT == 2) {
    *reinterpret_cast<int4*>(reinterpret_cast<int32_t*>(out) + idx) = make_int4(t0, t1, t2, t3);
  } else if constexpr (OUT == 1) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx) =
        make_float4(sc * (float)t0, sc * (float)t1, sc * (float)t2, sc * (float)t3);
  } else {
    const uint32_t lo = f32_to_bf16_rne(sc * (float)t0) | ((uint32_t)f32_to_bf16_rne(sc * (float)t1) << 16);
    const uint32_t hi = f32_to_bf16_rne(sc * (float)t2) | ((uint32_t)f32_to_bf16_rne(sc * (float)t3) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) = make_uint2(lo, hi);
  }
}

constexpr int BK = 128;           // k per LDS stage
constexpr int LROW = BK + 16;     // padded LDS row stride in bytes

template <int BITS, int OUT, int BM, int BN>
__global__ void __launch_bounds__(256, 1)
k_gemm(const void* __restrict__ codes, const float* __restrict__ scales,
       const int32_t* __restrict__ rowsum, const uint32_t* __restrict__ wp,
       const float* __restrict__ alpha, int64_t M, int64_t N, int64_t K,
       void* __restrict__ out, int64_t ldo, int tilesM, int tilesN) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int PA = BITS == 8 ? BM / 32 : BM / 64;  // 16-byte A loads per thread
  constexpr int PB = BN / 128;                        // 16-byte B loads per thread
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * LROW];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * LROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // Tile order: consecutive block ids go to different XCDs, so give each
  // XCD a contiguous range of tiles, then walk M-groups of 8 tiles.
  const int G = tilesM * tilesN;
  const int b = blockIdx.x;
  const int L = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  constexpr int GROUP_M = 8;
  const int per_group = GROUP_M * tilesN;
  const int first_m = (L / per_group) * GROUP_M;
  const int gsz = min(GROUP_M, tilesM - first_m);
  const int tm = first_m + (L % per_group) % gsz;
  const int tn = (L % per_group) / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t KW = K / 16;  // packed weight words per row
  uint4 ra[PA], rb[PB];

  auto gload = [&](int kt) {
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      if constexpr (BITS == 8) {
        const int r = tid / 8 + 32 * p, c = tid % 8;
        const int64_t k = (int64_t)kt * BK + 16 * c;
        ra[p] = (m0 + r < M && k < K)
                    ? *reinterpret_cast<const uint4*>(reinterpret_cast<const int8_t*>(codes) + (m0 + r) * K + k)
                    : make_uint4(0, 0, 0, 0);
      } else {
        const int r = tid / 4 + 64 * p, c = tid % 4;
        const int64_t k = (int64_t)kt * BK + 32 * c;
        ra[p] = (m0 + r < M && k < K)
                    ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(codes) + (m0 + r) * (K / 2) + k / 2)
                    : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int r = tid / 2 + 128 * p, c = tid % 2;
      const int64_t kw = (int64_t)kt * (BK / 16) + 4 * c;
      rb[p] = (n0 + r < N && kw < KW) ? *reinterpret_cast<const uint4*>(wp + (n0 + r) * KW + kw)
                                      : make_uint4(0, 0, 0, 0);
    }
  };

  auto sstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      if constexpr (BITS == 8) {
        const int r = tid / 8 + 32 * p, c = tid % 8;
        *reinterpret_cast<uint4*>(&As[buf][r * LROW + 16 * c]) = ra[p];
      } else {
        const int r = tid / 4 + 64 * p, c = tid % 4;
        const uint32_t w[4] = {ra[p].x, ra[p].y, ra[p].z, ra[p].w};
        uint32_t d[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          d[2 * i] = sext_nibbles(w[i] & 0x0f0f0f0fu);
          d[2 * i + 1] = sext_nibbles((w[i] >> 4) & 0x0f0f0f0fu);
        }
        uint4* dst = reinterpret_cast<uint4*>(&As[buf][r * LROW + 32 * c]);
        dst[0] = make_uint4(d[0], d[1], d[2], d[3]);
        dst[1] = make_uint4(d[4], d[5], d[6], d[7]);
      }
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int r = tid / 2 + 128 * p, c = tid % 2;
      const uint32_t w[4] = {rb[p].x, rb[p].y, rb[p].z, rb[p].w};
      uint4* dst = reinterpret_cast<uint4*>(&Bs[buf][r * LROW + 64 * c]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = make_uint4(w[i] & 0x03030303u, (w[i] >> 2) & 0x03030303u, (w[i] >> 4) & 0x03030303u,
                            (w[i] >> 6) & 0x03030303u);
    }
  };

  v4i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int nk = (int)((K + BK - 1) / BK);
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane % 16, fk = 16 * (lane / 16);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 64) {
      v4i bf[FN], af[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        bf[i] = *reinterpret_cast<const v4i*>(&Bs[cur][(wn * WN + 16 * i + fr) * LROW + ks + fk]);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        af[j] = *reinterpret_cast<const v4i*>(&As[cur][(wm * WM + 16 * j + fr) * LROW + ks + fk]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = mfma16x16x64(bf[i], af[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  const float al = *alpha;
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t m = m0 + wm * WM + 16 * j + fr;
    if (m >= M) continue;
    const int32_t R = rowsum[m];
    const float sc = scales[m] * al;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int64_t n = n0 + wn * WN + 16 * i + 4 * (lane / 16);
      if (n < N) store4<OUT>(out, m * ldo + n, acc[i][j], R, sc);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode: M <= 16 tokens, one block per 16 output features.
constexpr int kGemvBatch = 8;  // 16-byte weight loads in flight per lane

template <int BITS, int OUT>
__global__ void __launch_bounds__(256)
k_gemv(const void* __restrict__ codes, const float* __restrict__ scales,
       const int32_t* __restrict__ rowsum, const uint32_t* __restrict__ wp,
       const float* __restrict__ alpha, int M, int64_t N, int64_t K,
       void* __restrict__ out, int64_t ldo) {
  __shared__ v4i red[3][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int fr = lane % 16, g = lane / 16;
  const int64_t KW = K / 16;
  const int64_t steps = (KW + 15) / 16;  // a step is 16 words (256 k) per row
  const uint32_t* wrow = wp + (n0 + fr) * KW;
  const bool mlive = fr < M;

  v4i acc = {0, 0, 0, 0};
  for (int64_t s0 = wave; s0 < steps; s0 += 4 * kGemvBatch) {
    uint4 w[kGemvBatch];
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
      const int64_t kw = (s0 + 4 * b) * 16 + 4 * g;
      w[b] = (s0 + 4 * b < steps && kw < KW) ? load_stream(wrow + kw)
                                             : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
      const int64_t kw = (s0 + 4 * b) * 16 + 4 * g;
      // Skip only whole steps (a wave-uniform test): an MFMA always runs on
      // all 64 lanes, so lanes past the end of K feed zeros instead.
      if (s0 + 4 * b >= steps) continue;
      // activation codes for k = 16*kw .. 16*kw + 63 of token fr
      uint32_t x[16];
      if (mlive && kw < KW) {
        if constexpr (BITS == 8) {
          const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const int8_t*>(codes) + fr * K + 16 * kw);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 u = p[i];
            x[4 * i] = u.x; x[4 * i + 1] = u.y; x[4 * i + 2] = u.z; x[4 * i + 3] = u.w;
          }
        } else {
          const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint32_t*>(codes) + fr * (K / 8) + 2 * kw);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint4 u = p[i];
            const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              x[8 * i + 2 * q] = sext_nibbles(ww[q] & 0x0f0f0f0fu);
              x[8 * i + 2 * q + 1] = sext_nibbles((ww[q] >> 4) & 0x0f0f0f0fu);
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = 0;
      }
      const uint32_t ws[4] = {w[b].x, w[b].y, w[b].z, w[b].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i a = {(int)(ws[i] & 0x03030303u), (int)((ws[i] >> 2) & 0x03030303u),
                       (int)((ws[i] >> 4) & 0x03030303u), (int)((ws[i] >> 6) & 0x03030303u)};
        const v4i bx = {(int)x[4 * i], (int)x[4 * i + 1], (int)x[4 * i + 2], (int)x[4 * i + 3]};
        acc = mfma16x16x64(a, bx, acc);
      }
    }
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i) acc += red[i][lane];
    if (fr < M) {
      const float sc = scales[fr] * *alpha;
      store4<OUT>(out, fr * ldo + n0 + 4 * g, acc, rowsum[fr], sc);
    }
  }
}

template <int BITS, int OUT>
hipError_t launch_bits_out(const void* codes, const float* scales, const int32_t* rowsum,
                           const uint32_t* wp, const float* alpha, int64_t M, int64_t N, int64_t K,
                           void* out, int64_t ldo, int cu_count, hipStream_t s) {
  if (M <= kGemvMaxM) {
    hipLaunchKernelGGL((k_gemv<BITS, OUT>), dim3((unsigned)(N / 16)), dim3(256), 0, s, codes, scales,
                       rowsum, wp, alpha, (int)M, N, K, out, ldo);
    return hipGetLastError();
  }
  // Large tiles when they alone fill the chip; otherwise 128 x 128.
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  if (t256 >= cu_count) {
    const int tm = (int)((M + 255) / 256), tn = (int)((N + 255) / 256);
    hipLaunchKernelGGL((k_gemm<BITS, OUT, 256, 256>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, codes,
                       scales, rowsum, wp, alpha, M, N, K, out, ldo, tm, tn);
  } else {
    const int tm = (int)((M + 127) / 128), tn = (int)((N + 127) / 128);
    hipLaunchKernelGGL((k_gemm<BITS, OUT, 128, 128>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, codes,
                       scales, rowsum, wp, alpha, M, N, K, out, ldo, tm, tn);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ternary_gemm(const void* codes, int bits, const float* scales, const int32_t* rowsum,
                               const uint32_t* wp, const float* alpha, int64_t M, int64_t N, int64_t K,
                               int out_kind, void* out, int64_t ldo, int cu_count, hipStream_t s) {
  if (M == 0) return hipSuccess;
#define HBL_G(BITS, OUT) \
  return launch_bits_out<BITS, OUT>(codes, scales, rowsum, wp, alpha, M, N, K, out, ldo, cu_count, s)
  if (bits == 8) {
    if (out_kind == 0) HBL_G(8, 0);
    if (out_kind == 1) HBL_G(8, 1);
    HBL_G(8, 2);
  } else {
    if (out_kind == 0) HBL_G(4, 0);
    if (out_kind == 1) HBL_G(4, 1);
    HBL_G(4, 2);
  }
#undef HBL_G
}

}  // namespace hbl
