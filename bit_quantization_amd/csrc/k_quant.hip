// Per-token Walsh-Hadamard rotation fused with per-token activation
// quantisation, for gfx950.
//
// What is computed (architecture write-up of "BitNet v2", §3.4):
//   x_r = H_k x for each token row x of length K = 2^k, H_k the normalised
//   Sylvester-Hadamard matrix ("The Hadamard Transformation", Eq. 5-6),
//   evaluated as k radix-2 butterfly stages (a, b) -> (a + b, a - b) in fp32
//   and one final multiplication by 2^{-k/2};
//   then INT8 absmax (Eq. 7) or INT4 absmean (Eq. 8) per token:
//     factor = Qmax / (stat + eps), code = clip(rint(x_r * factor)),
//     scale = stat / Qmax.
//
// Work decomposition (one token row per group of T threads, T = 2^t):
//   A row of K = 2^k elements is held in registers, E = 2^e per thread,
//   e = max(3, ceil(k/2)), t = k - e.  Element index bits are split into
//   lo (bits 0-2, an 8-element chunk = one 16-byte bf16 load), mid (t bits,
//   the thread index in phase A) and hi (e - 3 bits).
//   Phase A: each thread loads its chunks (lo, hi vary) and applies the
//            butterfly stages of the lo and hi bits in registers.
//   Phase B: the row is exchanged through LDS so that each thread holds the
//            elements whose mid bits vary, and those t stages run in
//            registers.  The result goes back to LDS.
//   Output:  each thread re-reads contiguous 8-element chunks, applies the
//            1/sqrt(K) scale, the row statistic is reduced across the row,
//            and the codes are packed and stored contiguously.
// The butterfly stages commute, so applying them in this order gives the
// transform exactly in real arithmetic; fp32 rounding differs from a
// sequential evaluation by a few ulps.
//
// LDS addresses are XOR-swizzled so that both the 16-byte chunk accesses of
// phase A and the 4-byte strided accesses of phase B are free of bank
// conflicts.
#include "hbl_internal.h"
#include "k_dot.h"

namespace hbl {
namespace {

constexpr float kEps = 1e-5f;
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
// (float)sqrt(7): the INT4 clipping constant of Eq. 8.
constexpr float kSqrt7 = 2.6457513110645907f;

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
// Two fp32 values whose low 16 bits are zero (small integers) as packed bf16,
// the first in the low half: exact, no rounding.
__device__ __forceinline__ uint32_t pk_bf16_exact(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// Byte offsets of group g (32 codes) of token row m in the MX6 layout: the
// codes of 256-row block B = m / 256 and stage s = g / 4 (128 codes) form one
// 24 KB tile, a 16 KB main area (the first 16 bytes of each group: row r =
// m % 256 at units 4 r .. 4 r + 3, group gi = g % 4 at unit
// 4 r + (gi ^ ((r >> 2) & 3))) and an 8 KB tail area (the last 8 bytes: row r
// at units 2 r, 2 r + 1, groups 2 u, 2 u + 1 in the two halves of unit
// 2 r + (u ^ ((r >> 3) & 1))).  That is the matmul's LDS stage image, so its
// stage loads are plain contiguous copies.
__device__ __forceinline__ int64_t mx6_main_off(int64_t m, int g, int K) {
  const int64_t tile = (m >> 8) * (K / 128) + (g >> 2);
  const int r = (int)(m & 255), gi = g & 3;
  return tile * 24576 + 16 * (4 * r + (gi ^ ((r >> 2) & 3)));
}
__device__ __forceinline__ int64_t mx6_tail_off(int64_t m, int g, int K) {
  const int64_t tile = (m >> 8) * (K / 128) + (g >> 2);
  const int r = (int)(m & 255), gi = g & 3;
  return tile * 24576 + 16384 + 16 * (2 * r + ((gi >> 1) ^ ((r >> 3) & 1))) + 8 * (gi & 1);
}

// A 16-byte load with the non-temporal hint: data read once, which should
// not displace what the next kernel reads from the Infinity Cache.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  typedef unsigned v4u_ __attribute__((ext_vector_type(4)));
  const v4u_ v = __builtin_nontemporal_load(reinterpret_cast<const v4u_*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Loads 8 consecutive elements starting at p (16-byte aligned) as fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, float* v) {
  if constexpr (BF16) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16lo(u.x); v[1] = bf16hi(u.x);
    v[2] = bf16lo(u.y); v[3] = bf16hi(u.y);
    v[4] = bf16lo(u.z); v[5] = bf16hi(u.z);
    v[6] = bf16lo(u.w); v[7] = bf16hi(u.w);
  } else {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// In-register radix-2 stages over register-index bits [B0, B1).
template <int E, int B0, int B1>
__device__ __forceinline__ void butterflies(float (&v)[E]) {
#pragma unroll
  for (int b = B0; b < B1; ++b) {
    const int h = 1 << b;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], c = v[i + h];
        v[i] = a + c;
        v[i + h] = a - c;
      }
    }
  }
}

// LDS address swizzle: flips bits 2-4 from bits >= 5 (an involution).
template <int TL>
__device__ __forceinline__ int swz(int e) {
  if constexpr (TL >= 2) {
    const int hi = (e >> (3 + TL)) & 3;
    return e ^ (hi << 3) ^ (((e >> 5) & 1) << 2);
  } else {
    return e;
  }
}

// Reduction of one value over the T threads of a row.  Every thread of the
// row gets the same bits: the xor-butterfly pairs the same partials on
// both sides, and the cross-wave step combines the waves in a fixed order.
// The value of lane l ^ o, for a butterfly over lane distances o = 1, 2, 4,
// ... in that order.  Distances 1 and 2 are quad permutations; 4 and 8 are
// the half-row and row mirrors (lane i <-> 7 - i, 15 - i), which pair each
// lane with the other half of its group, equivalent to l ^ o once the
// earlier steps have made every 4- (8-) lane group uniform; 16 and 32 go
// through the LDS crossbar.  DPP moves cost one VALU slot instead of an
// LDS round trip.
template <int O>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (O == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  else if constexpr (O == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  else if constexpr (O == 4) return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  else if constexpr (O == 8) return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  else return __shfl_xor(v, O);
}

// Butterfly over the W lanes of a group: every lane ends with the same bits
// (each step combines the same two values in either order).
template <int W, bool IS_MAX>
__device__ __forceinline__ float lanes_reduce(float v) {
#define HBL_STEP(O)                                                   \
  if constexpr (W > O) {                                              \
    const float u = __int_as_float(lane_xor<O>(__float_as_int(v)));   \
    v = IS_MAX ? fmaxf(v, u) : v + u;                                 \
  }
  HBL_STEP(1) HBL_STEP(2) HBL_STEP(4) HBL_STEP(8) HBL_STEP(16) HBL_STEP(32)
#undef HBL_STEP
  return v;
}

template <int W>
__device__ __forceinline__ int lanes_reduce_int(int v) {
#define HBL_STEP(O) \
  if constexpr (W > O) v += lane_xor<O>(v);
  HBL_STEP(1) HBL_STEP(2) HBL_STEP(4) HBL_STEP(8) HBL_STEP(16) HBL_STEP(32)
#undef HBL_STEP
  return v;
}

// Sum (or max) of |v[0..N)|, a pairwise tree (log2 N dependent steps).
template <int N, bool IS_MAX>
__device__ __forceinline__ float abs_tree(const float* v) {
  static_assert(N >= 2 && (N & (N - 1)) == 0, "power of two");
  float t[N / 2];
#pragma unroll
  for (int i = 0; i < N / 2; ++i) t[i] = IS_MAX ? fmaxf(fabsf(v[i]), fabsf(v[i + N / 2])) : fabsf(v[i]) + fabsf(v[i + N / 2]);
#pragma unroll
  for (int w = N / 4; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = IS_MAX ? fmaxf(t[i], t[i + w]) : t[i] + t[i + w];
  return t[0];
}

// Sum of squares of v[0..N) as a pairwise tree (products rounded, then
// added; no fused multiply-add).
template <int N>
__device__ __forceinline__ float sq_tree(const float* v) {
  float a[N / 2];
#pragma unroll
  for (int i = 0; i < N / 2; ++i) a[i] = v[i] * v[i] + v[i + N / 2] * v[i + N / 2];
#pragma unroll
  for (int w = N / 4; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) a[i] = a[i] + a[i + w];
  return a[0];
}

template <int T, bool IS_MAX>
__device__ __forceinline__ float row_reduce(float v, float* red, int row, int tid) {
  constexpr int W = T < 64 ? T : 64;
  v = lanes_reduce<W, IS_MAX>(v);
  if constexpr (T > 64) {
    constexpr int NW = T / 64;
    if ((tid & 63) == 0) red[row * NW + (tid >> 6)] = v;
    __syncthreads();
    float r = red[row * NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      const float u = red[row * NW + i];
      r = IS_MAX ? fmaxf(r, u) : r + u;
    }
    v = r;
  }
  return v;
}

template <int T>
__device__ __forceinline__ int row_reduce_int(int v, int* red, int row, int tid) {
  constexpr int W = T < 64 ? T : 64;
  v = lanes_reduce_int<W>(v);
  if constexpr (T > 64) {
    constexpr int NW = T / 64;
    if ((tid & 63) == 0) red[row * NW + (tid >> 6)] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) r += red[row * NW + i];
    v = r;
  }
  return v;
}

// Normalisation layer of H-BitLinear (RMSNorm, Eq. 9): the row's values
// become v * r * g with r = 1 / sqrt(mean of the squares + eps) and g the
// per-channel gain (NULL: one).  ss is this thread's partial sum of squares;
// the row total is reduced through red (a buffer of its own, so that the
// statistic's reduction later in the row needs no extra barrier).  ge(i) is
// the element index of v[i].
template <int T, int N, typename GE>
__device__ __forceinline__ void rmsnorm_apply(float* v, float ss, float kf, const float* __restrict__ gain,
                                              float* red, int row, int tid, GE ge) {
  ss = row_reduce<T, false>(ss, red, row, tid);
  const float r = 1.0f / __builtin_sqrtf(ss / kf + kEps);
  if (gain) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 g = *reinterpret_cast<const float4*>(gain + ge(i));
      v[i] = (v[i] * r) * g.x; v[i + 1] = (v[i + 1] * r) * g.y;
      v[i + 2] = (v[i + 2] * r) * g.z; v[i + 3] = (v[i + 3] * r) * g.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = v[i] * r;
  }
}

template <int LOG2K>
struct Geom {
  static constexpr int K = 1 << LOG2K;
  static constexpr int EL = (LOG2K + 1) / 2 > 3 ? (LOG2K + 1) / 2 : 3;  // log2 E
  static constexpr int TL = LOG2K - EL;                                 // log2 T
  static constexpr int E = 1 << EL;
  static constexpr int T = 1 << TL;
  static constexpr int NC = E / 8;                 // 8-element chunks per thread
  static constexpr int RPB = T >= 128 ? 1 : 128 / T;  // rows per block
  static constexpr int THREADS = RPB * T;
  static constexpr int RED = RPB * (T > 64 ? T / 64 : 1);
};

// OUT: 0 = codes (BITS 8 or 4), 1 = fp32 rotated values.  NORM: the row
// goes through the RMSNorm layer (gain nullable) before the rotation.
template <int LOG2K, bool BF16, int BITS, bool HAD, int OUT, bool NORM>
__global__ void __launch_bounds__(Geom<LOG2K>::THREADS)
k_fwht_quant(const void* __restrict__ x, int64_t M, int64_t ldx,
             void* __restrict__ codes, float* __restrict__ scales,
             int32_t* __restrict__ rowsum, float* __restrict__ yout,
             const float* __restrict__ gain) {
  using G = Geom<LOG2K>;
  constexpr int K = G::K, E = G::E, T = G::T, TL = G::TL, EL = G::EL, NC = G::NC;
  constexpr int ESZ = BF16 ? 2 : 4;

  __shared__ __attribute__((aligned(16))) float lds[HAD ? G::RPB * K : 4];
  __shared__ float redf[G::RED];
  __shared__ int redi[G::RED];
  __shared__ float redn[NORM ? G::RED : 1];

  const int row = threadIdx.x / T;
  const int tid = threadIdx.x % T;
  const int64_t m = (int64_t)blockIdx.x * G::RPB + row;
  const bool live = m < M;
  float* L = lds + (HAD ? row * K : 0);

  // Phase A: chunk c of this thread covers elements (c << (3+TL)) | (tid << 3) | 0..7.
  float v[E];
  {
    const char* xr = reinterpret_cast<const char*>(x) + (live ? m : 0) * ldx * ESZ;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e0 = (c << (3 + TL)) | (tid << 3);
      if (live) {
        load8<BF16>(xr + (int64_t)e0 * ESZ, v + 8 * c);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * c + j] = 0.0f;
      }
    }
  }
  if constexpr (NORM)
    rmsnorm_apply<T, E>(v, sq_tree<E>(v), (float)K, gain, redn, row, tid,
                        [&](int i) { return ((i >> 3) << (3 + TL)) | (tid << 3) | (i & 7); });

  if constexpr (HAD) {
    // stages of the lo and hi bits: every register bit
    butterflies<E, 0, EL>(v);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e0 = (c << (3 + TL)) | (tid << 3);
      *reinterpret_cast<float4*>(L + swz<TL>(e0)) = make_float4(v[8 * c], v[8 * c + 1], v[8 * c + 2], v[8 * c + 3]);
      *reinterpret_cast<float4*>(L + swz<TL>(e0 + 4)) = make_float4(v[8 * c + 4], v[8 * c + 5], v[8 * c + 6], v[8 * c + 7]);
    }
    __syncthreads();
    // Phase B: register r holds mid = r & (T-1); the remaining e bits of the
    // element index are rho = ((r >> TL) << TL) | tid, split into lo and hi.
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int rho = ((r >> TL) << TL) | tid;
      const int e = ((rho >> 3) << (3 + TL)) | ((r & (T - 1)) << 3) | (rho & 7);
      v[r] = L[swz<TL>(e)];
    }
    butterflies<E, 0, TL>(v);
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int rho = ((r >> TL) << TL) | tid;
      const int e = ((rho >> 3) << (3 + TL)) | ((r & (T - 1)) << 3) | (rho & 7);
      L[swz<TL>(e)] = v[r];
    }
    __syncthreads();
    // back to the chunk layout of phase A, with the normalisation 2^{-k/2}
    const float scale = (LOG2K % 2 == 0) ? __uint_as_float((uint32_t)(127 - LOG2K / 2) << 23)
                                          : (float)(1.0 / __builtin_sqrt((double)K));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e0 = (c << (3 + TL)) | (tid << 3);
      const float4 a = *reinterpret_cast<const float4*>(L + swz<TL>(e0));
      const float4 b = *reinterpret_cast<const float4*>(L + swz<TL>(e0 + 4));
      v[8 * c + 0] = a.x * scale; v[8 * c + 1] = a.y * scale;
      v[8 * c + 2] = a.z * scale; v[8 * c + 3] = a.w * scale;
      v[8 * c + 4] = b.x * scale; v[8 * c + 5] = b.y * scale;
      v[8 * c + 6] = b.z * scale; v[8 * c + 7] = b.w * scale;
    }
  }

  if constexpr (OUT == 1) {
    if (live) {
      float* yr = yout + m * (int64_t)K;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int e0 = (c << (3 + TL)) | (tid << 3);
        reinterpret_cast<float4*>(yr + e0)[0] = make_float4(v[8 * c], v[8 * c + 1], v[8 * c + 2], v[8 * c + 3]);
        reinterpret_cast<float4*>(yr + e0)[1] = make_float4(v[8 * c + 4], v[8 * c + 5], v[8 * c + 6], v[8 * c + 7]);
      }
    }
    return;
  } else {
    // row statistic: gamma = max|x_r| (INT8) or sum|x_r| (INT4, divided by K)
    float st = abs_tree<E, BITS == 8>(v);
    st = row_reduce<T, BITS == 8>(st, redf, row, tid);
    float f, s;
    if constexpr (BITS == 8) {
      f = 127.0f / (st + kEps);
      s = st / 127.0f;
    } else {
      const float beta = st / (float)K;  // exact: K is a power of two
      f = kSqrt7 / (beta + kEps);
      s = beta / kSqrt7;
    }
    constexpr float lo = BITS == 8 ? -128.0f : -8.0f;
    constexpr float hi = BITS == 8 ? 127.0f : 7.0f;
    int qsum = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      int q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float r = __builtin_rintf(v[8 * c + j] * f);
        q[j] = (int)fminf(fmaxf(r, lo), hi);
        qsum += q[j];
      }
      const int e0 = (c << (3 + TL)) | (tid << 3);
      if (live) {
        if constexpr (BITS == 8) {
          uint32_t w0 = (q[0] & 0xff) | ((q[1] & 0xff) << 8) | ((q[2] & 0xff) << 16) | ((uint32_t)q[3] << 24);
          uint32_t w1 = (q[4] & 0xff) | ((q[5] & 0xff) << 8) | ((q[6] & 0xff) << 16) | ((uint32_t)q[7] << 24);
          *reinterpret_cast<uint2*>(reinterpret_cast<int8_t*>(codes) + m * (int64_t)K + e0) = make_uint2(w0, w1);
        } else {
          uint32_t w = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) w |= (uint32_t)(q[j] & 0xf) << (8 * (j & 3) + 4 * (j >> 2));
          reinterpret_cast<uint32_t*>(codes)[m * (int64_t)(K / 8) + (e0 >> 3)] = w;
        }
      }
    }
    qsum = row_reduce_int<T>(qsum, redi, row, tid);
    if (live && tid == 0) {
      scales[m] = s;
      if (rowsum) rowsum[m] = qsum;
    }
  }
}

// ---------------------------------------------------------------------------
// Rows of K = 2^k >= 1024 elements: 64 elements per thread, T = K/64 threads
// per row, 256 threads per block (256/T rows), persistent over row groups.
//
// The k butterfly stages are applied in three register passes; between
// passes the row goes through LDS, always as 16-byte groups of 4 consecutive
// elements (element bits 0-1 stay in registers as passengers):
//   pass 1: registers hold element bits 0-5 (64 contiguous elements, loaded
//           with eight 16-byte loads); 6 stages;
//   pass 2: registers hold bits 6-9 (and 0-1); thread index = bits 2-5 and
//           10..k-1; 4 stages;
//   pass 3: registers hold bits 10..k-1 (a3 = k-10 of them), the low ex =
//           4-a3 bits of 2-5 and bits 0-1; thread index = the other bits of
//           2-5 and bits 6-9; a3 stages (absent when k = 10).
// LDS holds the row in fp32 with 16-byte unit u stored at u ^ ((u >> 4) &
// 15): the unit-wise writes of pass 1 and the reads and writes of passes 2
// and 3 then each touch 16 distinct bank groups per 16 lanes.
// In the last layout each thread quantises groups of 4 consecutive elements
// (the 1/sqrt(K) scale is folded into the per-row factor), the packed codes
// go back through LDS in natural order, and each thread stores contiguous
// 16-byte units.  The next row group's input is loaded while the current
// one is transformed.
template <int LOG2K, int BS = 256>
struct G64 {
  static constexpr int K = 1 << LOG2K;
  static constexpr int T = K / 64;             // threads per row
  static constexpr int RPB = BS / T;           // rows per block (BS threads)
  static constexpr int A3 = LOG2K - 10;        // active bits of pass 3
  static constexpr int EX = 4 - A3;            // low bits of 2-5 kept in registers in pass 3
};

__device__ __forceinline__ int swz16(int e) {  // float index -> swizzled float index
  const int u = e >> 2;
  return ((u ^ ((u >> 4) & 15)) << 2) | (e & 3);
}

// With bf16 input, pass 1 (the 64-point transforms of the contiguous
// 64-element chunks) runs on the matrix cores instead: per wave, Y = H_64 X
// for X the 64 x 64 matrix of its 64 chunks, as 16 v_mfma_f32_32x32x16_bf16
// (2 x 2 output tiles of 32 x 32, 4 k-steps of 16).  The bf16 inputs and the
// +-1 entries are exact in bf16 and every product is exact; the sums are
// accumulated in fp32.  The chunks are loaded straight into the operand
// layout (lane l holds 8 consecutive elements of chunk l % 32 of its column
// group), and the result is written to LDS as groups of 4 consecutive
// elements, in the same swizzled layout as the register path.
// OUT: 0 = codes (BITS 8 or 4), 1 = fp32 rotated values, 2 = INT4 codes as
// MX6 operands of the FP6 x FP4 matmul (BITS 4): groups of 32 codes as
// 192-bit fields (code e at bit 6 e), placed in 24 KB tiles of 256 rows x 128
// codes (mx6_main_off, mx6_tail_off).
template <int LOG2K, bool BF16, int BITS, bool HAD, int OUT, bool NORM, int BS>
__global__ void __launch_bounds__(BS, 2)
k_fwht_quant64(const void* __restrict__ x, int64_t M, int64_t ldx,
               void* __restrict__ codes, float* __restrict__ scales,
               int32_t* __restrict__ rowsum, float* __restrict__ yout,
               const float* __restrict__ gain) {
  using G = G64<LOG2K, BS>;
  constexpr int K = G::K, T = G::T, RPB = G::RPB, A3 = G::A3, EX = G::EX;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int NL = BF16 ? 8 : 16;  // 16-byte loads per thread
  // the matrix-core first pass needs the bf16 inputs themselves as operands;
  // normalised rows take the register path
  constexpr bool MFMA1 = BF16 && HAD && !NORM;
  // bf16 rows without the rotation: lane t takes the 16-byte units t + T q
  // (8 elements each) of its row, so that every load instruction reads
  // consecutive bytes (and the INT8 / INT4 code stores write them).  INT8
  // (a maximum: the order of the elements changes no bits) for every K;
  // INT4 and MX6 codes (a sum, in the same order for both, so that the two
  // layouts keep identical codes) for K = 4096 and 8192, where a row spans
  // whole waves.  The four units of a group of 32 MX6 codes then lie in four
  // consecutive lanes of one wave: the codes go through a wave-private LDS
  // area as bytes to gather each group.  (At K = 16384 the MX6 form measured
  // slower this way: the rows keep 64 contiguous elements per lane there.)
  constexpr bool SPREAD = BF16 && !HAD && !NORM && OUT != 1 && (BITS == 8 || T == 64 || T == 128);
  // MX6 codes of rotated rows of whole waves: the last exchange stays in
  // the wave (see the output stage)
  constexpr bool WLOC = HAD && OUT == 2 && T >= 64 && !NORM;
  __shared__ __attribute__((aligned(16))) uint8_t cb[SPREAD && OUT == 2 ? (BS / 64) * 4096 : 16];
  __shared__ __attribute__((aligned(16))) float lds[RPB * K];
  __shared__ float redf[RPB * (T > 64 ? T / 64 : 1)];
  __shared__ int redi[RPB * (T > 64 ? T / 64 : 1)];
  __shared__ float redn[NORM ? RPB * (T > 64 ? T / 64 : 1) : 1];

  const int row = threadIdx.x / T;
  const int t = threadIdx.x % T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* L = lds + row * K;
  const int64_t ngroups = (M + RPB - 1) / RPB;

  // Chunk (64 contiguous elements) of the block held by this lane in the
  // matrix-core pass, for column group cg: block chunk 64*wave + 32*cg + lane%32.
  auto mchunk = [&](int cg) { return 64 * wave + 32 * cg + (lane & 31); };

  // H_64 operands A(rb, s)[i][kk] = H[32*rb + i][16*s + kk], i = lane % 32,
  // kk = 8*(lane/32) + p, as bf16 +-1.  Since i < 32 and kk < 16,
  // A(rb, s) = P(s & 1) * (-1)^(rb * (s >> 1)) with
  // P(0)[i][kk] = (-1)^popcount(i & kk) and P(1) = P(0) * (-1)^(bit 4 of i):
  // four distinct operands, hP[s & 1][rb * (s >> 1)].
  v8bf hP[2][2];
  if constexpr (MFMA1) {
#pragma unroll
    for (int odd = 0; odd < 2; ++odd)
#pragma unroll
      for (int neg = 0; neg < 2; ++neg) {
        uint32_t w[4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          uint32_t h2 = 0;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int i = lane & 31, kk = 8 * (lane >> 5) + 2 * pp + half;
            const int par = (__popc(i & kk) + odd * ((i >> 4) & 1) + neg) & 1;
            h2 |= (par ? 0xbf80u : 0x3f80u) << (16 * half);
          }
          w[pp] = h2;
        }
        hP[odd][neg] = __builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3]));
      }
  }

  // The next row group's input is loaded into the same registers as soon as
  // the current one's have been consumed.
  uint4 raw0[NL];
  auto load_rows = [&](auto& raw, int64_t grp) {
    if constexpr (MFMA1) {
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        const int bc = mchunk(cg), r = bc / T, tc = bc % T;
        const int64_t m = grp * RPB + r;
        const bool live = grp < ngroups && m < M;
        const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) + (live ? m : 0) * ldx * ESZ +
                                                          ((int64_t)tc * 64 + 8 * (lane >> 5)) * ESZ);
#pragma unroll
        for (int st = 0; st < 4; ++st) raw[4 * cg + st] = live ? src[2 * st] : make_uint4(0, 0, 0, 0);
      }
    } else if constexpr (SPREAD) {
      // 16-byte unit t + T q of the row: each load instruction reads
      // consecutive bytes, whole 128-byte lines, so they can carry the
      // non-temporal hint: the rows (read once) then leave the codes this
      // kernel writes in the Infinity Cache for the matmuls that read them
      // next (the first such matmul of the 7B block, 65536 x 4096 x 4096:
      // 577 -> 513 us).  The rotation paths read a line in four pieces,
      // one per load instruction, and keep plain loads (with the hint the
      // K = 16384 rotation ran 753 -> 1022 us).
      const int64_t m = grp * RPB + row;
      const bool live = grp < ngroups && m < M;
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) + (live ? m : 0) * ldx * ESZ);
#pragma unroll
      for (int q = 0; q < NL; ++q) raw[q] = live ? load_nt(src + t + T * q) : make_uint4(0, 0, 0, 0);
    } else {
      const int64_t m = grp * RPB + row;
      const bool live = grp < ngroups && m < M;
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) +
                                                        (live ? m : 0) * ldx * ESZ + (int64_t)t * 64 * ESZ);
#pragma unroll
      for (int q = 0; q < NL; ++q) raw[q] = live ? src[q] : make_uint4(0, 0, 0, 0);
    }
  };

  auto row_group = [&](auto& raw, int64_t grp, int64_t refill) {
    const int64_t m = grp * RPB + row;
    const bool live = m < M;
    float v[64];
    if constexpr (MFMA1) {
      // pass 1 on the matrix cores, result to LDS
      v16f acc[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) acc[rb][cg] = v16f{};
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
          const v8bf bx = __builtin_bit_cast(v8bf, raw[4 * cg + st]);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb][cg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hP[st & 1][rb * (st >> 1)], bx, acc[rb][cg], 0, 0, 0);
        }
      load_rows(raw, refill);  // prefetch the next row group
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        const int bc = mchunk(cg), r = bc / T, tc = bc % T;
        float* Lr = lds + r * K;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            // rows 32*rb + 8*blk + 4*(lane/32) + 0..3 of chunk tc
            const int e = tc * 64 + 32 * rb + 8 * blk + 4 * (lane >> 5);
            const v16f& a = acc[rb][cg];
            *reinterpret_cast<float4*>(Lr + swz16(e)) = make_float4(a[4 * blk], a[4 * blk + 1], a[4 * blk + 2], a[4 * blk + 3]);
          }
      }
      // each wave's chunks are exactly the elements its pass-2 lanes read
      // (the element's bits from 12 up, or its row, name the wave): with
      // WLOC no block barrier here
      if constexpr (WLOC) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); else __syncthreads();
    } else {
      if constexpr (BF16) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[8 * q + 2 * i] = bf16lo(w[i]);
            v[8 * q + 2 * i + 1] = bf16hi(w[i]);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          v[4 * q] = __uint_as_float(raw[q].x); v[4 * q + 1] = __uint_as_float(raw[q].y);
          v[4 * q + 2] = __uint_as_float(raw[q].z); v[4 * q + 3] = __uint_as_float(raw[q].w);
        }
      }
      // with the normalisation the prefetch is issued after it: the gain
      // and the prefetched rows would not both fit in registers
      if constexpr (NORM)
        rmsnorm_apply<T, 64>(v, sq_tree<64>(v), (float)K, gain, redn, row, t,
                             [&](int i) { return (t << 6) | i; });
      load_rows(raw, refill);  // prefetch the next row group
      if constexpr (HAD) {
        butterflies<64, 0, 6>(v);
#pragma unroll
        for (int q = 0; q < 16; ++q)
          *reinterpret_cast<float4*>(L + swz16((t << 6) | (4 * q))) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        __syncthreads();
      }
    }

    // layout of the last pass: register group g of 4 -> first element
    auto last_e = [&](int gidx) {
      if constexpr (A3 == 0) {  // pass 2 layout: j = gidx
        return ((t >> 4) << 10) | (gidx << 6) | ((t & 15) << 2);
      } else {
        const int j3 = gidx >> EX, xx = gidx & ((1 << EX) - 1);
        const int lo = t & ((1 << A3) - 1), mid = t >> A3;
        return (j3 << 10) | (mid << 6) | (lo << (2 + EX)) | (xx << 2);
      }
    };

    if constexpr (HAD) {
      // pass 2
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float4 a = *reinterpret_cast<const float4*>(L + swz16(((t >> 4) << 10) | (j << 6) | ((t & 15) << 2)));
        v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
      }
      butterflies<64, 2, 6>(v);
      if constexpr (A3 > 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          *reinterpret_cast<float4*>(L + swz16(((t >> 4) << 10) | (j << 6) | ((t & 15) << 2))) =
              make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
        __syncthreads();
        // pass 3
#pragma unroll
        for (int gi = 0; gi < 16; ++gi) {
          const float4 a = *reinterpret_cast<const float4*>(L + swz16(last_e(gi)));
          v[4 * gi] = a.x; v[4 * gi + 1] = a.y; v[4 * gi + 2] = a.z; v[4 * gi + 3] = a.w;
        }
        butterflies<64, 6 - A3, 6>(v);
      }
    }

    // normalisation 2^{-k/2} (or fl(1/sqrt(K)) for odd k)
    constexpr float scale = (LOG2K % 2 == 0) ? (float)(1.0 / (double)(1 << (LOG2K / 2))) : 0.0f;
    const float c = HAD ? ((LOG2K % 2 == 0) ? scale : (float)(1.0 / __builtin_sqrt((double)K))) : 1.0f;

    if constexpr (OUT == 1) {
      // rotated values in natural order through LDS, then contiguous stores
      __syncthreads();
#pragma unroll
      for (int gi = 0; gi < 16; ++gi)
        *reinterpret_cast<float4*>(L + swz16(last_e(gi))) =
            make_float4(v[4 * gi] * c, v[4 * gi + 1] * c, v[4 * gi + 2] * c, v[4 * gi + 3] * c);
      __syncthreads();
      if (live) {
        float* yr = yout + m * (int64_t)K;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int u = t + T * q;  // 16-byte unit of the row
          *reinterpret_cast<float4*>(yr + 4 * u) = *reinterpret_cast<const float4*>(L + swz16(4 * u));
        }
      }
      __syncthreads();
    } else {
      float st = abs_tree<64, BITS == 8>(v);
      st = row_reduce<T, BITS == 8>(st, redf, row, t);
      float f, s;
      if constexpr (BITS == 8) {
        const float gamma = st * c;
        f = 127.0f / (gamma + kEps);
        s = gamma / 127.0f;
      } else {
        const float beta = (st * c) / (float)K;
        f = kSqrt7 / (beta + kEps);
        s = beta / kSqrt7;
      }
      // The rotated value is v * c; quantise v * (c * f).  Rounding: the
      // clipped value plus 1.5 * 2^23 is rounded to an integer by the fp32
      // add (nearest-even), whose low byte is then the two's-complement code.
      const float fc = HAD ? c * f : f;
      constexpr float lo = BITS == 8 ? -128.0f : -8.0f;
      constexpr float hi = BITS == 8 ? 127.0f : 7.0f;
      constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: fp32 values in [2^23, 2^24) are integers
      constexpr int kMagicBits = 0x4b400000;
      // four codes as the bytes of one word: fma(v, fc, 1.5*2^23) rounds the
      // exact product v*fc to the nearest integer (ties to even) in the low
      // mantissa bits; the clip is done on those bits
      auto quant4 = [&](const float* vv) {
        int b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int bits = __float_as_int(__builtin_fmaf(vv[j], fc, kMagic));
          b[j] = min(max(bits, kMagicBits + (int)lo), kMagicBits + (int)hi);
        }
        const uint32_t p01 = __builtin_amdgcn_perm((uint32_t)b[1], (uint32_t)b[0], 0x0c0c0400u);
        const uint32_t p23 = __builtin_amdgcn_perm((uint32_t)b[3], (uint32_t)b[2], 0x04000c0cu);
        return p01 | p23;
      };
      int qs[4] = {0, 0, 0, 0};  // four independent row-sum chains
      // MX6 codes: the same rounding and clip, kept as fp32 integers
      // (exact), then 32 codes at a time converted to E3M2 by the gfx950
      // packed conversion (scale 1: exact for integers in [-8, 7]), whose
      // 192-bit result holds element 2 i of its first operand at field 2 i and
      // element i of its second at field 2 i + 1 (measured on the device)
      auto qf = [&](float vv) {
        const float r = __builtin_fmaf(vv, fc, kMagic);
        return __builtin_amdgcn_fmed3f(r, kMagic + lo, kMagic + hi) - kMagic;
      };
      auto mx6_group = [&](const float* e, int g) {  // e: the group's 32 codes in order
        v16f a, b;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          a[i] = e[2 * i];
          b[i] = e[2 * i + 1];
        }
        const auto r = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, 1.0f);
        uint8_t* dst = reinterpret_cast<uint8_t*>(codes);
        *reinterpret_cast<uint4*>(dst + mx6_main_off(m, g, K)) = make_uint4(r[0], r[1], r[2], r[3]);
        *reinterpret_cast<uint2*>(dst + mx6_tail_off(m, g, K)) = make_uint2(r[4], r[5]);
      };
      // the same from 32 codes in bf16 (16 words, code i in half i % 2 of
      // word i / 2): the bf16 form of the conversion, element i at field i
      auto mx6_group_bf16 = [&](const uint4 (&u)[4], int g) {
        typedef __bf16 v32bf __attribute__((ext_vector_type(32)));
        struct W16 { uint4 a, b, c, d; };
        const auto r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(__builtin_bit_cast(v32bf, W16{u[0], u[1], u[2], u[3]}), 1.0f);
        uint8_t* dst = reinterpret_cast<uint8_t*>(codes);
        *reinterpret_cast<uint4*>(dst + mx6_main_off(m, g, K)) = make_uint4(r[0], r[1], r[2], r[3]);
        *reinterpret_cast<uint2*>(dst + mx6_tail_off(m, g, K)) = make_uint2(r[4], r[5]);
      };
      if constexpr (SPREAD && OUT == 2) {
        // the wave's codes as bytes to its LDS area, slice q holding the 8
        // codes of unit t + T q of each lane in lane order; piece j (32
        // bytes) of slice q is then group (T / 4) q + 16 (t / 64) + j, and
        // each lane converts two pieces.  (The barrier is not needed for the
        // data, which stays within the wave; it keeps the block's waves in
        // step, measured 7 % faster at K = 4096.)
        uint8_t* const C = cb + wave * 4096;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          *reinterpret_cast<uint2*>(C + 512 * q + 8 * lane) = make_uint2(quant4(v + 8 * q), quant4(v + 8 * q + 4));
        __syncthreads();
        if (live) {
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int q = (lane >> 4) + 4 * qq, j = lane & 15;
            const int g = (T / 4) * q + 16 * (t >> 6) + j;
            const uint4 a = *reinterpret_cast<const uint4*>(C + 512 * q + 32 * j);
            const uint4 b = *reinterpret_cast<const uint4*>(C + 512 * q + 32 * j + 16);
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = (float)(int)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
            mx6_group(v, g);
          }
        }
      } else if constexpr (!HAD && OUT == 2) {
        // the thread's 64 elements are contiguous: groups 2t and 2t + 1
#pragma unroll
        for (int i = 0; i < 64; ++i) v[i] = qf(v[i]);
        if (live) {
          mx6_group(v, 2 * t);
          mx6_group(v + 32, 2 * t + 1);
        }
      } else if constexpr (WLOC) {
        // The lanes holding the 32 codes of a group share element bits 5 and
        // up (bits 2-4 come from the lane's low bits and its register index):
        // with T >= 64 they lie in one wave, which holds element bits 6-9
        // in MPW values and every higher bit.  Each wave stages its 4096
        // codes as bf16 (exact: integers in [-8, 7]) in the first 8 KB of
        // its own 16 KB of the row's area (the rotated values there are no
        // longer read: every wave's pass 3 read before the row reduction's
        // barrier), at local index (bits 10 and up, bits 6-9 - MPW wr, bits
        // 0-5), 16-byte unit q of local group lg at q ^ ((lg >> 2) & 3) so
        // that both the 8-byte writes and the 64-byte group reads of 16
        // lanes fall into distinct banks.  Each lane then converts two
        // groups with the bf16 form of the packed E3M2 conversion.
        constexpr int MPW = 1024 / T;
        const int wr = t >> 6;
        uint8_t* const S = reinterpret_cast<uint8_t*>(L) + 16384 * wr;
#pragma unroll
        for (int gi = 0; gi < 16; ++gi) {
          const int e = last_e(gi);
          const int li = ((((e >> 10) * MPW) + (((e >> 6) & 15) - MPW * wr)) << 6) | (e & 63);
          const int lg = li >> 5;
          const uint32_t lo = pk_bf16_exact(qf(v[4 * gi]), qf(v[4 * gi + 1]));
          const uint32_t hi = pk_bf16_exact(qf(v[4 * gi + 2]), qf(v[4 * gi + 3]));
          *reinterpret_cast<uint2*>(S + 64 * lg + 16 * (((li >> 3) & 3) ^ ((lg >> 2) & 3)) + 2 * (li & 7)) =
              make_uint2(lo, hi);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own area: no block barrier
        if (live) {
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int lg = (t & 63) + 64 * qq, hb = lg >> 1;
            uint4 u[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) u[q] = *reinterpret_cast<const uint4*>(S + 64 * lg + 16 * (q ^ ((lg >> 2) & 3)));
            const int e = ((hb / MPW) << 10) | ((MPW * wr + hb % MPW) << 6) | (32 * (lg & 1));
            mx6_group_bf16(u, e >> 5);
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next row's writes
      } else if constexpr (HAD && OUT == 2) {
        // codes as fp32 to LDS in natural order, then each thread converts
        // groups t and t + T (32 consecutive codes each)
#pragma unroll
        for (int gi = 0; gi < 16; ++gi)
          *reinterpret_cast<float4*>(L + swz16(last_e(gi))) =
              make_float4(qf(v[4 * gi]), qf(v[4 * gi + 1]), qf(v[4 * gi + 2]), qf(v[4 * gi + 3]));
        __syncthreads();
        if (live) {
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int g = t + T * qq;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const float4 a = *reinterpret_cast<const float4*>(L + swz16(32 * g + 4 * u));
              v[4 * u] = a.x; v[4 * u + 1] = a.y; v[4 * u + 2] = a.z; v[4 * u + 3] = a.w;
            }
            mx6_group(v, g);
          }
        }
      } else if constexpr (!HAD) {
        // the thread's 64 elements are contiguous: pack and store directly
#pragma unroll
        for (int gq = 0; gq < 8; ++gq) {
          const uint32_t w0 = quant4(v + 8 * gq), w1 = quant4(v + 8 * gq + 4);
          qs[(2 * gq) % 4] = __builtin_amdgcn_sdot4((int)w0, 0x01010101, qs[(2 * gq) % 4], false);
          qs[(2 * gq + 1) % 4] = __builtin_amdgcn_sdot4((int)w1, 0x01010101, qs[(2 * gq + 1) % 4], false);
          const int e0 = SPREAD ? 8 * (t + T * gq) : (t << 6) | (8 * gq);
          if (live) {
            if constexpr (BITS == 8) {
              *reinterpret_cast<uint2*>(reinterpret_cast<int8_t*>(codes) + m * (int64_t)K + e0) = make_uint2(w0, w1);
            } else {
              reinterpret_cast<uint32_t*>(codes)[m * (int64_t)(K / 8) + (e0 >> 3)] =
                  (w0 & 0x0f0f0f0fu) | ((w1 & 0x0f0f0f0fu) << 4);
            }
          }
        }
      } else {
        // quantise groups of 4 consecutive elements; codes to LDS in natural
        // order: INT8 one byte per code; INT4 one word per group holding its
        // nibbles in half h = (e >> 2) & 1 of each byte (the other half zero),
        // so that two neighbouring groups OR into one packed word
        uint8_t* C8 = reinterpret_cast<uint8_t*>(L);
#pragma unroll
        for (int gi = 0; gi < 16; ++gi) {
          const uint32_t w = quant4(v + 4 * gi);
          qs[gi % 4] = __builtin_amdgcn_sdot4((int)w, 0x01010101, qs[gi % 4], false);
          const int e = last_e(gi);
          if constexpr (BITS == 8) {
            *reinterpret_cast<uint32_t*>(C8 + e) = w;
          } else {
            *reinterpret_cast<uint32_t*>(C8 + e) = (w & 0x0f0f0f0fu) << (4 * ((e >> 2) & 1));
          }
        }
        __syncthreads();
        if (live) {
          if constexpr (BITS == 8) {
            int8_t* dst = reinterpret_cast<int8_t*>(codes) + m * (int64_t)K;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int u = t + T * qq;  // 16-byte unit = 16 codes
              *reinterpret_cast<uint4*>(dst + 16 * u) = *reinterpret_cast<const uint4*>(C8 + 16 * u);
            }
          } else {
            uint32_t* dst = reinterpret_cast<uint32_t*>(codes) + m * (int64_t)(K / 8);
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
              const int u = t + T * qq;  // 4 output words = 8 groups
              const uint4 a = *reinterpret_cast<const uint4*>(C8 + 32 * u);
              const uint4 b = *reinterpret_cast<const uint4*>(C8 + 32 * u + 16);
              *reinterpret_cast<uint4*>(dst + 4 * u) = make_uint4(a.x | a.y, a.z | a.w, b.x | b.y, b.z | b.w);
            }
          }
        }
      }
      // (the FP6 x FP4 matmul needs no row sums)
      const int qsum = OUT == 2 ? 0 : row_reduce_int<T>((qs[0] + qs[1]) + (qs[2] + qs[3]), redi, row, t);
      if (live && t == 0) {
        // the row index made opaque here, so that the store addresses are
        // formed now from the base pointers rather than kept (and spilled)
        // across the loop: a reload would wait for the prefetched rows
        int64_t mi = m;
        asm volatile("" : "+v"(mi));
        scales[mi] = s;
        if (rowsum) rowsum[mi] = qsum;
      }
      // LDS and reduction scratch are reused by the next row group (with
      // WLOC each wave reuses only its own area, after its own reads; the
      // reduction scratch is rewritten only past the next row's pass-2
      // barrier)
      if constexpr (!WLOC) __syncthreads();
    }
  };
  // Rows of K = 16384 with the rotation to MX6 codes, at least 32 per
  // block: each XCD (blocks b with the same b % 8) takes a contiguous range
  // of rows, so that the rows in flight at once are neighbours and the
  // 64-byte halves of the MX6 layout's lines, written by neighbouring
  // rows, meet in one L2 (M = 65536: 764 -> 747 us; with 8 rows per block,
  // M = 4096, it was 2.6 % slower).
  if constexpr (LOG2K == 14 && HAD && OUT == 2 && BF16 && !NORM) {
    const int64_t P = gridDim.x;
    if (P % 8 == 0 && ngroups >= 32 * P) {
      const int64_t PX = P / 8, chunk = (ngroups + 7) / 8;
      const int64_t lo = (int64_t)(blockIdx.x % 8) * chunk, hi = min(lo + chunk, ngroups);
      int64_t grp = lo + blockIdx.x / 8;
      load_rows(raw0, grp < hi ? grp : ngroups);
      for (; grp < hi; grp += PX) row_group(raw0, grp, grp + PX < hi ? grp + PX : ngroups);
      return;
    }
  }
  const int64_t S = gridDim.x;
  int64_t grp = blockIdx.x;
  load_rows(raw0, grp);
  for (; grp < ngroups; grp += S) row_group(raw0, grp, grp + S);
}

// Few-token form of the rotation + INT8 quantisation (decode): one token row
// per block of K / 16 threads (16 waves at K = 16384), 16 elements per
// thread, so that the row's latency chain is spread over 4 waves per SIMD
// instead of one.  K = 2^k, k = 10 ... 14; bf16 input.
//   pass 1: wave w holds elements 1024 w .. + 1023, 16 chunks of 64; the
//           64-point transforms of its chunks run on the matrix cores as
//           Y = H_64 X with v_mfma_f32_16x16x32_bf16 (X: 64 elements x 16
//           chunks, two k-steps of 32; the bf16 inputs and +-1 entries are
//           exact, the sums fp32).  Lane l then holds elements 16 rb +
//           4 (l / 16) + j of chunk l % 16 (rb, j = 0..3): bits 0-5 done.
//   pass 2: through LDS (16-byte unit u of a wave's 1024-element area at
//           16 (u / 16) + ((u % 16) ^ (u / 16))), lane l takes element bits
//           0-5 = l and the 16 chunks: bits 6-9 in registers.
//   pass 3: back through LDS, thread t takes bits 10 .. k-1 (the waves)
//           and 16 / 2^(k-10) consecutive passengers: the last k - 10 stages.
// Then the row maximum, the codes by one fma against 1.5 * 2^23 (as the
// row-group kernel), and the codes through LDS in natural order for
// contiguous 16-byte stores.
// (The row's work, for a block of exactly K / 16 threads, in two parts: the
// loads of the pass-1 operands (row_load), then the rest
// (row_quant).  L holds K floats of LDS, redf and redi K / 1024
// entries each.  codes, scales and rowsum may point to LDS.)
// pass 1's B operand of k-step ks = 8 consecutive inputs of chunk lane % 16
template <int LOG2K>
__device__ __forceinline__ void row_load(const void* __restrict__ x, int64_t ldx, int64_t m, int tid,
                                              v8bf (&bx)[2], bool live = true) {
  const int lane = tid & 63, wave = tid >> 6, cc = lane & 15, g = lane >> 4;
  const __bf16* xr = reinterpret_cast<const __bf16*>(x) + (live ? m : 0) * ldx;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    bx[ks] = live ? *reinterpret_cast<const v8bf*>(xr + 1024 * wave + 64 * cc + 32 * ks + 8 * g)
                  : __builtin_bit_cast(v8bf, make_uint4(0u, 0u, 0u, 0u));
}

// BITS 8: INT8 absmax codes (Eq. 7), int8 [K]; BITS 4: INT4 absmean codes
// (Eq. 8), packed as the public INT4 layout (code j = 4 h + b of a word at
// bits 8 b + 4 h), K / 2 bytes, or, with MX, as MX6 operands of the FP6 x
// FP4 matmul (mx6_main_off, mx6_tail_off; codes is then the buffer base).
// RSUM false: no row sum (rowsum and redi unused; the one-launch decode
// layer takes each thread's code sums into its matmul instead).
template <int LOG2K, int BITS = 8, bool MX = false, bool RSUM = true>
__device__ __forceinline__ void row_quant(const v8bf (&bx)[2], int8_t* __restrict__ codes,
                                               float* __restrict__ scales, int32_t* __restrict__ rowsum, int64_t m,
                                               int tid, float* __restrict__ L, float* __restrict__ redf,
                                               int* __restrict__ redi) {
  constexpr int K = 1 << LOG2K, TR = K / 16, WB = LOG2K - 10, NWV = 1 << WB;
  constexpr int PB = 4 - WB, P = 1 << PB;  // passengers of pass 3
  const int lane = tid & 63, wave = tid >> 6;
  const int cc = lane & 15, g = lane >> 4;
  // A operand (rb, ks): rows 16 rb + i of H_64 (i = l % 16), columns 32 ks +
  // kk (kk = 8 (l / 16) + e, e = 0..7).  The row and column bits split into
  // disjoint parts, so H_64[16 rb + i][32 ks + kk] = (-1)^popcount(i & kk) *
  // (-1)^((rb & 1) (kk >> 4)) * (-1)^((rb >> 1) ks), and kk >> 4 = (l / 16) / 2
  // is the lane's: one base operand per lane, the others its sign flips.
  uint32_t hb[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    uint32_t h2 = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kk = 8 * g + 2 * pp + half;
      h2 |= ((__popc(cc & kk) & 1) ? 0xbf80u : 0x3f80u) << (16 * half);
    }
    hb[pp] = h2;
  }
  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f c[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    c[rb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t neg = ((((rb & 1) & (g >> 1)) ^ ((rb >> 1) & ks)) != 0) ? 0x80008000u : 0u;
      const v8bf ha = __builtin_bit_cast(v8bf, make_uint4(hb[0] ^ neg, hb[1] ^ neg, hb[2] ^ neg, hb[3] ^ neg));
      c[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha, bx[ks], c[rb], 0, 0, 0);
    }
  }
  float* Lw = L + 1024 * wave;
  auto unit = [](int u) { return 16 * (u >> 4) + ((u & 15) ^ (u >> 4)); };
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    *reinterpret_cast<float4*>(Lw + 4 * unit(16 * cc + 4 * rb + g)) = make_float4(c[rb][0], c[rb][1], c[rb][2], c[rb][3]);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // pass 2 reads the wave's own 1024 elements
  // pass 2: element bits 0-5 = lane, bits 6-9 = register index
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) v[q] = Lw[4 * unit(16 * q + (lane >> 2)) + (lane & 3)];
  butterflies<16, 0, 4>(v);
#pragma unroll
  for (int q = 0; q < 16; ++q) Lw[4 * unit(16 * q + (lane >> 2)) + (lane & 3)] = v[q];
  __syncthreads();
  // pass 3: register i = p + P w', element 1024 w' + P t + p
#pragma unroll
  for (int wv = 0; wv < NWV; ++wv)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int f = P * tid + p;
      v[p + P * wv] = L[1024 * wv + 4 * unit(f >> 2) + (f & 3)];
    }
  butterflies<16, PB, 4>(v);

  // INT8 absmax (Eq. 7) or INT4 absmean (Eq. 8) of the rotated row x_r = c v
  constexpr float scale = (LOG2K % 2 == 0) ? (float)(1.0 / (double)(1 << (LOG2K / 2))) : 0.0f;
  const float cn = (LOG2K % 2 == 0) ? scale : (float)(1.0 / __builtin_sqrt((double)K));
  float st = abs_tree<16, BITS == 8>(v);
  st = row_reduce<TR, BITS == 8>(st, redf, 0, tid);
  float f, s_out;
  if constexpr (BITS == 8) {
    const float gamma = st * cn;
    f = 127.0f / (gamma + kEps);
    s_out = gamma / 127.0f;
  } else {
    const float beta = (st * cn) / (float)K;
    f = kSqrt7 / (beta + kEps);
    s_out = beta / kSqrt7;
  }
  const float fc = cn * f;
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  constexpr int kMagicBits = 0x4b400000;
  constexpr int kLo = BITS == 8 ? -128 : -8, kHi = BITS == 8 ? 127 : 7;
  // Every thread's pass-3 reads are done (the row reduction's barrier, or
  // in-order LDS within a one-wave row).  Wave w holds the codes of elements
  // 1024 wv + 64 P w .. + 64 P - 1 for each wv: 16 spans of 64 P bytes, 1 KB,
  // which it stages in its own area (local byte 64 P wv + P l + p) and
  // stores as 16-byte pieces, with no block barrier.
  if constexpr (TR <= 64) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  int8_t* C8 = reinterpret_cast<int8_t*>(Lw);
#pragma unroll
  for (int wv = 0; wv < NWV; ++wv)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int bits = __float_as_int(__builtin_fmaf(v[p + P * wv], fc, kMagic));
      C8[64 * P * wv + P * lane + p] = (int8_t)(min(max(bits, kMagicBits + kLo), kMagicBits + kHi) - kMagicBits);
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own codes
  const uint4 q4 = *reinterpret_cast<const uint4*>(C8 + 16 * lane);
  {
    const int wv = (16 * lane) / (64 * P), o = (16 * lane) % (64 * P);
    const int64_t e = m * (int64_t)K + 1024 * wv + 64 * P * wave + o;  // first of the 16 codes
    if constexpr (MX) {
      static_assert(BITS == 4, "MX6 operands hold INT4 codes");
      // lanes 2 i and 2 i + 1 hold the 32 codes of group (e - m K) / 32 (o
      // is a multiple of 32 in even lanes); the even lane converts them
      // with the gfx950 packed E3M2 conversion (scale 1: exact for integers
      // in [-8, 7]), element 2 j of its first operand at field 2 j and
      // element j of its second at field 2 j + 1
      const uint32_t nb[4] = {(uint32_t)__shfl_xor((int)q4.x, 1), (uint32_t)__shfl_xor((int)q4.y, 1),
                              (uint32_t)__shfl_xor((int)q4.z, 1), (uint32_t)__shfl_xor((int)q4.w, 1)};
      if ((lane & 1) == 0) {
        const uint32_t own[4] = {q4.x, q4.y, q4.z, q4.w};
        v16f a, b;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c0 = 2 * i, c1 = 2 * i + 1;  // codes of the group
          const uint32_t w0 = c0 < 16 ? own[c0 >> 2] : nb[(c0 - 16) >> 2];
          const uint32_t w1 = c1 < 16 ? own[c1 >> 2] : nb[(c1 - 16) >> 2];
          a[i] = (float)(int)(int8_t)(w0 >> (8 * (c0 & 3)));
          b[i] = (float)(int)(int8_t)(w1 >> (8 * (c1 & 3)));
        }
        const auto r = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, 1.0f);
        const int g = (int)((e - m * (int64_t)K) >> 5);
        uint8_t* dst = reinterpret_cast<uint8_t*>(codes);
        *reinterpret_cast<uint4*>(dst + mx6_main_off(m, g, K)) = make_uint4(r[0], r[1], r[2], r[3]);
        *reinterpret_cast<uint2*>(dst + mx6_tail_off(m, g, K)) = make_uint2(r[4], r[5]);
      }
    } else if constexpr (BITS == 8) {
      *reinterpret_cast<uint4*>(codes + e) = q4;
    } else {
      // codes 0-3 of each group of 8 in the low nibbles, 4-7 in the high ones
      *reinterpret_cast<uint2*>(codes + e / 2) =
          make_uint2((q4.x & 0x0f0f0f0fu) | ((q4.y & 0x0f0f0f0fu) << 4), (q4.z & 0x0f0f0f0fu) | ((q4.w & 0x0f0f0f0fu) << 4));
    }
  }
  if constexpr (RSUM) {
    int qs = __builtin_amdgcn_sdot4((int)q4.x, 0x01010101, 0, false);
    qs = __builtin_amdgcn_sdot4((int)q4.y, 0x01010101, qs, false);
    qs = __builtin_amdgcn_sdot4((int)q4.z, 0x01010101, qs, false);
    qs = __builtin_amdgcn_sdot4((int)q4.w, 0x01010101, qs, false);
    qs = row_reduce_int<TR>(qs, redi, 0, tid);
    if (tid == 0 && rowsum) rowsum[m] = qs;
  }
  if (tid == 0) scales[m] = s_out;
}

template <int LOG2K, int BITS, bool MX>
__global__ void __launch_bounds__((1 << LOG2K) / 16)
k_fwht_quant_row(const void* __restrict__ x, int64_t ldx, int8_t* __restrict__ codes, float* __restrict__ scales,
                 int32_t* __restrict__ rowsum) {
  constexpr int K = 1 << LOG2K, NWV = K / 1024;
  __shared__ __attribute__((aligned(16))) float L[K];
  __shared__ float redf[NWV];
  __shared__ int redi[NWV];
  v8bf bx[2];
  row_load<LOG2K>(x, ldx, blockIdx.x, threadIdx.x, bx);
  row_quant<LOG2K, BITS, MX>(bx, codes, scales, rowsum, blockIdx.x, threadIdx.x, L, redf, redi);
}

// Decode layer of one or two tokens in one launch (H-BitLinear forward,
// INT8 codes, bf16 input, K = 2^k, k = 10 ... 14, MT tokens with MT K / 16
// <= 1024): every block of the dot-product matmul (gemv_dot_body, NB output
// features per block) issues the loads of the token rows, then its weight
// loads, and, while the weights are in flight, rotates and quantises the
// rows itself, one group of K / 16 threads per row (row_quant, the same
// arithmetic as k_fwht_quant_row, so the same codes; the groups pass the
// same barriers), keeping the codes and scales in its LDS (no row sum: each
// matmul thread subtracts the sum of its own codes instead, which takes a
// block reduction and its barrier off the rotation's chain).  Every
// block repeats that work (an n log n transform per row, small beside its
// share of the weight stream) so that no block waits for another and the
// layer needs no second launch.  Rows m >= M are zero and their outputs are
// not stored.  (A wave's loads complete in issue
// order: the rows are loaded before the weights, whose arrival the rotation
// does not need.)  From 8192 row elements per block (two tokens at K =
// 4096, one from K = 8192) every block first waits for its rows and only
// then issues its weights: issued together, the weight requests (16.8 MB
// at K = 16384) queue in front of the rows' and the quantisation starts
// late.  Us per layer, rotated / plain: one token at K = 16384 8.4 ->
// 7.4-7.8 / 7.2 -> 6.2, at 8192 5.24 -> 4.95 / 4.4 -> 3.9, two at 4096
// 4.9 -> 4.6 / 4.1 -> 3.7; below, the wait costs: one token at 4096 3.78
// -> 3.87 / 2.96 -> 3.07, two at 2048 3.50 -> 3.67, one at 1024 2.84 ->
// 2.98 (one at 2048 gains, 3.54 -> 3.37 / 2.96 -> 2.70, and is left out
// of the rule).
// 16 output features per block (256 blocks at N = 4096).  Measured with one
// token, us per layer at K = 16384 / 4096 (two tokens at 4096): 8 features
// per block - / 4.3 (5.7), 16: 8.5 / 3.7 (4.8), 32: 9.9 / 4.2 (5.2), 64:
// 14.5 at K = 16384; blocks beyond one per CU would run in a second round
// at K = 16384 (80 KB of LDS each)
template <int LOG2K>
constexpr int DecodeNB = 16;

// HAD false: plain BitLinear (Eq. 9 without the rotation), INT8 codes only:
// the row's absmax (order-free), f = 127 / (gamma + eps) and the codes by
// one fma against 1.5 * 2^23 with an integer clip, as the many-row
// quantiser computes them for unrotated rows, so that the layer equals its
// two launches bit for bit.  A thread quantises the 16 elements row_load
// gave it (two runs of 8) and stores their codes in place.
template <int LOG2K, int MT, int BITS, bool HAD = true>
__global__ void __launch_bounds__(MT * (1 << LOG2K) / 16)
k_decode_token(const void* __restrict__ x, int64_t ldx, int M, const uint32_t* __restrict__ wp,
               const float* __restrict__ alpha, void* __restrict__ out, int64_t ldo) {
  static_assert(HAD || BITS == 8, "plain one-launch layer: INT8 codes");
  constexpr int K = 1 << LOG2K, TR = K / 16, NT = MT * TR, TK = K / 64, NWV = K / 1024;
  constexpr int CB = K * BITS / 8;  // code bytes per row
  static_assert(NT <= 1024, "one block holds the rows");
  static_assert(DotGeom<MT, TK, NT, DecodeNB<LOG2K>>::RED_INTS <= MT * K, "the matmul's sums fit the row buffers");
  __shared__ __attribute__((aligned(16))) float L[MT * K];
  __shared__ __attribute__((aligned(16))) int8_t cl[MT * CB];
  __shared__ float redf[MT * NWV];
  __shared__ int redi[MT * NWV];
  __shared__ float s_tok[MT];
  const int tid = threadIdx.x, grp = tid / TR, gt = tid % TR;
  v8bf bx[2];
  gemv_dot_body<BITS, 0, MT, TK, NT, DecodeNB<LOG2K>, false, true>(
      cl, s_tok, nullptr, wp, alpha, M, K, out, ldo, blockIdx.x, tid, reinterpret_cast<int*>(L),
      [&] {
        row_load<LOG2K>(x, ldx, grp, gt, bx, grp < M);
        if constexpr (MT * K >= 8192) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the rows first
        __builtin_amdgcn_sched_barrier(0);  // the rows' loads are issued before the weights'
      },
      [&] {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (HAD) {
          row_quant<LOG2K, BITS, false, false>(bx, cl + grp * CB, s_tok + grp, nullptr, 0, gt, L + grp * K,
                                               redf + grp * NWV, redi + grp * NWV);
        } else {
          // row_load's runs: elements 1024 w + 64 (l % 16) + 32 ks + 8 (l / 16) + 0..7
          const int lane = gt & 63, wave = gt >> 6;
          float v[16];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const uint4 u = __builtin_bit_cast(uint4, bx[ks]);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[8 * ks + 2 * i] = __uint_as_float(w[i] << 16);
              v[8 * ks + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
          }
          float st = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) st = fmaxf(st, fabsf(v[i]));
          st = row_reduce<TR, true>(st, redf + grp * NWV, 0, gt);
          const float f = 127.0f / (st + kEps);
          constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
          constexpr int kMagicBits = 0x4b400000;
          int8_t* c8 = cl + grp * CB + 1024 * wave + 64 * (lane & 15) + 8 * (lane >> 4);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            uint32_t wq[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int b = __float_as_int(__builtin_fmaf(v[8 * ks + j], f, kMagic));
              const int q = min(max(b, kMagicBits - 128), kMagicBits + 127) - kMagicBits;
              wq[j >> 2] |= (uint32_t)(q & 0xff) << (8 * (j & 3));
            }
            *reinterpret_cast<uint2*>(c8 + 32 * ks) = make_uint2(wq[0], wq[1]);
          }
          if (gt == 0) s_tok[grp] = st / 127.0f;
        }
        __syncthreads();  // codes and scales in LDS
      });
}

// Plain (no rotation) quantisation for any K % 64 == 0, K <= 16384: one row
// per block of 256 threads, each holding up to 8 chunks of 8 elements.
template <bool BF16, int BITS, bool NORM>
__global__ void __launch_bounds__(256)
k_quant_plain(const void* __restrict__ x, int64_t M, int K, int64_t ldx,
              void* __restrict__ codes, float* __restrict__ scales,
              int32_t* __restrict__ rowsum, const float* __restrict__ gain) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int CH = 8;
  __shared__ float redf[4];
  __shared__ int redi[4];
  __shared__ float redn[4];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x;
  const int nchunk = K / 8;
  const char* xr = reinterpret_cast<const char*>(x) + m * ldx * ESZ;
  float v[CH * 8];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = tid + 256 * c;
    if (ch < nchunk) {
      load8<BF16>(xr + (int64_t)ch * 8 * ESZ, v + 8 * c);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[8 * c + j] = 0.0f;
    }
  }
  if constexpr (NORM) {
    // chunks past the row end are zero and hold a zero gain index: clamp it
    rmsnorm_apply<256, CH * 8>(v, sq_tree<CH * 8>(v), (float)K, gain, redn, 0, tid,
                               [&](int i) { const int ch = tid + 256 * (i >> 3);
                                            return (ch < nchunk ? 8 * ch : 0) + (i & 7); });
  }
  float st = 0.0f;
#pragma unroll
  for (int i = 0; i < CH * 8; ++i) st = (BITS == 8) ? fmaxf(st, fabsf(v[i])) : st + fabsf(v[i]);
  st = row_reduce<256, BITS == 8>(st, redf, 0, tid);
  float f, s;
  if constexpr (BITS == 8) {
    f = 127.0f / (st + kEps);
    s = st / 127.0f;
  } else {
    // mean as (fp64 of the fp32 sum) / K rounded once, K need not be a power of two
    const float beta = (float)((double)st / (double)K);
    f = kSqrt7 / (beta + kEps);
    s = beta / kSqrt7;
  }
  constexpr float lo = BITS == 8 ? -128.0f : -8.0f;
  constexpr float hi = BITS == 8 ? 127.0f : 7.0f;
  int qsum = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = tid + 256 * c;
    if (ch >= nchunk) continue;
    int q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float r = __builtin_rintf(v[8 * c + j] * f);
      q[j] = (int)fminf(fmaxf(r, lo), hi);
      qsum += q[j];
    }
    if constexpr (BITS == 8) {
      uint32_t w0 = (q[0] & 0xff) | ((q[1] & 0xff) << 8) | ((q[2] & 0xff) << 16) | ((uint32_t)q[3] << 24);
      uint32_t w1 = (q[4] & 0xff) | ((q[5] & 0xff) << 8) | ((q[6] & 0xff) << 16) | ((uint32_t)q[7] << 24);
      *reinterpret_cast<uint2*>(reinterpret_cast<int8_t*>(codes) + m * (int64_t)K + 8 * ch) = make_uint2(w0, w1);
    } else {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) w |= (uint32_t)(q[j] & 0xf) << (8 * (j & 3) + 4 * (j >> 2));
      reinterpret_cast<uint32_t*>(codes)[m * (int64_t)(K / 8) + ch] = w;
    }
  }
  qsum = row_reduce_int<256>(qsum, redi, 0, tid);
  if (tid == 0) {
    scales[m] = s;
    if (rowsum) rowsum[m] = qsum;
  }
}

// Token counts up to this take k_fwht_quant_row (INT8 codes with the
// rotation, bf16 input): measured on MI355X against the row-group kernel
// (us per call, graph replay): K = 16384 M = 1 5.37 -> 4.98, M = 256 8.10 ->
// 7.63, M = 512 10.63 -> 10.89 (slower); K = 4096 M = 1 4.03 -> 2.90, M =
// 1024 7.47 -> 6.81; K = 8192 M = 256 6.71 -> 4.91.  Beyond the thresholds
// (row-group -> row kernel, INT8 / INT4 / MX6 codes): K = 4096 M = 2048
// 7.8 / 7.2 / 8.3 -> 7.8 / 7.3 / 8.7; K = 8192 M = 1024 8.3 / 7.5 / 9.1 ->
// 8.3 / 7.4 / 8.8; K = 16384 M = 512 8.5 / 7.9 / 9.2 -> 9.0 / 8.2 / 9.4.
template <int LOG2K>
constexpr int64_t kRowKernelMaxM = LOG2K >= 14 ? 256 : 1024;

// Block size: rows of K <= 4096 (a wave or less per row) run in blocks of
// 64 threads (codes; up to 8 blocks per CU) or 128 (MX6 codes; up to 4 per
// CU), which need no barrier across rows; measured at K = 4096 against 256
// threads and 2 blocks per CU: codes 7-15 % faster at M = 1 ... 65536, MX6
// codes 2-11 %.  Longer rows, and the fp32 output, keep 256 threads.
template <int LOG2K, bool BF16, int BITS, bool HAD, int OUT, bool NORM>
hipError_t launch_fq64(const void* x, int64_t M, int64_t ldx, void* codes, float* scales, int32_t* rowsum,
                       float* y, const float* gain, int cu_count, hipStream_t s) {
  constexpr int BS = (LOG2K <= 12 && OUT != 1) ? (OUT == 2 ? 128 : 64) : 256;
  using G = G64<LOG2K, BS>;
  // persistent: as many blocks per CU as 128 KB of row buffers hold (two of
  // 256 threads)
  constexpr int PER_CU = BS == 256 ? 2 : 128 * 1024 / (4 * G::RPB * G::K);
  const int64_t groups = (M + G::RPB - 1) / G::RPB;
  const int64_t cap = (int64_t)PER_CU * (cu_count > 0 ? cu_count : 256);
  const int64_t blocks = groups < cap ? groups : cap;
  hipLaunchKernelGGL((k_fwht_quant64<LOG2K, BF16, BITS, HAD, OUT, NORM, BS>), dim3((unsigned)blocks), dim3(BS), 0, s,
                     x, M, ldx, codes, scales, rowsum, y, gain);
  return hipGetLastError();
}

template <int LOG2K, bool BF16, int BITS, bool HAD, int OUT, bool NORM>
hipError_t launch_fq(const void* x, int64_t M, int64_t ldx, void* codes, float* scales,
                     int32_t* rowsum, float* y, const float* gain, hipStream_t s) {
  using G = Geom<LOG2K>;
  const int64_t blocks = (M + G::RPB - 1) / G::RPB;
  hipLaunchKernelGGL((k_fwht_quant<LOG2K, BF16, BITS, HAD, OUT, NORM>), dim3((unsigned)blocks),
                     dim3(G::THREADS), 0, s, x, M, ldx, codes, scales, rowsum, y, gain);
  return hipGetLastError();
}

template <int LOG2K, bool NORM>
hipError_t dispatch_quant_mx(const void* x, bool bf16, int64_t M, int64_t ldx, bool had, void* codes,
                             float* scales, int32_t* rowsum, const float* gain, int cu, hipStream_t s) {
  if constexpr (LOG2K >= 10) {
#define HBL_MXQ(B16, HAD) \
  return launch_fq64<LOG2K, B16, 4, HAD, 2, NORM>(x, M, ldx, codes, scales, rowsum, nullptr, gain, cu, s)
    if (bf16) { if (had) HBL_MXQ(true, true); else HBL_MXQ(true, false); }
    else { if (had) HBL_MXQ(false, true); else HBL_MXQ(false, false); }
#undef HBL_MXQ
  } else {
    return hipErrorInvalidValue;
  }
}

template <int LOG2K, bool NORM>
hipError_t dispatch_quant(const void* x, bool bf16, int64_t M, int64_t ldx, bool had, int bits,
                          void* codes, float* scales, int32_t* rowsum, const float* gain, int cu,
                          hipStream_t s) {
  if constexpr (!NORM && LOG2K >= 10) {
    // few rotated bf16 rows: one row per block of K / 16 threads, for every
    // code layout (INT8, INT4, MX6), so that INT4 and MX6 codes of the same
    // rows still come from the same arithmetic
    if (bf16 && had && M <= kRowKernelMaxM<LOG2K>) {
#define HBL_ROW(BITS, MX)                                                                                   \
  hipLaunchKernelGGL((k_fwht_quant_row<LOG2K, BITS, MX>), dim3((unsigned)M), dim3((1 << LOG2K) / 16), 0, s, x, \
                     ldx, static_cast<int8_t*>(codes), scales, rowsum);                                     \
  return hipGetLastError()
      if (bits == 8) { HBL_ROW(8, false); }
      if (bits == 4) { HBL_ROW(4, false); }
      if (bits == 6) { HBL_ROW(4, true); }
#undef HBL_ROW
    }
  }
  if constexpr (!NORM)  // MX6 codes are written without the normalisation layer
    if (bits == 6) return dispatch_quant_mx<LOG2K, NORM>(x, bf16, M, ldx, had, codes, scales, rowsum, gain, cu, s);
#define HBL_FQ(B16, BITS, HAD)                                                                              \
  if constexpr (LOG2K >= 10)                                                                                \
    return launch_fq64<LOG2K, B16, BITS, HAD, 0, NORM>(x, M, ldx, codes, scales, rowsum, nullptr, gain, cu, \
                                                       s);                                                  \
  else                                                                                                      \
    return launch_fq<LOG2K, B16, BITS, HAD, 0, NORM>(x, M, ldx, codes, scales, rowsum, nullptr, gain, s)
  if (bf16) {
    if (had) { if (bits == 8) HBL_FQ(true, 8, true); else HBL_FQ(true, 4, true); }
    else { if (bits == 8) HBL_FQ(true, 8, false); else HBL_FQ(true, 4, false); }
  } else {
    if (had) { if (bits == 8) HBL_FQ(false, 8, true); else HBL_FQ(false, 4, true); }
    else { if (bits == 8) HBL_FQ(false, 8, false); else HBL_FQ(false, 4, false); }
  }
#undef HBL_FQ
}

template <bool NORM>
hipError_t launch_plain(const void* x, bool x_bf16, int64_t M, int K, int64_t ldx, int bits, void* codes,
                        float* scales, int32_t* rowsum, const float* gain, hipStream_t s) {
  if (x_bf16) {
    if (bits == 8)
      hipLaunchKernelGGL((k_quant_plain<true, 8, NORM>), dim3((unsigned)M), dim3(256), 0, s, x, M, K, ldx, codes,
                         scales, rowsum, gain);
    else
      hipLaunchKernelGGL((k_quant_plain<true, 4, NORM>), dim3((unsigned)M), dim3(256), 0, s, x, M, K, ldx, codes,
                         scales, rowsum, gain);
  } else {
    if (bits == 8)
      hipLaunchKernelGGL((k_quant_plain<false, 8, NORM>), dim3((unsigned)M), dim3(256), 0, s, x, M, K, ldx, codes,
                         scales, rowsum, gain);
    else
      hipLaunchKernelGGL((k_quant_plain<false, 4, NORM>), dim3((unsigned)M), dim3(256), 0, s, x, M, K, ldx, codes,
                         scales, rowsum, gain);
  }
  return hipGetLastError();
}

int ilog2(int K);

template <bool NORM>
hipError_t quant_by_k(const void* x, bool x_bf16, int64_t M, int K, int64_t ldx, bool hadamard, int bits,
                      void* codes, float* scales, int32_t* rowsum, const float* gain, int cu, hipStream_t s) {
  if ((K & (K - 1)) != 0) {  // only reachable without the rotation (the ABI layer rejects it otherwise)
    if (bits == 6) return hipErrorInvalidValue;  // MX6 codes: K a power of two >= 1024
    return launch_plain<NORM>(x, x_bf16, M, K, ldx, bits, codes, scales, rowsum, gain, s);
  }
#define HBL_QK(L) \
  case L: return dispatch_quant<L, NORM>(x, x_bf16, M, ldx, hadamard, bits, codes, scales, rowsum, gain, cu, s);
  switch (ilog2(K)) {
    HBL_QK(4) HBL_QK(5) HBL_QK(6) HBL_QK(7) HBL_QK(8) HBL_QK(9)
    HBL_QK(10) HBL_QK(11) HBL_QK(12) HBL_QK(13) HBL_QK(14)
    default: return hipErrorInvalidValue;
  }
#undef HBL_QK
}

int ilog2(int K) {
  int l = 0;
  while ((1 << l) < K) ++l;
  return l;
}

}  // namespace

hipError_t launch_hadamard_quant(const void* x, bool x_bf16, int64_t M, int K, int64_t ldx,
                                 bool hadamard, int bits, void* codes, float* scales,
                                 int32_t* rowsum, bool norm, const float* gain, int cu, hipStream_t s) {
  if (M == 0) return hipSuccess;
  return norm ? quant_by_k<true>(x, x_bf16, M, K, ldx, hadamard, bits, codes, scales, rowsum, gain, cu, s)
              : quant_by_k<false>(x, x_bf16, M, K, ldx, hadamard, bits, codes, scales, rowsum, nullptr, cu, s);
}

// (Before the rows-first wait and the code-first two-launch GEMV, two
// rotated tokens at K = 8192 measured 10.8 us in one launch against about
// 8 in two; with both, 6.9 against 7.8.)
// Tokens the one-launch layer takes (at most 1024 threads, K / 16 per
// token), where it measured faster than the two launches: plain INT8,
// whose quantisation is one reduction, every such count; rotated, not
// three or four tokens at K = 4096 (us, two launches -> one: 6.56 -> 6.7,
// 6.58 -> 6.9), but four at K = 1024 (5.16 -> 3.50) and 2048 (5.68 ->
// 4.69) and two at 8192 (7.8 -> 6.9)
int decode_token_max_m(int64_t K, bool hadamard) {
  if (hadamard) return K > 8192 ? 1 : K > 2048 ? 2 : 4;
  return K > 8192 ? 1 : K > 4096 ? 2 : 4;
}

template <int L, int MT>
constexpr int decode_nb() { return DotGeom<MT, (1 << L) / 64, MT * (1 << L) / 16, DecodeNB<L>>::NB; }

bool decode_token_applies(bool x_bf16, int64_t M, int64_t N, int64_t K, bool hadamard, bool norm, int bits) {
  // rotated: INT8 or INT4 codes; plain: INT8 codes
  if (!((bits == 8 || (bits == 4 && hadamard)) && x_bf16 && !norm && K >= 1024 && K <= 16384 && (K & (K - 1)) == 0))
    return false;
  if (M < 1 || M > decode_token_max_m(K, hadamard)) return false;
  return N % 16 == 0;  // features per block (decode_nb)
}

hipError_t launch_decode_token(const void* x, int64_t ldx, int64_t M, int K, int bits, bool hadamard,
                               const uint32_t* wp, const float* alpha, int64_t N, void* out, int64_t ldo,
                               hipStream_t s) {
#define HBL_DT(L, MT)                                                                                            \
  {                                                                                                              \
    constexpr int NB = decode_nb<L, MT>();                                                                       \
    if (N % NB != 0) return hipErrorInvalidValue;                                                                \
    const dim3 grid((unsigned)(N / NB)), block(MT * (1 << L) / 16);                                              \
    if (!hadamard)                                                                                               \
      hipLaunchKernelGGL((k_decode_token<L, MT, 8, false>), grid, block, 0, s, x, ldx, (int)M, wp, alpha, out,   \
                         ldo);                                                                                   \
    else if (bits == 8)                                                                                          \
      hipLaunchKernelGGL((k_decode_token<L, MT, 8>), grid, block, 0, s, x, ldx, (int)M, wp, alpha, out, ldo);   \
    else                                                                                                         \
      hipLaunchKernelGGL((k_decode_token<L, MT, 4>), grid, block, 0, s, x, ldx, (int)M, wp, alpha, out, ldo);   \
    return hipGetLastError();                                                                                    \
  }
#define HBL_DTP(L, MT)                                                                                           \
  {                                                                                                              \
    constexpr int NB = decode_nb<L, MT>();                                                                       \
    if (N % NB != 0) return hipErrorInvalidValue;                                                                \
    hipLaunchKernelGGL((k_decode_token<L, MT, 8, false>), dim3((unsigned)(N / NB)), dim3(MT * (1 << L) / 16), 0, \
                       s, x, ldx, (int)M, wp, alpha, out, ldo);                                                  \
    return hipGetLastError();                                                                                    \
  }
  if (bits != 8 && (bits != 4 || !hadamard)) return hipErrorInvalidValue;
  if (M < 1 || M > decode_token_max_m(K, hadamard)) return hipErrorInvalidValue;
  if (M > 2) {  // 3 or 4 tokens: K <= 2048, or plain at 4096
    switch (ilog2(K)) {
      case 10: HBL_DT(10, 4)
      case 11: HBL_DT(11, 4)
      case 12: HBL_DTP(12, 4)
      default: return hipErrorInvalidValue;
    }
  }
  switch (ilog2(K)) {
    case 10: if (M == 1) HBL_DT(10, 1) else HBL_DT(10, 2)
    case 11: if (M == 1) HBL_DT(11, 1) else HBL_DT(11, 2)
    case 12: if (M == 1) HBL_DT(12, 1) else HBL_DT(12, 2)
    case 13: if (M == 1) HBL_DT(13, 1) else HBL_DT(13, 2)
    case 14: HBL_DT(14, 1)
    default: return hipErrorInvalidValue;
  }
#undef HBL_DTP
#undef HBL_DT
}

hipError_t launch_hadamard_f32(const void* x, bool x_bf16, int64_t M, int K, int64_t ldx, float* y, int cu,
                               hipStream_t s) {
  if (M == 0) return hipSuccess;
#define HBL_HF(L)                                                                              \
  case L:                                                                                      \
    return x_bf16 ? launch_fq<L, true, 8, true, 1, false>(x, M, ldx, nullptr, nullptr, nullptr, y, nullptr, s) \
                  : launch_fq<L, false, 8, true, 1, false>(x, M, ldx, nullptr, nullptr, nullptr, y, nullptr, s);
#define HBL_HF64(L)                                                                                      \
  case L:                                                                                                \
    return x_bf16 ? launch_fq64<L, true, 8, true, 1, false>(x, M, ldx, nullptr, nullptr, nullptr, y, nullptr, cu, s)     \
                  : launch_fq64<L, false, 8, true, 1, false>(x, M, ldx, nullptr, nullptr, nullptr, y, nullptr, cu, s);
  switch (ilog2(K)) {
    HBL_HF(4) HBL_HF(5) HBL_HF(6) HBL_HF(7) HBL_HF(8) HBL_HF(9)
    HBL_HF64(10) HBL_HF64(11) HBL_HF64(12) HBL_HF64(13) HBL_HF64(14)
    default: return hipErrorInvalidValue;
  }
#undef HBL_HF
#undef HBL_HF64
}

}  // namespace hbl
