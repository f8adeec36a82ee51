// Post-RoPE QKV / KV-cache quantiser (architecture write-up of "BitNet v2",
// §3.4 "QKV Attention Quantization: Post-RoPE INT4/3-bit").
//
// The QKV heads are quantised to unsigned integers with the absmax
// function, without calibration; the KV heads of the [BOS] token stay at
// 8 bits.  Reading of the unsigned mapping (the pages give no formula): the
// absmax quantiser of Eq. 7 at b bits, Q = 2^(b-1) - 1, shifted by 2^(b-1):
//   gamma = max |x| over the head's D elements, f = Q / (gamma + eps),
//   u = RoundClip(x f, -2^(b-1), 2^(b-1) - 1) + 2^(b-1),   scale = gamma / Q.
// The factor is formed once per head with an IEEE divide; each code is
// rint of the fp32 product (no fused multiply-add), like Eq. 7's path.
//
// Layout: x is [B][S][H][D] contiguous; codes [B][S][H][D b / 8] bytes
// (b = 8 one byte per code; b = 4 code 2i in the low nibble of byte i; b = 3
// eight codes per three bytes, code j of the eight at bits 3 j of the
// 24-bit little-endian value); scales [B][S][H].  With keep_bos8, position
// 0 of each sequence is also written at 8 bits to bos_codes [B][H][D] and
// bos_scales [B][H].
//
// One lane per 32 consecutive elements, D / 32 consecutive lanes per head
// (D a power of two, 32 .. 2048), a grid of up to 128 blocks per CU that
// strides over larger inputs; the head's maximum is reduced across its lanes
// with xor shuffles.  Memory-bound: 2 (bf16) or 4 (fp32) bytes read
// and b / 8 written per element.
#include "hbl_internal.h"

namespace hbl {
namespace {

constexpr float kKvEps = 1e-5f;

__device__ __forceinline__ float bf16lo_kv(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi_kv(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// unsigned b-bit codes of the 32 values in v
template <int BITS>
__device__ __forceinline__ void kv_codes(const float* v, float f, uint32_t (&u)[32]) {
  constexpr int HALF = 1 << (BITS - 1);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float r = __builtin_rintf(v[i] * f);
    const float c = fminf(fmaxf(r, (float)-HALF), (float)(HALF - 1));
    u[i] = (uint32_t)((int)c + HALF);
  }
}

// the 32 codes packed into 32 b / 8 bytes, stored at dst (4-byte aligned)
template <int BITS>
__device__ __forceinline__ void kv_store(const uint32_t (&u)[32], uint8_t* dst) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int w = 0; w < 8; w += 4) {
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = u[4 * (w + q)] | (u[4 * (w + q) + 1] << 8) | (u[4 * (w + q) + 2] << 16) | (u[4 * (w + q) + 3] << 24);
      *reinterpret_cast<uint4*>(dst + 4 * w) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else if constexpr (BITS == 4) {
    uint32_t o[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t t = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) t |= u[8 * w + n] << (4 * n);
      o[w] = t;
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    uint32_t g[4];  // 24-bit groups of 8 codes
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t t = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) t |= u[8 * k + j] << (3 * j);
      g[k] = t;
    }
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);
    d[0] = g[0] | (g[1] << 24);
    d[1] = (g[1] >> 8) | (g[2] << 16);
    d[2] = (g[2] >> 16) | (g[3] << 8);
  }
}

template <bool BF16, int BITS, int L>  // L lanes per head (D = 32 L)
__global__ void __launch_bounds__(256)
k_kv_quant(const void* __restrict__ x, int64_t groups, int64_t S, int64_t H, int keep_bos8,
           uint8_t* __restrict__ codes, float* __restrict__ scales, uint8_t* __restrict__ bos_codes,
           float* __restrict__ bos_scales) {
  constexpr int D = 32 * L;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int CB = D * BITS / 8;  // code bytes per head
  const int64_t lanes = groups * L;
  for (int64_t gl = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gl - (threadIdx.x & 63) < lanes;
       gl += (int64_t)gridDim.x * blockDim.x) {
    // the whole wave runs each iteration (the reductions below need every
    // lane); lanes past the end compute on zeros and store nothing
    const bool live = gl < lanes;
    const int64_t g = live ? gl / L : 0;
    const int j = (int)(gl % L);
    float v[32];
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) + (g * D + 32 * j) * ESZ);
    if constexpr (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 a = live ? src[q] : make_uint4(0, 0, 0, 0);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * q + 2 * i] = bf16lo_kv(w[i]);
          v[8 * q + 2 * i + 1] = bf16hi_kv(w[i]);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 a = live ? src[q] : make_uint4(0, 0, 0, 0);
        v[4 * q] = __uint_as_float(a.x); v[4 * q + 1] = __uint_as_float(a.y);
        v[4 * q + 2] = __uint_as_float(a.z); v[4 * q + 3] = __uint_as_float(a.w);
      }
    }
    float m[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) m[i] = fmaxf(fabsf(v[i]), fabsf(v[i + 16]));
#pragma unroll
    for (int w = 8; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) m[i] = fmaxf(m[i], m[i + w]);
    float gamma = m[0];
#pragma unroll
    for (int o = 1; o < L; o *= 2) gamma = fmaxf(gamma, __shfl_xor(gamma, o));
    constexpr float Q = (float)((1 << (BITS - 1)) - 1);
    const float f = Q / (gamma + kKvEps);
    uint32_t u[32];
    kv_codes<BITS>(v, f, u);
    if (live) {
      kv_store<BITS>(u, codes + g * CB + j * (32 * BITS / 8));
      if (j == 0) scales[g] = gamma / Q;
    }
    if constexpr (BITS != 8) {
      const int64_t t = g / H;  // token index b S + s
      if (keep_bos8 && live && t % S == 0) {
        const int64_t bh = (t / S) * H + g % H;
        const float f8 = 127.0f / (gamma + kKvEps);
        kv_codes<8>(v, f8, u);
        kv_store<8>(u, bos_codes + bh * D + 32 * j);
        if (j == 0) bos_scales[bh] = gamma / 127.0f;
      }
    } else {
      const int64_t t = g / H;
      if (keep_bos8 && live && t % S == 0) {
        const int64_t bh = (t / S) * H + g % H;
        kv_store<8>(u, bos_codes + bh * D + 32 * j);
        if (j == 0) bos_scales[bh] = gamma / Q;
      }
    }
  }
}

template <bool BF16, int BITS>
hipError_t launch_kv_l(const void* x, int64_t groups, int64_t S, int64_t H, int D, int keep, uint8_t* c, float* s,
                       uint8_t* bc, float* bs, int cu, hipStream_t st) {
  const int L = D / 32;
  const int64_t lanes = groups * L;
  const int64_t want = (lanes + 255) / 256;
  // up to 128 blocks per CU: at one 7B layer's K states (2^23 lanes) every
  // lane then quantises one group (122 us), against 135 us when 16 blocks
  // per CU stride over the groups
  const int64_t cap = 128 * (int64_t)(cu > 0 ? cu : 256);
  const unsigned blocks = (unsigned)(want < cap ? want : cap);
#define HBL_KV(LL)                                                                                               \
  case LL:                                                                                                       \
    hipLaunchKernelGGL((k_kv_quant<BF16, BITS, LL>), dim3(blocks), dim3(256), 0, st, x, groups, S, H, keep, c, s, \
                       bc, bs);                                                                                  \
    break;
  switch (L) {
    HBL_KV(1) HBL_KV(2) HBL_KV(4) HBL_KV(8) HBL_KV(16) HBL_KV(32) HBL_KV(64)
    default: return hipErrorInvalidValue;
  }
#undef HBL_KV
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_quant(const void* x, bool x_bf16, int64_t B, int64_t S, int64_t H, int D, int bits,
                           int keep_bos8, void* codes, float* scales, void* bos_codes, float* bos_scales, int cu,
                           hipStream_t s) {
  const int64_t groups = B * S * H;
  if (groups == 0) return hipSuccess;
  uint8_t* c = static_cast<uint8_t*>(codes);
  uint8_t* bc = static_cast<uint8_t*>(bos_codes);
#define HBL_KVB(BF, BITS) return launch_kv_l<BF, BITS>(x, groups, S, H, D, keep_bos8, c, scales, bc, bos_scales, cu, s)
  if (x_bf16) {
    if (bits == 3) HBL_KVB(true, 3);
    if (bits == 4) HBL_KVB(true, 4);
    HBL_KVB(true, 8);
  } else {
    if (bits == 3) HBL_KVB(false, 3);
    if (bits == 4) HBL_KVB(false, 4);
    HBL_KVB(false, 8);
  }
#undef HBL_KVB
}

}  // namespace hbl
