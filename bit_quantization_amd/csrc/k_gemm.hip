// Ternary-weight integer matmul with the rescale of Eq. 9 (architecture
// write-up of "BitNet v2", §3.4 "H-BitLinear"), for gfx950:
//   acc[m][n] = sum_k q_x[m][k] q_w[n][k],  out = (scale_m * alpha) * acc.
//
// Two kernels:
//   k_gemm -- large token counts.  Block tile 256 x 256 (8 waves of
//     128 x 64) or 128 x 128 (4 waves of 64 x 64), each wave a tile of
//     16x16x64 int8 MFMAs with int32 accumulators.  Codes and weights are staged to LDS
//     as they are stored (packed) and widened by each wave after its LDS
//     read.  Weights are decoded from two bits to the unsigned byte
//     c = q + 1 in {0, 1, 2}, so the MFMA sums q_x * c; the epilogue
//     subtracts sum_k q_x (the token's row sum of codes) to obtain
//     sum_k q_x * q_w exactly.
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

// An LDS stage holds S = 2 MFMA k-steps (128 codes: 64 bytes per row for
// INT4, 128 for INT8).  Lane group g = lane/16 of
// a fragment covers the S consecutive weight words S*g .. S*g + S-1 of the
// stage: one LDS read per lane brings the weights of all S steps, and step s
// uses word S*g + s with the matching 16 codes.  Widening:
//   weights:  word -> {w & m, w>>2 & m, w>>4 & m, w>>6 & m}, m = 0x03030303,
//             the bytes c = q_w + 1;
//   INT4:     word -> {(w << 4) & 0xf0f0f0f0, w & 0xf0f0f0f0}, the bytes
//             16 q_x (a nibble in the high half of a byte is 16 times its
//             value as a signed byte), so the sums carry a factor 16;
//   INT8:     bytes as stored.
// Epilogue: sum q_x q_w = sum q_x c / (16 for INT4) - rowsum.
//
// LDS rows are not padded; 16-byte units are XOR-swizzled by row so that
// the 16-lane column reads of the fragments and the row-contiguous staging
// writes both touch distinct banks (64 banks of 4 bytes):
//   INT8 codes row (128 B):    unit u of row r at u ^ ((r >> 1) & 7)
//   INT4 codes row (64 B):     unit u of row r at u ^ ((r >> 2) & 3)
//   weights row (32 B):        unit u of row r at u ^ ((r >> 3) & 1)
template <int BITS, int OUT, int BM, int BN, int WGM, int WGN, int MINB>
__global__ void __launch_bounds__(64 * WGM * WGN, MINB)
k_gemm(const void* __restrict__ codes, const float* __restrict__ scales,
       const int32_t* __restrict__ rowsum, const uint32_t* __restrict__ wp,
       const float* __restrict__ alpha, int64_t M, int64_t N, int64_t K,
       void* __restrict__ out, int64_t ldo, int tilesM, int tilesN) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int S = 2;                         // MFMA k-steps per stage
  constexpr int BKC = 64 * S;                  // codes per row per stage
  constexpr int AROW = BKC * BITS / 8;         // code bytes per row per stage
  constexpr int BROW = 16 * S;                 // weight bytes per row per stage
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int BCPR = BROW / 16;              // weight chunks per row
  constexpr int PA = BM * AROW / 16 / NT;      // 16-byte staging chunks per thread
  constexpr int PB = BN * BROW / 16 / NT;
  static_assert(PA * NT * 16 == BM * AROW && PB * NT * 16 == BN * BROW, "staging must divide evenly");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "fragment rows");
  constexpr int SPR = BITS == 4 ? 2 : 1;       // MFMA steps per 16-byte code read
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * AROW];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * BROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;

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

  const int64_t arow_bytes = BITS == 4 ? K / 2 : K;  // global code row stride
  const int64_t brow_bytes = K / 4;                  // global weight row stride
  const uint8_t* A8 = reinterpret_cast<const uint8_t*>(codes);
  const uint8_t* B8 = reinterpret_cast<const uint8_t*>(wp);

  // LDS byte offsets (swizzled) of 16-byte unit u of row r
  auto aoff = [](int r, int u) {
    if constexpr (BITS == 8) return r * AROW + 16 * (u ^ ((r >> 1) & 7));
    else return r * AROW + 16 * (u ^ ((r >> 2) & 3));
  };
  auto boff = [](int r, int u) { return r * BROW + 16 * (u ^ ((r >> 3) & 1)); };

  // Staging: chunk p of this thread is row r0 + RPP*p of the tile, 16-byte
  // unit col.  Every load is issued at a valid address (rows past the end
  // re-read the last row, k past the end re-reads offset 0) and zeroed when
  // out of range, so the stage body has no branches.  RPP is a multiple of
  // 16, so the swizzle of a chunk's row does not depend on p and every LDS
  // offset is one base plus a constant.
  constexpr int ACPR = AROW / 16;                    // code chunks per row
  constexpr int A_RPP = NT / ACPR, B_RPP = NT / BCPR;  // rows per staging pass
  static_assert(A_RPP % 16 == 0 && B_RPP % 16 == 0, "swizzle period");
  const int ar0 = tid / ACPR, acol = tid % ACPR;
  const int br0 = tid / BCPR, bcol = tid % BCPR;
  const int la0 = aoff(ar0, acol), lb0 = boff(br0, bcol);
  // The staging loads of a stage are issued in two halves, each written to
  // LDS halfway through the compute, to halve the registers they hold.
  static_assert(PA % 2 == 0 && (PB % 2 == 0 || PB == 1), "halves");
  constexpr int HA = PA / 2, HB = PB >= 2 ? PB / 2 : PB;
  uint4 ra[HA], rb[HB];
  auto gload = [&](int kt, int part) {
    const int64_t ka = (int64_t)kt * AROW + 16 * acol, kb = (int64_t)kt * BROW + 16 * bcol;
    const bool oka = ka < arow_bytes, okb = kb < brow_bytes;
#pragma unroll
    for (int q = 0; q < HA; ++q) {
      const int64_t row = m0 + ar0 + A_RPP * (part * HA + q);
      const bool ok = oka && row < M;
      const uint4 v = *reinterpret_cast<const uint4*>(A8 + (row < M ? row : M - 1) * arow_bytes +
                                                      (oka ? ka : 16 * acol));
      ra[q] = ok ? v : make_uint4(0, 0, 0, 0);
    }
    if (PB >= 2 || part == 0) {
#pragma unroll
      for (int q = 0; q < HB; ++q) {
        const int64_t row = n0 + br0 + B_RPP * (part * HB + q);
        const bool ok = okb && row < N;
        const uint4 v = *reinterpret_cast<const uint4*>(B8 + (row < N ? row : N - 1) * brow_bytes +
                                                        (okb ? kb : 16 * bcol));
        rb[q] = ok ? v : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf, int part) {
#pragma unroll
    for (int q = 0; q < HA; ++q)
      *reinterpret_cast<uint4*>(&As[buf][la0 + A_RPP * AROW * (part * HA + q)]) = ra[q];
    if (PB >= 2 || part == 0) {
#pragma unroll
      for (int q = 0; q < HB; ++q)
        *reinterpret_cast<uint4*>(&Bs[buf][lb0 + B_RPP * BROW * (part * HB + q)]) = rb[q];
    }
  };

  v4i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int nk = (int)((K + BKC - 1) / BKC);
  const int fr = lane % 16, g = lane / 16;
  // Fragment rows are wm*WM + 16*j + fr (codes) and wn*WN + 16*i + fr
  // (weights): the swizzle depends on fr only, and fragment j (i) sits at a
  // constant offset from fragment 0.
  // codes of lane group g: unit g (INT4: both steps) or units 2g, 2g+1
  // (INT8: one per step); weights: 8 bytes, half (g & 1) of unit g >> 1
  const int abase0 = BITS == 4 ? aoff(wm * WM + fr, g) : aoff(wm * WM + fr, 2 * g);
  const int abase1 = BITS == 4 ? abase0 : aoff(wm * WM + fr, 2 * g + 1);
  const int bbase = boff(wn * WN + fr, g >> 1) + 8 * (g & 1);
  constexpr int AFRAG = 16 * AROW, BFRAG = 16 * BROW;  // bytes between fragments

  gload(0, 0);
  sstore(0, 0);
  gload(0, 1);
  sstore(0, 1);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const uint8_t* Ab = As[cur];
    const uint8_t* Bb = Bs[cur];
    const int kn = kt + 1 < nk ? kt + 1 : kt;  // the last stage re-reads itself into the spare buffer
    gload(kn, 0);
    uint32_t bw[FN][S];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const uint2 u = *reinterpret_cast<const uint2*>(Bb + bbase + BFRAG * i);
      bw[i][0] = u.x;
      bw[i][1] = u.y;
    }
#pragma unroll
    for (int h = 0; h < S / SPR; ++h) {
      uint4 ar[FM];
#pragma unroll
      for (int j = 0; j < FM; ++j) ar[j] = *reinterpret_cast<const uint4*>(Ab + (h ? abase1 : abase0) + AFRAG * j);
#pragma unroll
      for (int t = 0; t < SPR; ++t) {
        const int s = h * SPR + t;
        v4i bf[FN];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const uint32_t w = bw[i][s];
          bf[i] = v4i{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
                      (int)((w >> 6) & 0x03030303u)};
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          v4i af;
          if constexpr (BITS == 4) {
            const uint32_t x0 = t == 0 ? ar[j].x : ar[j].z, x1 = t == 0 ? ar[j].y : ar[j].w;
            af = v4i{(int)((x0 << 4) & 0xf0f0f0f0u), (int)(x0 & 0xf0f0f0f0u), (int)((x1 << 4) & 0xf0f0f0f0u),
                     (int)(x1 & 0xf0f0f0f0u)};
          } else {
            af = v4i{(int)ar[j].x, (int)ar[j].y, (int)ar[j].z, (int)ar[j].w};
          }
#pragma unroll
          for (int i = 0; i < FN; ++i) acc[i][j] = mfma16x16x64(bf[i], af, acc[i][j]);
        }
        if (s == S / 2 - 1) {
          sstore(cur ^ 1, 0);
          gload(kn, 1);
        }
      }
    }
    sstore(cur ^ 1, 1);
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
      const int64_t n = n0 + wn * WN + 16 * i + 4 * g;
      if (n >= N) continue;
      v4i a = acc[i][j];
      if constexpr (BITS == 4) a = a >> 4;  // exact: every product carries a factor 16
      store4<OUT>(out, m * ldo + n, a, R, sc);
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

// ---------------------------------------------------------------------------
// Decode with very few tokens (M <= 4), K % 1024 == 0: dot-product kernel.
// A block of 512 threads owns NB output features.  Thread t covers the 64
// codes k = 64*(t % TK) .. +63 (TK = min(256, K/64) threads per feature row)
// of RPT = NB / (512 / TK) of those features; it loads the tokens' codes for
// its k-range once (registers) and streams the rows' packed weights with one
// 16-byte load per row (consecutive threads read consecutive 16 bytes of a
// row).  Each weight word gives 4 dwords of bytes c = q_w + 1, multiplied
// into the codes with v_dot4_i32_i8; INT4 codes are widened to 16 q_x (the
// sums are divided by 16 at the end, exactly).  Partial sums are reduced
// over the TK threads of a row (xor-butterflies within a wave, then a fixed
// order over the waves), then rescaled.
template <int BITS, int OUT, int MT, int TK>
struct DotGeom {
  static constexpr int NTH = 512;                          // threads per block
  static constexpr int RP = NTH / TK;                      // feature rows side by side
  static constexpr int NB = RP > 8 ? RP : 8;               // features per block
  static constexpr int RPT = NB / RP;                      // rows per thread
};

template <int BITS, int OUT, int MT, int TK>
__global__ void __launch_bounds__(512)
k_gemv_dot(const void* __restrict__ codes, const float* __restrict__ scales,
           const int32_t* __restrict__ rowsum, const uint32_t* __restrict__ wp,
           const float* __restrict__ alpha, int M, int64_t N, int64_t K,
           void* __restrict__ out, int64_t ldo) {
  using DG = DotGeom<BITS, OUT, MT, TK>;
  constexpr int NB = DG::NB;
  __shared__ int red[DG::NTH / 64][NB][MT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  static_assert(TK >= 16 && TK <= 256, "threads per feature row");
  constexpr int RP = DG::RP;
  constexpr int RPT = DG::RPT;
  const int kt = tid % TK, rg = tid / TK;
  const int64_t n0 = (int64_t)blockIdx.x * NB;
  const int64_t KW = K / 16;

  // the weights: rows n0 + rg + RP*i, words 4*kt .. 4*kt+3; issue every load first
  uint4 w[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) w[i] = load_stream(wp + (n0 + rg + (int64_t)RP * i) * KW + 4 * kt);

  // the tokens' codes for k = 64*kt .. +63, as 16 dwords of signed bytes
  uint32_t x[MT][16];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < M) {
      if constexpr (BITS == 8) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const int8_t*>(codes) + (int64_t)m * K + 64 * kt);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 u = p[q];
          x[m][4 * q] = u.x; x[m][4 * q + 1] = u.y; x[m][4 * q + 2] = u.z; x[m][4 * q + 3] = u.w;
        }
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint32_t*>(codes) + (int64_t)m * (K / 8) + 8 * kt);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint4 u = p[q];
          const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[m][8 * q + 2 * j] = (ww[j] << 4) & 0xf0f0f0f0u;  // codes 0-3 of the word, as 16 q
            x[m][8 * q + 2 * j + 1] = ww[j] & 0xf0f0f0f0u;     // codes 4-7
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) x[m][j] = 0;
    }
  }

  int acc[RPT][MT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = 0;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t c0 = ws[q] & 0x03030303u, c1 = (ws[q] >> 2) & 0x03030303u;
      const uint32_t c2 = (ws[q] >> 4) & 0x03030303u, c3 = (ws[q] >> 6) & 0x03030303u;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int a = acc[i][m];
        a = __builtin_amdgcn_sdot4((int)c0, (int)x[m][4 * q], a, false);
        a = __builtin_amdgcn_sdot4((int)c1, (int)x[m][4 * q + 1], a, false);
        a = __builtin_amdgcn_sdot4((int)c2, (int)x[m][4 * q + 2], a, false);
        a = __builtin_amdgcn_sdot4((int)c3, (int)x[m][4 * q + 3], a, false);
        acc[i][m] = a;
      }
    }
  }
  // reduce over the TK threads of each row: within the wave over the lanes
  // of the same row group, then over the waves holding that row group
  constexpr int lanes_per_row = TK < 64 ? TK : 64;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      int v = acc[i][m];
#pragma unroll
      for (int o = 1; o < lanes_per_row; o <<= 1) v += __shfl_xor(v, o);
      acc[i][m] = v;
    }
  }
  // lane 0 of each row group in each wave publishes its partials
  if ((lane % lanes_per_row) == 0) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + RP * i;  // feature within the block
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wave][row][m] = acc[i][m];
    }
  }
  __syncthreads();
  if (tid < NB * MT) {
    const int row = tid / MT, m = tid % MT;
    if (m < M) {
      // the row belongs to row group row % RP, held by TK threads = TK/64 waves
      // (or part of one wave when TK < 64)
      int v = 0;
      if constexpr (TK >= 64) {
        constexpr int nw = TK / 64;            // waves per row group
        const int w0 = (row % RP) * nw;        // first wave of the row's group
#pragma unroll
        for (int wv = 0; wv < nw; ++wv) v += red[w0 + wv][row][m];
      } else {
        v = red[(row % RP) * TK / 64][row][m];
      }
      if constexpr (BITS == 4) v >>= 4;  // exact: every product carries a factor 16
      const int64_t n = n0 + row;
      const float sc = scales[m] * *alpha;
      const int t = v - rowsum[m];
      if constexpr (OUT == 2) {
        reinterpret_cast<int32_t*>(out)[(int64_t)m * ldo + n] = t;
      } else if constexpr (OUT == 1) {
        reinterpret_cast<float*>(out)[(int64_t)m * ldo + n] = sc * (float)t;
      } else {
        reinterpret_cast<uint16_t*>(out)[(int64_t)m * ldo + n] = f32_to_bf16_rne(sc * (float)t);
      }
    }
  }
}

template <int BITS, int OUT>
hipError_t launch_bits_out(const void* codes, const float* scales, const int32_t* rowsum,
                           const uint32_t* wp, const float* alpha, int64_t M, int64_t N, int64_t K,
                           void* out, int64_t ldo, int cu_count, hipStream_t s) {
  if (M <= 4 && K % 1024 == 0) {
    const int64_t tk = K / 64 < 256 ? K / 64 : 256;
#define HBL_DOT(MT, TK)                                                                                      \
  if (N % DotGeom<BITS, OUT, MT, TK>::NB == 0) {                                                           \
    hipLaunchKernelGGL((k_gemv_dot<BITS, OUT, MT, TK>), dim3((unsigned)(N / DotGeom<BITS, OUT, MT, TK>::NB)), \
                       dim3(512), 0, s, codes, scales, rowsum, wp, alpha, (int)M, N, K, out, ldo);           \
    return hipGetLastError();                                                                                \
  }
#define HBL_DOT_TK(MT)                          \
  if (tk == 256) { HBL_DOT(MT, 256) }           \
  else if (tk == 128) { HBL_DOT(MT, 128) }      \
  else if (tk == 64) { HBL_DOT(MT, 64) }        \
  else if (tk == 32) { HBL_DOT(MT, 32) }        \
  else { HBL_DOT(MT, 16) }
    if (M == 1) { HBL_DOT_TK(1) }
    else if (M == 2) { HBL_DOT_TK(2) }
    else { HBL_DOT_TK(4) }
#undef HBL_DOT_TK
#undef HBL_DOT
  }
  if (M <= kGemvMaxM) {
    hipLaunchKernelGGL((k_gemv<BITS, OUT>), dim3((unsigned)(N / 16)), dim3(256), 0, s, codes, scales,
                       rowsum, wp, alpha, (int)M, N, K, out, ldo);
    return hipGetLastError();
  }
  // 256 x 256 tiles (8 waves of 128 x 64, one block per CU) when there are
  // enough of them to fill the chip; otherwise 128 x 128 tiles (4 waves of
  // 64 x 64, several blocks per CU).
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  if (t256 >= cu_count) {
    const int tm = (int)((M + 255) / 256), tn = (int)((N + 255) / 256);
    hipLaunchKernelGGL((k_gemm<BITS, OUT, 256, 256, 2, 4, 1>), dim3((unsigned)(tm * tn)), dim3(512), 0, s, codes,
                       scales, rowsum, wp, alpha, M, N, K, out, ldo, tm, tn);
  } else {
    const int tm = (int)((M + 127) / 128), tn = (int)((N + 127) / 128);
    hipLaunchKernelGGL((k_gemm<BITS, OUT, 128, 128, 2, 2, 2>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, codes,
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
