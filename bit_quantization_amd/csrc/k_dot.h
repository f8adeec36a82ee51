// Dot-product form of the ternary matmul for one or two tokens (decode),
// shared by the matmul entry point (k_gemm.hip) and the one-launch decode
// layer (k_quant.hip).  Computes Eq. 9 of the architecture write-up of
// "BitNet v2" (§3.4 "H-BitLinear"):
//   out[m][n] = (scale_m * alpha) * sum_k q_x[m][k] q_w[n][k].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hbl {
namespace {

typedef unsigned dot_v4u __attribute__((ext_vector_type(4)));

// Streaming 16-byte load (data used once: do not keep it in the caches).
__device__ __forceinline__ uint4 load_stream(const uint32_t* p) {
  const dot_v4u v = __builtin_nontemporal_load(reinterpret_cast<const dot_v4u*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Value of the partner lane in an xor-butterfly sum over lane distances o =
// 1, 2, 4, ... taken in that order: 1 and 2 are quad permutations; 4 and 8
// the half-row and row mirrors (lane i <-> 7 - i, 15 - i), which pair each
// lane with the other half of its group, the same sum as l ^ o once the
// earlier steps have made every 4- (8-) lane group hold one value; 16 and 32
// through the LDS crossbar.  Integer sums: any pairing order gives the same
// result.
__device__ __forceinline__ int lane_sum_partner(int v, int o) {
  switch (o) {
    case 1: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    case 4: return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    case 8: return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    default: return __shfl_xor(v, o);
  }
}

// Decode with very few tokens, K a power of two from 1024 to 16384.
// A block of NTH threads owns NB output features.  Thread t covers 64 codes
// of RPT = NB / (NTH / TK) of those features (TK = K / 64 threads per
// feature row; kt = t % TK): k = 64 kt .. + 63 (one 16-byte weight load
// per row, consecutive threads reading consecutive 16 bytes of a row), or,
// for INT8 codes up to K = 8192, the four 16-code groups kt + TK j (j =
// 0..3, so that consecutive threads also read consecutive 16-byte pieces
// of the codes); it loads the tokens' codes once (registers) and streams
// the rows' packed weights, every load issued first.  Each weight word gives
// 4 dwords of bytes c = q_w + 1, multiplied into the codes with
// v_dot4_i32_i8; INT4 codes are widened to 16 q_x (the sums are divided by
// 16 at the end, exactly).  Partial sums are reduced over the TK threads of
// a row (xor-butterflies within a wave, then a fixed order over the waves),
// then rescaled: sum q_x q_w = sum q_x c - rowsum.
template <int MT, int TK, int NTH = 512, int NBMIN = 8>
struct DotGeom {
  static constexpr int RP = NTH / TK;                 // feature rows side by side
  static constexpr int NB = RP > NBMIN ? RP : NBMIN;  // features per block
  static constexpr int RPT = NB / RP;                 // rows per thread
  static constexpr int RED_INTS = (NTH / 64) * NB * MT;  // LDS of the cross-wave sums
};

// One block's share: features fb * NB .. + NB - 1.  red: RED_INTS ints of
// LDS.  before_weights() runs first, before_codes() after the weight loads
// are issued and before the scales and row sums are read (the one-launch
// decode layer issues its token-row loads in the first and computes the
// codes in the second; the codes may then live in LDS).  The codes are
// loaded after before_codes(), or, with XFIRST, before the weight loads
// are issued (codes in global memory, written by an earlier launch).  With
// SELF, rowsum is not read: each thread starts its sums at minus the sum
// of its own codes, so that the reduction over the row's threads yields
// sum q_x c - sum q_x = sum q_x q_w directly (the same integers).
template <int BITS, int OUT, int MT, int TK, int NTH, int NBMIN = 8, bool XFIRST = false, bool SELF = false,
          typename Pre, typename Hook>
__device__ __forceinline__ void gemv_dot_body(const void* __restrict__ codes, const float* __restrict__ scales,
                                              const int32_t* __restrict__ rowsum, const uint32_t* __restrict__ wp,
                                              const float* __restrict__ alpha, int M, int64_t K, void* __restrict__ out,
                                              int64_t ldo, int64_t fb, int tid, int* red, Pre before_weights,
                                              Hook before_codes) {
  using DG = DotGeom<MT, TK, NTH, NBMIN>;
  constexpr int NB = DG::NB;
  const int lane = tid & 63, wave = tid >> 6;
  static_assert(TK >= 16 && TK <= 256, "threads per feature row");
  static_assert(NTH % TK == 0 && NB % DG::RP == 0, "block shape");
  constexpr int RP = DG::RP;
  constexpr int RPT = DG::RPT;
  const int kt = tid % TK, rg = tid / TK;
  const int64_t n0 = fb * NB;
  const int64_t KW = K / 16;

  // IL: the thread's codes are the four 16-code groups kt + TK j (j =
  // 0..3), so that the lanes of a wave read consecutive 16-byte pieces of
  // codes and consecutive weight words (INT8 codes up to K = 8192: M = 1,
  // K = 4096 3.5 -> 3.1 us, M = 2 4.4 -> 3.7; at K = 16384 and with INT4
  // codes, read as 8-byte pieces, 3-11 % slower); else the 64 consecutive
  // codes 64 kt .. + 63 and one 16-byte weight load per row.  Weights: rows
  // n0 + rg + RP i; every weight load is issued before any is used.
  constexpr bool IL = BITS == 8 && TK <= 128;
  // the tokens' codes for k = 64*kt .. +63, as 16 dwords of signed bytes
  // (16-byte piece j of token m at byte m K BITS/8 + 16 j)
  auto piece = [&](int m, int64_t j) -> uint4 {
    return reinterpret_cast<const uint4*>(reinterpret_cast<const int8_t*>(codes) + (int64_t)m * K * BITS / 8)[j];
  };
  uint32_t x[MT][16];
  auto load_codes = [&] {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        if constexpr (BITS == 8) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 u = piece(m, IL ? kt + TK * q : 4 * kt + q);
            x[m][4 * q] = u.x; x[m][4 * q + 1] = u.y; x[m][4 * q + 2] = u.z; x[m][4 * q + 3] = u.w;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint4 u = piece(m, 2 * kt + q);
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
  };

  before_weights();
  if constexpr (XFIRST) load_codes();
  uint4 w[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const uint32_t* row = wp + (n0 + rg + (int64_t)RP * i) * KW;
    if constexpr (IL)
      w[i] = make_uint4(__builtin_nontemporal_load(row + kt), __builtin_nontemporal_load(row + kt + TK),
                        __builtin_nontemporal_load(row + kt + 2 * TK), __builtin_nontemporal_load(row + kt + 3 * TK));
    else
      w[i] = load_stream(row + 4 * kt);
  }
  before_codes();
  if constexpr (!XFIRST) load_codes();

  int acc[RPT][MT];
  int xsum[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    xsum[m] = 0;
    if constexpr (SELF)
#pragma unroll
      for (int j = 0; j < 16; ++j) xsum[m] = __builtin_amdgcn_sdot4((int)x[m][j], 0x01010101, xsum[m], false);
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = -xsum[m];
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
      for (int o = 1; o < lanes_per_row; o <<= 1) v += lane_sum_partner(v, o);
      acc[i][m] = v;
    }
  }
  // lane 0 of each row group in each wave publishes its partials
  // (red[wave][row][m])
  if ((lane % lanes_per_row) == 0) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + RP * i;  // feature within the block
#pragma unroll
      for (int m = 0; m < MT; ++m) red[(wave * NB + row) * MT + m] = acc[i][m];
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
        for (int wv = 0; wv < nw; ++wv) v += red[((w0 + wv) * NB + row) * MT + m];
      } else {
        v = red[(((row % RP) * TK / 64) * NB + row) * MT + m];
      }
      if constexpr (BITS == 4) v >>= 4;  // exact: every product carries a factor 16
      const int64_t n = n0 + row;
      const float sc = scales[m] * *alpha;
      const int t = SELF ? v : v - rowsum[m];
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

}  // namespace
}  // namespace hbl
