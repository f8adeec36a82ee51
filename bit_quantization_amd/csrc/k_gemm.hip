// Ternary-weight integer matmul with the rescale of Eq. 9 (architecture
// write-up of "BitNet v2", §3.4 "H-BitLinear"), for gfx950:
//   acc[m][n] = sum_k q_x[m][k] q_w[n][k],  out = (scale_m * alpha) * acc.
//
// Two kernels:
//   k_gemm -- large token counts.  Block tile 256 x 256 (8 waves of
//     128 x 64) or 128 x 128 (4 waves of 64 x 64), each wave a tile of
//     16x16x64 int8 MFMAs with int32 accumulators.  Codes and weights are
//     copied to LDS as they are stored (packed), by direct-to-LDS buffer
//     loads three stages ahead, and widened by each wave after its LDS
//     read.  Weights are decoded from two bits to the unsigned byte
//     c = q + 1 in {0, 1, 2}, so the MFMA sums q_x * c; the epilogue
//     subtracts sum_k q_x (the token's row sum of codes) to obtain
//     sum_k q_x * q_w exactly.
//   k_gemv -- token counts up to 128 (decode and small batches).  Each block
//     owns 16 output features and streams their packed weights once with
//     16-byte loads; the 4 waves of a block split K and are reduced through
//     LDS.  The tokens, in groups of 16, are the 16 columns of the MFMA's
//     second operand (columns beyond M are zero); each decoded weight
//     fragment serves every group.
//
// In both kernels the MFMA's first operand is the weight fragment and its
// second the activation fragment, so each lane ends with four consecutive
// output features of one token: one 8-byte bf16 store.
#include "hbl_internal.h"
#include "k_dot.h"

#include <climits>

#include <algorithm>
#include <type_traits>
#include <utility>

namespace hbl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Two's-complement nibbles (bytes 0..15) to signed bytes, bytewise:
// ((u ^ 8) + 0x78) ^ 0x80 never carries between bytes.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t u) {
  return ((u ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
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
  // The body is compiled for the device only: the host pass (which only
  // needs the launch stub) drops this template's instantiation otherwise.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = WGM * WGN;                // waves
  constexpr int S = 2;                         // MFMA k-steps per stage
  constexpr int NST = 3;                       // LDS stages in flight
  constexpr int BKC = 64 * S;                  // codes per row per stage
  constexpr int AROW = BKC * BITS / 8;         // code bytes per row per stage
  constexpr int BROW = 16 * S;                 // weight bytes per row per stage
  constexpr int ACPR = AROW / 16, BCPR = BROW / 16;  // 16-byte units per row
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int ADMA = BM * AROW / 1024 / NW;  // 1 KB direct-to-LDS loads per wave per stage
  constexpr int BDMA = BN * BROW / 1024 / NW;
  static_assert(ADMA * NW * 1024 == BM * AROW && BDMA * NW * 1024 == BN * BROW, "staging must divide evenly");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "fragment rows");
  constexpr int SPR = BITS == 4 ? 2 : 1;       // MFMA steps per 16-byte code read
  __shared__ __attribute__((aligned(1024))) uint8_t As[NST][BM * AROW];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs[NST][BN * BROW];

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
  const int arows = (int)min<int64_t>(BM, M - m0), brows = (int)min<int64_t>(BN, N - n0);

  // LDS byte offsets (swizzled) of 16-byte unit u of row r
  auto aoff = [](int r, int u) {
    if constexpr (BITS == 8) return r * AROW + 16 * (u ^ ((r >> 1) & 7));
    else return r * AROW + 16 * (u ^ ((r >> 2) & 3));
  };
  auto boff = [](int r, int u) { return r * BROW + 16 * (u ^ ((r >> 3) & 1)); };

  // Staging by direct-to-LDS buffer loads: each wave instruction fills 1 KB
  // of a stage (lane l -> 16 bytes at base + 16 l).  Lane l of instruction j
  // of wave w writes physical unit P = 64 (w + NW j) + l, i.e. row P / CPR,
  // physical unit P % CPR, which holds logical unit (P % CPR) ^ swizzle(row).
  // Rows and k past the end get an offset beyond the buffer's range, which
  // reads as zero.  The buffers start at the block's first row.
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(codes) + m0 * arow_bytes), (short)0,
      (int)(arows * arow_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(wp) + n0 * brow_bytes), (short)0,
      (int)(brows * brow_bytes), 0x00020000);
  constexpr uint32_t kOut = 0x80000000u;  // beyond any buffer range
  uint32_t aoffg[ADMA], boffg[BDMA];      // global byte offset of the unit at stage 0 (or kOut)
  int acolb[ADMA], bcolb[BDMA];           // byte offset of the unit within a stage row
#pragma unroll
  for (int j = 0; j < ADMA; ++j) {
    const int P = 64 * (wave + NW * j) + lane, r = P / ACPR, p = P % ACPR;
    const int u = BITS == 8 ? (p ^ ((r >> 1) & 7)) : (p ^ ((r >> 2) & 3));
    acolb[j] = 16 * u;
    aoffg[j] = r < arows ? (uint32_t)(r * arow_bytes + 16 * u) : kOut;
  }
#pragma unroll
  for (int j = 0; j < BDMA; ++j) {
    const int P = 64 * (wave + NW * j) + lane, r = P / BCPR, p = P % BCPR;
    const int u = p ^ ((r >> 3) & 1);
    bcolb[j] = 16 * u;
    boffg[j] = r < brows ? (uint32_t)(r * brow_bytes + 16 * u) : kOut;
  }
  auto stage_load = [&](int kt, int buf) {
    const uint32_t ka = (uint32_t)kt * AROW, kb = (uint32_t)kt * BROW;
#pragma unroll
    for (int j = 0; j < ADMA; ++j) {
      const bool ok = aoffg[j] != kOut && ka + acolb[j] < arow_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, &As[buf][1024 * (wave + NW * j)], 16, ok ? aoffg[j] + ka : kOut, 0, 0,
                                               0);
    }
#pragma unroll
    for (int j = 0; j < BDMA; ++j) {
      const bool ok = boffg[j] != kOut && kb + bcolb[j] < brow_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, &Bs[buf][1024 * (wave + NW * j)], 16, ok ? boffg[j] + kb : kOut, 0, 0,
                                               0);
    }
  };
  constexpr int DMA_PER_STAGE = ADMA + BDMA;

  v4i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int nk = (int)((K + BKC - 1) / BKC);
  const int fr = lane % 16, g = lane / 16;
  // Fragment rows are wm*WM + 16*j + fr (codes) and wn*WN + 16*i + fr
  // (weights): the swizzle depends on fr only, and fragment j (i) sits at a
  // constant offset from fragment 0.  Codes of lane group g: unit g (INT4:
  // both steps) or units 2g, 2g+1 (INT8: one per step); weights: 8 bytes,
  // half (g & 1) of unit g >> 1.
  const int abase0 = BITS == 4 ? aoff(wm * WM + fr, g) : aoff(wm * WM + fr, 2 * g);
  const int abase1 = BITS == 4 ? abase0 : aoff(wm * WM + fr, 2 * g + 1);
  const int bbase = boff(wn * WN + fr, g >> 1) + 8 * (g & 1);
  constexpr int AFRAG = 16 * AROW, BFRAG = 16 * BROW;  // bytes between fragments

  // prologue: stages 0 and 1 in flight
  stage_load(0, 0);
  if (nk > 1) stage_load(1, 1);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt must have landed: at most the loads of stage kt + 1 may be
    // outstanding; then every wave's share is visible after the barrier
    if (kt + 1 < nk) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_PER_STAGE) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    // the buffer of stage kt + 2 was last read in stage kt - 1: free now
    if (kt + 2 < nk) stage_load(kt + 2, (kt + 2) % NST);
    const uint8_t* Ab = As[kt % NST];
    const uint8_t* Bb = Bs[kt % NST];
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
      }
    }
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
#endif
}

// ---------------------------------------------------------------------------
// Persistent matmul for large token counts (K a multiple of 512).
//
// One block of 4 waves (2 x 2) per CU, one wave per SIMD.  Block tile
// BM x BN (256 x 256 when the tiles fill the chip, else 256 x 128), wave
// tile BM/2 x BN/2 built from 32x32x32 int8 MFMAs whose int32 accumulators
// live in the accumulation registers.  A stage is BK = 128 codes; four
// stage buffers, each its own LDS variable, are refilled by direct-to-LDS
// buffer loads four stages ahead.  Each block walks its tiles in sequence
// and numbers the stages of all of them consecutively, so the loads and the
// fragment prefetch of a tile's last stages already bring in the next tile.
//
// Fragment layout (32x32x32): lane l covers row / column l % 32 of its
// fragment and, for MFMA step t of a stage, the 16 codes
// k = 64 (l / 32) + 16 t .. + 15 of the stage (the same k for both
// operands, so the MFMA's own k order does not matter).  The accumulator of
// a fragment holds, in lane l and register r, token l % 32 and feature
// 8 (r / 4) + 4 (l / 32) + r % 4.
//
// Within stage kt the waves meet once, halfway through the MFMAs: past that
// barrier every wave has read stage kt's buffer (so its refill may start)
// and stage kt + 1 has landed (so its fragments may be read while the
// second half of stage kt's MFMAs runs).  Each MFMA step's operands are
// widened during the previous step's MFMAs.  The barrier carries no memory
// fence (a fence would wait for every load in flight, the prefetch
// included); each wave has waited for its own loads of the stage first.
//
// LDS rows are not padded; 16-byte units are XOR-swizzled by row
// (unit u of row r at u ^ ((r >> s) & (U - 1)), U units per row,
// s = log2(16 / U)) so that the 16 rows a b128 read touches at once fall
// into distinct banks.
constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// smallest M K at which the int8 layer takes the split persistent matmul
constexpr int64_t kSplitMinMK = int64_t(1) << 20;

// the plan of k_gemm_pt
// narrow tiles (fewer 256 x 256 tiles than CUs) are 128 x 256, split or not
SplitPlan pt_plan(int64_t M, int64_t N, int64_t K, int cu_count, bool may_split) {
  return split_plan(M, N, K, cu_count, may_split, true);
}

// int32 partial sums of a split plan's items (0: no split)
size_t pt_partial_bytes(const SplitPlan& p) {
  return p.ksplit > 1 ? (size_t)p.items() * p.bm * p.bn * sizeof(int32_t) : 0;
}

template <int BITS, int OUT, int BM, int BN, int NWV>
__global__ void __launch_bounds__(64 * NWV, 1)
k_gemm_pt(const void* __restrict__ codes, const float* __restrict__ scales,
          const int32_t* __restrict__ rowsum, const uint32_t* __restrict__ wp,
          const float* __restrict__ alpha, int64_t M, int64_t N, int64_t K,
          void* __restrict__ out, int64_t ldo, int tilesM, int tilesN, int gm, int ksplit,
          int4* __restrict__ part) {
#if defined(__HIP_DEVICE_COMPILE__)
  // NW waves as a (NW / 2) x 2 grid of 256-row tiles, 4 (one per SIMD) or
  // 8 (two per SIMD), or 2 x 4 for 128 x 256 tiles (64 x 64 wave tiles)
  constexpr int NW = NWV, WGM = BM == 128 ? 2 : NW / 2, WGN = NW / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(BM == 256 || (BM == 128 && BN == 256 && NW == 8), "tile shapes 256 x BN and 128 x 256");
  constexpr int BK = 128, NSTEP = BK / 32, NST = 4;  // NST stage buffers; also the unroll
  constexpr int AROW = BK * BITS / 8, BROW = BK / 4;  // bytes per row per stage
  constexpr int AU = AROW / 16, BU = BROW / 16;       // 16-byte units per row
  constexpr int ASH = ilog2c(16 / AU), BSH = ilog2c(16 / BU);
  constexpr int NAU = AU / 2, NBU = BU / 2;           // units per lane half per fragment
  // the weights of a 256 x 128 tile's stage (4 KB) are half a load per wave
  // with 8 waves: each wave then loads 512 bytes with its lanes 0-31
  constexpr bool BHALF = BN * BROW / 1024 == NW / 2;
  // waves issuing the stage loads: for INT8 codes on 256 x 256 tiles one per
  // SIMD (waves 0-3, twice the loads each), so that each SIMD keeps a wave
  // that never waits to issue a load (bit-identical; us against all eight
  // waves loading: 65536 x 4096 x 4096 976 -> 950, 4096 x 4096 x 16384 219
  // -> 215, 65536 x 16384 x 4096 3788 -> 3747; INT4 codes 1 % slower)
  constexpr int PW = (BITS == 8 && BM == 256 && BN == 256 && NW == 8) ? 4 : NW;
  constexpr int ADMA = BM * AROW / 1024 / PW, BDMA = BHALF ? 1 : BN * BROW / 1024 / PW;
  static_assert(ADMA * PW * 1024 == BM * AROW && (BHALF || BDMA * PW * 1024 == BN * BROW) && (PW == NW || !BHALF),
                "staging must divide evenly");
  static_assert(NBU == 1, "one weight unit per lane half");
  constexpr int DPS = ADMA + BDMA;  // loads per wave per stage
  constexpr int ASZ = BM * AROW, BSZ = BN * BROW;
  __shared__ __attribute__((aligned(1024))) uint8_t As0[ASZ], As1[ASZ], As2[ASZ], As3[ASZ];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs0[BSZ], Bs1[BSZ], Bs2[BSZ], Bs3[BSZ];
  // bf16 outputs of 64 x 64 wave tiles are staged through LDS when it has
  // room besides the stages; the 256 x 256 tile stores fragments directly
  // (staging its 128-wide rows costs more registers than it saves)
  constexpr int OROW = WN * 2 + 16;  // bytes per staged output row of a wave
  constexpr bool STAGE_OUT = OUT == 0 && WN == 64 && NST * (ASZ + BSZ) + NW * 32 * OROW <= 160 * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t Os[STAGE_OUT ? NW * 32 * OROW : 16];
  auto abuf = [&]<int I>(std::integral_constant<int, I>) -> uint8_t* {
    if constexpr (I == 0) return As0; else if constexpr (I == 1) return As1; else if constexpr (I == 2) return As2; else return As3;
  };
  auto bbuf = [&]<int I>(std::integral_constant<int, I>) -> uint8_t* {
    if constexpr (I == 0) return Bs0; else if constexpr (I == 1) return Bs1; else if constexpr (I == 2) return Bs2; else return Bs3;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int64_t arow_bytes = BITS == 4 ? K / 2 : K;  // global code row stride
  const int64_t brow_bytes = K / 4;                  // global weight row stride
  const int nks = (int)(K / BK) / ksplit;            // stages of one item (a multiple of NST)

  // Items of this block: r P + slot for r = 0, 1, ... (P blocks, a multiple
  // of 8).  Consecutive block ids go to different XCDs; slot gives each XCD
  // a contiguous range of each round's items (split_item: a tile and one of
  // ksplit K slices, tiles walked in M-groups of gm so that an XCD's blocks
  // share codes and weights in its L2).  With ksplit > 1 an item leaves its
  // int32 partial sums in part for k_pt_reduce.
  const int G = tilesM * tilesN * ksplit, P = gridDim.x, b = blockIdx.x;
  const int slot = (b % 8) * (P / 8) + b / 8;
  const int ntiles = slot < G ? (G - slot + P - 1) / P : 0;
  auto tile_of = [&](int r, int64_t& m0, int64_t& n0, int& ks) {
    split_item<BM, BN>(r * P + slot, tilesM, tilesN, gm, m0, n0, ks);
  };

  auto aswz = [](int r, int u) { return u ^ ((r >> ASH) & (AU - 1)); };
  auto bswz = [](int r, int u) { return u ^ ((r >> BSH) & (BU - 1)); };
  // Lane l of load j of wave w fills physical unit P = 64 (w + NW j) + l of
  // a stage: row P / U, physical unit l % U, holding logical unit
  // (l % U) ^ swizzle(row); the swizzle term is the same for every j, so one
  // column offset per lane serves all loads.  Rows past the end of the
  // matrix lie beyond the buffer's range and read as zero.
  constexpr int AJR = 64 * PW / AU, BJR = 64 * PW / BU;  // rows between loads j and j + 1
  // (half loads: unit 32 w + l of the weight stage, lanes l < 32)
  const int ar0 = (64 * wave + lane) / AU, br0 = (BHALF ? 32 * wave + (lane & 31) : 64 * wave + lane) / BU;
  const uint32_t aoff0 = (uint32_t)ar0 * (uint32_t)arow_bytes + 16u * (uint32_t)aswz(ar0, lane % AU);
  const uint32_t boff0 = (uint32_t)br0 * (uint32_t)brow_bytes + 16u * (uint32_t)bswz(br0, lane % BU);
  const uint32_t astep = (uint32_t)AJR * (uint32_t)arow_bytes, bstep = (uint32_t)BJR * (uint32_t)brow_bytes;
  constexpr uint32_t kOut = 0x80000000u;  // beyond any buffer range: reads zero

  // load cursor: tile dr (of this block), stage dk, and that tile's buffers
  int dr = 0, dk = 0;
  __amdgpu_buffer_rsrc_t rA, rB;
  auto set_tile = [&](int r) {
    int64_t m0 = 0, n0 = 0;
    int ks = 0;
    if (r < ntiles) tile_of(r, m0, n0, ks);
    const int arows = r < ntiles ? (int)min<int64_t>(BM, M - m0) : 0;
    const int brows = r < ntiles ? (int)min<int64_t>(BN, N - n0) : 0;
    // both ranges start at the item's first column (rows keep their stride;
    // the range still ends with the tile's last row)
    const int64_t ka = (int64_t)ks * nks * AROW, kb = (int64_t)ks * nks * BROW;
    rA = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(codes) + m0 * arow_bytes + ka), (short)0,
        arows > 0 ? (int)(arows * arow_bytes - ka) : 0, 0x00020000);
    rB = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(wp) + n0 * brow_bytes + kb), (short)0,
        brows > 0 ? (int)(brows * brow_bytes - kb) : 0, 0x00020000);
  };
  // loads of stage (dr, dk) into buffer I; advances the cursor
  auto stage_load = [&]<int I, bool SW = true>(std::integral_constant<int, I> bi, std::bool_constant<SW> = {}) {
    uint8_t* const Ad = abuf(bi);
    uint8_t* const Bd = bbuf(bi);
    const bool live = dr < ntiles;
    const uint32_t va = live ? aoff0 + (uint32_t)dk * AROW : kOut;
    const uint32_t vb = live ? boff0 + (uint32_t)dk * BROW : kOut;
    if (PW == NW || wave < PW) {
#pragma unroll
    for (int j = 0; j < ADMA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, Ad + 1024 * (wave + PW * j), 16, va + j * astep, 0, 0, 0);
    if constexpr (BHALF) {
      if (lane < 32) __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, Bd + 512 * wave, 16, vb, 0, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < BDMA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, Bd + 1024 * (wave + PW * j), 16, vb + j * bstep, 0, 0, 0);
    }
    }
    ++dk;
    if constexpr (SW) {
      if (dk == nks) {
        dk = 0;
        set_tile(++dr);
      }
    }
  };

  v16i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v16i{};

  const int fr = lane % 32, h = lane / 32;
  const int ar = wm * WM + fr, br = wn * WN + fr;
  int abase[NAU];
#pragma unroll
  for (int v = 0; v < NAU; ++v) abase[v] = ar * AROW + 16 * aswz(ar, NAU * h + v);
  const int bbase = br * BROW + 16 * bswz(br, h);
  constexpr int AFRAG = 32 * AROW, BFRAG = 32 * BROW;  // bytes between fragments

  // A stage's fragments: the head (weights, and the code units of the first
  // half of the MFMA steps) is read across the mid-stage barrier of the
  // previous stage; the tail (code units of the second half) at the start of
  // the stage itself, landing while the first half runs.
  constexpr int HU = NAU / 2;
  struct Head {
    uint4 b[FN];
    uint4 a[FM][HU];
  };
  struct Tail {
    uint4 a[FM][HU];
  };
  auto read_head = [&]<int I>(Head& f, std::integral_constant<int, I> bi) {
    const uint8_t* Ab = abuf(bi);
    const uint8_t* Bb = bbuf(bi);
#pragma unroll
    for (int i = 0; i < FN; ++i) f.b[i] = *reinterpret_cast<const uint4*>(Bb + bbase + BFRAG * i);
#pragma unroll
    for (int v = 0; v < HU; ++v)
#pragma unroll
      for (int j = 0; j < FM; ++j) f.a[j][v] = *reinterpret_cast<const uint4*>(Ab + abase[v] + AFRAG * j);
  };
  auto read_tail = [&]<int I>(Tail& f, std::integral_constant<int, I> bi) {
    const uint8_t* Ab = abuf(bi);
#pragma unroll
    for (int v = 0; v < HU; ++v)
#pragma unroll
      for (int j = 0; j < FM; ++j) f.a[j][v] = *reinterpret_cast<const uint4*>(Ab + abase[HU + v] + AFRAG * j);
  };
  // The operands of one MFMA step, widened: weights from two bits to the
  // bytes c = q + 1 (word -> {w, w >> 2, w >> 4, w >> 6} & 0x03030303); INT4
  // codes to the bytes 16 q (low nibbles shifted up, high nibbles in place);
  // INT8 codes as stored.  Step t uses weight word t of the lane's unit and
  // code unit t / 2 (INT4) or t (INT8) of its half of the stage.
  struct Dec {
    v4i bf[FN];
    v4i af[FM];
  };
  auto decode = [&](Dec& d, const uint4 (&bq)[FN], const uint4 (&aq)[FM][HU], int t) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const uint4 q = bq[i];
      const uint32_t w = (t == 0) ? q.x : (t == 1) ? q.y : (t == 2) ? q.z : q.w;
      d.bf[i] = v4i{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
                    (int)((w >> 6) & 0x03030303u)};
    }
    const int th = t % (NSTEP / 2);  // step within the half (head or tail units)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      if constexpr (BITS == 4) {
        const uint4 q = aq[j][th / 2];
        const uint32_t x0 = (th % 2 == 0) ? q.x : q.z, x1 = (th % 2 == 0) ? q.y : q.w;
        d.af[j] = v4i{(int)((x0 << 4) & 0xf0f0f0f0u), (int)(x0 & 0xf0f0f0f0u), (int)((x1 << 4) & 0xf0f0f0f0u),
                      (int)(x1 & 0xf0f0f0f0u)};
      } else {
        const uint4 q = aq[j][th];
        d.af[j] = v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
      }
    }
  };
  auto mfmas = [&](const Dec& d) {
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int i = 0; i < FN; ++i) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(d.bf[i], d.af[j], acc[i][j], 0, 0, 0);
  };
  auto bar = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Epilogue of compute tile r: sum q_x q_w = sum q_x c (/ 16 for INT4) - rowsum.
  auto epilogue = [&](int r) {
    // r made opaque here: nothing of the epilogue is computed early and kept
    // live through the stage loop
    asm volatile("" : "+s"(r));
    if ((BM == 128 || BN == 128) && ksplit > 1) {
      // raw int32 partial sums in fragment order: each store is 1 KB
      // contiguous (splits use the narrow tiles only)
      int4* dst = part + ((int64_t)(r * P + slot) * NW + wave) * (FN * FM * 4 * 64) + lane;
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v16i& a = acc[i][j];
            dst[((i * FM + j) * 4 + q) * 64] = make_int4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v16i{};
      return;
    }
    int64_t m0, n0;
    int ks;
    tile_of(r, m0, n0, ks);
    const float al = *alpha;
    if constexpr (STAGE_OUT) {
      // bf16 through LDS: for fragment row j the wave writes its 32 tokens x
      // WN features to its own [32][WN] tile (rows padded by 16 bytes), then
      // stores whole rows, 16 bytes per lane: far fewer and larger write
      // requests than the fragments' 16-byte row pieces
      uint8_t* const Ow = Os + wave * 32 * OROW;
      constexpr int U = WN * 2 / 16;  // 16-byte units per staged row
      const bool wide = (ldo & 7) == 0;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int64_t m = m0 + wm * WM + 32 * j + fr;
        const int32_t R = m < M ? rowsum[m] : 0;
        const float sc = m < M ? scales[m] * al : 0.0f;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v4i a = v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            if constexpr (BITS == 4) a = a >> 4;  // exact: every product carries a factor 16
            const uint32_t lo = f32_to_bf16_rne(sc * (float)(a[0] - R)) | ((uint32_t)f32_to_bf16_rne(sc * (float)(a[1] - R)) << 16);
            const uint32_t hi = f32_to_bf16_rne(sc * (float)(a[2] - R)) | ((uint32_t)f32_to_bf16_rne(sc * (float)(a[3] - R)) << 16);
            *reinterpret_cast<uint2*>(Ow + fr * OROW + 2 * (32 * i + 8 * q + 4 * h)) = make_uint2(lo, hi);
          }
          __builtin_amdgcn_sched_barrier(0);  // one fragment's values live at a time
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile is the wave's own: no barrier
#pragma unroll
        for (int pp = 0; pp < 32 * U / 64; ++pp) {
          const int row = lane / U + (64 / U) * pp, u = lane % U;
          const int64_t mm = m0 + wm * WM + 32 * j + row, nn = n0 + wn * WN + 8 * u;
          const uint4 v = *reinterpret_cast<const uint4*>(Ow + row * OROW + 16 * u);
          if (mm < M && nn < N) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(out) + mm * ldo + nn;
            if (wide) {
              *reinterpret_cast<uint4*>(dst) = v;
            } else {
              reinterpret_cast<uint2*>(dst)[0] = make_uint2(v.x, v.y);
              reinterpret_cast<uint2*>(dst)[1] = make_uint2(v.z, v.w);
            }
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next row's writes
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = m0 + wm * WM + 32 * j + fr;
      if (m < M) {
        const int32_t R = rowsum[m];
        const float sc = scales[m] * al;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + wn * WN + 32 * i + 8 * q + 4 * h;
            if (n < N) {
              v4i a = v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              if constexpr (BITS == 4) a = a >> 4;  // exact: every product carries a factor 16
              store4<OUT>(out, m * ldo + n, a, R, sc);
            }
          }
      }
    }
    }
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = v16i{};
  };

  if (ntiles == 0) return;
  set_tile(0);
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (stage_load(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, NST>{});
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 1) * DPS) : "memory");
  bar();
  Head h0, h1;
  Tail tl;
  read_head(h0, std::integral_constant<int, 0>{});
  // Stage Q of a group of NST: buffer Q, heads h0 / h1 by parity.  The
  // operands of step t + 1 are widened while step t's MFMAs run (an MFMA
  // whose operand was just written by the VALU waits for it).
  static_assert(NSTEP == 4, "four MFMA steps per stage");
  auto body = [&]<int Q>(std::integral_constant<int, Q>) {
    Head& cur = (Q % 2 == 0) ? h0 : h1;
    Head& nxt = (Q % 2 == 0) ? h1 : h0;
    read_tail(tl, std::integral_constant<int, Q>{});
    Dec d0, d1;
    decode(d0, cur.b, cur.a, 0);
    decode(d1, cur.b, cur.a, 1);
    mfmas(d0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tail has landed
    decode(d0, cur.b, tl.a, 2);
    mfmas(d1);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((NST - 2) * DPS) : "memory");
    bar();
    // nks is a multiple of NST and the loads run NST stages ahead, so the
    // load cursor reaches the end of a tile only in the group's last body
    stage_load(std::integral_constant<int, Q>{}, std::bool_constant<Q == NST - 1>{});
    read_head(nxt, std::integral_constant<int, (Q + 1) % NST>{});
    decode(d1, cur.b, tl.a, 3);
    mfmas(d0);
    mfmas(d1);
    __builtin_amdgcn_iglp_opt(0);
  };
  const int groups_per_tile = nks / NST;
  for (int r = 0; r < ntiles; ++r) {
    for (int gq = 0; gq < groups_per_tile; ++gq) {
      [&]<int... I>(std::integer_sequence<int, I...>) {
        (body(std::integral_constant<int, I>{}), ...);
      }(std::make_integer_sequence<int, NST>{});
    }
    epilogue(r);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

// ---------------------------------------------------------------------------
// Decode: M <= 16 tokens, one block per 16 output features.

// MG groups of 16 tokens (M <= 16 MG): every block streams its 16 features'
// weights once and applies each decoded weight fragment to all token groups,
// whose codes are read from the L2 (every block reads all of them).
template <int BITS, int OUT, int MG, int NWV = 8, int BATCH = 4>
__global__ void __launch_bounds__(64 * NWV)
k_gemv(const void* __restrict__ codes, const float* __restrict__ scales,
       const int32_t* __restrict__ rowsum, const uint32_t* __restrict__ wp,
       const float* __restrict__ alpha, int M, int64_t N, int64_t K,
       void* __restrict__ out, int64_t ldo) {
  __shared__ v4i red[MG][NWV - 1][64];
  // One group of tokens: each step's codes (16 tokens x RB bytes: 256 for
  // INT8, 128 for INT4) are copied into the wave's LDS area by direct-to-LDS
  // loads in which RB / 16 consecutive lanes read one token's RB bytes, then
  // read back as MFMA operands.  (Read straight into registers, each 16-byte
  // load of a wave touches 16 token rows at a 64- or 32-byte lane stride.)
  // Unit u of token t is stored at slot u ^ t (INT8) or u ^ (t / 2 mod 8)
  // (INT4) of its row, so that the 16 rows read at once fall into distinct
  // banks.
  constexpr bool XLDS = MG == 1;
  constexpr int RB = BITS == 8 ? 256 : 128, XU = RB / 16, TPL = 1024 / RB;
  auto xswz = [](int t) { return BITS == 8 ? t : (t >> 1) & 7; };
  __shared__ __attribute__((aligned(1024))) uint8_t xs[XLDS ? NWV * BATCH * 16 * RB : 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int fr = lane % 16, g = lane / 16;
  const int64_t KW = K / 16;
  const int64_t steps = (KW + 15) / 16;  // a step is 16 words (256 k) per row
  const uint32_t* wrow = wp + (n0 + fr) * KW;
  // every block reads every token's codes: each starts its walk over K at
  // its own step, so that the blocks do not all read the same code lines of
  // the L2 at once (the integer sums do not depend on the order; measured at
  // N = 4096, K = 16384: M = 16 13.4 -> 12.9 us, M = 8 10.7 -> 10.2)
  const int64_t rot = ((int64_t)blockIdx.x * 13) % steps;

  v4i acc[MG];
#pragma unroll
  for (int tg = 0; tg < MG; ++tg) acc[tg] = v4i{0, 0, 0, 0};
  __amdgpu_buffer_rsrc_t rX;
  if constexpr (XLDS)
    rX = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(codes), (short)0, (int)(M * K * BITS / 8), 0x00020000);
  for (int64_t s0 = wave; s0 < steps; s0 += NWV * BATCH) {
    uint4 w[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int64_t st = s0 + NWV * b, ps = st + rot < steps ? st + rot : st + rot - steps;
      const int64_t kw = ps * 16 + 4 * g;
      w[b] = (st < steps && kw < KW) ? load_stream(wrow + kw) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (XLDS) {
      // the previous batch's operand reads are done before its area is refilled
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int t0 = lane / XU, q = lane % XU;
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int64_t st = s0 + NWV * b, ps = st + rot < steps ? st + rot : st + rot - steps;
        if (st >= steps) break;  // wave-uniform
        uint8_t* dst = xs + (wave * BATCH + b) * 16 * RB;
#pragma unroll
        for (int j = 0; j < 16 / TPL; ++j) {
          // TPL tokens per load; groups wholly past M are not loaded (their
          // output columns are not stored), tokens past M in a partly
          // filled group lie beyond the range and read as zero
          if (TPL * j >= M) break;  // wave-uniform
          const int t = TPL * j + t0;
          const uint32_t off = (uint32_t)(t * (K * BITS / 8) + ps * RB + 16 * (q ^ xswz(t)));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, dst + 1024 * j, 16, off, 0, 0, 0);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the batch's weights and codes
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int64_t st = s0 + NWV * b, ps = st + rot < steps ? st + rot : st + rot - steps;
      const int64_t kw = ps * 16 + 4 * g;
      // Skip only whole steps (a wave-uniform test): an MFMA always runs on
      // all 64 lanes, so lanes past the end of K feed zeros instead.
      if (s0 + NWV * b >= steps) continue;
      const uint32_t ws[4] = {w[b].x, w[b].y, w[b].z, w[b].w};
      v4i a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = v4i{(int)(ws[i] & 0x03030303u), (int)((ws[i] >> 2) & 0x03030303u),
                   (int)((ws[i] >> 4) & 0x03030303u), (int)((ws[i] >> 6) & 0x03030303u)};
#pragma unroll
      for (int tg = 0; tg < MG; ++tg) {
        const int tok = 16 * tg + fr;
        if (MG > 1 && 16 * tg >= M) break;  // wave-uniform: no token of this group
        // activation codes for k = 16*kw .. 16*kw + 63 of token tok
        uint32_t x[16];
        if constexpr (XLDS) {
          const uint8_t* row = xs + (wave * BATCH + b) * 16 * RB + fr * RB;
          if constexpr (BITS == 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint4 u = *reinterpret_cast<const uint4*>(row + 16 * ((4 * g + i) ^ fr));
              x[4 * i] = u.x; x[4 * i + 1] = u.y; x[4 * i + 2] = u.z; x[4 * i + 3] = u.w;
            }
          } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const uint4 u = *reinterpret_cast<const uint4*>(row + 16 * ((2 * g + i) ^ xswz(fr)));
              const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) {
                x[8 * i + 2 * qq] = sext_nibbles(ww[qq] & 0x0f0f0f0fu);
                x[8 * i + 2 * qq + 1] = sext_nibbles((ww[qq] >> 4) & 0x0f0f0f0fu);
              }
            }
          }
        } else if (tok < M && kw < KW) {
          if constexpr (BITS == 8) {
            const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const int8_t*>(codes) + tok * K + 16 * kw);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint4 u = p[i];
              x[4 * i] = u.x; x[4 * i + 1] = u.y; x[4 * i + 2] = u.z; x[4 * i + 3] = u.w;
            }
          } else {
            const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint32_t*>(codes) + tok * (K / 8) + 2 * kw);
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
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4i bx = {(int)x[4 * i], (int)x[4 * i + 1], (int)x[4 * i + 2], (int)x[4 * i + 3]};
          acc[tg] = mfma16x16x64(a[i], bx, acc[tg]);
        }
      }
    }
  }
#pragma unroll
  for (int tg = 0; tg < MG; ++tg)
    if (wave > 0) red[tg][wave - 1][lane] = acc[tg];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int tg = 0; tg < MG; ++tg) {
      v4i t = acc[tg];
#pragma unroll
      for (int i = 0; i < NWV - 1; ++i) t += red[tg][i][lane];
      const int tok = 16 * tg + fr;
      if (tok < M) {
        const float sc = scales[tok] * *alpha;
        store4<OUT>(out, tok * ldo + n0 + 4 * g, t, rowsum[tok], sc);
      }
    }
  }
}

// Decode with one or two tokens, K a power of two from 1024 to 16384: the dot-product form (k_dot.h), one
// block of 512 threads per DotGeom::NB output features.  The codes are loaded before the weights, so that
// they do not queue behind the weight stream (graph-replayed, matrices cycled, us: one token at K = 16384
// 5.41 -> 5.23, at 4096 2.99 -> 2.96; two at K = 8192 4.66 -> 4.30, at 16384 6.61 -> 6.57).
template <int BITS, int OUT, int MT, int TK>
__global__ void __launch_bounds__(512)
k_gemv_dot(const void* __restrict__ codes, const float* __restrict__ scales,
           const int32_t* __restrict__ rowsum, const uint32_t* __restrict__ wp,
           const float* __restrict__ alpha, int M, int64_t K, void* __restrict__ out, int64_t ldo) {
  __shared__ int red[DotGeom<MT, TK>::RED_INTS];
  gemv_dot_body<BITS, OUT, MT, TK, 512, 8, true>(codes, scales, rowsum, wp, alpha, M, K, out, ldo, blockIdx.x,
                                                 threadIdx.x, red, [] {}, [] {});
}

// Sum of the ksplit int32 partial sums of k_gemm_pt's 128 x 256 split items, then
// the epilogue of Eq. 9 (/ 16 for INT4, minus the row sum, rescale).  One
// thread per four outputs of one lane's fragment, reading the partials in
// the order k_gemm_pt wrote them.
template <int BITS, int OUT, int BM, int BN, int NWV>
__global__ void __launch_bounds__(256)
k_pt_reduce(const int4* __restrict__ part, int ksplit, int tilesM, int tilesN, int gm, const float* __restrict__ scales,
            const int32_t* __restrict__ rowsum, const float* __restrict__ alpha, int64_t M, int64_t N,
            void* __restrict__ out, int64_t ldo) {
  // the wave grid of k_gemm_pt for the tile shape
  constexpr int NW = NWV, WGM = BM == 128 ? 2 : NW / 2, WGN = NW / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  const int64_t units = (int64_t)tilesM * tilesN * (BM * BN / 4);
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  const int lane = (int)(u % 64);
  int64_t t = u / 64;
  const int q = (int)(t % 4);
  t /= 4;
  const int ij = (int)(t % (FN * FM));
  t /= FN * FM;
  const int wave = (int)(t % NW);
  const int T = (int)(t / NW);
  const int i = ij / FM, j = ij % FM, wm = wave % WGM, wn = wave / WGM, fr = lane % 32, h = lane / 32;
  int64_t m0, n0;
  int ks;
  split_item<BM, BN>(T, tilesM, tilesN, gm, m0, n0, ks);
  const int64_t m = m0 + wm * WM + 32 * j + fr, n = n0 + wn * WN + 32 * i + 8 * q + 4 * h;
  if (m >= M || n >= N) return;
  int4 a = part[u];
  for (int s = 1; s < ksplit; ++s) {
    const int4 b = part[u + s * units];
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  v4i v = v4i{a.x, a.y, a.z, a.w};
  if constexpr (BITS == 4) v = v >> 4;  // exact: every product carries a factor 16
  store4<OUT>(out, m * ldo + n, v, rowsum[m], scales[m] * *alpha);
}

template <int BITS, int OUT>
hipError_t launch_bits_out(const void* codes, const float* scales, const int32_t* rowsum,
                           const uint32_t* wp, const float* alpha, int64_t M, int64_t N, int64_t K,
                           void* out, int64_t ldo, void* part, size_t part_bytes, int cu_count, hipStream_t s) {
  // with room for a K split, the persistent matmul beats weight streaming
  // from M K >= 2^20 (measured at N = 4096: M >= 64 at K = 16384, M >= 256
  // at K = 4096); 16 tokens or fewer always stream
  const bool split_ok = part != nullptr && K % 512 == 0 && M > 16 && M * K >= kSplitMinMK &&
                        part_bytes >= pt_partial_bytes(pt_plan(M, N, K, cu_count, true));
  if (split_ok) {
    const SplitPlan p = pt_plan(M, N, K, cu_count, true);
    if (p.ksplit > 1) {
      const int64_t cap = cu_count >= 8 ? (cu_count / 8) * 8 : 8;
      const int64_t P = std::min<int64_t>(((p.items() + 7) / 8) * 8, cap);
      int4* pt = static_cast<int4*>(part);
      // (splits use the narrow tiles, 128 x 256)
      hipLaunchKernelGGL((k_gemm_pt<BITS, OUT, 128, 256, 8>), dim3((unsigned)P), dim3(512), 0, s, codes, scales,
                         rowsum, wp, alpha, M, N, K, out, ldo, p.tm, p.tn, p.gm, p.ksplit, pt);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t units = (int64_t)p.tm * p.tn * (128 * 256 / 4);
      hipLaunchKernelGGL((k_pt_reduce<BITS, OUT, 128, 256, 8>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s,
                         pt, p.ksplit, p.tm, p.tn, p.gm, scales, rowsum, alpha, M, N, out, ldo);
      return hipGetLastError();
    }
  }
  // the dot-product kernel for 1-2 tokens; its per-token code loads grow
  // with M, and the matrix-core GEMV is faster from 3 tokens on (measured
  // at N = 4096, 32 or 128 matrices cycled, us dot against MFMA: K = 16384,
  // M = 2 INT4 6.9 / 7.7, INT8 6.6 / 7.0; M = 3 INT4 8.6 / 7.6; M = 4 INT4
  // 8.9 / 7.6; K = 4096, M = 2 INT4 3.5 / 3.8, INT8 3.5 / 3.6)
  // (a thread covers 64 codes of each of its rows, TK = K / 64 a power of
  // two from 16 to 256: K = 1024 ... 16384)
  if (M <= 2 && K >= 1024 && K <= 16384 && (K & (K - 1)) == 0) {
    const int64_t tk = K / 64;
#define HBL_DOT(MT, TK)                                                                                  \
  if (N % DotGeom<MT, TK>::NB == 0) {                                                                  \
    hipLaunchKernelGGL((k_gemv_dot<BITS, OUT, MT, TK>), dim3((unsigned)(N / DotGeom<MT, TK>::NB)), dim3(512), 0, \
                       s, codes, scales, rowsum, wp, alpha, (int)M, K, out, ldo);                        \
    return hipGetLastError();                                                                            \
  }
#define HBL_DOT_TK(MT)                          \
  if (tk == 256) { HBL_DOT(MT, 256) }           \
  else if (tk == 128) { HBL_DOT(MT, 128) }      \
  else if (tk == 64) { HBL_DOT(MT, 64) }        \
  else if (tk == 32) { HBL_DOT(MT, 32) }        \
  else { HBL_DOT(MT, 16) }
    if (M == 1) { HBL_DOT_TK(1) }
    else { HBL_DOT_TK(2) }
#undef HBL_DOT_TK
#undef HBL_DOT
  }
  if (M <= kGemvMaxM && !split_ok) {
    // weight streaming with the tokens in groups of 16: every CU busy (one
    // block per 16 features) where the matrix-core tiles would leave most
    // of them idle
#define HBL_GV(MG)                                                                                              \
  hipLaunchKernelGGL((k_gemv<BITS, OUT, MG>), dim3((unsigned)(N / 16)), dim3(512), 0, s, codes, scales, rowsum, wp, \
                     alpha, (int)M, N, K, out, ldo)
    // (one group stages its codes by buffer loads, whose range is 16 K BITS / 8
    // bytes < 2^31; longer rows take the two-group kernel)
    if (M <= 16 && 16 * K * BITS / 8 <= (int64_t)INT_MAX) HBL_GV(1);
    else if (M <= 32) HBL_GV(2);
    else if (M <= 64) HBL_GV(4);
    else HBL_GV(8);
#undef HBL_GV
    return hipGetLastError();
  }
  if (K % 512 == 0) {
    // persistent: one block per CU, 256 x 256 tiles when they fill the chip
    const SplitPlan p = pt_plan(M, N, K, cu_count, false);
    const int64_t cap = cu_count >= 8 ? (cu_count / 8) * 8 : 8;
    const int64_t P = std::min<int64_t>(((p.items() + 7) / 8) * 8, cap);
    if (p.bm == 256) {
      // 256 x 256 tiles run 8 waves (two per SIMD)
      hipLaunchKernelGGL((k_gemm_pt<BITS, OUT, 256, 256, 8>), dim3((unsigned)P), dim3(512), 0, s, codes, scales,
                         rowsum, wp, alpha, M, N, K, out, ldo, p.tm, p.tn, p.gm, 1, nullptr);
    } else {
      // narrower tiles as 128 x 256: the same outputs per tile as 256 x 128
      // from 24 instead of 36 KB (INT8 codes) or 16 instead of 20 KB (INT4)
      // of operands per stage
      hipLaunchKernelGGL((k_gemm_pt<BITS, OUT, 128, 256, 8>), dim3((unsigned)P), dim3(512), 0, s, codes, scales,
                         rowsum, wp, alpha, M, N, K, out, ldo, p.tm, p.tn, p.gm, 1, nullptr);
    }
    return hipGetLastError();
  }
  // Other K: 256 x 256 tiles (8 waves of 128 x 64, one block per CU) when
  // there are enough of them to fill the chip; otherwise 128 x 128 tiles
  // (4 waves of 64 x 64, several blocks per CU).
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

size_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 || N <= 0 || K % 512 != 0 || M * K < kSplitMinMK) return 0;
  return pt_partial_bytes(pt_plan(M, N, K, kSplitItems, true));
}

hipError_t launch_ternary_gemm(const void* codes, int bits, const float* scales, const int32_t* rowsum,
                               const uint32_t* wp, const float* alpha, int64_t M, int64_t N, int64_t K,
                               int out_kind, void* out, int64_t ldo, void* part, size_t part_bytes, int cu_count,
                               hipStream_t s) {
  if (M == 0) return hipSuccess;
#define HBL_G(BITS, OUT)                                                                                      \
  return launch_bits_out<BITS, OUT>(codes, scales, rowsum, wp, alpha, M, N, K, out, ldo, part, part_bytes, \
                                    cu_count, s)
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
