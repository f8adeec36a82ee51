// INT4 H-BitLinear matmul on the FP6 x FP4 matrix cores of gfx950 (the
// rescale of Eq. 9, architecture write-up of "BitNet v2", §3.4
// "H-BitLinear"):
//   acc[m][n] = sum_k q_x[m][k] q_w[n][k],  out = (scale_m * alpha) * acc.
//
// The INT4 activation codes q_x in [-8, 7] are exact in the 6-bit float
// E3M2 (OCP "BF6": 1 sign, 3 exponent (bias 3), 2 mantissa bits) and the
// ternary weights in the 4-bit float E2M1 (1 sign, 2 exponent (bias 1), 1
// mantissa bit), every product is an integer of magnitude <= 8, and the
// fp32 accumulator holds every partial sum exactly (|sum| <= 8 K < 2^24 for
// K <= 2^21).  So v_mfma_f32_32x32x64_f8f6f4 computes the integer matmul
// exactly, at twice the rate per clock of the int8 matrix cores.
//
// Operand layouts (both produced by this library; see include/hbl.h): each
// stage of the matmul (256 token rows or 128 feature rows x 128 k) is stored
// as the LDS image the kernel needs, so that its stage loads are contiguous
// 1 KB copies.
//   codes, "MX6": groups of 32 codes as 192-bit fields (code e at bits 6 e,
//     little endian) in 24 KB tiles of 256 rows x 128 codes: a 16 KB main
//     area (the first 16 bytes of each group; row r, group gi at unit
//     4 r + (gi ^ ((r >> 2) & 3))) and an 8 KB tail area (the last 8 bytes;
//     row r, groups 2 u and 2 u + 1 in the halves of unit
//     2 r + (u ^ ((r >> 3) & 1))).  Tiles run over the stages of a 256-row
//     block, then the blocks; the buffer holds whole blocks.
//   weights, "MX4": uint32 words, two bits per weight: for a word holding
//     k = 16 w .. 16 w + 15 and n = 0..7, bit 4n+1 = (q_{16w+n} != 0),
//     bit 4n+3 = (q_{16w+n} < 0), bit 4n = (q_{16w+8+n} != 0),
//     bit 4n+2 = (q_{16w+8+n} < 0); word & 0xAAAAAAAA then holds the E2M1
//     codes of k = 16w .. 16w+7 (nibble n, sign at bit 3, exponent bit at
//     bit 1) and (word << 1) & 0xAAAAAAAA those of k = 16w+8 .. 16w+15.
//     4 KB tiles of 128 rows x 128 k: row r's units (64 k each) at
//     2 r + (u ^ ((r >> 3) & 1)); tiles over the stages of a block, then the
//     blocks; rows past N are zero.
//
// Kernel structure (k_gemm_mx): persistent, one block of 8 waves (two per
// SIMD) per CU, block tile 256 x 256 (4 x 2 waves) when those tiles fill the
// chip, else 128 tokens x 256 features (2 x 4 waves), also for the items of
// a K split; wave tile 64 x 128 or 64 x 64 of 32x32x64 MFMAs with fp32
// accumulators.  (The kernel also builds with 4 waves, one per
// SIMD, 128 x BN/2 wave tiles: 5-20 % slower, since a wave's barrier and
// operand waits then leave its matrix core idle.)  A stage is 128 codes (two MFMA steps);
// four stage buffers, each its own LDS variable, are refilled four stages
// ahead by direct-to-LDS buffer loads; the stage sequence runs through the
// block's tiles, so the last stages of a tile already load the next one.
// For bf16 outputs of 256 x 256 tiles up to K = 8192 the stage loads are
// issued by one wave per SIMD only, so that each SIMD keeps a wave that
// never waits to issue a load.
// The waves meet once per stage, between its two MFMA steps: past that
// barrier the stage's buffer may be refilled and the next stage's fragments
// are read while the second step runs.  The barrier carries no memory fence
// (a fence would also wait for the prefetch in flight); each wave has waited
// for its own loads of the next stage first.
//
// Output of bf16 tiles: every block finishes its tiles at about the same
// time, so the stores come in bursts.  Each wave writes its fragments to
// its own LDS area and stores whole 128-byte row pieces from there (16
// bytes per lane; rows or features outside the matrix take an offset past
// the buffer range and are dropped, so the number of stores is fixed; the
// stores are non-temporal), and the next tile's first stages do not wait
// for those stores: their load waits count them (vmcnt retires in issue
// order), so only the fourth stage of the next tile waits for them.
//
// Fragment layout (32x32x64, measured on the device): lane l of an operand
// holds row l % 32 and the 32 k's 32 (l / 32) .. + 31 of the MFMA step,
// as consecutive 6-bit (codes) or 4-bit (weights) fields; in the
// accumulator, lane l and register r hold token l % 32 and feature
// 8 (r / 4) + 4 (l / 32) + r % 4.  Step t of a stage gives lane half h the
// stage's k = 64 h + 32 t .. + 31, i.e. code group 2 h + t: the lane's
// weight unit (16 bytes, k = 64 h .. 64 h + 63) serves both steps, its code
// main parts are units 2 h and 2 h + 1, and one tail unit (h) holds the
// last 8 bytes of both groups.
//
// LDS rows are not padded; 16-byte units are XOR-swizzled by row (unit u of
// row r at u ^ ((r >> s) & (U - 1)), U units per row, s = log2(16 / U)) so
// that the 16 rows one b128 read touches at once fall into distinct banks.
#include "hbl_internal.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace hbl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Two fp32 values to packed bf16 (first in the low half), round to nearest
// even: gfx950's v_cvt_pk_bf16_f32, one instruction for both.  For the
// finite values the epilogues produce this is the same rounding as adding
// 0x7fff plus the lowest kept bit and truncating.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
}

// four consecutive features of one token: acc holds exact integers
template <int OUT>
__device__ __forceinline__ void store4f(void* out, int64_t idx, float a0, float a1, float a2, float a3, float sc) {
  if constexpr (OUT == 2) {
    *reinterpret_cast<int4*>(reinterpret_cast<int32_t*>(out) + idx) = make_int4((int)a0, (int)a1, (int)a2, (int)a3);
  } else if constexpr (OUT == 1) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx) = make_float4(sc * a0, sc * a1, sc * a2, sc * a3);
  } else {
    const uint32_t lo = pk_bf16(sc * a0, sc * a1);
    const uint32_t hi = pk_bf16(sc * a2, sc * a3);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) = make_uint2(lo, hi);
  }
}

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }



template <int OUT, int BM, int BN, int NWV, int PWV = NWV>
__global__ void __launch_bounds__(64 * NWV, 1)
k_gemm_mx(const uint8_t* __restrict__ codes, const float* __restrict__ scales, const uint32_t* __restrict__ wq,
          const float* __restrict__ alpha, int64_t M, int64_t N, int64_t K, void* __restrict__ out, int64_t ldo,
          int tilesM, int tilesN, int gm, int ksplit, int p16, void* __restrict__ part) {
#if defined(__HIP_DEVICE_COMPILE__)
  // NW waves as a (NW / 2) x 2 grid of 256-row tiles (4 waves, one per
  // SIMD, or 8, two per SIMD), or 2 x 4 for 128 x 256 tiles: 64 x 64 wave
  // tiles with 8 waves
  constexpr int NW = NWV, WGM = BM == 128 ? 2 : NW / 2, WGN = NW / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int BK = 128, NST = 4;                  // codes per stage; stage buffers (also the unroll)
  constexpr int MROW = 64, TROW = 32, BROW = 32;    // bytes per row per stage: code mains, code tails, weights
  constexpr int MU = MROW / 16, TU = TROW / 16, BU = BROW / 16;
  constexpr int MSH = ilog2c(16 / MU), TSH = ilog2c(16 / TU), BSH = ilog2c(16 / BU);
  // the weights of a 256 x 128 tile's stage (4 KB), and the code tails of a
  // 128 x 256 tile's (4 KB), are half a load per wave with 8 waves: each
  // wave then loads 512 bytes with its lanes 0-31
  constexpr bool BHALF = BN * BROW / 1024 == NW / 2;
  constexpr bool THALF = BM * TROW / 1024 == NW / 2;
  // PW waves issue the stage loads: all of them, or (256 x 256 tiles, PWV
  // = 4) one wave per SIMD, so that each SIMD keeps a wave that never waits
  // to issue a load
  constexpr int PW = PWV;
  static_assert(PW == NW || (PW == 4 && NW == 8 && BM == 256 && BN == 256), "loading waves: all, or one per SIMD");
  constexpr int MDMA = BM * MROW / 1024 / PW, TDMA = THALF ? 1 : BM * TROW / 1024 / PW,
                BDMA = BHALF ? 1 : BN * BROW / 1024 / PW;
  static_assert(MDMA * PW * 1024 == BM * MROW && (THALF || TDMA * PW * 1024 == BM * TROW) &&
                    (BHALF || BDMA * PW * 1024 == BN * BROW) && (PW == NW || (!THALF && !BHALF)),
                "staging must divide evenly");
  constexpr int DPS = MDMA + TDMA + BDMA;  // loads per wave per stage
  constexpr int MSZ = BM * MROW, TSZ = BM * TROW, BSZ = BN * BROW;
  static_assert((BM == 256 || (BM == 128 && BN == 256 && NW == 8)) && BN % 128 == 0,
                "the MX6 tile is 256 rows x 128 codes (a block takes all of it or one half), the MX4 tile "
                "128 rows x 128 weights");
  __shared__ __attribute__((aligned(1024))) uint8_t Am0[MSZ], Am1[MSZ], Am2[MSZ], Am3[MSZ];
  __shared__ __attribute__((aligned(1024))) uint8_t At0[TSZ], At1[TSZ], At2[TSZ], At3[TSZ];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs0[BSZ], Bs1[BSZ], Bs2[BSZ], Bs3[BSZ];
  // bf16 outputs of 256 x 128 tiles are staged through LDS (whole-row stores)
  constexpr int OROW = WN * 2 + 16;
  constexpr bool STAGE_OUT = OUT == 0 && WN == 64 && NST * (MSZ + TSZ + BSZ) + NW * 32 * OROW <= 160 * 1024;
  // 256 x 256 tiles stage them by halves of the wave's 128 features: 32 rows
  // x 64 features (128 bytes, 16-byte units XOR-swizzled by row) per wave,
  // the 32 KB of LDS the four stage buffers leave
  constexpr bool STAGE_HALF = OUT == 0 && WN == 128 && NST * (MSZ + TSZ + BSZ) + NW * 32 * 128 <= 160 * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t Os[STAGE_OUT ? NW * 32 * OROW : (STAGE_HALF ? NW * 32 * 128 : 16)];
  auto mbuf = [&]<int I>(std::integral_constant<int, I>) -> uint8_t* {
    if constexpr (I == 0) return Am0; else if constexpr (I == 1) return Am1; else if constexpr (I == 2) return Am2; else return Am3;
  };
  auto tbuf = [&]<int I>(std::integral_constant<int, I>) -> uint8_t* {
    if constexpr (I == 0) return At0; else if constexpr (I == 1) return At1; else if constexpr (I == 2) return At2; else return At3;
  };
  auto bbuf = [&]<int I>(std::integral_constant<int, I>) -> uint8_t* {
    if constexpr (I == 0) return Bs0; else if constexpr (I == 1) return Bs1; else if constexpr (I == 2) return Bs2; else return Bs3;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int64_t arow_bytes = K / 4 * 3;  // global code row stride (MX6)
  const int64_t brow_bytes = K / 4;      // global weight row stride (MX4)
  const int nk = (int)(K / BK);          // stages of the whole K
  const int nks = nk / ksplit;           // stages of one item (a multiple of NST)

  // Items of this block: r P + slot (P blocks, a multiple of 8); slot gives
  // each XCD a contiguous range of each round's items.  An item is a tile
  // and one of ksplit K slices; with ksplit > 1 it leaves its exact partial
  // sums in part for k_mx_reduce, as int16 when p16 (|sum| <= 8 K / ksplit
  // fits), else as fp32.
  const int G = tilesM * tilesN * ksplit, P = gridDim.x, b = blockIdx.x;
  const int slot = (b % 8) * (P / 8) + b / 8;
  const int ntiles = slot < G ? (G - slot + P - 1) / P : 0;
  auto tile_of = [&](int r, int64_t& m0, int64_t& n0, int& ks) { split_item<BM, BN>(r * P + slot, tilesM, tilesN, gm, m0, n0, ks); };

  auto mswz = [](int r, int u) { return u ^ ((r >> MSH) & (MU - 1)); };
  auto tswz = [](int r, int u) { return u ^ ((r >> TSH) & (TU - 1)); };
  auto bswz = [](int r, int u) { return u ^ ((r >> BSH) & (BU - 1)); };
  // The MX6 and MX4 layouts store each stage as the LDS image (rows in
  // 16-byte units, XOR-swizzled by row), so lane l of load j of wave w copies
  // the 16 contiguous bytes of physical unit 64 (w + NW j) + l: every load
  // instruction moves 1 KB of consecutive addresses.  Codes: 24 KB per
  // 256-row block and stage (16 KB main area, then 8 KB tail area); a
  // 128-row half takes the half of each area that holds its rows (the
  // swizzles depend on r % 16 only, so each half is itself the image of its
  // rows); weights: 4 KB per 128-row block and stage.
  const uint32_t cl0 = 16u * (uint32_t)(64 * wave + lane);
  const uint32_t tl0 = THALF ? 16u * (uint32_t)(32 * wave + (lane & 31)) : cl0;
  const uint32_t wblk = (uint32_t)(K / BK) * 4096u;  // bytes of one 128-row weight block
  // weight unit 64 (w + PW j) + l lies in 128-row block (64 w + l) / 256 + j PW / 4
  // (half loads: unit 32 w + l of the one block, lanes l < 32)
  const uint32_t wb0 = BHALF ? 16u * (uint32_t)(32 * wave + (lane & 31))
                             : (uint32_t)((64 * wave + lane) / 256) * wblk + 16u * (uint32_t)((64 * wave + lane) % 256);
  constexpr uint32_t kOut = 0x80000000u;  // beyond any buffer range: reads zero, stores dropped
  constexpr int kNT = 2;                  // buffer store cache policy: non-temporal

  int dr = 0, dk = 0;  // load cursor: tile dr of this block, stage dk
  uint32_t amo = 0, ato = 16384;  // offsets of the tile's main and tail areas in a stage image
  __amdgpu_buffer_rsrc_t rA, rB;
  auto set_tile = [&](int r) {
    int64_t m0 = 0, n0 = 0;
    int ks = 0;
    if (r < ntiles) tile_of(r, m0, n0, ks);
    // the code buffer holds whole 256-row blocks (rows past M are padding,
    // their outputs are not stored); the weight buffer whole 128-row blocks.
    // Both ranges start at the item's first stage.
    const int64_t wrows = (N + 127) / 128 * 128;
    const int brows = r < ntiles ? (int)min<int64_t>(BN, wrows - n0) : 0;
    const int64_t ka = (int64_t)ks * nks * 24576, kb = (int64_t)ks * nks * 4096;
    const int64_t mb = m0 & ~(int64_t)255;  // the 256-row block holding the tile
    const uint32_t half = (uint32_t)((m0 >> 7) & 1);
    amo = half * 8192u;
    ato = 16384u + half * 4096u;
    rA = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(codes + mb * arow_bytes + ka), (short)0,
                                           r < ntiles ? (int)(256 * arow_bytes - ka) : 0, 0x00020000);
    rB = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(wq) + n0 * brow_bytes + kb), (short)0,
        r < ntiles ? (int)(brows * brow_bytes - kb) : 0, 0x00020000);
  };
  auto stage_load = [&]<int I, bool SW = true>(std::integral_constant<int, I> bi, std::bool_constant<SW> = {}) {
    uint8_t* const Md = mbuf(bi);
    uint8_t* const Td = tbuf(bi);
    uint8_t* const Bd = bbuf(bi);
    const bool live = dr < ntiles;
    const uint32_t vm = live ? (uint32_t)dk * 24576u + amo + cl0 : kOut;
    const uint32_t vt = live ? (uint32_t)dk * 24576u + ato + tl0 : kOut;
    const uint32_t vb = live ? (uint32_t)dk * 4096u + wb0 : kOut;
    if (PW == NW || wave < PW) {
#pragma unroll
    for (int j = 0; j < MDMA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, Md + 1024 * (wave + PW * j), 16, vm + j * (PW * 1024u), 0, 0, 0);
    if constexpr (THALF) {
      if (lane < 32) __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, Td + 512 * wave, 16, vt, 0, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < TDMA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, Td + 1024 * (wave + PW * j), 16, vt + j * (PW * 1024u), 0, 0,
                                                 0);
    }
    if constexpr (BHALF) {
      if (lane < 32) __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, Bd + 512 * wave, 16, vb, 0, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < BDMA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, Bd + 1024 * (wave + PW * j), 16, vb + j * (PW / 4) * wblk, 0, 0,
                                                 0);
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

  v16f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v16f{};

  const int fr = lane % 32, h = lane / 32;
  const int ar = wm * WM + fr, br = wn * WN + fr;
  const int mbase0 = ar * MROW + 16 * mswz(ar, 2 * h), mbase1 = ar * MROW + 16 * mswz(ar, 2 * h + 1);
  const int tbase = ar * TROW + 16 * tswz(ar, h);
  const int bbase = br * BROW + 16 * bswz(br, h);
  constexpr int MFRAG = 32 * MROW, TFRAG = 32 * TROW, BFRAG = 32 * BROW;  // bytes between fragments

  // a stage's fragments: per weight fragment one unit (both steps); per
  // code fragment and step the main unit and the tail half, read straight
  // into the six operand registers
  struct Frag {
    uint4 w[FN];
    v6i c0[FM], c1[FM];
  };
  auto read_frag = [&]<int I>(Frag& f, std::integral_constant<int, I> bi) {
    const uint8_t* Mb = mbuf(bi);
    const uint8_t* Tb = tbuf(bi);
    const uint8_t* Bb = bbuf(bi);
#pragma unroll
    for (int i = 0; i < FN; ++i) f.w[i] = *reinterpret_cast<const uint4*>(Bb + bbase + BFRAG * i);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const uint4 a = *reinterpret_cast<const uint4*>(Mb + mbase0 + MFRAG * j);
      const uint2 ta = *reinterpret_cast<const uint2*>(Tb + tbase + TFRAG * j);
      f.c0[j] = v6i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)ta.x, (int)ta.y};
      const uint4 c = *reinterpret_cast<const uint4*>(Mb + mbase1 + MFRAG * j);
      const uint2 tc = *reinterpret_cast<const uint2*>(Tb + tbase + 8 + TFRAG * j);
      f.c1[j] = v6i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, (int)tc.x, (int)tc.y};
    }
  };
  // weights of step t: words 2t, 2t+1 of the unit -> four E2M1 words
  auto decw = [&](v4i (&wf)[FN], const uint4 (&w)[FN], int t) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const uint32_t w0 = t == 0 ? w[i].x : w[i].z, w1 = t == 0 ? w[i].y : w[i].w;
      wf[i] = v4i{(int)(w0 & 0xAAAAAAAAu), (int)((w0 << 1) & 0xAAAAAAAAu), (int)(w1 & 0xAAAAAAAAu),
                  (int)((w1 << 1) & 0xAAAAAAAAu)};
    }
  };
  // the operand registers beyond the format's width (4 for E2M1, 6 for
  // E3M2) are not read: left undefined
  auto step = [&](const v4i (&wf)[FN], const v6i (&cf)[FM]) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const v8i b8 = __builtin_shufflevector(cf[j], cf[j], 0, 1, 2, 3, 4, 5, -1, -1);
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const v8i a8 = __builtin_shufflevector(wf[i], wf[i], 0, 1, 2, 3, -1, -1, -1, -1);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 4, 3, 0, 0, 0, 0);
      }
    }
  };
  auto bar = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto epilogue = [&](int r) {
    // r and the lane's coordinates made opaque here: nothing of the epilogue
    // (addresses included) is computed early and kept live through the loop
    asm volatile("" : "+s"(r));
    int fr = lane % 32, h = lane / 32;
    asm volatile("" : "+v"(fr), "+v"(h));
    if ((BM == 128 || BN == 128) && ksplit > 1) {
      // exact partial sums, in fragment order: each store is 1 KB contiguous
      // (splits use the narrow tiles only)
      const int64_t item = r * P + slot;
      if (p16) {
        uint4* dst = static_cast<uint4*>(part) + (item * NW + wave) * (FN * FM * 2 * 64) + lane;
        auto pk = [](float lo, float hi) { return ((uint32_t)(int)lo & 0xffffu) | ((uint32_t)(int)hi << 16); };
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
              const v16f& a = acc[i][j];
              const int e = 8 * qq;
              dst[((i * FM + j) * 2 + qq) * 64] =
                  make_uint4(pk(a[e], a[e + 1]), pk(a[e + 2], a[e + 3]), pk(a[e + 4], a[e + 5]), pk(a[e + 6], a[e + 7]));
            }
      } else {
        float4* dst = static_cast<float4*>(part) + (item * NW + wave) * (FN * FM * 4 * 64) + lane;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const v16f& a = acc[i][j];
              dst[((i * FM + j) * 4 + q) * 64] = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
            }
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v16f{};
      return;
    }
    int64_t m0, n0;
    int ks;
    tile_of(r, m0, n0, ks);
    const float al = *alpha;
    if constexpr (STAGE_OUT) {
      uint8_t* const Ow = Os + wave * 32 * OROW;
      constexpr int U = WN * 2 / 16;  // 16-byte units per staged row
      const bool wide = (ldo & 7) == 0;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int64_t m = m0 + wm * WM + 32 * j + fr;
        const float sc = m < M ? scales[m] * al : 0.0f;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v16f& a = acc[i][j];
            const uint32_t lo = pk_bf16(sc * a[4 * q], sc * a[4 * q + 1]);
            const uint32_t hi = pk_bf16(sc * a[4 * q + 2], sc * a[4 * q + 3]);
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
    } else if constexpr (STAGE_HALF) {
      // per fragment row and half of the wave's features: the fragments'
      // 8-byte pieces go to the wave's own [32][64] bf16 area (unit u of
      // row r at u ^ (r % 8)), then each lane stores 16 bytes: a store
      // instruction writes 8 whole 128-byte rows
      uint8_t* const Ow = Os + wave * 32 * 128;
      const bool wide = (ldo & 7) == 0;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int64_t m = m0 + wm * WM + 32 * j + fr;
        const float sc = m < M ? scales[m] * al : 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) {
            const v16f& a = acc[2 * half + ii][j];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t lo = pk_bf16(sc * a[4 * q], sc * a[4 * q + 1]);
              const uint32_t hi = pk_bf16(sc * a[4 * q + 2], sc * a[4 * q + 3]);
              *reinterpret_cast<uint2*>(Ow + fr * 128 + 16 * ((4 * ii + q) ^ (fr & 7)) + 8 * h) = make_uint2(lo, hi);
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the area is the wave's own: no barrier
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            // 8 rows per store; lanes outside the matrix take an offset
            // past the range (dropped), so every store is issued
            const int rl = (fr >> 3) + 4 * h, u = fr & 7, row = rl + 8 * pp;
            const int64_t mr = m0 + wm * WM + 32 * j + 8 * pp, nc = n0 + wn * WN + 64 * half;
            const uint4 v = *reinterpret_cast<const uint4*>(Ow + row * 128 + 16 * (u ^ (row & 7)));
            const __amdgpu_buffer_rsrc_t rO = __builtin_amdgcn_make_buffer_rsrc(
                reinterpret_cast<uint16_t*>(out) + mr * ldo + nc, (short)0, 0x7fffffff, 0x00020000);
            const bool ok = mr + rl < M && nc + 8 * u < N;
            const uint32_t off = ok ? (uint32_t)(rl * ldo + 8 * u) * 2u : kOut;
            // non-temporal (cache policy bit 1, "nt"): a round of tiles writes
            // about an L2's worth of outputs per XCD, which would otherwise
            // displace the code and weight rows the next tiles read again
            if (wide) {
              __builtin_amdgcn_raw_buffer_store_b128(v4u{v.x, v.y, v.z, v.w}, rO, (int)off, 0, kNT);
            } else {  // rows 8-byte aligned: two stores (more in flight than EPI_STORES: waits only lengthen)
              __builtin_amdgcn_raw_buffer_store_b64(v2u{v.x, v.y}, rO, (int)off, 0, kNT);
              __builtin_amdgcn_raw_buffer_store_b64(v2u{v.z, v.w}, rO, (int)(off + 8u), 0, kNT);
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next half's writes
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int64_t m = m0 + wm * WM + 32 * j + fr;
        if (m < M) {
          const float sc = scales[m] * al;
#pragma unroll
          for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int64_t n = n0 + wn * WN + 32 * i + 8 * q + 4 * h;
              const v16f& a = acc[i][j];
              if (n < N) store4f<OUT>(out, m * ldo + n, a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3], sc);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // one fragment row's values live at a time
      }
    }
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = v16f{};
  };

  if (ntiles == 0) return;
  set_tile(0);
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (stage_load(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, NST>{});
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 1) * DPS) : "memory");
  bar();
  Frag f0, f1;
  v4i wf0[FN], wf1[FN];
  read_frag(f0, std::integral_constant<int, 0>{});
  decw(wf0, f0.w, 0);
  // Stage Q of a group of NST: buffer Q, fragments f0 / f1 by parity.  The
  // weight operands of the next step are formed while a step's MFMAs run
  // (an MFMA whose operand was just written by the VALU waits for it).
  // A staged epilogue leaves EPI_STORES stores per wave in flight.  In
  // the next tile's first group, the stage loads a body waits for were
  // issued before them in its first NST - 1 bodies: those bodies let them
  // run on while the tile's MFMAs start (counts retire in issue order).
  constexpr int EPI_STORES = STAGE_HALF ? FM * 2 * 4 : 0;
  auto body = [&]<int Q, bool AFTER = false>(std::integral_constant<int, Q>, std::bool_constant<AFTER> = {}) {
    Frag& cur = (Q % 2 == 0) ? f0 : f1;
    Frag& nxt = (Q % 2 == 0) ? f1 : f0;
    step(wf0, cur.c0);
    decw(wf1, cur.w, 1);
    constexpr int inflight = (NST - 2) * DPS + (AFTER && Q < NST - 1 ? EPI_STORES : 0);
    static_assert(inflight <= 63, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(inflight) : "memory");
    bar();
    // nks is a multiple of NST and the loads run NST stages ahead, so the
    // load cursor reaches the end of a tile only in the group's last body
    stage_load(std::integral_constant<int, Q>{}, std::bool_constant<Q == NST - 1>{});
    read_frag(nxt, std::integral_constant<int, (Q + 1) % NST>{});
    step(wf1, cur.c1);
    decw(wf0, nxt.w, 0);
    if constexpr (Q != NST - 1) {
      // the next stage's fragment reads spread over this step's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x020, DPS, 0);
#pragma unroll
      for (int g = 0; g < (FM * 4 + FN + 1) / 2; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * FM * FN - (FM * 4 + FN + 1) / 2, 0);
    }
  };
  const int groups_per_tile = nks / NST;
  if constexpr (EPI_STORES > 0) {
    // the first tile starts as every later one: EPI_STORES stores issued
    // after its first stages' loads (an empty range: all dropped)
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(out, (short)0, 0, 0x00020000);
#pragma unroll
    for (int e = 0; e < EPI_STORES; ++e) __builtin_amdgcn_raw_buffer_store_b128(v4u{0u, 0u, 0u, 0u}, rz, 16 * e, 0, 0);
  }
  for (int r = 0; r < ntiles; ++r) {
    int gq = 0;
    if constexpr (EPI_STORES > 0) {
      if (r > 0) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
          (body(std::integral_constant<int, I>{}, std::true_type{}), ...);
        }(std::make_integer_sequence<int, NST>{});
        gq = 1;
      }
    }
    for (; gq < groups_per_tile; ++gq) {
      [&]<int... I>(std::integer_sequence<int, I...>) {
        (body(std::integral_constant<int, I>{}), ...);
      }(std::make_integer_sequence<int, NST>{});
    }
    epilogue(r);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

// Ternary layout of the library (c = q + 1 at bits 8b + 2s of each word,
// weight 4s + b) -> MX4 words in the tiled stage images; one thread per
// output word.  Output word w4 of tile (block nb of 128 rows, stage s of 128
// k) at physical unit p = w4 / 4: row r = p / 2 of the block, logical unit
// u = (p % 2) ^ ((r >> 3) & 1), i.e. k = 128 s + 64 u + 16 (w4 % 4) ..+ 15.
// Rows past N are zero.
__global__ void k_prepare_mx4(const uint32_t* __restrict__ wp, int64_t N, int64_t K, int64_t n_out,
                              uint32_t* __restrict__ wq) {
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= n_out) return;
  const int64_t stages = K / 128;
  const int64_t tile = o >> 10, within = o & 1023;
  const int64_t nb = tile / stages, st = tile % stages;
  const int p = (int)(within >> 2), wi = (int)(within & 3);
  const int r = p >> 1, u = (p & 1) ^ ((r >> 3) & 1);
  const int64_t n = nb * 128 + r;
  uint32_t res = 0;
  if (n < N) {
    const uint32_t w = wp[n * (K / 16) + st * 8 + u * 4 + wi];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t c = (w >> (8 * (j & 3) + 2 * (j >> 2))) & 3u;  // weight j: s = j / 4, b = j % 4
      const uint32_t nz = c != 1u, neg = c == 0u;
      const int nn = j & 7, hi = j >> 3;  // k < 8: bits 4n+1, 4n+3; else 4n, 4n+2
      res |= (nz << (4 * nn + 1 - hi)) | (neg << (4 * nn + 3 - hi));
    }
  }
  wq[o] = res;
}

}  // namespace

hipError_t launch_prepare_mx4(const uint32_t* wp, int64_t N, int64_t K, uint32_t* wq, hipStream_t s) {
  const int64_t n_out = (N + 127) / 128 * 128 * (K / 16);
  if (n_out == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prepare_mx4, dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, s, wp, N, K, n_out, wq);
  return hipGetLastError();
}

namespace {

// Sum of the ksplit partial sums of each output (exact integers: any order
// gives the same value), then the rescale of Eq. 9.  One thread per four
// (fp32 partials) or eight (int16) outputs of one lane's fragment, reading
// the partials in the order k_gemm_mx wrote them.
template <int OUT, int BM, int BN, bool P16, int NWV>
__global__ void __launch_bounds__(256)
k_mx_reduce(const void* __restrict__ part, int ksplit, int tilesM, int tilesN, int gm, const float* __restrict__ scales,
            const float* __restrict__ alpha, int64_t M, int64_t N, void* __restrict__ out, int64_t ldo) {
  // the wave grid of k_gemm_mx for the tile shape
  constexpr int NW = NWV, WGM = BM == 128 ? 2 : NW / 2, WGN = NW / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  constexpr int QU = P16 ? 2 : 4;                         // 16-byte units per fragment and lane
  const int64_t per_tile = (int64_t)NW * FN * FM * QU * 64;  // units of one tile
  const int64_t units = (int64_t)tilesM * tilesN * per_tile;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  const int lane = (int)(u % 64);
  int64_t t = u / 64;
  const int q = (int)(t % QU);
  t /= QU;
  const int ij = (int)(t % (FN * FM));
  t /= FN * FM;
  const int wave = (int)(t % NW);
  const int T = (int)(t / NW);
  const int i = ij / FM, j = ij % FM, wm = wave % WGM, wn = wave / WGM, fr = lane % 32, h = lane / 32;
  int64_t m0, n0;
  int ks;
  split_item<BM, BN>(T, tilesM, tilesN, gm, m0, n0, ks);
  const int64_t m = m0 + wm * WM + 32 * j + fr;
  const int64_t n = n0 + wn * WN + 32 * i + (P16 ? 16 : 8) * q + 4 * h;
  if (m >= M || n >= N) return;
  const float sc = scales[m] * *alpha;
  if constexpr (P16) {
    const uint4* p = static_cast<const uint4*>(part) + u;
    int v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s = 0; s < ksplit; ++s) {
      const uint4 b = p[s * units];
      const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] += (int)(int16_t)(w[e] & 0xffffu);
        v[2 * e + 1] += (int)(int16_t)(w[e] >> 16);
      }
    }
    store4f<OUT>(out, m * ldo + n, (float)v[0], (float)v[1], (float)v[2], (float)v[3], sc);
    if (n + 8 < N) store4f<OUT>(out, m * ldo + n + 8, (float)v[4], (float)v[5], (float)v[6], (float)v[7], sc);
  } else {
    const float4* p = static_cast<const float4*>(part) + u;
    float4 a = p[0];
    for (int s = 1; s < ksplit; ++s) {
      const float4 b = p[s * units];
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    store4f<OUT>(out, m * ldo + n, a.x, a.y, a.z, a.w, sc);
  }
}

struct MxPlan : SplitPlan {
  bool p16;  // int16 partial sums
  size_t part_bytes() const { return ksplit > 1 ? (size_t)ksplit * tm * tn * bm * bn * (p16 ? 2 : 4) : 0; }
};

// narrow tiles (fewer 256 x 256 tiles than CUs) are 128 x 256, split or not
MxPlan mx_plan(int64_t M, int64_t N, int64_t K, int cu_count, bool may_split) {
  MxPlan p;
  static_cast<SplitPlan&>(p) = split_plan(M, N, K, cu_count, may_split, true);
  p.p16 = 8 * (K / p.ksplit) <= 32767;  // |partial sum| <= 8 K / ksplit
  return p;
}

}  // namespace

size_t gemm_mx_partial_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return mx_plan(M, N, K, kSplitItems, true).part_bytes();
}

hipError_t launch_gemm_mx(const void* codes, const float* scales, const uint32_t* wq, const float* alpha, int64_t M,
                          int64_t N, int64_t K, int out_kind, void* out, int64_t ldo, void* part, size_t part_bytes,
                          int cu_count, hipStream_t s) {
  if (M == 0) return hipSuccess;
  // the split is sized for kSplitItems CUs; with a workspace too small for it
  // (or none) the matmul runs unsplit
  MxPlan p = mx_plan(M, N, K, cu_count, part != nullptr);
  if (p.ksplit > 1 && part_bytes < p.part_bytes()) p.ksplit = 1;
  const int64_t G = (int64_t)p.tm * p.tn * p.ksplit;
  const int64_t cap = cu_count >= 8 ? (cu_count / 8) * 8 : 8;
  const int64_t P = std::min<int64_t>(((G + 7) / 8) * 8, cap);
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  const int ksplit = p.ksplit, tm = p.tm, tn = p.tn, gm = p.gm, p16 = p.p16 ? 1 : 0;
  // 8 waves (two per SIMD: one wave's barrier and operand waits are covered
  // by the other's MFMAs).  Narrow tiles are 128 x 256: the same outputs per
  // tile as 256 x 128 from 20 instead of 28 KB of operands per stage (6-bit
  // codes cost more bytes per row than 2-bit weights).  Measured on MI355X
  // against 256 x 128 (bit-identical), unsplit: layer at M = 2048, N = K =
  // 4096 35.1 -> 32.9 us, M = 1024 28.8 -> 27.2, M = 3072 55.1 -> 53.4;
  // M = 2048, K = 16384 102 -> 99.
#define HBL_MXT(OUT, BM, BN, PWV)                                                                          \
  hipLaunchKernelGGL((k_gemm_mx<OUT, BM, BN, 8, PWV>), dim3((unsigned)P), dim3(512), 0, s, c, scales, wq, alpha, M, N, \
                     K, out, ldo, tm, tn, gm, ksplit, p16, part)
  // bf16 outputs of 256 x 256 tiles up to K = 8192: the stage loads from one
  // wave per SIMD (bit-identical; us against all eight waves loading: 65536
  // x 4096 x 4096 508 -> 496, 65536 x 16384 x 4096 2033 -> 1991; at K =
  // 16384 slower, 1835 -> 1895)
  if (p.bm == 128) {
    if (out_kind == 0) HBL_MXT(0, 128, 256, 8); else if (out_kind == 1) HBL_MXT(1, 128, 256, 8); else HBL_MXT(2, 128, 256, 8);
  } else {
    if (out_kind == 0) {
      if (K <= 8192) HBL_MXT(0, 256, 256, 4); else HBL_MXT(0, 256, 256, 8);
    } else if (out_kind == 1) {
      HBL_MXT(1, 256, 256, 8);
    } else {
      HBL_MXT(2, 256, 256, 8);
    }
  }
#undef HBL_MXT
  if (ksplit == 1) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // (splits use the 128 x 256 tiles only)
  const int64_t units = (int64_t)tm * tn * 128 * 256 / (p16 ? 8 : 4);
  const unsigned rb = (unsigned)((units + 255) / 256);
#define HBL_MXR(OUT, P16)                                                                                          \
  hipLaunchKernelGGL((k_mx_reduce<OUT, 128, 256, P16, 8>), dim3(rb), dim3(256), 0, s, part, ksplit, tm, tn, gm, scales, \
                     alpha, M, N, out, ldo)
  if (p16) {
    if (out_kind == 0) { HBL_MXR(0, true); } else if (out_kind == 1) { HBL_MXR(1, true); } else { HBL_MXR(2, true); }
  } else {
    if (out_kind == 0) { HBL_MXR(0, false); } else if (out_kind == 1) { HBL_MXR(1, false); } else { HBL_MXR(2, false); }
  }
#undef HBL_MXR
  return hipGetLastError();
}

}  // namespace hbl
