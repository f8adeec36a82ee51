// Measured peaks of the device, the denominators the matmul and streaming
// kernels of libhbl are compared against:
//   * dense int8 matrix-core throughput: every SIMD of every CU runs
//     independent chains of v_mfma_i32_16x16x64_i8 / v_mfma_i32_32x32x32_i8
//     on register-resident operands, reading the same registers or rotating
//     over four sets, for five kinds of operand bits (the datapath's
//     switching activity, hence its power and clock, depends on them);
//   * dense FP6 x FP4 matrix-core throughput (v_mfma_f32_32x32x64_f8f6f4,
//     E2M1 first operand, E3M2 second: the INT4 matmul's formats), one and
//     four waves per SIMD, for operands like the matmul's and random bits;
//   * HBM read bandwidth: one streaming read of 2 GiB;
//   * the streaming floor of one launch: graph replays of launches that each
//     read 16 MiB or 4 MiB from buffers cycled through more memory than the
//     caches hold (the decode weight sizes), and of an empty launch.
// A stand-alone program (no library code); prints one line per measurement.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

#define CK(x)                                                                                  \
  do {                                                                                         \
    hipError_t e_ = (x);                                                                       \
    if (e_ != hipSuccess) {                                                                    \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);    \
      std::exit(1);                                                                            \
    }                                                                                          \
  } while (0)

// NACC independent accumulators per wave.  ROT: the operands rotate over 4
// register sets, so that consecutive MFMAs read different registers (as a
// matmul does); otherwise every MFMA reads the same two operands.
template <int NACC, bool BIG, bool ROT>
__global__ void __launch_bounds__(256) k_mfma(int iters, const uint32_t* __restrict__ ops, int* __restrict__ sink,
                                              long long* __restrict__ clk) {
  v4i a[4], b[4];
  const uint4* src = reinterpret_cast<const uint4*>(ops) + (size_t)(blockIdx.x * 256 + threadIdx.x) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = src[i], w = src[4 + i];
    a[i] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
    b[i] = v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
  }
  const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  int s = 0;
  if constexpr (BIG) {
    v16i acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = v16i{};
    for (int it = 0; it < iters; it += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < NACC; ++i)
          acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ROT ? (i + u) % 4 : 0], b[ROT ? (i + 2 * u) % 4 : 0], acc[i],
                                                         0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NACC; ++i) s += acc[i][0] ^ acc[i][15];
  } else {
    v4i acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = v4i{0, 0, 0, 0};
    for (int it = 0; it < iters; it += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < NACC; ++i)
          acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[ROT ? (i + u) % 4 : 0], b[ROT ? (i + 2 * u) % 4 : 0], acc[i],
                                                         0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NACC; ++i) s += acc[i][0] ^ acc[i][3];
  }
  const long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// FP6 x FP4: per thread 40 words, four 4-word E2M1 operands then four
// 6-word E3M2 operands, rotated as in k_mfma.
template <int NACC>
__global__ void __launch_bounds__(256) k_mfma_mx(int iters, const uint32_t* __restrict__ ops, int* __restrict__ sink,
                                                 long long* __restrict__ clk) {
  v4i a[4];
  v6i b[4];
  const uint32_t* src = ops + (size_t)(blockIdx.x * 256 + threadIdx.x) * 40;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = v4i{(int)src[4 * i], (int)src[4 * i + 1], (int)src[4 * i + 2], (int)src[4 * i + 3]};
    b[i] = v6i{(int)src[16 + 6 * i], (int)src[17 + 6 * i], (int)src[18 + 6 * i], (int)src[19 + 6 * i],
               (int)src[20 + 6 * i], (int)src[21 + 6 * i]};
  }
  const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  v16f acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = v16f{};
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NACC; ++i) {
        const v4i& x = a[(i + u) % 4];
        const v6i& y = b[(i + 2 * u) % 4];
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_shufflevector(x, x, 0, 1, 2, 3, -1, -1, -1, -1),
                                                                 __builtin_shufflevector(y, y, 0, 1, 2, 3, 4, 5, -1, -1),
                                                                 acc[i], 4, 3, 0, 0, 0, 0);
      }
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < NACC; ++i) s += (int)acc[i][0] ^ (int)acc[i][15];
  const long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// FP6 x FP4 operand bits, per thread 16 E2M1 words then 24 E3M2 words:
//   0 like the INT4 matmul: E2M1 nibbles of random ternary weights, E3M2
//     codes of random integers in [-8, 7] (one per byte)
//   1 random bits
__global__ void k_fill_mx(uint32_t* p, size_t n, int mode) {
  static constexpr uint8_t kE3M2[16] = {56, 55, 54, 53, 52, 50, 48, 44, 0, 12, 16, 18, 20, 21, 22, 23};  // -8 .. 7
  static constexpr uint8_t kE2M1[3] = {10, 0, 2};                                                     // -1, 0, 1
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    uint64_t z = (uint64_t)i * 0x9E3779B97F4A7C15ull + 777u;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    uint32_t v = (uint32_t)z;
    if (mode == 0) {
      v = 0;
      if (i % 40 < 16) {
        for (int j = 0; j < 8; ++j) v |= (uint32_t)kE2M1[((z >> (5 * j)) & 31) % 3] << (4 * j);
      } else {
        for (int j = 0; j < 4; ++j) v |= (uint32_t)kE3M2[(z >> (8 * j)) & 15] << (8 * j);
      }
    }
    p[i] = v;
  }
}

// Each block streams R 16-byte units per thread (unit t + 256 r of its
// slab) and folds them into one word per wave.
template <int R>
__global__ void __launch_bounds__(256) k_read(const uint4* __restrict__ p, uint32_t* __restrict__ sink) {
  const uint4* q = p + (size_t)blockIdx.x * 256 * R + threadIdx.x;
  uint32_t s = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(q + 256 * r));
    s ^= t[0] ^ t[1] ^ t[2] ^ t[3];
  }
  for (int o = 32; o > 0; o >>= 1) s ^= __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + threadIdx.x / 64] = s;
}

// Operand bits, per thread 16 words of first operand then 16 of second:
//   0 low switching: the bytes 1 and 0 in a fixed pattern
//   1 every byte 0x11
//   2 like the INT4 matmul: first operand random high nibbles (16 q),
//     second random bytes in {0, 1, 2} (the widened ternary weights)
//   3 like the INT8 matmul: first operand random bytes, second as in 2
//   4 random bytes
__global__ void k_fill(uint32_t* p, size_t n, int mode) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    uint64_t z = (uint64_t)i * 0x9E3779B97F4A7C15ull + 12345u;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    const uint32_t r = (uint32_t)(z ^ (z >> 31));
    const bool first = (i % 32) < 16;
    const uint32_t c3 = (r & 0x01010101u) + ((r >> 8) & 0x01010101u);  // bytes in {0, 1, 2}
    uint32_t v;
    switch (mode) {
      case 0: v = (i % 4 == 0) ? 0x00000001u : 0u; break;
      case 1: v = 0x11111111u; break;
      case 2: v = first ? (r & 0xf0f0f0f0u) : c3; break;
      case 3: v = first ? r : c3; break;
      default: v = r; break;
    }
    p[i] = v;
  }
}

}  // namespace

int main() {
  int dev = 0, cus = 0;
  CK(hipGetDevice(&dev));
  CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  hipDeviceProp_t prop;
  CK(hipGetDeviceProperties(&prop, dev));
  std::printf("device %s, %d CUs\n", prop.gcnArchName, cus);

  // ---- int8 matrix cores
  const int max_blocks = 4 * cus;  // up to four 256-thread blocks per CU: four waves per SIMD
  const size_t nops = (size_t)max_blocks * 256 * 8 * 4;  // words: 8 uint4 per thread
  uint32_t* ops;
  int* sink;
  long long* clk;
  CK(hipMalloc(&ops, nops * 4));
  CK(hipMalloc(&sink, (size_t)max_blocks * 256 * 4));
  CK(hipMalloc(&clk, (size_t)max_blocks * 2 * 8));
  static const char* kData[] = {"low-switching", "0x11 bytes", "INT4-like", "INT8-like", "random"};
  auto mfma = [&](auto kern, const char* name, double ops_per_mfma, int nacc, int mode, int waves_per_simd) {
    const int blocks = waves_per_simd * cus;
    hipLaunchKernelGGL(k_fill, dim3(1024), dim3(256), 0, 0, ops, nops, mode);
    const int iters = 2048;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, 0, iters, ops, sink, clk);
    CK(hipDeviceSynchronize());
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    const int reps = 5;
    CK(hipEventRecord(a, 0));
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, 0, iters, ops, sink, clk);
    CK(hipEventRecord(b, 0));
    CK(hipEventSynchronize(b));
    float ms;
    CK(hipEventElapsedTime(&ms, a, b));
    std::vector<long long> h((size_t)blocks * 2);
    CK(hipMemcpy(h.data(), clk, h.size() * 8, hipMemcpyDeviceToHost));
    double c = 0, r = 0;
    for (size_t i = 0; i < h.size(); i += 2) { c += (double)h[i]; r += (double)h[i + 1]; }
    const double total = (double)reps * blocks * 4 * iters * nacc * ops_per_mfma;
    const double ghz = c / (r * 10.0), tops = total / (ms * 1e-3) / 1e12;
    std::printf("mfma %-22s %d wave(s)/SIMD %-14s operands: %7.1f TOP/s at %.2f GHz (%.0f ops/clock/SIMD of 2048)\n",
                name, waves_per_simd, kData[mode], tops, ghz, tops * 1e12 / (ghz * 1e9 * 4 * cus));
    std::fflush(stdout);
  };
  for (int wps : {1, 4})
    for (int mode = 0; mode < 5; ++mode) {
      mfma(k_mfma<8, false, false>, "16x16x64 fixed regs", 32768.0, 8, mode, wps);
      mfma(k_mfma<8, false, true>, "16x16x64 rotating", 32768.0, 8, mode, wps);
      mfma(k_mfma<4, true, false>, "32x32x32 fixed regs", 65536.0, 4, mode, wps);
      mfma(k_mfma<4, true, true>, "32x32x32 rotating", 65536.0, 4, mode, wps);
    }
  // ---- FP6 x FP4 matrix cores
  {
    const size_t nmx = (size_t)max_blocks * 256 * 40;
    uint32_t* mx;
    CK(hipMalloc(&mx, nmx * 4));
    static const char* kMxData[] = {"INT4-like", "random"};
    for (int wps : {1, 4})
      for (int mode = 0; mode < 2; ++mode) {
        const int blocks = wps * cus, iters = 2048, nacc = 4;
        hipLaunchKernelGGL(k_fill_mx, dim3(1024), dim3(256), 0, 0, mx, nmx, mode);
        hipLaunchKernelGGL(k_mfma_mx<4>, dim3(blocks), dim3(256), 0, 0, iters, mx, sink, clk);
        CK(hipDeviceSynchronize());
        hipEvent_t a, b;
        CK(hipEventCreate(&a));
        CK(hipEventCreate(&b));
        const int reps = 5;
        CK(hipEventRecord(a, 0));
        for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(k_mfma_mx<4>, dim3(blocks), dim3(256), 0, 0, iters, mx, sink, clk);
        CK(hipEventRecord(b, 0));
        CK(hipEventSynchronize(b));
        float ms;
        CK(hipEventElapsedTime(&ms, a, b));
        std::vector<long long> h((size_t)blocks * 2);
        CK(hipMemcpy(h.data(), clk, h.size() * 8, hipMemcpyDeviceToHost));
        double c = 0, r = 0;
        for (size_t i = 0; i < h.size(); i += 2) { c += (double)h[i]; r += (double)h[i + 1]; }
        const double total = (double)reps * blocks * 4 * iters * nacc * 131072.0;
        const double ghz = c / (r * 10.0), tops = total / (ms * 1e-3) / 1e12;
        std::printf("mfma fp4 x bf6 32x32x64 %d wave(s)/SIMD %-14s operands: %7.1f TOP/s at %.2f GHz (%.0f ops/clock/SIMD of 4096)\n",
                    wps, kMxData[mode], tops, ghz, tops * 1e12 / (ghz * 1e9 * 4 * cus));
        std::fflush(stdout);
      }
    CK(hipFree(mx));
  }
  CK(hipFree(ops));
  CK(hipFree(sink));
  CK(hipFree(clk));

  // ---- HBM read: 2 GiB once
  {
    const size_t bytes = (size_t)2 << 30;
    uint4* buf;
    uint32_t* s2;
    CK(hipMalloc(&buf, bytes));
    CK(hipMemset(buf, 1, bytes));
    constexpr int R = 16;
    const size_t nblk = bytes / (16 * 256 * R);
    CK(hipMalloc(&s2, nblk * 4 * 4));
    hipLaunchKernelGGL(k_read<R>, dim3((unsigned)nblk), dim3(256), 0, 0, buf, s2);
    CK(hipDeviceSynchronize());
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    const int reps = 5;
    CK(hipEventRecord(a, 0));
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(k_read<R>, dim3((unsigned)nblk), dim3(256), 0, 0, buf, s2);
    CK(hipEventRecord(b, 0));
    CK(hipEventSynchronize(b));
    float ms;
    CK(hipEventElapsedTime(&ms, a, b));
    std::printf("hbm read 2 GiB: %.0f GB/s\n", (double)bytes * reps / (ms * 1e-3) / 1e9);
    std::fflush(stdout);
    CK(hipFree(buf));
    CK(hipFree(s2));
  }

  // ---- one launch per weight matrix: 16 MiB and 4 MiB, cycled over 768 MiB
  {
    const size_t slab = (size_t)16 << 20;
    const int nbuf = 48;
    std::vector<uint4*> bufs(nbuf);
    for (auto& p : bufs) {
      CK(hipMalloc(&p, slab));
      CK(hipMemset(p, 3, slab));
    }
    uint32_t* s3;
    CK(hipMalloc(&s3, 1 << 20));
    hipStream_t st;
    CK(hipStreamCreate(&st));
    auto floor = [&](size_t bytes) {
      constexpr int R = 8;
      const unsigned nblk = bytes ? (unsigned)(bytes / (16 * 256 * R)) : 1;
      hipGraph_t g;
      hipGraphExec_t ge;
      CK(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
      for (int i = 0; i < nbuf; ++i) hipLaunchKernelGGL(k_read<R>, dim3(nblk), dim3(256), 0, st, bufs[i], s3);
      CK(hipStreamEndCapture(st, &g));
      CK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
      CK(hipGraphLaunch(ge, st));
      CK(hipStreamSynchronize(st));
      hipEvent_t a, b;
      CK(hipEventCreate(&a));
      CK(hipEventCreate(&b));
      const int reps = 10;
      CK(hipEventRecord(a, st));
      for (int r = 0; r < reps; ++r) CK(hipGraphLaunch(ge, st));
      CK(hipEventRecord(b, st));
      CK(hipEventSynchronize(b));
      float ms;
      CK(hipEventElapsedTime(&ms, a, b));
      const double us = ms * 1e3 / (reps * nbuf);
      const double rb = bytes ? (double)bytes : 256.0 * 16 * R;
      std::printf("one launch reading %8zu bytes (graph replay, %d distinct buffers): %.2f us per launch, %.0f GB/s\n",
                  (size_t)rb, nbuf, us, rb / us / 1e3);
      std::fflush(stdout);
      CK(hipGraphExecDestroy(ge));
      CK(hipGraphDestroy(g));
    };
    floor(slab);
    floor(slab / 4);
    floor(0);
    for (auto& p : bufs) CK(hipFree(p));
    CK(hipFree(s3));
  }
  return 0;
}
