// Absmean ternary weight quantiser for gfx950 (architecture write-up of
// "BitNet v2", §3.4 "Weight Quantization", Eq. 1-2):
//   alpha = mean |W| over the whole matrix,
//   q     = RoundClip(W / (alpha + eps), -1, 1), round = nearest-even,
// packed two bits per weight (c = q + 1) in the layout of include/hbl.h.
//
// Three launches, all deterministic:
//   1. each block sums |W| over a fixed contiguous range in fp64;
//   2. one block adds the partial sums in a fixed tree order and writes
//      alpha = (float)(sum / (N*K));
//   3. one thread per packed word quantises 16 weights and packs them.
// The matrix is static, so this runs once per weight matrix, off the token
// path.
#include "hbl_internal.h"

namespace hbl {
namespace {

constexpr float kEps = 1e-5f;
constexpr int kPartialThreads = 256;
constexpr int kMaxPartials = 1024;

__device__ __forceinline__ float wload(const void* w, bool bf16, int64_t i) {
  if (bf16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(w)[i] << 16);
  return reinterpret_cast<const float*>(w)[i];
}

__device__ double block_sum_f64(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  return sh[0];
}

__global__ void __launch_bounds__(kPartialThreads)
k_abs_partial(const void* __restrict__ w, bool bf16, int64_t total, int64_t chunk,
              double* __restrict__ partials) {
  __shared__ double sh[kPartialThreads];
  const int64_t begin = (int64_t)blockIdx.x * chunk;
  int64_t end = begin + chunk;
  if (end > total) end = total;
  double acc = 0.0;
  for (int64_t i = begin + threadIdx.x; i < end; i += kPartialThreads)
    acc += fabs((double)wload(w, bf16, i));
  const double s = block_sum_f64(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__global__ void __launch_bounds__(kMaxPartials)
k_alpha(const double* __restrict__ partials, int n, int64_t total, float* __restrict__ alpha) {
  __shared__ double sh[kMaxPartials];
  const double v = (int)threadIdx.x < n ? partials[threadIdx.x] : 0.0;
  const double s = block_sum_f64(v, sh);
  if (threadIdx.x == 0) *alpha = (float)(s / (double)total);
}

__global__ void __launch_bounds__(256)
k_ternarize_pack(const void* __restrict__ w, bool bf16, int64_t n_words,
                 const float* __restrict__ alpha, uint32_t* __restrict__ packed) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_words) return;
  const float d = *alpha + kEps;
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float q = fminf(fmaxf(__builtin_rintf(wload(w, bf16, 16 * i + j) / d), -1.0f), 1.0f);
    const uint32_t c = (uint32_t)((int)q + 1);
    word |= c << (8 * (j & 3) + 2 * (j >> 2));
  }
  packed[i] = word;
}

}  // namespace

int ternarize_partials(int64_t N, int64_t K) {
  const int64_t total = N * K;
  int64_t p = (total + 65535) / 65536;
  if (p < 1) p = 1;
  if (p > kMaxPartials) p = kMaxPartials;
  return (int)p;
}

hipError_t launch_ternarize(const void* w, bool w_bf16, int64_t N, int64_t K, uint32_t* packed,
                            float* alpha, double* partials, int n_partials, hipStream_t s) {
  const int64_t total = N * K;
  const int64_t chunk = (total + n_partials - 1) / n_partials;
  hipLaunchKernelGGL(k_abs_partial, dim3(n_partials), dim3(kPartialThreads), 0, s, w, w_bf16, total,
                     chunk, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_alpha, dim3(1), dim3(kMaxPartials), 0, s, partials, n_partials, total, alpha);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_words = total / 16;
  hipLaunchKernelGGL(k_ternarize_pack, dim3((unsigned)((n_words + 255) / 256)), dim3(256), 0, s, w,
                     w_bf16, n_words, alpha, packed);
  return hipGetLastError();
}

}  // namespace hbl
