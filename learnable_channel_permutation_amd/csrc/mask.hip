// N:M mask from fp32 scores. One thread per 32-position word of one row:
// it loads the 32 scores, ranks each group of M in registers and writes the
// packed word (bit k mod 32 = position k, 1 = kept). The keep rule is
// nm_keep in common.h: ties to the lower position, NaN as -inf.
#include "common.h"
#include "kernels.h"

namespace lcp {

template <int M>
__global__ __launch_bounds__(256) void nm_mask_kernel(const float* __restrict__ scores, int rows,
                                                      int words, int N, uint32_t* __restrict__ bits) {
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  if (id >= (long long)rows * words) return;
  const float* src = scores + id * 32;
  float v[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const floatx4 x = *reinterpret_cast<const floatx4*>(src + 4 * q);
    v[4 * q + 0] = nan_to_ninf(x[0]);
    v[4 * q + 1] = nan_to_ninf(x[1]);
    v[4 * q + 2] = nan_to_ninf(x[2]);
    v[4 * q + 3] = nan_to_ninf(x[3]);
  }
  uint32_t w = 0;
#pragma unroll
  for (int g = 0; g < 32 / M; ++g) w |= nm_keep<M>(v + g * M, N) << (g * M);
  bits[id] = w;
}

hipError_t launch_nm_mask(const float* scores, int rows, int cin, int N, int M, uint32_t* bits,
                          hipStream_t s) {
  const int words = cin / 32;
  const long long n = (long long)rows * words;
  const int grid = (int)((n + 255) / 256);
  if (M == 4) nm_mask_kernel<4><<<grid, 256, 0, s>>>(scores, rows, words, N, bits);
  else if (M == 8) nm_mask_kernel<8><<<grid, 256, 0, s>>>(scores, rows, words, N, bits);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Mask words of the step (block-major: word a of row i in block b at
// (b * rows + i) * (B / 32) + a) to the row-major layout [rows][cin / 32].
__global__ __launch_bounds__(256) void bits_rowmajor_kernel(const uint32_t* __restrict__ bm, int rows,
                                                            int words, int tt, uint32_t* __restrict__ out) {
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  if (id >= (long long)rows * words) return;
  const int i = (int)(id / words), wd = (int)(id % words);
  const int b = wd / tt, a = wd % tt;
  out[id] = bm[((size_t)b * rows + i) * tt + a];
}

hipError_t launch_bits_rowmajor(const uint32_t* bm, int rows, int cin, int B, uint32_t* out, hipStream_t s) {
  const int words = cin / 32;
  const long long n = (long long)rows * words;
  bits_rowmajor_kernel<<<(int)((n + 255) / 256), 256, 0, s>>>(bm, rows, words, B / 32, out);
  return hipGetLastError();
}

}  // namespace lcp
