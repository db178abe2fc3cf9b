// N:M mask from fp32 scores. Each thread loads 4 consecutive scores per
// 16-byte load (a wave's load covers 1 KB, fully coalesced; MASK_U loads in
// flight per thread, non-temporal: the scores are read once);
// a group of M = 8 spans two lanes, which exchange their halves. The 4 bits
// of a lane are ORed over the 8 lanes that hold one 32-position word and
// the first of them writes the packed word (bit k mod 32 = position k,
// 1 = kept). The keep rule is nm_keep in common.h: ties to the lower
// position, NaN as -inf.
#include "common.h"
#include "kernels.h"

namespace lcp {

constexpr int MASK_U = 4;   // 16-byte loads in flight per thread

template <int M>
__global__ __launch_bounds__(256) void nm_mask_kernel(const float* __restrict__ scores, long long n4, int N,
                                                      uint32_t* __restrict__ bits) {
  const int l = threadIdx.x & 63;
  const long long base = (long long)blockIdx.x * (256 * MASK_U) + threadIdx.x;   // index of 4 scores
  floatx4 x[MASK_U];
#pragma unroll
  for (int u = 0; u < MASK_U; ++u) {
    const long long id = base + 256 * u;
    x[u] = id < n4 ? __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(scores) + id)
                   : floatx4{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
  }
#pragma unroll
  for (int u = 0; u < MASK_U; ++u) {
    const long long id = base + 256 * u;
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = nan_to_ninf(x[u][c]);
    uint32_t nib;
    if constexpr (M == 4) {
      nib = nm_keep<4>(v, N);
    } else {
      // lanes 2k and 2k + 1 hold one group of 8; both rank it, the even lane keeps its bits
      float g[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float o = shfl_xor(v[c], 1);
        g[c] = (l & 1) ? o : v[c];
        g[4 + c] = (l & 1) ? v[c] : o;
      }
      const uint32_t k = nm_keep<8>(g, N);
      nib = (l & 1) ? 0u : k;
    }
    // lane l contributes bits 4 (l % 8) .. of the word held by lanes 8 (l / 8) ..
    uint32_t w = nib << (4 * (l & 7));
    w |= (uint32_t)__shfl_xor((int)w, 1, 64);
    w |= (uint32_t)__shfl_xor((int)w, 2, 64);
    w |= (uint32_t)__shfl_xor((int)w, 4, 64);
    if ((l & 7) == 0 && id < n4) bits[id >> 3] = w;
  }
}

hipError_t launch_nm_mask(const float* scores, int rows, int cin, int N, int M, uint32_t* bits,
                          hipStream_t s) {
  const long long n4 = (long long)rows * (cin / 4);
  const int grid = (int)((n4 + 256 * MASK_U - 1) / (256 * MASK_U));
  if (M == 4) nm_mask_kernel<4><<<grid, 256, 0, s>>>(scores, n4, N, bits);
  else if (M == 8) nm_mask_kernel<8><<<grid, 256, 0, s>>>(scores, n4, N, bits);
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
