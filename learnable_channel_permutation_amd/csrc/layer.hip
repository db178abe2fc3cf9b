// Per-layer setup, constant across the LCP steps on one layer: the column
// norms ||X[:, j]||_2 (the activation factor of Wanda's importance) and, for
// bf16 layers, the transposed activations Xt [cin][pitch] that the backward
// GEMM reads with the token index contiguous.
//
// Both kernels walk one strip of 64 channels down all T tokens, so each
// column's sum of squares is accumulated by fixed threads in a fixed order
// (deterministic, no atomics).
#include "common.h"
#include "kernels.h"

namespace lcp {

__global__ __launch_bounds__(256) void colnorm_f32_kernel(const float* __restrict__ X, int T,
                                                          int cin, float* __restrict__ norms) {
  __shared__ float part[4][64];
  const int t = threadIdx.x, col = t & 63, rg = t >> 6;
  const int c = blockIdx.x * 64 + col;
  float s = 0.f;
  if (c < cin)
    for (int r = rg; r < T; r += 4) {
      const float v = X[(size_t)r * cin + c];
      s += v * v;
    }
  part[rg][col] = s;
  __syncthreads();
  if (rg == 0 && c < cin) norms[c] = sqrtf((part[0][col] + part[1][col]) + (part[2][col] + part[3][col]));
}

// Tile of 64 tokens x 64 channels, bf16. Loads are 16-byte chunks, 8 per
// token row; the transposed stores are 16-byte chunks of 8 tokens.
__global__ __launch_bounds__(256) void layer_init_bf16_kernel(const uint16_t* __restrict__ X,
                                                              int T, int cin, int pitch,
                                                              float* __restrict__ norms,
                                                              uint16_t* __restrict__ Xt) {
  constexpr int LD = 64 + 8;  // padded row (uint16) of the LDS tile
  __shared__ uint16_t tile[64 * LD];
  __shared__ float part[4][64];
  const int t = threadIdx.x;
  const int c0 = blockIdx.x * 64;
  const int col = t & 63, rg = t >> 6;
  float ss = 0.f;
  const int t_end = Xt != nullptr ? pitch : T;
  for (int t0 = 0; t0 < t_end; t0 += 64) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int id = t + 256 * q;
      const int row = id >> 3, ch = id & 7;
      const int gr = t0 + row, gc = c0 + ch * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gr < T && gc < cin) v = *reinterpret_cast<const u32x4*>(X + (size_t)gr * cin + gc);
      uint32_t* dst = reinterpret_cast<uint32_t*>(tile + row * LD + ch * 8);
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = bf2f(tile[(rg * 16 + r) * LD + col]);
      ss += v * v;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int id = t + 256 * q;
      const int cc = id >> 3, tq = id & 7;
      if (Xt != nullptr && c0 + cc < cin) {
        u32x4 v;
        v.x = tile[(8 * tq + 0) * LD + cc] | ((uint32_t)tile[(8 * tq + 1) * LD + cc] << 16);
        v.y = tile[(8 * tq + 2) * LD + cc] | ((uint32_t)tile[(8 * tq + 3) * LD + cc] << 16);
        v.z = tile[(8 * tq + 4) * LD + cc] | ((uint32_t)tile[(8 * tq + 5) * LD + cc] << 16);
        v.w = tile[(8 * tq + 6) * LD + cc] | ((uint32_t)tile[(8 * tq + 7) * LD + cc] << 16);
        *reinterpret_cast<u32x4*>(Xt + (size_t)(c0 + cc) * pitch + t0 + 8 * tq) = v;
      }
    }
    __syncthreads();
  }
  part[rg][col] = ss;
  __syncthreads();
  if (rg == 0 && c0 + col < cin)
    norms[c0 + col] = sqrtf((part[0][col] + part[1][col]) + (part[2][col] + part[3][col]));
}

hipError_t launch_colnorm_f32(const float* X, int T, int cin, float* norms, hipStream_t s) {
  colnorm_f32_kernel<<<(cin + 63) / 64, 256, 0, s>>>(X, T, cin, norms);
  return hipGetLastError();
}

hipError_t launch_layer_init_bf16(const uint16_t* X, int T, int cin, int pitch, float* norms,
                                  uint16_t* Xt, hipStream_t s) {
  layer_init_bf16_kernel<<<(cin + 63) / 64, 256, 0, s>>>(X, T, cin, pitch, norms, Xt);
  return hipGetLastError();
}

}  // namespace lcp
