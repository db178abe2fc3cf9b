// Per-layer setup, constant across the LCP steps on one layer: the column
// norms ||X[:, j]||_2 (the activation factor of Wanda's importance) and, for
// bf16 layers, the transposed activations Xt [cin][pitch] that the backward
// GEMM reads with the token index contiguous.
//
// Both kernels walk strips of channels down all T tokens, so each column's
// sum of squares is accumulated by fixed lanes in a fixed order
// (deterministic, no atomics).
#include "common.h"
#include "kernels.h"

namespace lcp {

// fp32: 16 row groups of 64 channels per workgroup; row group g sums rows
// g, g + 16, ... with four loads in flight, and the 16 group sums are added
// in a fixed order.
__global__ __launch_bounds__(1024) void colnorm_f32_kernel(const float* __restrict__ X, int T,
                                                           int cin, float* __restrict__ norms) {
  __shared__ float part[16][64];
  const int t = threadIdx.x, col = t & 63, rg = t >> 6;
  const int c = blockIdx.x * 64 + col;
  float s = 0.f;
  if (c < cin) {
    int r = rg;
    for (; r + 48 < T; r += 64) {
      const float v0 = X[(size_t)r * cin + c], v1 = X[(size_t)(r + 16) * cin + c];
      const float v2 = X[(size_t)(r + 32) * cin + c], v3 = X[(size_t)(r + 48) * cin + c];
      s += v0 * v0;
      s += v1 * v1;
      s += v2 * v2;
      s += v3 * v3;
    }
    for (; r < T; r += 16) {
      const float v = X[(size_t)r * cin + c];
      s += v * v;
    }
  }
  part[rg][col] = s;
  __syncthreads();
  if (rg == 0 && c < cin) {
    float tot = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) tot += part[g][col];
    norms[c] = sqrtf(tot);
  }
}

// bf16: one workgroup per strip of 32 channels, 4 waves; consecutive strips
// go to the same XCD (workgroup ids are dealt round-robin over the 8 XCDs), so
// the two 64-byte halves of a 128-byte row segment meet in one L2. Lane
// (cb, rb) of a wave owns an 8 x 8 block (tokens 8rb.., channels 8cb..) of
// each 128-token x 32-channel tile: it loads the 8 token rows (16 bytes
// each), transposes the block in registers (one v_perm_b32 per output word)
// and stores the 8 channel rows of Xt (16 bytes each), while summing squares
// for its 8 channels. Four tiles are in flight per wave (all of a wave's
// tiles at 2,048 tokens). Column sums are
// reduced over the 16 lanes of a column block (one DPP row) and then over the
// 4 waves (LDS), in a fixed order. X is read and Xt written through the
// caches: the error GEMM reads X again soon after, and finds much of it
// there.
__device__ __forceinline__ void transpose8x8(const u32x4 (&r)[8], u32x4 (&o)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    uint32_t wq[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = r[2 * p][c >> 1], b = r[2 * p + 1][c >> 1];
      wq[p] = __builtin_amdgcn_perm(b, a, sel);
    }
    o[c] = u32x4{wq[0], wq[1], wq[2], wq[3]};
  }
}

__global__ __launch_bounds__(256) void layer_init_bf16_kernel(const uint16_t* __restrict__ X,
                                                              int T, int cin, int pitch,
                                                              float* __restrict__ norms,
                                                              uint16_t* __restrict__ Xt) {
  __shared__ float part[4][32];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int rb = l & 15, cb = l >> 4;
  const int G = gridDim.x;
  const int strip = ((G & 7) == 0) ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int c0 = strip * 32 + 8 * cb;               // this lane's 8 channels
  const bool cok = c0 < cin;                         // cin % 8 == 0: all 8 or none
  const int t_end = Xt != nullptr ? pitch : T;
  float ss[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) ss[c] = 0.f;

  auto load = [&](int t0, u32x4 (&r)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = t0 + 8 * rb + e;
      r[e] = (cok && row < T) ? *reinterpret_cast<const u32x4*>(X + (size_t)row * cin + c0) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto consume = [&](int t0, const u32x4 (&r)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = lo_bf(r[e][q]), hi = hi_bf(r[e][q]);
        ss[2 * q] = fmaf(lo, lo, ss[2 * q]);
        ss[2 * q + 1] = fmaf(hi, hi, ss[2 * q + 1]);
      }
    // pitch is a multiple of 64, so a group of 8 tokens is entirely inside or outside it
    if (Xt != nullptr && cok && t0 + 8 * rb < pitch) {
      u32x4 o[8];
      transpose8x8(r, o);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<u32x4*>(Xt + (size_t)(c0 + c) * pitch + t0 + 8 * rb) = o[c];
    }
  };

  // wave w covers token tiles w, w + 4, w + 8, ... (128 tokens each), four at a time
  u32x4 ra[8], rb2[8], rc[8], rd[8];
  int t0 = 128 * w;
  for (; t0 + 1536 < t_end; t0 += 2048) {
    load(t0, ra);
    load(t0 + 512, rb2);
    load(t0 + 1024, rc);
    load(t0 + 1536, rd);
    consume(t0, ra);
    consume(t0 + 512, rb2);
    consume(t0 + 1024, rc);
    consume(t0 + 1536, rd);
  }
  for (; t0 + 512 < t_end; t0 += 1024) {
    load(t0, ra);
    load(t0 + 512, rb2);
    consume(t0, ra);
    consume(t0 + 512, rb2);
  }
  if (t0 < t_end) {
    load(t0, ra);
    consume(t0, ra);
  }

  // column sums: the 16 lanes rb of a column block (one DPP row), then the 4 waves
#pragma unroll
  for (int c = 0; c < 8; ++c) ss[c] = row16_sum(ss[c]);
  if (rb == 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c) part[w][8 * cb + c] = ss[c];
  }
  __syncthreads();
  if (t < 32) {
    const int c = strip * 32 + t;
    if (c < cin) norms[c] = sqrtf((part[0][t] + part[1][t]) + (part[2][t] + part[3][t]));
  }
}

hipError_t launch_colnorm_f32(const float* X, int T, int cin, float* norms, hipStream_t s) {
  colnorm_f32_kernel<<<(cin + 63) / 64, 1024, 0, s>>>(X, T, cin, norms);
  return hipGetLastError();
}

hipError_t launch_layer_init_bf16(const uint16_t* X, int T, int cin, int pitch, float* norms,
                                  uint16_t* Xt, hipStream_t s) {
  layer_init_bf16_kernel<<<(cin + 31) / 32, 256, 0, s>>>(X, T, cin, pitch, norms, Xt);
  return hipGetLastError();
}

}  // namespace lcp
