// Cosine objective of the LCP step ([PermLLM] optimisation objective:
// L = 1 - y . y~ / (|y| |y~|) between the dense and the sparse outputs, taken
// over the layer's whole output y = W X^T, y~ = W_tilde X^T).
//
// The step already forms the residual R = D X^T = Y - Y~ (the error GEMM),
// so the objective needs three scalars: r = |R|^2 and a = <Y, R> (partials
// written by the error GEMM's epilogue) and y2 = |Y|^2 (constant per layer).
// With p = <Y, Y~> = y2 - a and m2 = |Y~|^2 = y2 - 2a + r:
//   L = 1 - p / (|Y| |Y~|)      = (r y2 - a^2) / (|Y||Y~| (|Y||Y~| + p))
// (the second form has no cancellation when L is small), and the quotient
// rule gives
//   dL/dY~ = -Y / (|Y||Y~|) + p Y~ / (|Y| |Y~|^3) = ((a - r) Y - p R) / (|Y| |Y~|^3),
// a combination of Y and R with two scalar coefficients (no cancellation
// between large terms: both coefficients carry the small residual).
#include "common.h"
#include "kernels.h"

namespace lcp {

// One wave: fixed-order double sums of the partials, then the scalars.
__global__ __launch_bounds__(64) void cosine_finalize_kernel(const float* __restrict__ part,
                                                             const float* __restrict__ party, int n,
                                                             const float* __restrict__ y2p,
                                                             float* __restrict__ coef,
                                                             float* __restrict__ err) {
  // eight far-memory loads of each array in flight per lane, added in order
  // (a slot past n adds +0)
  double r = 0.0, a = 0.0;
  for (int i = threadIdx.x; i < n; i += 512) {
    float vr[8], va[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool in = i + 64 * q < n;
      vr[q] = in ? part[i + 64 * q] : 0.f;
      va[q] = in ? party[i + 64 * q] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      r += (double)vr[q];
      a += (double)va[q];
    }
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) {
    r += __shfl_xor(r, x, 64);
    a += __shfl_xor(a, x, 64);
  }
  if (threadIdx.x == 0) {
    const double y2 = (double)*y2p;
    const double m2 = y2 - 2.0 * a + r;
    const double p = y2 - a;
    double L = 1.0, cy = 0.0, cr = 0.0;
    if (y2 > 0.0 && m2 > 1e-12 * y2) {
      const double nm = sqrt(y2 * m2);
      if (p > 0.0) L = fmax(r * y2 - a * a, 0.0) / (nm * (nm + p));
      else L = 1.0 - p / nm;
      const double d = nm * m2;
      cy = (a - r) / d;
      cr = -p / d;
    }
    coef[0] = (float)sqrt(r);
    coef[1] = 1.f;
    coef[2] = (float)cy;
    coef[3] = (float)cr;
    *err = (float)L;
  }
}

// dY~ = cy Y + cr R, eight bf16 elements per thread.
__global__ __launch_bounds__(256) void cosine_grad_bf16_kernel(const u32x4* __restrict__ Y,
                                                               const u32x4* __restrict__ R, size_t n8,
                                                               const float* __restrict__ coef,
                                                               u32x4* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float cy = coef[2], cr = coef[3];
  const u32x4 y = Y[i], r = R[i];
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = pack2(cy * lo_bf(y[q]) + cr * lo_bf(r[q]), cy * hi_bf(y[q]) + cr * hi_bf(r[q]));
  out[i] = o;
}

// fp32: four elements per thread.
__global__ __launch_bounds__(256) void cosine_grad_f32_kernel(const floatx4* __restrict__ Y,
                                                              const floatx4* __restrict__ R, size_t n4,
                                                              const float* __restrict__ coef,
                                                              floatx4* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float cy = coef[2], cr = coef[3];
  const floatx4 y = Y[i], r = R[i];
  out[i] = floatx4{cy * y[0] + cr * r[0], cy * y[1] + cr * r[1], cy * y[2] + cr * r[2], cy * y[3] + cr * r[3]};
}

hipError_t launch_cosine_finalize(const float* part, const float* party, int nparts, const float* y2,
                                  float* coef, float* err, hipStream_t s) {
  cosine_finalize_kernel<<<1, 64, 0, s>>>(part, party, nparts, y2, coef, err);
  return hipGetLastError();
}

hipError_t launch_cosine_grad(const void* Y, const void* R, size_t n, int bf16, const float* coef, void* out,
                              hipStream_t s) {
  if (n % 8) return hipErrorInvalidValue;
  const size_t v = bf16 ? n / 8 : n / 4;
  const size_t grid = (v + 255) / 256;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  if (bf16)
    cosine_grad_bf16_kernel<<<(unsigned)grid, 256, 0, s>>>((const u32x4*)Y, (const u32x4*)R, v, coef, (u32x4*)out);
  else
    cosine_grad_f32_kernel<<<(unsigned)grid, 256, 0, s>>>((const floatx4*)Y, (const floatx4*)R, v, coef,
                                                           (floatx4*)out);
  return hipGetLastError();
}

}  // namespace lcp
