// Batched log-domain Sinkhorn normalisation of B x B block logits, forward
// and reverse, for gfx950.
//
// Definition ([PermLLM] Method 1): S_0(X) = exp(X), S_i(X) = T_c(T_r(S_{i-1})),
// P = S_L(L / tau); [blog] section 2.2 gives the log-domain form used here:
// each iteration subtracts the row log-sum-exp, then the column log-sum-exp,
// and the output is exp of the result.
//
// Design: one workgroup per block, B/16 waves. Wave w holds rows
// 16w .. 16w+15; inside a wave lane l = 16*lr + lc holds rows 16w + 4lr + a
// (a < 4) and columns lc*CPL + c (c < CPL = B/16), all in registers for every
// iteration (no HBM or LDS round trip of the block). Row reductions run over
// the 16 lanes of a lane row (xor 1, 2, 4, 8); column reductions over the 4
// lane rows (xor 16, 32) and then across waves through LDS. Work is done in
// base 2: z = logits * log2(e) / tau, lse2 = max + log2(sum exp2(z - max)), so
// each normalisation costs one v_exp_f32 per element. The row offsets r_i and
// column offsets c_i (base 2) are kept for the reverse pass.
#include "common.h"
#include "kernels.h"

namespace lcp {

template <int B>
struct SkGeom {
  static constexpr int WAVES = B / 16;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int CPL = B / 16;
};

// Load one block (times `scale`) into the lane's registers.
template <int B>
__device__ __forceinline__ void sk_load(const float* __restrict__ src, float scale,
                                        float (&z)[4][SkGeom<B>::CPL], int w, int lr, int lc) {
  constexpr int CPL = SkGeom<B>::CPL;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const float* p = src + (16 * w + 4 * lr + a) * B + lc * CPL;
#pragma unroll
    for (int c = 0; c < CPL; c += 2) {
      float2 v = *reinterpret_cast<const float2*>(p + c);
      z[a][c] = v.x * scale;
      z[a][c + 1] = v.y * scale;
    }
  }
}

// One forward iteration on the register block. Writes the row offsets of this
// lane's rows to roff[row] (if lc == 0) and the column offsets to coff[col]
// (if w == 0 && lr == 0); both pointers may be global or LDS (flat).
template <int B>
__device__ __forceinline__ void sk_iter(float (&z)[4][SkGeom<B>::CPL], float* red_m, float* red_s,
                                        float* roff, float* coff, int w, int lr, int lc) {
  constexpr int CPL = SkGeom<B>::CPL;
  constexpr int WAVES = SkGeom<B>::WAVES;
  // ---- row step: U = Z - lse_row(Z)
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float m = z[a][0];
#pragma unroll
    for (int c = 1; c < CPL; ++c) m = fmaxf(m, z[a][c]);
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) m = fmaxf(m, shfl_xor(m, x));
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) s += exp2_(z[a][c] - m);
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) s += shfl_xor(s, x);
    const float r = m + log2_(s);
#pragma unroll
    for (int c = 0; c < CPL; ++c) z[a][c] -= r;
    if (roff != nullptr && lc == 0) roff[16 * w + 4 * lr + a] = r;
  }
  // ---- column step: Z = U - lse_col(U)
  float mc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float m = fmaxf(fmaxf(z[0][c], z[1][c]), fmaxf(z[2][c], z[3][c]));
    m = fmaxf(m, shfl_xor(m, 16));
    m = fmaxf(m, shfl_xor(m, 32));
    if (lr == 0) red_m[w * B + lc * CPL + c] = m;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float m = red_m[lc * CPL + c];
#pragma unroll
    for (int v = 1; v < WAVES; ++v) m = fmaxf(m, red_m[v * B + lc * CPL + c]);
    mc[c] = m;
    float s = exp2_(z[0][c] - m) + exp2_(z[1][c] - m) + exp2_(z[2][c] - m) + exp2_(z[3][c] - m);
    s += shfl_xor(s, 16);
    s += shfl_xor(s, 32);
    if (lr == 0) red_s[w * B + lc * CPL + c] = s;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float s = red_s[lc * CPL + c];
#pragma unroll
    for (int v = 1; v < WAVES; ++v) s += red_s[v * B + lc * CPL + c];
    const float cc = mc[c] + log2_(s);
#pragma unroll
    for (int a = 0; a < 4; ++a) z[a][c] -= cc;
    if (coff != nullptr && w == 0 && lr == 0) coff[lc * CPL + c] = cc;
  }
}

// Forward: P = exp2(Z^L); optional offsets off[b][i][0][row], off[b][i][1][col].
template <int B>
__global__ __launch_bounds__(SkGeom<B>::THREADS) void sinkhorn_fwd_kernel(
    const float* __restrict__ logits, float* P, float* __restrict__ off, int iters, float scale) {
  constexpr int CPL = SkGeom<B>::CPL;
  constexpr int WAVES = SkGeom<B>::WAVES;
  __shared__ float red_m[WAVES * B];
  __shared__ float red_s[WAVES * B];
  const int b = blockIdx.x;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, lr = l >> 4, lc = l & 15;
  float z[4][CPL];
  sk_load<B>(logits + (size_t)b * B * B, scale, z, w, lr, lc);
  for (int it = 0; it < iters; ++it) {
    float* ro = off ? off + ((size_t)(b * iters + it) * 2 + 0) * B : nullptr;
    float* co = off ? off + ((size_t)(b * iters + it) * 2 + 1) * B : nullptr;
    sk_iter<B>(z, red_m, red_s, ro, co, w, lr, lc);
  }
  float* dst = P + (size_t)b * B * B;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float* p = dst + (16 * w + 4 * lr + a) * B + lc * CPL;
#pragma unroll
    for (int c = 0; c < CPL; c += 2) {
      float2 v;
      v.x = exp2_(z[a][c]);
      v.y = exp2_(z[a][c + 1]);
      *reinterpret_cast<float2*>(p + c) = v;
    }
  }
}

// Reverse pass. Gamma = dP . P; for i = L .. 1: undo the column step
// (Gamma -= exp(Z^i) . colsum(Gamma)), then the row step
// (Gamma -= exp(U^i) . rowsum(Gamma)); dlogits = Gamma / tau. Z^i and U^i are
// rebuilt from the logits and the offsets by the same sequence of
// subtractions the forward performed, so they match it bit for bit.
// dP is dense [nb][B][B] (seg_tpw == 0) or the block adjoint's partials: the
// workgroups g_lo..g_hi whose tile ranges cover block b each left one B x B
// partial at slot g * maxseg + (b - first block of g); they are summed in
// workgroup order. Offsets come from `off` ([nb][iters][2][B], as written by the
// forward) or, when off == nullptr, are recomputed here. Dynamic LDS holds
// 2 * iters * B floats.
template <int B>
__global__ __launch_bounds__(SkGeom<B>::THREADS) void sinkhorn_bwd_kernel(
    const float* __restrict__ logits, const float* __restrict__ dP, int seg_tpw, int seg_tpb,
    int seg_maxseg, int seg_grid, const float* __restrict__ off, float* __restrict__ dlogits, int iters,
    float scale, float inv_tau) {
  constexpr int CPL = SkGeom<B>::CPL;
  constexpr int WAVES = SkGeom<B>::WAVES;
  extern __shared__ float sh_off[];          // [iters][2][B]
  __shared__ float red_m[WAVES * B];
  __shared__ float red_s[WAVES * B];
  __shared__ float red_g[2][WAVES * B];
  const int b = blockIdx.x;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, lr = l >> 4, lc = l & 15;

  float z0[4][CPL];
  sk_load<B>(logits + (size_t)b * B * B, scale, z0, w, lr, lc);
  if (off != nullptr) {
    const float* src = off + (size_t)b * iters * 2 * B;
    for (int i = t; i < iters * 2 * B; i += SkGeom<B>::THREADS) sh_off[i] = src[i];
  } else {
    float z[4][CPL];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPL; ++c) z[a][c] = z0[a][c];
    for (int it = 0; it < iters; ++it)
      sk_iter<B>(z, red_m, red_s, sh_off + (2 * it) * B, sh_off + (2 * it + 1) * B, w, lr, lc);
  }
  __syncthreads();

  // rebuild Z^L and form Gamma = dP . exp(Z^L)
  float g[4][CPL];
  {
    int g_lo = 0, g_hi = 0;
    if (seg_tpw > 0) {
      g_lo = (b * seg_tpb) / seg_tpw;
      g_hi = min(seg_grid - 1, ((b + 1) * seg_tpb - 1) / seg_tpw);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int row = 16 * w + 4 * lr + a;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int col = lc * CPL + c;
        float v = z0[a][c];
        for (int it = 0; it < iters; ++it) {
          v = v - sh_off[(2 * it) * B + row];
          v = v - sh_off[(2 * it + 1) * B + col];
        }
        float d;
        if (seg_tpw == 0) {
          d = dP[(size_t)b * B * B + row * B + col];
        } else {
          d = 0.f;
          for (int gg = g_lo; gg <= g_hi; ++gg) {
            const int k = b - (gg * seg_tpw) / seg_tpb;
            d += dP[((size_t)gg * seg_maxseg + k) * B * B + row * B + col];
          }
        }
        g[a][c] = d * exp2_(v);
      }
    }
  }

  for (int it = iters - 1; it >= 0; --it) {
    float* red = red_g[it & 1];
    // exp(U^i) and exp(Z^i) for this iteration
    float eu[4][CPL], ez[4][CPL];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int row = 16 * w + 4 * lr + a;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int col = lc * CPL + c;
        float v = z0[a][c];
        for (int k = 0; k < it; ++k) {
          v = v - sh_off[(2 * k) * B + row];
          v = v - sh_off[(2 * k + 1) * B + col];
        }
        const float u = v - sh_off[(2 * it) * B + row];
        const float zz = u - sh_off[(2 * it + 1) * B + col];
        eu[a][c] = exp2_(u);
        ez[a][c] = exp2_(zz);
      }
    }
    // undo the column step: column sums of Gamma
    float cs[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float s = (g[0][c] + g[1][c]) + (g[2][c] + g[3][c]);
      s += shfl_xor(s, 16);
      s += shfl_xor(s, 32);
      if (lr == 0) red[w * B + lc * CPL + c] = s;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float s = red[lc * CPL + c];
#pragma unroll
      for (int v = 1; v < WAVES; ++v) s += red[v * B + lc * CPL + c];
      cs[c] = s;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPL; ++c) g[a][c] -= ez[a][c] * cs[c];
    // undo the row step: row sums of Gamma (within the wave)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) s += g[a][c];
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) s += shfl_xor(s, x);
#pragma unroll
      for (int c = 0; c < CPL; ++c) g[a][c] -= eu[a][c] * s;
    }
  }

  float* dst = dlogits + (size_t)b * B * B;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float* p = dst + (16 * w + 4 * lr + a) * B + lc * CPL;
#pragma unroll
    for (int c = 0; c < CPL; c += 2) {
      float2 v;
      v.x = g[a][c] * inv_tau;
      v.y = g[a][c + 1] * inv_tau;
      *reinterpret_cast<float2*>(p + c) = v;
    }
  }
}

// ---- launchers ---------------------------------------------------------------
static inline float sk_scale(float tau) { return (float)(1.4426950408889634 / (double)tau); }

hipError_t launch_sinkhorn_fwd(const float* logits, float* P, float* off, int nb, int B,
                               int iters, float tau, hipStream_t s) {
  const float scale = sk_scale(tau);
  switch (B) {
    case 32: sinkhorn_fwd_kernel<32><<<nb, SkGeom<32>::THREADS, 0, s>>>(logits, P, off, iters, scale); break;
    case 64: sinkhorn_fwd_kernel<64><<<nb, SkGeom<64>::THREADS, 0, s>>>(logits, P, off, iters, scale); break;
    case 128: sinkhorn_fwd_kernel<128><<<nb, SkGeom<128>::THREADS, 0, s>>>(logits, P, off, iters, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sinkhorn_bwd(const float* logits, const float* dP, const AdjSplit* seg,
                               const float* off, float* dlogits, int nb, int B, int iters,
                               float tau, hipStream_t s) {
  const int tpw = seg ? seg->tpw : 0, tpb = seg ? seg->tpb : 0;
  const int maxseg = seg ? seg->maxseg : 0, grid = seg ? seg->grid : 0;
  const float scale = sk_scale(tau);
  const float inv_tau = (float)(1.0 / (double)tau);
  const size_t lds = (size_t)iters * 2 * B * sizeof(float);
  switch (B) {
    case 32: sinkhorn_bwd_kernel<32><<<nb, SkGeom<32>::THREADS, lds, s>>>(logits, dP, tpw, tpb, maxseg, grid, off, dlogits, iters, scale, inv_tau); break;
    case 64: sinkhorn_bwd_kernel<64><<<nb, SkGeom<64>::THREADS, lds, s>>>(logits, dP, tpw, tpb, maxseg, grid, off, dlogits, iters, scale, inv_tau); break;
    case 128: sinkhorn_bwd_kernel<128><<<nb, SkGeom<128>::THREADS, lds, s>>>(logits, dP, tpw, tpb, maxseg, grid, off, dlogits, iters, scale, inv_tau); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lcp
