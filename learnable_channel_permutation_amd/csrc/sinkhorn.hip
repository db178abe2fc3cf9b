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
// the 16 lanes of a DPP row; column reductions pair lanes 16 and 32 apart
// (permlane swaps), then the waves' partial sums meet in LDS: wave w merges
// columns 16w .. 16w+15 (four lanes per column, each taking every fourth
// wave, merged across lanes 16 and 32 apart) and publishes the column
// results, two barriers per column step. Work is done in base 2:
// z = logits * log2(e) / tau.
// The forward exponentiates the block once (K = exp2(z - row max)) and
// iterates row and column scalings on it, one multiply-add per element and
// normalisation (the iterates are diag(u) K diag(v) exactly as the
// log-domain ones are exp2 of Z^i); a block whose row or column sum leaves
// the range where that is accurate restarts on the exact log-domain
// iteration. The row offsets r_i and column offsets c_i (base 2) of every
// iteration are kept for the reverse pass, which works in the log domain.
#include "common.h"
#include "kernels.h"

namespace lcp {

template <int B>
struct SkGeom {
  static constexpr int WAVES = B / 16;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int CPL = B / 16;
};

// CPL consecutive floats (16-byte aligned for CPL >= 4, 8-byte for CPL = 2);
// NT: non-temporal access (data used once, kept out of the caches)
template <int CPL, bool NT = false>
__device__ __forceinline__ void ld_cols(const float* p, float (&v)[CPL]) {
  if constexpr (CPL % 4 == 0) {
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
      const floatx4* a = reinterpret_cast<const floatx4*>(p + c);
      const floatx4 q = NT ? __builtin_nontemporal_load(a) : *a;
      v[c] = q[0]; v[c + 1] = q[1]; v[c + 2] = q[2]; v[c + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPL; c += 2) {
      const float2 q = *reinterpret_cast<const float2*>(p + c);
      v[c] = q.x; v[c + 1] = q.y;
    }
  }
}
template <int CPL, bool NT = false>
__device__ __forceinline__ void st_cols(float* p, const float (&v)[CPL]) {
  if constexpr (CPL % 4 == 0) {
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
      const floatx4 q = floatx4{v[c], v[c + 1], v[c + 2], v[c + 3]};
      floatx4* a = reinterpret_cast<floatx4*>(p + c);
      if (NT) __builtin_nontemporal_store(q, a);
      else *a = q;
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPL; c += 2) *reinterpret_cast<float2*>(p + c) = float2{v[c], v[c + 1]};
  }
}

// The lane's 4 x CPL elements of a row-major B x B block.
template <int B, bool NT = false>
__device__ __forceinline__ void ld_block(const float* __restrict__ src, float (&v)[4][SkGeom<B>::CPL], int w,
                                         int lr, int lc) {
  constexpr int CPL = SkGeom<B>::CPL;
#pragma unroll
  for (int a = 0; a < 4; ++a) ld_cols<CPL, NT>(src + (16 * w + 4 * lr + a) * B + lc * CPL, v[a]);
}

// Value of the lane 16 (or 32) apart, from the permlane swaps (the swap
// returns the pair in lane order, so the partner is the other element).
__device__ __forceinline__ float partner16(float v, int l) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((l & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float partner32(float v, int l) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((l & 32) ? r[0] : r[1]);
}
// (m, s) <- the (max, sum of exp2(x - max)) pair of the union of two sets;
// an empty set is (-inf, 0). Symmetric in its operands, bit for bit.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float a = (s > 0.f) ? s * exp2_(m - mn) : 0.f;
  const float b = (s2 > 0.f) ? s2 * exp2_(m2 - mn) : 0.f;
  m = mn;
  s = a + b;
}

// Column step of one iteration from the values themselves: Z = U - lse_col(U)
// with each wave's (max, sum) pairs over its 16 rows merged in LDS.
template <int B>
__device__ __forceinline__ void col_step_exact(float (&z)[4][SkGeom<B>::CPL], float2* red, float* ccb, int w,
                                               int lr, int lc) {
  constexpr int CPL = SkGeom<B>::CPL;
  constexpr int WAVES = SkGeom<B>::WAVES;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float m = fmaxf(fmaxf(z[0][c], z[1][c]), fmaxf(z[2][c], z[3][c]));
    m = xor32_max(xor16_max(m));
    float s = (exp2_(z[0][c] - m) + exp2_(z[1][c] - m)) + (exp2_(z[2][c] - m) + exp2_(z[3][c] - m));
    s = xor32_sum(xor16_sum(s));
    if (lr == 0) red[w * B + lc * CPL + c] = float2{m, s};
  }
  __syncthreads();
  // wave w merges columns 16w + lc over the waves: quarter lr takes waves
  // lr, lr + 4, ..., then the quarters meet across lanes 16 and 32 apart
  {
    const int l = 16 * lr + lc, col = 16 * w + lc;
    float m = -__builtin_inff(), s = 0.f;
#pragma unroll
    for (int v = lr; v < WAVES; v += 4) {
      const float2 pv = red[v * B + col];
      lse_merge(m, s, pv.x, pv.y);
    }
    lse_merge(m, s, partner16(m, l), partner16(s, l));
    lse_merge(m, s, partner32(m, l), partner32(s, l));
    if (lr == 0) ccb[col] = m + log2_(s);
  }
  __syncthreads();
}

// One forward iteration on the register block, using reduction buffer `red`
// (WAVES * B (max, sum) pairs; alternate two buffers between iterations),
// `ccb` (B column offsets) and the flag word `flag` (alternate two as well).
// The row step keeps its exponentials: exp2(U) = exp2(Z - rowmax) / rowsum,
// so the column sums of exp2(U) need no second exponential. A column whose
// sum falls below 2^-90 (its terms may have underflowed in the row step)
// sends the whole block through the exact log-domain column step instead.
// Writes the row offsets of this lane's rows to roff[row] (if lc == 0) and the
// column offsets to coff[col] (if w == 0 && lr == 0); either may be null.
template <int B>
__device__ __forceinline__ void sk_iter(float (&z)[4][SkGeom<B>::CPL], float2* red, float* ccb, int* flag,
                                        float* roff, float* coff, int w, int lr, int lc) {
  constexpr int CPL = SkGeom<B>::CPL;
  constexpr int WAVES = SkGeom<B>::WAVES;
  // ---- row step: U = Z - lse_row(Z), q = exp2(U)
  float q[4][CPL];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float m = z[a][0];
#pragma unroll
    for (int c = 1; c < CPL; ++c) m = fmaxf(m, z[a][c]);
    m = row16_max(m);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      q[a][c] = exp2_(z[a][c] - m);
      s += q[a][c];
    }
    s = row16_sum(s);
    const float r = m + log2_(s);
    const float inv = 1.f / s;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      z[a][c] -= r;
      q[a][c] *= inv;
    }
    if (roff != nullptr && lc == 0) roff[16 * w + 4 * lr + a] = r;
  }
  // ---- column step: Z = U - log2(colsum(q)); each wave's sums over its 16 rows
  if (w == 0 && lr == 0 && lc == 0) *flag = 0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float s = (q[0][c] + q[1][c]) + (q[2][c] + q[3][c]);
    s = xor32_sum(xor16_sum(s));
    if (lr == 0) red[w * B + lc * CPL + c] = float2{s, 0.f};
  }
  __syncthreads();
  {
    const int l = 16 * lr + lc, col = 16 * w + lc;
    float s = 0.f;
#pragma unroll
    for (int v = lr; v < WAVES; v += 4) s += red[v * B + col].x;
    s += partner16(s, l);
    s += partner32(s, l);
    if (lr == 0) {
      ccb[col] = log2_(s);
      if (!(s >= 0x1p-90f)) *flag = 1;
    }
  }
  __syncthreads();
  if (*flag != 0) col_step_exact<B>(z, red, ccb, w, lr, lc);   // block-uniform
  float cv[CPL];
  ld_cols<CPL>(ccb + lc * CPL, cv);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
#pragma unroll
    for (int a = 0; a < 4; ++a) z[a][c] -= cv[c];
    if (coff != nullptr && w == 0 && lr == 0) coff[lc * CPL + c] = cv[c];
  }
}

// Quad broadcast (DPP quad_perm [a, a, a, a]): every lane of a quad gets the
// value of the quad's lane a.
template <int A>
__device__ __forceinline__ float quad_bcast(float v) {
  return dpp<A | (A << 2) | (A << 4) | (A << 6)>(v);
}

// Smallest row or column sum the scaled iteration accepts. Scalings stay
// below 2^45 each, so an entry whose exponential underflowed (K < 2^-126)
// stands for P < 2^-36: below the parity tolerance's absolute floor, and a
// negligible share (< 2^-36) of every sum it belongs to.
constexpr float kScaledFloor = 0x1p-45f;

// Forward: P = exp2(Z^L); optional offsets off[b][i][0][row], off[b][i][1][col].
// The iterations run on scalings of a block exponentiated once
// (Sinkhorn-Knopp in the form of Schmitzer's stabilized scaling): with
// K_jk = exp2(z_jk - m_j), m_j the row maximum, every iterate is
// exp2(Z^i) = diag(u) K diag(v), so one row step is u_j = 1 / sum_k K_jk v_k
// and one column step v_k = 1 / sum_j K_jk u_j: one multiply-add per element
// and step, no exponential. The log-domain offsets of iteration i follow from
// the sums (row: r = log2 s_i - log2 s_(i-1), with m_j + log2 s_1 for i = 1;
// column alike with t), so the reverse pass rebuilds Z^i from them as from the
// log-domain forward. If any sum falls below kScaledFloor the block restarts
// on the log-domain iteration of sk_iter (block-uniform decision).
// With fwd != nullptr the block of P and its column norms are staged in LDS
// and the MFMA operand fragments (frag.h) are written as well.
template <int B, bool OFFS, bool FRAGS>
__global__ __launch_bounds__(SkGeom<B>::THREADS) __attribute__((amdgpu_waves_per_eu(B == 128 ? 4 : 8))) void sinkhorn_fwd_kernel(
    const float* __restrict__ logits, float* P, float* __restrict__ off, int iters, float scale,
    const float* __restrict__ n, u32x4* __restrict__ fwd, u32x4* __restrict__ adj) {
  constexpr int CPL = SkGeom<B>::CPL;
  constexpr int WAVES = SkGeom<B>::WAVES;
  constexpr int PP = B + 2;                       // LDS row pitch of the staged block
  __shared__ float2 red[2][WAVES * B];
  __shared__ __attribute__((aligned(16))) float ccb[B];
  __shared__ __attribute__((aligned(16))) float vsh[2][B];
  __shared__ int skflag[2];
  extern __shared__ float ps[];                   // [B][PP] P block, then [B] norms
  const int b = blockIdx.x;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, lr = l >> 4, lc = l & 15;
  const int q = lc & 3;                           // the row 4 lr + q of this lane's quad position
  const float* src = logits + (size_t)b * B * B;
  float* ob = OFFS ? off + (size_t)b * iters * 2 * B : nullptr;

  // the standalone call (no offsets) reads each logit once and writes each
  // entry of P once: non-temporal; the step's logits and P are read again
  constexpr bool NT = !OFFS;
  float K[4][CPL];                                 // exp2(z - m), at the end the block of P
  ld_block<B, NT>(src, K, w, lr, lc);
  float m[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float mm = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      K[a][c] *= scale;
      mm = fmaxf(mm, K[a][c]);
    }
    m[a] = row16_max(mm);
#pragma unroll
    for (int c = 0; c < CPL; ++c) K[a][c] = exp2_(K[a][c] - m[a]);
  }
  const float m_mine = q == 0 ? m[0] : q == 1 ? m[1] : q == 2 ? m[2] : m[3];

  float v[CPL], u[4];
#pragma unroll
  for (int c = 0; c < CPL; ++c) v[c] = 1.f;
  float ls_prev = 0.f, lt_prev = 0.f;             // log2 of this lane's previous row / column sum
  bool scaled = true;
  for (int it = 0; it < iters; ++it) {
    float* rg = reinterpret_cast<float*>(red[it & 1]);
    if (w == 0 && l == 0) skflag[it & 1] = 0;
    // ---- row step: s_j = sum_k K_jk v_k, u_j = 1 / s_j (lane q of each
    // quad takes row 4 lr + q, the quad shares the four results)
    float s[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float acc = K[a][0] * v[0];
#pragma unroll
      for (int c = 1; c < CPL; ++c) acc = fmaf(K[a][c], v[c], acc);
      s[a] = row16_sum(acc);
    }
    const float s_mine = q == 0 ? s[0] : q == 1 ? s[1] : q == 2 ? s[2] : s[3];
    const bool row_bad = !(s_mine >= kScaledFloor);
    const float u_mine = __builtin_amdgcn_rcpf(s_mine);
    u[0] = quad_bcast<0>(u_mine);
    u[1] = quad_bcast<1>(u_mine);
    u[2] = quad_bcast<2>(u_mine);
    u[3] = quad_bcast<3>(u_mine);
    if (OFFS) {
      const float ls = log2_(s_mine);
      if (lc < 4) ob[(2 * it) * B + 16 * w + 4 * lr + q] = (it == 0) ? m_mine + ls : ls - ls_prev;
      ls_prev = ls;
    }
    // ---- column step: t_k = sum_j K_jk u_j over the lane's rows, the wave's
    // 16 rows (lanes 16 and 32 apart), then the waves (LDS)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float acc = K[0][c] * u[0];
#pragma unroll
      for (int a = 1; a < 4; ++a) acc = fmaf(K[a][c], u[a], acc);
      acc = xor32_sum(xor16_sum(acc));
      if (lr == 0) rg[w * B + lc * CPL + c] = acc;
    }
    __syncthreads();
    {
      const int col = 16 * w + lc;
      float tk = 0.f;
#pragma unroll
      for (int vw = lr; vw < WAVES; vw += 4) tk += rg[vw * B + col];
      tk += partner16(tk, l);
      tk += partner32(tk, l);
      if (row_bad || !(tk >= kScaledFloor)) skflag[it & 1] = 1;
      if (lr == 0) vsh[it & 1][col] = __builtin_amdgcn_rcpf(tk);
      if (OFFS) {
        const float lt = log2_(tk);
        if (lr == 0) ob[(2 * it + 1) * B + col] = (it == 0) ? lt : lt - lt_prev;
        lt_prev = lt;
      }
    }
    __syncthreads();
    if (skflag[it & 1] != 0) {                    // block-uniform
      scaled = false;
      break;
    }
    ld_cols<CPL>(&vsh[it & 1][lc * CPL], v);
  }

  if (scaled) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPL; ++c) K[a][c] = (K[a][c] * u[a]) * v[c];
  } else {
    // exact log-domain restart of the whole block (every thread has read the
    // flag before sk_iter reuses it)
    __syncthreads();
    float z[4][CPL];
    ld_block<B>(src, z, w, lr, lc);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPL; ++c) z[a][c] *= scale;
    for (int it = 0; it < iters; ++it) {
      float* ro = OFFS ? ob + (2 * it) * B : nullptr;
      float* co = OFFS ? ob + (2 * it + 1) * B : nullptr;
      sk_iter<B>(z, red[it & 1], ccb, &skflag[it & 1], ro, co, w, lr, lc);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPL; ++c) K[a][c] = exp2_(z[a][c]);
  }

  float* dst = P + (size_t)b * B * B;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int row = 16 * w + 4 * lr + a;
    st_cols<CPL, NT>(dst + row * B + lc * CPL, K[a]);
    if (FRAGS) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) ps[row * PP + lc * CPL + c] = K[a][c];
    }
  }
  if (FRAGS) {
    for (int i = t; i < B; i += SkGeom<B>::THREADS) ps[B * PP + i] = n[(size_t)b * B + i];
    __syncthreads();
    frag_build<B, PP>(ps, ps + B * PP, fwd + (size_t)b * FragGeom<B>::NARR * FragGeom<B>::FRAG,
                      adj + (size_t)b * FragGeom<B>::FRAG, t, SkGeom<B>::THREADS);
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
// workgroup order, the loads of the next partial in flight while the current
// one is added. Offsets come from `off` ([nb][iters][2][B], as written by the
// forward) or, when off == nullptr, are recomputed here. Dynamic LDS holds
// 2 * iters * B floats.
template <int B>
__global__ __launch_bounds__(SkGeom<B>::THREADS) void sinkhorn_bwd_kernel(
    const float* logits, const float* __restrict__ dP, int seg_tpw, int seg_tpb,
    int seg_maxseg, int seg_grid, const float* __restrict__ off, float* __restrict__ dlogits, int iters,
    float scale, float inv_tau, AdamW opt) {
  constexpr int CPL = SkGeom<B>::CPL;
  constexpr int WAVES = SkGeom<B>::WAVES;
  extern __shared__ float sh_off[];          // [iters][2][B]
  __shared__ float2 red[2][WAVES * B];
  __shared__ float red_g[2][WAVES * B];
  __shared__ __attribute__((aligned(16))) float ccb[B];
  __shared__ int skflag[2];
  const int b = blockIdx.x;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, lr = l >> 4, lc = l & 15;
  const int row0 = 16 * w + 4 * lr;          // this lane's rows row0 .. row0 + 3

  float z0[4][CPL];
  ld_block<B>(logits + (size_t)b * B * B, z0, w, lr, lc);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < CPL; ++c) z0[a][c] *= scale;

  // dP of this block: dense, or the sum of the adjoint's partials
  float d[4][CPL];
  if (seg_tpw == 0) {
    ld_block<B>(dP + (size_t)b * B * B, d, w, lr, lc);
  } else {
    // (workgroup, segment) partials of the block adjoint, or with seg_tpw < 0
    // one partial per row panel [panel][nb][B][B]
    const bool panels = seg_tpw < 0;
    const int g_lo = panels ? 0 : (b * seg_tpb) / seg_tpw;
    const int g_hi = panels ? seg_grid - 1 : min(seg_grid - 1, ((b + 1) * seg_tpb - 1) / seg_tpw);
    auto slot = [&](int gg) {
      return panels ? dP + ((size_t)gg * gridDim.x + b) * B * B
                    : dP + ((size_t)gg * seg_maxseg + (b - (gg * seg_tpw) / seg_tpb)) * B * B;
    };
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPL; ++c) d[a][c] = 0.f;
    // up to four partials in flight at once, added in workgroup order
    for (int g0 = g_lo; g0 <= g_hi; g0 += 4) {
      float q[4][4][CPL];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (g0 + k <= g_hi) ld_block<B, true>(slot(g0 + k), q[k], w, lr, lc);   // read once: non-temporal
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (g0 + k <= g_hi) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < CPL; ++c) d[a][c] += q[k][a][c];
        }
    }
  }

  if (off != nullptr) {
    const float* src = off + (size_t)b * iters * 2 * B;
    for (int i = 4 * t; i < iters * 2 * B; i += 4 * SkGeom<B>::THREADS)
      *reinterpret_cast<floatx4*>(sh_off + i) = *reinterpret_cast<const floatx4*>(src + i);
  } else {
    float z[4][CPL];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPL; ++c) z[a][c] = z0[a][c];
    for (int it = 0; it < iters; ++it)
      sk_iter<B>(z, red[it & 1], ccb, &skflag[it & 1], sh_off + (2 * it) * B, sh_off + (2 * it + 1) * B, w, lr, lc);
  }
  __syncthreads();

  // Z^k for this lane's elements: z0 minus the offsets of iterations < k, in
  // the forward's order (row offset, then column offset, per iteration).
  // Z^kc (kc = ceil(L/2)) is kept as a checkpoint, and an iterate past it
  // continues from there: the same operations on the same values, about
  // half the passes (the reverse sweep would otherwise cost O(L^2) of them).
  auto advance = [&](int from, int to, float (&v)[4][CPL]) {
    for (int i = from; i < to; ++i) {
      const floatx4 r = *reinterpret_cast<const floatx4*>(sh_off + (2 * i) * B + row0);
      float cv[CPL];
      ld_cols<CPL>(sh_off + (2 * i + 1) * B + lc * CPL, cv);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[a][c] = (v[a][c] - r[a]) - cv[c];
    }
  };
  const int kc = (iters + 1) / 2;
  float zc[4][CPL];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < CPL; ++c) zc[a][c] = z0[a][c];
  advance(0, kc, zc);
  auto rebuild = [&](int k, float (&v)[4][CPL]) {
    const bool past = k >= kc;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPL; ++c) v[a][c] = past ? zc[a][c] : z0[a][c];
    advance(past ? kc : 0, k, v);
  };

  float g[4][CPL];
  {
    float v[4][CPL];
    rebuild(iters, v);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPL; ++c) g[a][c] = d[a][c] * exp2_(v[a][c]);
  }

  for (int it = iters - 1; it >= 0; --it) {
    float* rg = red_g[it & 1];
    // exp(U^i) and exp(Z^i) of this iteration
    float eu[4][CPL], ez[4][CPL];
    {
      float v[4][CPL];
      rebuild(it, v);
      const floatx4 r = *reinterpret_cast<const floatx4*>(sh_off + (2 * it) * B + row0);
      float cv[CPL];
      ld_cols<CPL>(sh_off + (2 * it + 1) * B + lc * CPL, cv);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float u = v[a][c] - r[a];
          eu[a][c] = exp2_(u);
          ez[a][c] = exp2_(u - cv[c]);
        }
    }
    // undo the column step: column sums of Gamma over the 4 lane rows, then the waves
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float s = (g[0][c] + g[1][c]) + (g[2][c] + g[3][c]);
      s = xor32_sum(xor16_sum(s));
      if (lr == 0) rg[w * B + lc * CPL + c] = s;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float s = rg[lc * CPL + c];
#pragma unroll
      for (int v = 1; v < WAVES; ++v) s += rg[v * B + lc * CPL + c];
#pragma unroll
      for (int a = 0; a < 4; ++a) g[a][c] -= ez[a][c] * s;
    }
    // undo the row step: row sums of Gamma (within the wave)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) s += g[a][c];
      s = row16_sum(s);
#pragma unroll
      for (int c = 0; c < CPL; ++c) g[a][c] -= eu[a][c] * s;
    }
  }

#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const size_t o = (size_t)b * B * B + (row0 + a) * B + lc * CPL;
    float gr[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) gr[c] = g[a][c] * inv_tau;
    if (dlogits != nullptr) st_cols<CPL>(dlogits + o, gr);
    if (opt.param != nullptr) {
      // AdamW on this lane's logits: the block's values were read at the
      // start by this same lane, so the in-place update is race-free. No
      // contraction: the same rounded operations as adamw_kernel.
#pragma clang fp contract(off)
      float p[CPL], mm[CPL], vv[CPL];
      ld_cols<CPL>(opt.param + o, p);
      ld_cols<CPL>(opt.m + o, mm);
      ld_cols<CPL>(opt.v + o, vv);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        mm[c] = opt.b1 * mm[c] + (1.f - opt.b1) * gr[c];
        vv[c] = opt.b2 * vv[c] + (1.f - opt.b2) * gr[c] * gr[c];
        const float step = (mm[c] / opt.bc1) / (__builtin_sqrtf(vv[c] / opt.bc2) + opt.eps);
        p[c] = p[c] * (1.f - opt.lr * opt.wd) - opt.lr * step;
      }
      st_cols<CPL>(opt.m + o, mm);
      st_cols<CPL>(opt.v + o, vv);
      st_cols<CPL>(opt.param + o, p);
    }
  }
}

// Standalone AdamW, the same arithmetic as the fused epilogue above.
__global__ __launch_bounds__(256) void adamw_kernel(const float* __restrict__ grad, int n, AdamW opt) {
#pragma clang fp contract(off)
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float gr = grad[i];
  const float mm = opt.b1 * opt.m[i] + (1.f - opt.b1) * gr;
  const float vv = opt.b2 * opt.v[i] + (1.f - opt.b2) * gr * gr;
  const float step = (mm / opt.bc1) / (__builtin_sqrtf(vv / opt.bc2) + opt.eps);
  opt.m[i] = mm;
  opt.v[i] = vv;
  opt.param[i] = opt.param[i] * (1.f - opt.lr * opt.wd) - opt.lr * step;
}

hipError_t launch_adamw(const float* grad, int n, const AdamW& opt, hipStream_t s) {
  adamw_kernel<<<(n + 255) / 256, 256, 0, s>>>(grad, n, opt);
  return hipGetLastError();
}

// ---- launchers ---------------------------------------------------------------
static inline float sk_scale(float tau) { return (float)(1.4426950408889634 / (double)tau); }

hipError_t launch_sinkhorn_fwd(const float* logits, float* P, float* off, int nb, int B,
                               int iters, float tau, const float* n, u32x4* fwd, u32x4* adj,
                               hipStream_t s) {
  const float scale = sk_scale(tau);
  const size_t lds = fwd ? (size_t)(B * (B + 2) + B) * sizeof(float) : 0;
  // variants: plain (no offsets, no fragments), offsets only (fp32 layers),
  // offsets and fragments (bf16 layers)
  const bool o = off != nullptr, f = fwd != nullptr;
  if (f && !o) return hipErrorInvalidValue;
  switch (B) {
    case 32: (f ? sinkhorn_fwd_kernel<32, true, true> : o ? sinkhorn_fwd_kernel<32, true, false> : sinkhorn_fwd_kernel<32, false, false>)<<<nb, SkGeom<32>::THREADS, lds, s>>>(logits, P, off, iters, scale, n, fwd, adj); break;
    case 64: (f ? sinkhorn_fwd_kernel<64, true, true> : o ? sinkhorn_fwd_kernel<64, true, false> : sinkhorn_fwd_kernel<64, false, false>)<<<nb, SkGeom<64>::THREADS, lds, s>>>(logits, P, off, iters, scale, n, fwd, adj); break;
    case 128: (f ? sinkhorn_fwd_kernel<128, true, true> : o ? sinkhorn_fwd_kernel<128, true, false> : sinkhorn_fwd_kernel<128, false, false>)<<<nb, SkGeom<128>::THREADS, lds, s>>>(logits, P, off, iters, scale, n, fwd, adj); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sinkhorn_bwd(const float* logits, const float* dP, const AdjSplit* seg,
                               const float* off, float* dlogits, int nb, int B, int iters,
                               float tau, const AdamW* opt, hipStream_t s) {
  const AdamW o = opt ? *opt : AdamW{nullptr, nullptr, nullptr, 0.f, 0.f, 0.f, 0.f, 0.f, 1.f, 1.f};
  const int tpw = seg ? seg->tpw : 0, tpb = seg ? seg->tpb : 0;
  const int maxseg = seg ? seg->maxseg : 0, grid = seg ? seg->grid : 0;
  const float scale = sk_scale(tau);
  const float inv_tau = (float)(1.0 / (double)tau);
  const size_t lds = (size_t)iters * 2 * B * sizeof(float);
  switch (B) {
    case 32: sinkhorn_bwd_kernel<32><<<nb, SkGeom<32>::THREADS, lds, s>>>(logits, dP, tpw, tpb, maxseg, grid, off, dlogits, iters, scale, inv_tau, o); break;
    case 64: sinkhorn_bwd_kernel<64><<<nb, SkGeom<64>::THREADS, lds, s>>>(logits, dP, tpw, tpb, maxseg, grid, off, dlogits, iters, scale, inv_tau, o); break;
    case 128: sinkhorn_bwd_kernel<128><<<nb, SkGeom<128>::THREADS, lds, s>>>(logits, dP, tpw, tpb, maxseg, grid, off, dlogits, iters, scale, inv_tau, o); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lcp
