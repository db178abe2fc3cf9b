// MFMA operand fragments of one soft block permutation P_b, in exactly the
// per-lane order in which the permute and block-adjoint kernels read them
// from LDS (one 16-byte entry = 8 bf16 = the K slots one lane feeds to one
// 32x32x16 MFMA). Built once per step, from P_b and the column norms n staged
// in LDS, at the end of the Sinkhorn forward.
//
// Forward set, per block (see permute.hip):
//   F1[t][p][lane]      Pb[j][k]              row k = 32t + remap(rho), K j
//   FQ[s][t][p][lane]   split_s(n_j Pb[j][k])  (s < NSPLIT exact bf16 terms)
//   F2[t2][p][lane]     Pb[j][k]              row j = 32t2 + remap(rho), K k
// with lane = 32h + rho and, for F1/FQ, K step p = 2 t2 + u covering
// j = 32 t2 + 16h + 8u + e; for F2, p = 2t + u covering k = 32t + 16h + 8u + e.
// Adjoint set, per block (see adjoint.hip):
//   FB[t][p][lane]      Pb[j][32t + n]   (lane = 32h + n), K step p covering
//                       j = 32(p/2) + 16h + 8(p%2) + e as in F1
#pragma once

#include "common.h"

namespace lcp {

template <int B>
struct FragGeom {
  static constexpr int KS = B / 16, TT = B / 32, FRAG = TT * KS * 64;
  static constexpr int NSPLIT = (B == 128) ? 2 : 3;
  static constexpr int NARR = 2 + NSPLIT;          // F1, FQ[NSPLIT], F2
};

// Eight floats -> one 16-byte entry of bf16, round to nearest even
// (v_cvt_pk_bf16_f32); split terms are exact in bf16 and convert unchanged.
__device__ __forceinline__ u32x4 pack8(const float (&v)[8]) {
  return u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
}
__device__ __forceinline__ void unpack8(const u32x4& w, float (&v)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = lo_bf(w[q]);
    v[2 * q + 1] = hi_bf(w[q]);
  }
}

// Ps: P_b in LDS with row pitch PP floats (PP even); ns: the block's B norms
// in LDS. Threads tid = 0 .. nthr-1 of the workgroup share the entries; each
// entry index yields one entry of every array (the FQ terms of an entry come
// from one split of the same eight products).
template <int B, int PP>
__device__ __forceinline__ void frag_build(const float* Ps, const float* ns, u32x4* __restrict__ fo,
                                           u32x4* __restrict__ ao, int tid, int nthr) {
  using G = FragGeom<B>;
  constexpr int KS = G::KS, FRAG = G::FRAG, NSPLIT = G::NSPLIT;
  static_assert(PP % 2 == 0, "F2 rows are read as float2");
  for (int ent = tid; ent < FRAG; ent += nthr) {
    const int lane = ent & 63, tp = ent >> 6;          // tp = t * KS + p
    const int t = tp / KS, p = tp % KS;
    const int h = lane >> 5, rho = lane & 31;
    const int half = 16 * h + 8 * (p & 1);
    // F1 and FQ: row k = 32t + remap(rho), K = source channels jb .. jb + 7
    {
      const int k = 32 * t + remap_row(rho);
      const int jb = 32 * (p >> 1) + half;
      float pv[8], q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = Ps[(jb + e) * PP + k];
        q[e] = ns[jb + e] * pv[e];
      }
      fo[ent] = pack8(pv);
      const u32x4 hi = pack8(q);
      float hv[8], r[8];
      unpack8(hi, hv);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = q[e] - hv[e];     // exact
      const u32x4 mid = pack8(r);
      fo[FRAG + ent] = hi;
      fo[2 * FRAG + ent] = mid;
      if (NSPLIT > 2) {
        float mv[8], lo[8];
        unpack8(mid, mv);
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = r[e] - mv[e];  // exact, a bf16 value
        fo[3 * FRAG + ent] = pack8(lo);
      }
    }
    // F2: row j = 32t + remap(rho), K = positions kb .. kb + 7 (contiguous in a row)
    {
      const int j = 32 * t + remap_row(rho);
      const int kb = 32 * (p >> 1) + half;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float2 x = *reinterpret_cast<const float2*>(Ps + j * PP + kb + e);
        v[e] = x.x;
        v[e + 1] = x.y;
      }
      fo[(1 + NSPLIT) * FRAG + ent] = pack8(v);
    }
    // FB (adjoint): Pb[jb + e][32t + rho], the K slots of F1
    {
      const int k = 32 * t + rho;
      const int jb = 32 * (p >> 1) + half;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Ps[(jb + e) * PP + k];
      ao[ent] = pack8(v);
    }
  }
}

inline size_t frag_fwd_entries(int B) {
  const int KS = B / 16, TT = B / 32, FRAG = TT * KS * 64;
  return (size_t)(2 + (B == 128 ? 2 : 3)) * FRAG;
}
inline size_t frag_adj_entries(int B) { return (size_t)(B / 32) * (B / 16) * 64; }

}  // namespace lcp
