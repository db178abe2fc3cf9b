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
//   FB[t][p][lane]      Pb[16p + 8h + e][32t + n]     (lane = 32h + n)
#pragma once

#include "common.h"

namespace lcp {

template <int B>
struct FragGeom {
  static constexpr int KS = B / 16, TT = B / 32, FRAG = TT * KS * 64;
  static constexpr int NSPLIT = (B == 128) ? 2 : 3;
  static constexpr int NARR = 2 + NSPLIT;          // F1, FQ[NSPLIT], F2
};

// Ps: P_b in LDS with row pitch PP floats; ns: the block's B norms in LDS.
// Threads tid = 0 .. nthr-1 of the workgroup share the entries.
template <int B, int PP>
__device__ __forceinline__ void frag_build(const float* Ps, const float* ns, u32x4* __restrict__ fo,
                                           u32x4* __restrict__ ao, int tid, int nthr) {
  using G = FragGeom<B>;
  constexpr int KS = G::KS, FRAG = G::FRAG, NSPLIT = G::NSPLIT;
  for (int id = tid; id < (G::NARR + 1) * FRAG; id += nthr) {
    const int arr = id / FRAG, ent = id % FRAG;
    const int lane = ent & 63, tp = ent >> 6;          // tp = t * KS + p
    const int t = tp / KS, p = tp % KS;
    const int h = lane >> 5, rho = lane & 31;
    float v[8];
    if (arr < 1 + NSPLIT) {                            // F1 or FQ[arr - 1]
      const int k = 32 * t + remap_row(rho);
      const int jb = 32 * (p >> 1) + 16 * h + 8 * (p & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = Ps[(jb + e) * PP + k];
        if (arr == 0) {
          v[e] = pv;
        } else {
          const float q = ns[jb + e] * pv;
          const float hi = bf2f(f2bf(q));
          const float r1 = q - hi;
          const float mid = bf2f(f2bf(r1));
          v[e] = (arr == 1) ? hi : (arr == 2) ? mid : (r1 - mid);
        }
      }
    } else if (arr == 1 + NSPLIT) {                    // F2
      const int j = 32 * t + remap_row(rho);
      const int kb = 32 * (p >> 1) + 16 * h + 8 * (p & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Ps[j * PP + kb + e];
    } else {                                           // FB (adjoint)
      const int k = 32 * t + rho;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Ps[(16 * p + 8 * h + e) * PP + k];
    }
    // the split terms are exact bf16 values; the others round to nearest even
    const u32x4 o = {f2bf(v[0]) | (f2bf(v[1]) << 16), f2bf(v[2]) | (f2bf(v[3]) << 16),
                     f2bf(v[4]) | (f2bf(v[5]) << 16), f2bf(v[6]) | (f2bf(v[7]) << 16)};
    if (arr <= 1 + NSPLIT) fo[arr * FRAG + ent] = o;
    else ao[ent] = o;
  }
}

inline size_t frag_fwd_entries(int B) {
  const int KS = B / 16, TT = B / 32, FRAG = TT * KS * 64;
  return (size_t)(2 + (B == 128 ? 2 : 3)) * FRAG;
}
inline size_t frag_adj_entries(int B) { return (size_t)(B / 32) * (B / 16) * 64; }

}  // namespace lcp
