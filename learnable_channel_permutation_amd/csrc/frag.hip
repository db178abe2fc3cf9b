// MFMA operand fragments of the soft block permutations, built once per step
// from P (fp32) and the column norms n, in exactly the per-lane order the
// permute and block-adjoint kernels read them from LDS (one 16-byte entry =
// 8 bf16 = the K slots one lane feeds to one 32x32x16 MFMA).
//
// Forward set, per block (see permute.hip):
//   F1[t][p][lane]      Pb[j][k]           row k = 32t + remap(rho), K j
//   FQ[s][t][p][lane]   split_s(n_j Pb[j][k]) (s < NSPLIT bf16 terms)
//   F2[t2][p][lane]     Pb[j][k]           row j = 32t2 + remap(rho), K k
// with lane = 32h + rho and, for F1/FQ, K step p = 2 t2 + u covering
// j = 32 t2 + 16h + 8u + e; for F2, p = 2t + u covering k = 32t + 16h + 8u + e.
// Adjoint set, per block (see adjoint.hip):
//   FB[t][p][lane]      Pb[16p + 8h + e][32t + n]     (lane = 32h + n)
// One thread writes one 16-byte entry; the 8 values it gathers come from L2.
#include "common.h"
#include "kernels.h"

namespace lcp {

template <int B>
__global__ __launch_bounds__(256) void frag_kernel(const float* __restrict__ P, const float* __restrict__ n,
                                                   u32x4* __restrict__ fwd, u32x4* __restrict__ adj) {
  constexpr int KS = B / 16, TT = B / 32, FRAG = TT * KS * 64;
  constexpr int NSPLIT = (B == 128) ? 2 : 3;
  constexpr int NARR = 2 + NSPLIT;                   // F1, FQ[NSPLIT], F2
  const int b = blockIdx.x;
  const float* Pb = P + (size_t)b * B * B;
  const float* nb = n + (size_t)b * B;
  u32x4* fo = fwd + (size_t)b * NARR * FRAG;
  u32x4* ao = adj + (size_t)b * FRAG;
  for (int id = threadIdx.x; id < (NARR + 1) * FRAG; id += 256) {
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
        const float pv = Pb[(jb + e) * B + k];
        if (arr == 0) {
          v[e] = pv;
        } else {
          const float q = nb[jb + e] * pv;
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
      for (int e = 0; e < 8; ++e) v[e] = Pb[j * B + kb + e];
    } else {                                           // FB (adjoint)
      const int k = 32 * t + rho;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Pb[(16 * p + 8 * h + e) * B + k];
    }
    // the split terms are exact bf16 values; rounding the others matches the
    // in-kernel preparation (round to nearest even)
    const u32x4 o = {f2bf(v[0]) | (f2bf(v[1]) << 16), f2bf(v[2]) | (f2bf(v[3]) << 16),
                     f2bf(v[4]) | (f2bf(v[5]) << 16), f2bf(v[6]) | (f2bf(v[7]) << 16)};
    if (arr <= 1 + NSPLIT) fo[arr * FRAG + ent] = o;
    else ao[ent] = o;
  }
}

size_t frag_fwd_entries(int B) {
  const int KS = B / 16, TT = B / 32, FRAG = TT * KS * 64;
  return (size_t)(2 + (B == 128 ? 2 : 3)) * FRAG;
}
size_t frag_adj_entries(int B) { return (size_t)(B / 32) * (B / 16) * 64; }

hipError_t launch_frag(const float* P, const float* n, int nb, int B, u32x4* fwd, u32x4* adj,
                       hipStream_t s) {
  switch (B) {
    case 32: frag_kernel<32><<<nb, 256, 0, s>>>(P, n, fwd, adj); break;
    case 64: frag_kernel<64><<<nb, 256, 0, s>>>(P, n, fwd, adj); break;
    case 128: frag_kernel<128><<<nb, 256, 0, s>>>(P, n, fwd, adj); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lcp
