// Hardening of the soft block permutations ([PermLLM] Method 2): per block,
// the permutation matrix P that maximises Tr(P^T P_hat), i.e. the maximum-
// weight assignment of source channels (rows j) to permuted positions
// (columns k).
//
// One wavefront per block runs the shortest-augmenting-path method of
// Jonker and Volgenant: rows are inserted one at a time; for each, a
// Dijkstra-style search over the reduced costs c[j][k] - u[j] - v[k]
// (c = -P_hat) grows from the new row until it reaches a free column, then
// the duals are updated and the matching is flipped along the path. Lane l
// owns columns l and l + 64: it keeps their shortest-path lengths, path
// predecessors and duals in registers and relaxes them in parallel; the
// column to settle next is chosen by a wave-wide reduction on (length,
// occupied, index), so the choice is deterministic. Arithmetic is double
// precision on the fp32 P_hat. Optionally the kernel also writes the MFMA
// operand fragments of the hard P (frag.h) for the permute and the adjoint.
#include "common.h"
#include "kernels.h"

namespace lcp {

__device__ __forceinline__ bool sap_better(double d, int occ, int c, double od, int oocc, int oc) {
  return d < od || (d == od && (occ < oocc || (occ == oocc && c < oc)));
}

template <int B>
__global__ __launch_bounds__(64) void harden_kernel(const float* __restrict__ P, float* __restrict__ P_hard,
                                                    int* __restrict__ perm, const float* __restrict__ n,
                                                    u32x4* __restrict__ fwd, u32x4* __restrict__ adj) {
  typedef unsigned long long u64;
  constexpr int CPL = (B + 63) / 64;            // columns per lane
  constexpr int PP = B + 2;                     // LDS pitch of the staged block (even, for frag_build)
  constexpr double INF = __builtin_huge_val();
  __shared__ float ps[B * PP + B];              // P_hat, later the hard P; then the block's norms
  __shared__ double u[B], dm[B];
  __shared__ int col4row[B], row4col[B], pathm[B];
  const int l = threadIdx.x, b = blockIdx.x;

  const float* src = P + (size_t)b * B * B;
  for (int e = l; e < B * B; e += 64) ps[(e / B) * PP + e % B] = src[e];
  for (int j = l; j < B; j += 64) {
    u[j] = 0.0;
    col4row[j] = -1;
    row4col[j] = -1;
  }
  double v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) v[c] = 0.0;
  __syncthreads();

  for (int cur = 0; cur < B; ++cur) {
    double d[CPL];
    int path[CPL];
    bool done[CPL];                             // settled, or not a column of this block
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      d[c] = INF;
      path[c] = -1;
      done[c] = (l + 64 * c) >= B;
    }
    u64 rvis[2] = {0ull, 0ull};
    int i = cur, sink = -1;
    double minv = 0.0;
    // each pass settles one new column, and a free column exists, so at most
    // B passes
    for (int pass = 0; pass < B && sink < 0; ++pass) {
      rvis[i >> 6] |= 1ull << (i & 63);
      const double ui = u[i];
      const float* crow = ps + i * PP;
      double bd = INF;
      int bocc = 2, bc = 1 << 30;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int col = l + 64 * c;
        if (!done[c]) {
          const double r = minv - (double)crow[col] - ui - v[c];
          if (r < d[c]) {
            d[c] = r;
            path[c] = i;
          }
          const int occ = row4col[col] >= 0;
          if (sap_better(d[c], occ, col, bd, bocc, bc)) {
            bd = d[c];
            bocc = occ;
            bc = col;
          }
        }
      }
      // wave-wide choice; a total order, so every lane ends with the same one
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) {
        const double od = __shfl_xor(bd, x, 64);
        const int oocc = __shfl_xor(bocc, x, 64), oc = __shfl_xor(bc, x, 64);
        if (sap_better(od, oocc, oc, bd, bocc, bc)) {
          bd = od;
          bocc = oocc;
          bc = oc;
        }
      }
      if (bc >= B) break;                       // cannot happen: an unsettled column is left
      minv = bd;
      if ((bc & 63) == l) done[bc >> 6] = true;
      const int r4 = row4col[bc];
      if (r4 < 0) sink = bc;
      else i = r4;
    }
    // duals: u[cur] += minv; other rows on the tree by minv - d(their column);
    // settled columns v -= minv - d
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int col = l + 64 * c;
      if (col < B) {
        dm[col] = d[c];
        pathm[col] = path[c];
        const bool settled = done[c];
        if (settled) v[c] -= minv - d[c];
      }
    }
    __syncthreads();
    for (int r = l; r < B; r += 64) {
      if (r == cur) u[r] += minv;
      else if ((rvis[r >> 6] >> (r & 63)) & 1ull) u[r] += minv - dm[col4row[r]];
    }
    __syncthreads();
    // flip the matching along the path from the sink back to row cur
    if (l == 0 && sink >= 0) {
      int j = sink;
      for (int step = 0; step < B; ++step) {
        const int ii = pathm[j];
        if (ii < 0) break;                      // only for non-finite P_hat
        row4col[j] = ii;
        const int t = col4row[ii];
        col4row[ii] = j;
        j = t;
        if (ii == cur || j < 0) break;
      }
    }
    __syncthreads();
  }

  if (perm != nullptr)
    for (int k = l; k < B; k += 64) perm[(size_t)b * B + k] = row4col[k];
  if (P_hard != nullptr) {
    float* dst = P_hard + (size_t)b * B * B;
    for (int e = l; e < B * B; e += 64) dst[e] = (row4col[e % B] == e / B) ? 1.f : 0.f;
  }
  if (fwd != nullptr) {
    for (int e = l; e < B * B; e += 64) ps[(e / B) * PP + e % B] = (row4col[e % B] == e / B) ? 1.f : 0.f;
    for (int k = l; k < B; k += 64) ps[B * PP + k] = n[(size_t)b * B + k];
    __syncthreads();
    frag_build<B, PP>(ps, ps + B * PP, fwd + (size_t)b * FragGeom<B>::NARR * FragGeom<B>::FRAG,
                      adj + (size_t)b * FragGeom<B>::FRAG, l, 64);
  }
}

hipError_t launch_harden(const float* P, int nb, int B, float* P_hard, int* perm, const float* n, u32x4* fwd,
                         u32x4* adj, hipStream_t s) {
  switch (B) {
    case 32: harden_kernel<32><<<nb, 64, 0, s>>>(P, P_hard, perm, n, fwd, adj); break;
    case 64: harden_kernel<64><<<nb, 64, 0, s>>>(P, P_hard, perm, n, fwd, adj); break;
    case 128: harden_kernel<128><<<nb, 64, 0, s>>>(P, P_hard, perm, n, fwd, adj); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lcp
