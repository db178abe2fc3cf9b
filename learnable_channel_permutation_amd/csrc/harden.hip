// Hardening of the soft block permutations ([PermLLM] Method 2): per block,
// the permutation matrix P that maximises Tr(P^T P_hat), i.e. the maximum-
// weight assignment of source channels (rows j) to permuted positions
// (columns k).
//
// One workgroup per block. Its first wavefront runs the shortest-augmenting-
// path method of Jonker and Volgenant: a feasible start (column minima as
// column duals, every row that is the unique best of some column matched to
// it) leaves only the contested rows; they are inserted one at a time, each
// by a Dijkstra-style search over the reduced costs c[j][k] - u[j] - v[k]
// (c = -P_hat) that grows from the new row until it reaches a free column,
// then the duals are updated and the matching is flipped along the path.
// Lane l owns columns l and l + 64: it keeps their shortest-path lengths,
// path predecessors and duals in registers and relaxes them in parallel; the
// column to settle next is chosen by a wave-wide DPP / permlane reduction on
// (length, occupied, index), so the choice is deterministic. Arithmetic is
// double precision on the fp32 P_hat. Staging, the start and the outputs use
// all four waves. Optionally the kernel also writes the MFMA operand
// fragments of the hard P (frag.h) for the permute and the adjoint.
#include "common.h"
#include "kernels.h"

namespace lcp {

// (length, key) ordering of candidate columns, key = 256 * occupied + column
__device__ __forceinline__ bool sap_better(double d, int key, double od, int okey) {
  return d < od || (d == od && key < okey);
}

// Partner values for the wave-wide choice: DPP moves inside rows of 16 lanes
// (quad swaps, half-row and row mirrors), then the permlane swaps pair lanes
// 16 and 32 apart. Every step combines two candidates under a total order,
// so after the six steps all 64 lanes hold the same (the best) candidate.
template <int CTRL>
__device__ __forceinline__ void sap_step_dpp(double& d, int& key) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)__double2loint(d), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)__double2hiint(d), CTRL, 0xf, 0xf, false);
  const int ok = __builtin_amdgcn_update_dpp(0, key, CTRL, 0xf, 0xf, false);
  const double od = __hiloint2double(hi, lo);
  if (sap_better(od, ok, d, key)) {
    d = od;
    key = ok;
  }
}
template <int DIST>
__device__ __forceinline__ void sap_step_swap(double& d, int& key, int lane) {
  const uint32_t lo = (uint32_t)__double2loint(d), hi = (uint32_t)__double2hiint(d), k = (uint32_t)key;
  uint32_t plo, phi, pk;
  if (DIST == 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(k, k, false, false);
    const bool upper = lane & 16;
    plo = upper ? a[0] : a[1];
    phi = upper ? b[0] : b[1];
    pk = upper ? c[0] : c[1];
  } else {
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const auto c = __builtin_amdgcn_permlane32_swap(k, k, false, false);
    const bool upper = lane & 32;
    plo = upper ? a[0] : a[1];
    phi = upper ? b[0] : b[1];
    pk = upper ? c[0] : c[1];
  }
  const double od = __hiloint2double((int)phi, (int)plo);
  if (sap_better(od, (int)pk, d, key)) {
    d = od;
    key = (int)pk;
  }
}

template <int B>
__global__ __launch_bounds__(256) void harden_kernel(const float* __restrict__ P, float* __restrict__ P_hard,
                                                     int* __restrict__ perm, const float* __restrict__ n,
                                                     u32x4* __restrict__ fwd, u32x4* __restrict__ adj) {
  typedef unsigned long long u64;
  constexpr int CPL = (B + 63) / 64;            // columns per lane of the searching wave
  constexpr int PP = B + 2;                     // LDS pitch of the staged block (even, for frag_build)
  constexpr double INF = __builtin_huge_val();
  __shared__ float ps[B * PP + B];              // P_hat, later the hard P; then the block's norms
  __shared__ double u[B], dm[B], vs[B];
  __shared__ int col4row[B], row4col[B], pathm[B], cnt[B], props[B];
  const int t = threadIdx.x, l = t & 63, w = t >> 6, b = blockIdx.x;

  // stage P_hat (16-byte loads)
  const floatx4* src4 = reinterpret_cast<const floatx4*>(P + (size_t)b * B * B);
  for (int e4 = t; e4 < B * B / 4; e4 += 256) {
    const floatx4 x = src4[e4];
    const int row = (4 * e4) / B, col = (4 * e4) % B;
    float* dst = ps + row * PP + col;
    *reinterpret_cast<float2*>(dst) = float2{x[0], x[1]};
    *reinterpret_cast<float2*>(dst + 2) = float2{x[2], x[3]};
  }
  for (int j = t; j < B; j += 256) {
    u[j] = 0.0;
    col4row[j] = -1;
    row4col[j] = -1;
    cnt[j] = 0;
  }
  __syncthreads();

  // feasible start: v[k] = min_j c[j][k] (c = -P_hat) with u = 0, so every
  // reduced cost is >= 0; each column proposes its first minimising row, and
  // a row proposed by exactly one column is matched to it (a tight edge)
  if (t < B) {
    float best = ps[t];
    int arg = 0;
    for (int j = 1; j < B; ++j) {
      const float x = ps[j * PP + t];
      if (x > best) {
        best = x;
        arg = j;
      }
    }
    vs[t] = -(double)best;
    props[t] = arg;
    atomicAdd(&cnt[arg], 1);
  }
  __syncthreads();
  if (t < B && cnt[props[t]] == 1) {
    row4col[t] = props[t];
    col4row[props[t]] = t;
  }
  __syncthreads();

  // contested rows: wave 0 alone, so its LDS traffic only needs ordering
  // inside the wave (wavefront-scope fences)
  if (w == 0) {
    double v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = (l + 64 * c < B) ? vs[l + 64 * c] : 0.0;
    for (int cur = 0; cur < B; ++cur) {
      if (col4row[cur] >= 0) continue;          // matched already (uniform)
      double d[CPL];
      int path[CPL];
      bool done[CPL];                           // settled, or not a column of this block
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        d[c] = INF;
        path[c] = -1;
        done[c] = (l + 64 * c) >= B;
      }
      u64 rvis[2] = {0ull, 0ull};
      int i = cur, sink = -1;
      double minv = 0.0;
      // each pass settles one new column, and a free column exists, so at
      // most B passes
      for (int pass = 0; pass < B && sink < 0; ++pass) {
        rvis[i >> 6] |= 1ull << (i & 63);
        const double ui = u[i];
        const float* crow = ps + i * PP;
        double bd = INF;
        int bkey = 1 << 30;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int col = l + 64 * c;
          if (!done[c]) {
            const double r = minv - (double)crow[col] - ui - v[c];
            if (r < d[c]) {
              d[c] = r;
              path[c] = i;
            }
            const int key = (row4col[col] >= 0 ? 256 : 0) + col;
            if (sap_better(d[c], key, bd, bkey)) {
              bd = d[c];
              bkey = key;
            }
          }
        }
        sap_step_dpp<0xB1>(bd, bkey);
        sap_step_dpp<0x4E>(bd, bkey);
        sap_step_dpp<0x141>(bd, bkey);
        sap_step_dpp<0x140>(bd, bkey);
        sap_step_swap<16>(bd, bkey, l);
        sap_step_swap<32>(bd, bkey, l);
        const int bc = bkey & 255;
        if (bkey >= (1 << 30) || bc >= B) break;  // cannot happen: an unsettled column is left
        minv = bd;
        if ((bc & 63) == l) done[bc >> 6] = true;
        const int r4 = row4col[bc];
        if (r4 < 0) sink = bc;
        else i = r4;
      }
      // duals: u[cur] += minv; other rows on the tree by minv - d(their
      // column); settled columns v -= minv - d
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int col = l + 64 * c;
        if (col < B) {
          dm[col] = d[c];
          pathm[col] = path[c];
          if (done[c]) v[c] -= minv - d[c];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      for (int r = l; r < B; r += 64) {
        if (r == cur) u[r] += minv;
        else if ((rvis[r >> 6] >> (r & 63)) & 1ull) u[r] += minv - dm[col4row[r]];
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      // flip the matching along the path from the sink back to row cur
      if (l == 0 && sink >= 0) {
        int j = sink;
        for (int step = 0; step < B; ++step) {
          const int ii = pathm[j];
          if (ii < 0) break;                    // only for non-finite P_hat
          row4col[j] = ii;
          const int tt = col4row[ii];
          col4row[ii] = j;
          j = tt;
          if (ii == cur || j < 0) break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
  }
  __syncthreads();

  if (perm != nullptr)
    for (int k = t; k < B; k += 256) perm[(size_t)b * B + k] = row4col[k];
  if (P_hard != nullptr) {
    floatx4* dst4 = reinterpret_cast<floatx4*>(P_hard + (size_t)b * B * B);
    for (int e4 = t; e4 < B * B / 4; e4 += 256) {
      const int row = (4 * e4) / B, col = (4 * e4) % B;
      dst4[e4] = floatx4{row4col[col] == row ? 1.f : 0.f, row4col[col + 1] == row ? 1.f : 0.f,
                         row4col[col + 2] == row ? 1.f : 0.f, row4col[col + 3] == row ? 1.f : 0.f};
    }
  }
  if (fwd != nullptr) {
    for (int e = t; e < B * B; e += 256) ps[(e / B) * PP + e % B] = (row4col[e % B] == e / B) ? 1.f : 0.f;
    for (int k = t; k < B; k += 256) ps[B * PP + k] = n[(size_t)b * B + k];
    __syncthreads();
    frag_build<B, PP>(ps, ps + B * PP, fwd + (size_t)b * FragGeom<B>::NARR * FragGeom<B>::FRAG,
                      adj + (size_t)b * FragGeom<B>::FRAG, t, 256);
  }
}

hipError_t launch_harden(const float* P, int nb, int B, float* P_hard, int* perm, const float* n, u32x4* fwd,
                         u32x4* adj, hipStream_t s) {
  switch (B) {
    case 32: harden_kernel<32><<<nb, 256, 0, s>>>(P, P_hard, perm, n, fwd, adj); break;
    case 64: harden_kernel<64><<<nb, 256, 0, s>>>(P, P_hard, perm, n, fwd, adj); break;
    case 128: harden_kernel<128><<<nb, 256, 0, s>>>(P, P_hard, perm, n, fwd, adj); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lcp
