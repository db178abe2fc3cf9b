// Block-wise channel permutation ([PermLLM] Method 3: P_B = diag(P_1..P_nb),
// W_hat = W P_B), the permuted importance S_hat = S P_B with S = |W| n
// ([PermLLM] integration formula; n = column norms of X), the N:M mask, and
// the return to source order W_tilde = (W_hat . M) P_B^T with D = W - W_tilde.
//
// bf16 path (gfx950 MFMA 32x32x16): a workgroup owns one channel block b and
// a range of rows; each wave takes 32-row tiles. Everything for one tile stays
// in registers:
//   product 1  W_hat^T[k][i] = sum_j Pb[j][k] W[i][j]    (A = P fragments,
//              B = 16-byte loads of the W row segment)
//   importance S_hat^T[k][i] = sum_j (n_j Pb[j][k]) |W[i][j]|, with n_j Pb
//              split into bf16 hi + mid (+ lo) so every product is exact in
//              fp32 and only the fp32 accumulation rounds
//   mask       the MFMA rows are remapped so that a lane of half h holds the
//              16 consecutive permuted positions 32t + 16h + r of its row i;
//              an N:M group is therefore inside one lane and is ranked in
//              registers
//   product 2  W_tilde^T[j][i] = sum_k Pb[j][k] A[i][k], with A = W_hat . M
//              (bf16) fed straight from the product-1 registers; the same
//              remap puts W_tilde[i][32t + 16h + r] in the lane that loaded
//              W[i][32t + 16h + r], so D = W - W_tilde needs no exchange.
// The P operands are built once per workgroup in LDS, already in the order in
// which each lane reads them (one 16-byte LDS read per MFMA operand).
//
// fp32 path: a plain VALU kernel (one workgroup per block and 8 rows) for
// float32 layers, where every product and sum is an fp32 FMA.
#include "common.h"
#include "kernels.h"

namespace lcp {

__device__ __forceinline__ uint16_t bf16_bits(float f) { return (uint16_t)f2bf(f); }

typedef __attribute__((address_space(3))) void* perm_lds_t;

template <int B, int MODE>
struct PermGeom {
  static constexpr int KS = B / 16;              // K steps of 16 over a block
  static constexpr int TT = B / 32;              // 32-wide tiles over a block
  static constexpr int FRAG = TT * KS * 64;      // u32x4 entries per fragment array
  static constexpr int NSPLIT = (MODE == PERM_PLAIN) ? 0 : (B == 128 ? 2 : 3);
  static constexpr int NARR = 1 + NSPLIT + (MODE == PERM_FWD ? 1 : 0);
  static constexpr int WAVES = (B == 128) ? 8 : 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr size_t LDS = (size_t)NARR * FRAG * 16;
};

// Build the fragment arrays for block b in LDS.
//   F1  product-1 A operand: row k (remapped), K index j
//   FQ  importance A operands (NSPLIT bf16 terms of colscale[j] * Pb[j][k])
//   F2  product-2 A operand: row j (remapped), K index k
template <int B, int MODE>
__device__ __forceinline__ void perm_prep(const float* __restrict__ P, const float* __restrict__ colscale,
                                          int b, int transposeP, uint16_t* lds) {
  using G = PermGeom<B, MODE>;
  constexpr int KS = G::KS;
  const float* src = P + (size_t)b * B * B;
  for (int e_idx = threadIdx.x; e_idx < B * B; e_idx += G::THREADS) {
    const int r = e_idx / B, c = e_idx % B;
    const float p = src[e_idx];
    const int j = transposeP ? c : r;
    const int k = transposeP ? r : c;
    // product 1 / importance position
    {
      const int t = k >> 5, rho = remap_inv(k & 31);
      const int t2 = j >> 5, h = (j >> 4) & 1, u = (j >> 3) & 1, e = j & 7;
      const int idx = (((t * KS + 2 * t2 + u) * 64) + 32 * h + rho) * 8 + e;
      lds[idx] = bf16_bits(p);
      if (G::NSPLIT > 0) {
        const float v = colscale[b * B + j] * p;
        const float hi = bf2f(f2bf(v));
        const float r1 = v - hi;
        const float mid = bf2f(f2bf(r1));
        lds[(size_t)1 * G::FRAG * 8 + idx] = bf16_bits(hi);
        lds[(size_t)2 * G::FRAG * 8 + idx] = bf16_bits(mid);
        if (G::NSPLIT > 2) lds[(size_t)3 * G::FRAG * 8 + idx] = bf16_bits(r1 - mid);
      }
    }
    if (MODE == PERM_FWD) {
      const int t2 = j >> 5, rho = remap_inv(j & 31);
      const int t = k >> 5, h = (k >> 4) & 1, u = (k >> 3) & 1, e = k & 7;
      const int idx = (((t2 * KS + 2 * t + u) * 64) + 32 * h + rho) * 8 + e;
      lds[(size_t)(1 + G::NSPLIT) * G::FRAG * 8 + idx] = bf16_bits(p);
    }
  }
}

// Persistent grid: workgroup g takes the contiguous range of 32-row tiles
// [g * tpw, (g + 1) * tpw) of the block-major tile sequence (tpb tiles per
// block), so every workgroup gets the same amount of work and a range spans
// at most a few blocks; the P fragments are (re)loaded into LDS when the
// block changes. With `gfrag` the fragments come precomputed from global
// memory (a coalesced copy), otherwise they are built here.
// NK: for M = 4, the N of N:M fixed at compile time (1..3), 0 = runtime N.
template <int B, int MODE, int M, int NK>
__global__ __launch_bounds__((PermGeom<B, MODE>::THREADS)) void permute_bf16_kernel(
    const uint16_t* __restrict__ A, int rows, int cin, const float* __restrict__ colscale,
    const float* __restrict__ P, int transposeP, const u32x4* __restrict__ gfrag, int tpw,
    void* __restrict__ out, int out_f32, uint32_t* __restrict__ bits, int N) {
  using G = PermGeom<B, MODE>;
  constexpr int KS = G::KS, TT = G::TT;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const u32x4* F1 = reinterpret_cast<const u32x4*>(lds);
  const u32x4* FQ = F1 + G::FRAG;
  const u32x4* F2 = F1 + (size_t)(1 + G::NSPLIT) * G::FRAG;

  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = l >> 5, n = l & 31;
  const int tpb = (rows + 31) / 32;
  const int total = (cin / B) * tpb;
  // workgroup g runs on XCD g % 8: consecutive tile ranges go to one XCD, so
  // the few workgroups that share a block fetch its P fragments into one L2
  // (the grid is a multiple of 8; ranges past the end are empty)
  const int g = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int t_begin = g * tpw;
  const int t_end = min(total, t_begin + tpw);

  for (int seg = t_begin; seg < t_end;) {
    const int b = seg / tpb;
    const int seg_end = min(t_end, (b + 1) * tpb);
    __syncthreads();                      // previous block's fragments no longer read
    if (gfrag != nullptr) {
      // every 16-byte entry goes global -> LDS directly; all of a thread's
      // copies are in flight at once and one wait covers them (entry counts
      // are multiples of 64, so each wave copies whole 1 KB rows or none)
      const u32x4* src = gfrag + (size_t)b * G::NARR * G::FRAG;
      constexpr int NE = G::NARR * G::FRAG, PER = (NE + G::THREADS - 1) / G::THREADS;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e0 = k * G::THREADS + 64 * w;
        if (e0 < NE)
          __builtin_amdgcn_global_load_lds(src + e0 + l, (perm_lds_t)(lds + (size_t)e0 * 8), 16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));   // vmcnt(0)
    } else {
      perm_prep<B, MODE>(P, colscale, b, transposeP, lds);
    }
    __syncthreads();

    const int colbase = b * B + 16 * h;
    u32x4 wop[KS];
    auto load_tile = [&](int tile) {
      const int i = (tile - b * tpb) * 32 + n;
#pragma unroll
      for (int p = 0; p < KS; ++p) {
        const int col = colbase + 32 * (p >> 1) + 8 * (p & 1);
        if (i < rows) wop[p] = *reinterpret_cast<const u32x4*>(A + (size_t)i * cin + col);
        else wop[p] = u32x4{0u, 0u, 0u, 0u};
      }
    };

    int tile = seg + w;
    if (tile < seg_end) load_tile(tile);
    for (; tile < seg_end; tile += G::WAVES) {
      // keep the P fragments in LDS: re-read them per tile instead of letting
      // the compiler hoist all of them into registers (which caps occupancy)
      __asm__ volatile("" ::: "memory");
      const int i = (tile - b * tpb) * 32 + n;
      u32x4 cur[KS];
#pragma unroll
      for (int p = 0; p < KS; ++p) cur[p] = wop[p];
      if (tile + G::WAVES < seg_end) load_tile(tile + G::WAVES);   // prefetch the next tile

      if (MODE == PERM_PLAIN) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          floatx16 acc = {};
#pragma unroll
          for (int p = 0; p < KS; ++p) acc = mfma32(F1[(t * KS + p) * 64 + l], cur[p], acc);
          if (i < rows) {
            const size_t o = (size_t)i * cin + colbase + 32 * t;
            if (out_f32) {
              floatx4* dst = reinterpret_cast<floatx4*>(reinterpret_cast<float*>(out) + o);
#pragma unroll
              for (int q = 0; q < 4; ++q) dst[q] = floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
            } else {
              u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + o);
#pragma unroll
              for (int q = 0; q < 2; ++q)
                dst[q] = u32x4{pack2(acc[8 * q], acc[8 * q + 1]), pack2(acc[8 * q + 2], acc[8 * q + 3]),
                               pack2(acc[8 * q + 4], acc[8 * q + 5]), pack2(acc[8 * q + 6], acc[8 * q + 7])};
            }
          }
        }
        continue;
      }

      u32x4 absw[KS];
#pragma unroll
      for (int p = 0; p < KS; ++p)
        absw[p] = u32x4{cur[p].x & 0x7fff7fffu, cur[p].y & 0x7fff7fffu, cur[p].z & 0x7fff7fffu, cur[p].w & 0x7fff7fffu};

      if (MODE == PERM_IMPORTANCE) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          floatx16 acc = {};
#pragma unroll
          for (int s = G::NSPLIT - 1; s >= 0; --s)
#pragma unroll
            for (int p = 0; p < KS; ++p) acc = mfma32(FQ[(size_t)s * G::FRAG + (t * KS + p) * 64 + l], absw[p], acc);
          if (i < rows) {
            float* dst = reinterpret_cast<float*>(out) + (size_t)i * cin + colbase + 32 * t;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              reinterpret_cast<floatx4*>(dst)[q] = floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
          }
        }
        continue;
      }

      // ---- PERM_FWD: mask, A = W_hat . M, product 2, D = W - W_tilde
      u32x4 aop[KS];
      uint32_t kw[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        floatx16 sh = {};
#pragma unroll
        for (int s = G::NSPLIT - 1; s >= 0; --s)
#pragma unroll
          for (int p = 0; p < KS; ++p) sh = mfma32(FQ[(size_t)s * G::FRAG + (t * KS + p) * 64 + l], absw[p], sh);
        floatx16 wh = {};
#pragma unroll
        for (int p = 0; p < KS; ++p) wh = mfma32(F1[(t * KS + p) * 64 + l], cur[p], wh);
        float v[16], a[16];
        uint32_t keep = 0;
        if constexpr (M == 4 && NK > 0) {
          // the scores are sums of products of |W|, n_j and P (all >= +0), so
          // nm_keep4_nonneg applies; each group's keep masks are used at once
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = sh[r];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bool k4[4];
            nm_keep4_nonneg<NK>(v + 4 * g, k4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              keep |= k4[q] ? (1u << (4 * g + q)) : 0u;
              a[4 * g + q] = k4[q] ? wh[4 * g + q] : 0.f;
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = nan_to_ninf(sh[r]);
#pragma unroll
          for (int g = 0; g < 16 / M; ++g) keep |= nm_keep<M>(v + g * M, N) << (g * M);
#pragma unroll
          for (int r = 0; r < 16; ++r) a[r] = ((keep >> r) & 1u) ? wh[r] : 0.f;
        }
        const uint32_t other = (uint32_t)__shfl_xor((int)keep, 32, 64);
        kw[t] = keep | (other << 16);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          aop[2 * t + u] = u32x4{pack2(a[8 * u], a[8 * u + 1]), pack2(a[8 * u + 2], a[8 * u + 3]),
                                 pack2(a[8 * u + 4], a[8 * u + 5]), pack2(a[8 * u + 6], a[8 * u + 7])};
      }
      // mask words, block-major: the tile's 32 rows x TT words are contiguous;
      // stored non-temporally (read again only by the backward's adjoint)
      if (h == 0 && i < rows) {
        uint32_t* bw = bits + ((size_t)b * rows + i) * TT;
        if constexpr (TT == 4) __builtin_nontemporal_store(u32x4{kw[0], kw[1], kw[2], kw[3]}, reinterpret_cast<u32x4*>(bw));
        else if constexpr (TT == 2) {
          typedef uint32_t v2u __attribute__((ext_vector_type(2)));
          __builtin_nontemporal_store(v2u{kw[0], kw[1]}, reinterpret_cast<v2u*>(bw));
        }
        else bw[0] = kw[0];
      }
#pragma unroll
      for (int t2 = 0; t2 < TT; ++t2) {
        floatx16 wt = {};
#pragma unroll
        for (int p2 = 0; p2 < KS; ++p2) wt = mfma32(F2[(t2 * KS + p2) * 64 + l], aop[p2], wt);
        if (i < rows) {
          u32x4 dv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const u32x4 wv = cur[2 * t2 + u];
            const uint32_t wq[4] = {wv.x, wv.y, wv.z, wv.w};
            uint32_t d[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              d[q] = pack2(lo_bf(wq[q]) - wt[8 * u + 2 * q], hi_bf(wq[q]) - wt[8 * u + 2 * q + 1]);
            dv[u] = u32x4{d[0], d[1], d[2], d[3]};
          }
          u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + (size_t)i * cin + colbase + 32 * t2);
          dst[0] = dv[0];
          dst[1] = dv[1];
        }
      }
    }
    seg = seg_end;
  }
}

// ---- fp32 VALU path -----------------------------------------------------------
// One workgroup of 256 threads per (block b, 8 rows): thread (row rr = t/32,
// lane q = t%32) produces positions q, q+32, ... of its row.
template <int B, int MODE, int M>
__global__ __launch_bounds__(256) void permute_f32_kernel(const float* __restrict__ A, int rows, int cin,
                                                          const float* __restrict__ colscale,
                                                          const float* __restrict__ P, int transposeP,
                                                          float* __restrict__ out,
                                                          uint32_t* __restrict__ bits, int N) {
  __shared__ float pb[B][B + 1];
  __shared__ float arow[8][B];
  __shared__ float what[8][B];
  __shared__ float shat[8][B];
  __shared__ uint32_t kw[8][B / 32];
  const int b = blockIdx.x;
  const int t = threadIdx.x, rr = t >> 5, q = t & 31;
  const int i = blockIdx.y * 8 + rr;
  const float* src = P + (size_t)b * B * B;
  for (int e = t; e < B * B; e += 256) {
    const int r = e / B, c = e % B;
    if (transposeP) pb[c][r] = src[e];
    else pb[r][c] = src[e];
  }
  for (int c = q; c < B; c += 32) arow[rr][c] = (i < rows) ? A[(size_t)i * cin + b * B + c] : 0.f;
  __syncthreads();
  for (int k = q; k < B; k += 32) {
    float s1 = 0.f, s2 = 0.f;
    for (int j = 0; j < B; ++j) {
      const float a = arow[rr][j];
      s1 = fmaf(a, pb[j][k], s1);
      if (MODE != PERM_PLAIN) s2 = fmaf(fabsf(a) * colscale[b * B + j], pb[j][k], s2);
    }
    what[rr][k] = s1;
    shat[rr][k] = s2;
  }
  __syncthreads();
  if (MODE == PERM_PLAIN || MODE == PERM_IMPORTANCE) {
    if (i < rows)
      for (int k = q; k < B; k += 32)
        out[(size_t)i * cin + b * B + k] = (MODE == PERM_PLAIN) ? what[rr][k] : shat[rr][k];
    return;
  }
  if (q < B / 32) {
    uint32_t wbits = 0;
    float v[32];
    for (int e = 0; e < 32; ++e) v[e] = nan_to_ninf(shat[rr][32 * q + e]);
    for (int g = 0; g < 32 / M; ++g) wbits |= nm_keep<M>(v + g * M, N) << (g * M);
    kw[rr][q] = wbits;
    if (i < rows) bits[((size_t)b * rows + i) * (B >> 5) + q] = wbits;
  }
  __syncthreads();
  for (int k = q; k < B; k += 32)
    if (!((kw[rr][k >> 5] >> (k & 31)) & 1u)) what[rr][k] = 0.f;
  __syncthreads();
  if (i < rows)
    for (int j = q; j < B; j += 32) {
      float s = 0.f;
      for (int k = 0; k < B; ++k) s = fmaf(what[rr][k], pb[j][k], s);
      out[(size_t)i * cin + b * B + j] = arow[rr][j] - s;
    }
}

// ---- elementwise difference for lcp_error --------------------------------------
__global__ __launch_bounds__(256) void diff_kernel(const void* __restrict__ W, const void* __restrict__ Wt,
                                                   int n, int bf16, void* __restrict__ D) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  if (bf16) {
    const uint16_t* a = reinterpret_cast<const uint16_t*>(W);
    const uint16_t* c = reinterpret_cast<const uint16_t*>(Wt);
    reinterpret_cast<uint16_t*>(D)[i] = (uint16_t)f2bf(bf2f(a[i]) - bf2f(c[i]));
  } else {
    reinterpret_cast<float*>(D)[i] = reinterpret_cast<const float*>(W)[i] - reinterpret_cast<const float*>(Wt)[i];
  }
}

// ---- launchers -------------------------------------------------------------------
// Grid: about one round of resident workgroups on 256 CUs (LDS and registers
// allow 4 per CU for B = 32, 3 for B = 64 with the forward's six fragment
// arrays, 1 for B = 128). Every tile is computed independently, so results do
// not depend on the split.
static int perm_grid(int B, int mode) { return B == 128 ? 256 : (B == 64 && mode == PERM_FWD) ? 768 : 1024; }

template <int B, int MODE, int M, int NK = 0>
static hipError_t perm_bf16_launch(const uint16_t* A, int rows, int cin, const float* colscale,
                                   const float* P, int transposeP, const u32x4* gfrag, void* out,
                                   int out_f32, uint32_t* bits, int N, hipStream_t s) {
  using G = PermGeom<B, MODE>;
  const int total = (cin / B) * ((rows + 31) / 32);
  int grid = perm_grid(B, MODE);
  const int tpw = (total + grid - 1) / grid;
  grid = ((total + tpw - 1) / tpw + 7) / 8 * 8;          // whole XCD rounds
  permute_bf16_kernel<B, MODE, M, NK><<<grid, G::THREADS, G::LDS, s>>>(A, rows, cin, colscale, P, transposeP,
                                                                    gfrag, tpw, out, out_f32, bits, N);
  return hipGetLastError();
}

template <int B, int MODE>
static hipError_t perm_bf16_m(const uint16_t* A, int rows, int cin, const float* colscale, const float* P,
                              int transposeP, const u32x4* gfrag, void* out, int out_f32, uint32_t* bits,
                              int N, int M, hipStream_t s) {
  if (M == 8) return perm_bf16_launch<B, MODE, 8>(A, rows, cin, colscale, P, transposeP, gfrag, out, out_f32, bits, N, s);
  switch (N) {
    case 1: return perm_bf16_launch<B, MODE, 4, 1>(A, rows, cin, colscale, P, transposeP, gfrag, out, out_f32, bits, N, s);
    case 2: return perm_bf16_launch<B, MODE, 4, 2>(A, rows, cin, colscale, P, transposeP, gfrag, out, out_f32, bits, N, s);
    case 3: return perm_bf16_launch<B, MODE, 4, 3>(A, rows, cin, colscale, P, transposeP, gfrag, out, out_f32, bits, N, s);
  }
  return perm_bf16_launch<B, MODE, 4>(A, rows, cin, colscale, P, transposeP, gfrag, out, out_f32, bits, N, s);
}

template <int B>
static hipError_t perm_bf16_b(const uint16_t* A, int rows, int cin, const float* colscale, const float* P,
                              int transposeP, const u32x4* gfrag, int mode, void* out, int out_f32,
                              uint32_t* bits, int N, int M, hipStream_t s) {
  switch (mode) {
    case PERM_PLAIN: return perm_bf16_launch<B, PERM_PLAIN, 4>(A, rows, cin, colscale, P, transposeP, nullptr, out, out_f32, bits, N, s);
    case PERM_IMPORTANCE: return perm_bf16_launch<B, PERM_IMPORTANCE, 4>(A, rows, cin, colscale, P, transposeP, nullptr, out, 1, bits, N, s);
    default: return perm_bf16_m<B, PERM_FWD>(A, rows, cin, colscale, P, transposeP, gfrag, out, 0, bits, N, M, s);
  }
}

hipError_t launch_permute_bf16(const uint16_t* A, int rows, int cin, const float* colscale,
                               const float* P, int B, int transposeP, const u32x4* gfrag, int mode,
                               void* out, int out_f32, uint32_t* bits, int N, int M, hipStream_t s) {
  switch (B) {
    case 32: return perm_bf16_b<32>(A, rows, cin, colscale, P, transposeP, gfrag, mode, out, out_f32, bits, N, M, s);
    case 64: return perm_bf16_b<64>(A, rows, cin, colscale, P, transposeP, gfrag, mode, out, out_f32, bits, N, M, s);
    case 128: return perm_bf16_b<128>(A, rows, cin, colscale, P, transposeP, gfrag, mode, out, out_f32, bits, N, M, s);
  }
  return hipErrorInvalidValue;
}

template <int B, int MODE, int M>
static hipError_t perm_f32_launch(const float* A, int rows, int cin, const float* colscale, const float* P,
                                  int transposeP, float* out, uint32_t* bits, int N, hipStream_t s) {
  dim3 grid(cin / B, (rows + 7) / 8);
  permute_f32_kernel<B, MODE, M><<<grid, 256, 0, s>>>(A, rows, cin, colscale, P, transposeP, out, bits, N);
  return hipGetLastError();
}

template <int B>
static hipError_t perm_f32_b(const float* A, int rows, int cin, const float* colscale, const float* P,
                             int transposeP, int mode, float* out, uint32_t* bits, int N, int M,
                             hipStream_t s) {
  switch (mode) {
    case PERM_PLAIN: return perm_f32_launch<B, PERM_PLAIN, 4>(A, rows, cin, colscale, P, transposeP, out, bits, N, s);
    case PERM_IMPORTANCE: return perm_f32_launch<B, PERM_IMPORTANCE, 4>(A, rows, cin, colscale, P, transposeP, out, bits, N, s);
    default:
      if (M == 8) return perm_f32_launch<B, PERM_FWD, 8>(A, rows, cin, colscale, P, transposeP, out, bits, N, s);
      return perm_f32_launch<B, PERM_FWD, 4>(A, rows, cin, colscale, P, transposeP, out, bits, N, s);
  }
}

hipError_t launch_permute_f32(const float* A, int rows, int cin, const float* colscale,
                              const float* P, int B, int transposeP, int mode, float* out,
                              uint32_t* bits, int N, int M, hipStream_t s) {
  switch (B) {
    case 32: return perm_f32_b<32>(A, rows, cin, colscale, P, transposeP, mode, out, bits, N, M, s);
    case 64: return perm_f32_b<64>(A, rows, cin, colscale, P, transposeP, mode, out, bits, N, M, s);
    case 128: return perm_f32_b<128>(A, rows, cin, colscale, P, transposeP, mode, out, bits, N, M, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_diff(const void* W, const void* Wt, int n, int bf16, void* D, hipStream_t s) {
  diff_kernel<<<(n + 255) / 256, 256, 0, s>>>(W, Wt, n, bf16, D);
  return hipGetLastError();
}

}  // namespace lcp
