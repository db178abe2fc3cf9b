// GEMMs of the LCP step: the output error R = D X^T (E = ||R||_F) and the
// backward product dD = (1/E) R X, both written as C[m][n] = sum_k A[m][k] B[n][k]
// with A and B row-major and K contiguous (the backward reads X transposed,
// prepared once per layer).
//
// bf16 kernel (gfx950): 256 x 128 x 64 tiles, 4 waves in a 2 x 2 layout, each
// wave 128 x 64 = 4 x 2 MFMA 32x32x16 blocks with fp32 accumulators. Global
// tiles are loaded as 16-byte chunks into registers and stored to LDS
// (double-buffered, one barrier per K step); chunk c of row r sits at
// position c ^ (r & 7) so the 16-byte fragment reads of 8 consecutive rows hit
// distinct banks. The MFMA A operand is taken from the B matrix with the row
// remap of common.h, so each lane ends up holding 16 consecutive output
// columns of one output row and writes them as two 16-byte stores.
// Workgroups are ordered so that each XCD (workgroup id mod 8) works on a
// compact group of 4 row panels x 8 column panels, which keeps the panels
// shared inside that XCD's L2.
//
// Epilogues: ERR stores C in bf16 and one sum of squares of the fp32
// accumulators per workgroup (reduced later in a fixed order); DD scales by
// -1/E (E read from device memory; 0 when E == 0) and stores bf16.
#include "common.h"
#include "kernels.h"

namespace lcp {

enum { EPI_ERR = 0, EPI_DD = 1 };

constexpr int GBM = 256, GBN = 128, GBK = 64;
constexpr int GROUP_M = 4;

__device__ __forceinline__ void tile_coords(int g, int G, int tiles_m, int tiles_n, int& tm, int& tn) {
  int logical = g;
  if ((G & 7) == 0) logical = (g & 7) * (G >> 3) + (g >> 3);
  const int in_group = GROUP_M * tiles_n;
  const int gid = logical / in_group;
  const int first_m = gid * GROUP_M;
  const int gsm = min(tiles_m - first_m, GROUP_M);
  const int rem = logical - gid * in_group;
  tm = first_m + rem % gsm;
  tn = rem / gsm;
}

__device__ __forceinline__ int swz(int row, int ch) { return row * GBK + ((ch ^ (row & 7)) << 3); }

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ Bm, int ldb, int M,
    int N_valid, int N_store, int K, uint16_t* __restrict__ C, int ldc, float* __restrict__ part,
    const float* __restrict__ Eptr) {
  constexpr int WM = GBM / 2, WN = GBN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int ACH = GBM * 8 / 256, BCH = GBN * 8 / 256;   // 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t As[2][GBM * GBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][GBN * GBK];

  const int tiles_m = (M + GBM - 1) / GBM, tiles_n = (N_store + GBN - 1) / GBN;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * GBM, n0 = tn * GBN;
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int h = l >> 5, ln = l & 31;

  u32x4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
      const int id = t + 256 * q, row = id >> 3, ch = id & 7;
      const int gm = m0 + row, gk = k0 + ch * 8;
      ra[q] = (gm < M && gk < K) ? *reinterpret_cast<const u32x4*>(A + (size_t)gm * lda + gk)
                                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < BCH; ++q) {
      const int id = t + 256 * q, row = id >> 3, ch = id & 7;
      const int gn = n0 + row, gk = k0 + ch * 8;
      rb[q] = (gn < N_valid && gk < K) ? *reinterpret_cast<const u32x4*>(Bm + (size_t)gn * ldb + gk)
                                       : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
      const int id = t + 256 * q, row = id >> 3, ch = id & 7;
      *reinterpret_cast<u32x4*>(&As[buf][swz(row, ch)]) = ra[q];
    }
#pragma unroll
    for (int q = 0; q < BCH; ++q) {
      const int id = t + 256 * q, row = id >> 3, ch = id & 7;
      *reinterpret_cast<u32x4*>(&Bs[buf][swz(row, ch)]) = rb[q];
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

  // rows of this lane's fragments inside the LDS tiles
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * WM + i * 32 + ln;
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = wn * WN + j * 32 + remap_row(ln);

  const int nk = (K + GBK - 1) / GBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GBK);
#pragma unroll
    for (int p = 0; p < GBK / 16; ++p) {
      u32x4 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const u32x4*>(&As[cur][swz(arow[i], 2 * p + h)]);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const u32x4*>(&Bs[cur][swz(brow[j], 2 * p + h)]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(fb[j], fa[i], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane (h, ln) of block (i, j) holds row m0 + wm*WM + 32i + ln,
  // columns n0 + wn*WN + 32j + 16h + r, r < 16.
  float scale = 1.f;
  if (EPI == EPI_DD) {
    const float E = *Eptr;
    scale = (E > 0.f) ? -1.f / E : 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WM + 32 * i + ln;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nb = n0 + wn * WN + 32 * j + 16 * h;
      const floatx16 a = acc[i][j];
      if (EPI == EPI_ERR) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ss += a[r] * a[r];
      }
      if (m < M && nb < N_store) {
        u32x4* dst = reinterpret_cast<u32x4*>(C + (size_t)m * ldc + nb);
        dst[0] = u32x4{pack2(a[0] * scale, a[1] * scale), pack2(a[2] * scale, a[3] * scale),
                       pack2(a[4] * scale, a[5] * scale), pack2(a[6] * scale, a[7] * scale)};
        dst[1] = u32x4{pack2(a[8] * scale, a[9] * scale), pack2(a[10] * scale, a[11] * scale),
                       pack2(a[12] * scale, a[13] * scale), pack2(a[14] * scale, a[15] * scale)};
      }
    }
  }
  if (EPI == EPI_ERR) {
    __shared__ float wsum[4];
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) ss += shfl_xor(ss, x);
    if (l == 0) wsum[w] = ss;
    __syncthreads();
    if (t == 0) part[blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  }
}

// ---- fp32 VALU GEMM ------------------------------------------------------------
// 64 x 64 tiles, 16 x 16 threads, 4 x 4 outputs per thread, K step 16.
// B_NN = 0: B is [N][K] (ldb); B_NN = 1: B is [K][N] (ldb).
template <int EPI, int B_NN>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda,
                                                       const float* __restrict__ Bm, int ldb, int M,
                                                       int N_valid, int N_store, int K,
                                                       float* __restrict__ C, int ldc,
                                                       float* __restrict__ part,
                                                       const float* __restrict__ Eptr) {
  __shared__ float as[16][64 + 1];
  __shared__ float bs[16][64 + 1];
  const int tiles_n = (N_store + 63) / 64;
  const int m0 = (blockIdx.x / tiles_n) * 64, n0 = (blockIdx.x % tiles_n) * 64;
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = t; e < 16 * 64; e += 256) {
      const int kk = e & 15, r = e >> 4;
      const int gm = m0 + r, gk = k0 + kk;
      as[kk][r] = (gm < M && gk < K) ? A[(size_t)gm * lda + gk] : 0.f;
      const int gn = n0 + r;
      float bv = 0.f;
      if (gn < N_valid && gk < K) bv = B_NN ? Bm[(size_t)gk * ldb + gn] : Bm[(size_t)gn * ldb + gk];
      bs[kk][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(as[kk][ty * 4 + a], bs[kk][tx * 4 + c], acc[a][c]);
    __syncthreads();
  }
  float scale = 1.f;
  if (EPI == EPI_DD) {
    const float E = *Eptr;
    scale = (E > 0.f) ? -1.f / E : 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int m = m0 + ty * 4 + a, n = n0 + tx * 4 + c;
      if (EPI == EPI_ERR) ss += acc[a][c] * acc[a][c];
      if (m < M && n < N_store) C[(size_t)m * ldc + n] = acc[a][c] * scale;
    }
  if (EPI == EPI_ERR) {
    __shared__ float wsum[4];
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) ss += shfl_xor(ss, x);
    if ((t & 63) == 0) wsum[t >> 6] = ss;
    __syncthreads();
    if (t == 0) part[blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  }
}

// E = sqrt(sum of partials), summed in a fixed order by one workgroup.
__global__ __launch_bounds__(256) void error_finalize_kernel(const float* __restrict__ part, int n,
                                                             float* __restrict__ E_ws,
                                                             float* __restrict__ err) {
  __shared__ float red[256];
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k >= 1; k >>= 1) {
    if ((int)threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float E = sqrtf(red[0]);
    if (E_ws) *E_ws = E;
    if (err) *err = E;
  }
}

// ---- launchers -------------------------------------------------------------------
int gemm_error_parts(int M, int N, int bf16) {
  if (bf16) return ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
  return ((M + 63) / 64) * ((N + 63) / 64);
}

hipError_t launch_gemm_error_bf16(const uint16_t* A, int lda, const uint16_t* Bm, int ldb, int M,
                                  int N_valid, int N_store, int K, uint16_t* C, int ldc,
                                  float* part, hipStream_t s) {
  const int G = gemm_error_parts(M, N_store, 1);
  gemm_bf16_kernel<EPI_ERR><<<G, 256, 0, s>>>(A, lda, Bm, ldb, M, N_valid, N_store, K, C, ldc, part, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_dd_bf16(const uint16_t* A, int lda, const uint16_t* Bm, int ldb, int M,
                               int N, int K, const float* E, uint16_t* C, int ldc, hipStream_t s) {
  const int G = gemm_error_parts(M, N, 1);
  gemm_bf16_kernel<EPI_DD><<<G, 256, 0, s>>>(A, lda, Bm, ldb, M, N, N, K, C, ldc, nullptr, E);
  return hipGetLastError();
}

hipError_t launch_gemm_error_f32(const float* A, int lda, const float* Bm, int ldb, int M,
                                 int N_valid, int N_store, int K, float* C, int ldc, float* part,
                                 hipStream_t s) {
  const int G = gemm_error_parts(M, N_store, 0);
  gemm_f32_kernel<EPI_ERR, 0><<<G, 256, 0, s>>>(A, lda, Bm, ldb, M, N_valid, N_store, K, C, ldc, part, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_dd_f32(const float* R, int ldr, const float* X, int ldx, int M, int N,
                              int K, const float* E, float* C, int ldc, hipStream_t s) {
  const int G = gemm_error_parts(M, N, 0);
  gemm_f32_kernel<EPI_DD, 1><<<G, 256, 0, s>>>(R, ldr, X, ldx, M, N, N, K, C, ldc, nullptr, E);
  return hipGetLastError();
}

hipError_t launch_error_finalize(const float* part, int nparts, float* E_ws, float* err,
                                 hipStream_t s) {
  error_finalize_kernel<<<1, 256, 0, s>>>(part, nparts, E_ws, err);
  return hipGetLastError();
}

}  // namespace lcp
