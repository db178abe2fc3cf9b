// Block adjoint of the LCP forward with the mask held constant.
//
// Forward (per block b): W_hat_b = W_b P_b, A_b = W_hat_b . M_b,
// W_tilde_b = A_b P_b^T. Given G = dE/dW_tilde (= -dE/dD), the chain rule gives
//   dE/dP_b = G_b^T A_b + W_b^T ((G_b P_b) . M_b),
// a sum over the Cout rows. Each workgroup reduces one block over one chunk of
// rows and writes that partial B x B matrix; the Sinkhorn adjoint kernel adds
// the chunk partials in chunk order (deterministic, no atomics).
//
// bf16 kernel: 4 waves; wave w takes the 32-wide column block t = w % (B/32)
// of the permuted positions and the 32-row sub-tile w / (B/32). Per sub-tile it
//   1. forms W_hat[i][k] and Y[i][k] = (G P_b)[i][k] for its 32 positions k
//      with MFMA (A operand: W or G rows from LDS, row-remapped so that a lane
//      ends up holding 16 consecutive rows i of one position k; B operand:
//      P_b fragments prepared in LDS),
//   2. applies the mask bits, rounds A = W_hat . M and Y . M to bf16,
//   3. accumulates dP^T[k][j] += sum_i A[i][k] G[i][j] + (Y . M)[i][k] W[i][j]
//      with MFMA, the rows i in the K slots (the lane's 16 rows are exactly
//      the K slots it supplies) and G / W columns read from the LDS tiles.
// Waves sharing t add their accumulators through LDS in a fixed order.
#include "common.h"
#include "kernels.h"

namespace lcp {

template <int B>
struct AdjGeom {
  static constexpr int KS = B / 16;
  static constexpr int TT = B / 32;
  static constexpr int RS = 4 / TT;             // 32-row sub-tiles per workgroup tile
  static constexpr int ROWS = 32 * RS;          // rows per workgroup tile
  static constexpr int LDT = B + 8;             // padded LDS row (uint16)
  static constexpr int FRAG = TT * KS * 64;     // u32x4 entries of the P fragments
};

template <int B>
__global__ __launch_bounds__(256) void adjoint_bf16_kernel(const uint16_t* __restrict__ G,
                                                           const uint16_t* __restrict__ W,
                                                           const float* __restrict__ P,
                                                           const uint32_t* __restrict__ bits,
                                                           int cout, int cin, int chunk_rows,
                                                           float* __restrict__ part) {
  using Gm = AdjGeom<B>;
  constexpr int KS = Gm::KS, TT = Gm::TT, RS = Gm::RS, ROWS = Gm::ROWS, LDT = Gm::LDT;
  __shared__ __attribute__((aligned(16))) uint16_t fb[Gm::FRAG * 8];
  // W and G tiles; after the row loop the same space holds the cross-wave sums
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2 * ROWS * LDT];
  static_assert((RS - 1) * TT * TT * 16 * 64 * 4 <= 2 * ROWS * LDT * 2, "combine buffer");
  uint16_t* tw = tiles;
  uint16_t* tg = tiles + ROWS * LDT;

  const int b = blockIdx.x, chunk = blockIdx.y;
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int h = l >> 5, n = l & 31;
  const int tb = w % TT, rs = w / TT;
  const int words = cin >> 5;

  // P fragments: fb[(t*KS + p)*64 + lane][e] = P_b[16p + 8h + e][32t + n]
  {
    const float* src = P + (size_t)b * B * B;
    for (int e_idx = t; e_idx < B * B; e_idx += 256) {
      const int j = e_idx / B, k = e_idx % B;
      const int tt = k >> 5, nn = k & 31, p = j >> 4, hh = (j >> 3) & 1, e = j & 7;
      fb[(((tt * KS + p) * 64) + 32 * hh + nn) * 8 + e] = (uint16_t)f2bf(src[e_idx]);
    }
  }

  floatx16 acc[TT];
#pragma unroll
  for (int q = 0; q < TT; ++q) acc[q] = floatx16{};

  const int r0 = chunk * chunk_rows;
  const int r1 = min(cout, r0 + chunk_rows);
  const u32x4* F = reinterpret_cast<const u32x4*>(fb);
  for (int i0 = r0; i0 < r1; i0 += ROWS) {
    __syncthreads();  // previous tile fully consumed (and fragments written)
    // cooperative load of ROWS x B of W and G (16-byte chunks)
    for (int id = t; id < ROWS * (B / 8); id += 256) {
      const int row = id / (B / 8), ch = id % (B / 8);
      const int gi = i0 + row;
      u32x4 vw = {0u, 0u, 0u, 0u}, vg = {0u, 0u, 0u, 0u};
      if (gi < r1) {
        const size_t o = (size_t)gi * cin + b * B + ch * 8;
        vw = *reinterpret_cast<const u32x4*>(W + o);
        vg = *reinterpret_cast<const u32x4*>(G + o);
      }
      *reinterpret_cast<u32x4*>(&tw[row * LDT + ch * 8]) = vw;
      *reinterpret_cast<u32x4*>(&tg[row * LDT + ch * 8]) = vg;
    }
    __syncthreads();

    // 1. W_hat and Y for positions 32*tb + n, rows 32*rs + 16h + r
    const int arow = 32 * rs + remap_row(n);
    floatx16 wh = {}, yy = {};
#pragma unroll
    for (int p = 0; p < KS; ++p) {
      const u32x4 fw = *reinterpret_cast<const u32x4*>(&tw[arow * LDT + 16 * p + 8 * h]);
      const u32x4 fg = *reinterpret_cast<const u32x4*>(&tg[arow * LDT + 16 * p + 8 * h]);
      const u32x4 fp = F[(tb * KS + p) * 64 + l];
      wh = mfma32(fw, fp, wh);
      yy = mfma32(fg, fp, yy);
    }
    // 2. mask (bit n of word (row, 32*b*B/32 + tb)), round to bf16
    u32x4 aop[2], yop[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float av[8], yv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int gi = i0 + 32 * rs + 16 * h + 8 * u + e;
        uint32_t keep = 0;
        if (gi < r1) keep = (bits[(size_t)gi * words + ((b * B) >> 5) + tb] >> n) & 1u;
        av[e] = keep ? wh[8 * u + e] : 0.f;
        yv[e] = keep ? yy[8 * u + e] : 0.f;
      }
      aop[u] = u32x4{pack2(av[0], av[1]), pack2(av[2], av[3]), pack2(av[4], av[5]), pack2(av[6], av[7])};
      yop[u] = u32x4{pack2(yv[0], yv[1]), pack2(yv[2], yv[3]), pack2(yv[4], yv[5]), pack2(yv[6], yv[7])};
    }
    // 3. dP^T[k][j] += sum_i A[i][k] G[i][j] + Ym[i][k] W[i][j]
#pragma unroll
    for (int t2 = 0; t2 < TT; ++t2) {
      const int col = 32 * t2 + n;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rb = 32 * rs + 16 * h + 8 * u;
        uint32_t g4[4], w4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          g4[q] = tg[(rb + 2 * q) * LDT + col] | ((uint32_t)tg[(rb + 2 * q + 1) * LDT + col] << 16);
          w4[q] = tw[(rb + 2 * q) * LDT + col] | ((uint32_t)tw[(rb + 2 * q + 1) * LDT + col] << 16);
        }
        acc[t2] = mfma32(aop[u], u32x4{g4[0], g4[1], g4[2], g4[3]}, acc[t2]);
        acc[t2] = mfma32(yop[u], u32x4{w4[0], w4[1], w4[2], w4[3]}, acc[t2]);
      }
    }
  }
  __syncthreads();

  // combine the RS waves that share tb (fixed order), then store:
  // lane (h, n) of block t2 holds dP^T[k = 32tb + 8(r/4) + 4h + r%4][j = 32t2 + n]
  float* red = reinterpret_cast<float*>(tiles);   // (RS-1) * TT * TT * 16 * 64 floats
  if (RS > 1 && rs > 0) {
#pragma unroll
    for (int t2 = 0; t2 < TT; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        red[((((rs - 1) * TT + tb) * TT + t2) * 16 + r) * 64 + l] = acc[t2][r];
  }
  __syncthreads();
  if (rs == 0) {
    for (int s = 1; s < RS; ++s)
#pragma unroll
      for (int t2 = 0; t2 < TT; ++t2)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t2][r] += red[((((s - 1) * TT + tb) * TT + t2) * 16 + r) * 64 + l];
    float* dst = part + ((size_t)chunk * (cin / B) + b) * B * B;
#pragma unroll
    for (int t2 = 0; t2 < TT; ++t2) {
      const int j = 32 * t2 + n;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = 32 * tb + 8 * q + 4 * h;
        *reinterpret_cast<floatx4*>(dst + j * B + k) =
            floatx4{acc[t2][4 * q], acc[t2][4 * q + 1], acc[t2][4 * q + 2], acc[t2][4 * q + 3]};
      }
    }
  }
}

// fp32 VALU version: one thread per (j, k) group of outputs, rows streamed
// through LDS one at a time.
template <int B>
__global__ __launch_bounds__(256) void adjoint_f32_kernel(const float* __restrict__ G,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ P,
                                                          const uint32_t* __restrict__ bits,
                                                          int cout, int cin, int chunk_rows,
                                                          float* __restrict__ part) {
  constexpr int PER = (B * B + 255) / 256;
  __shared__ float pb[B][B + 1];
  __shared__ float wr[B], gr[B], am[B], ym[B];
  const int b = blockIdx.x, chunk = blockIdx.y, t = threadIdx.x;
  const float* src = P + (size_t)b * B * B;
  for (int e = t; e < B * B; e += 256) pb[e / B][e % B] = src[e];
  float acc[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) acc[q] = 0.f;
  const int r0 = chunk * chunk_rows, r1 = min(cout, r0 + chunk_rows);
  const int words = cin >> 5;
  for (int i = r0; i < r1; ++i) {
    __syncthreads();
    if (t < B) {
      wr[t] = W[(size_t)i * cin + b * B + t];
      gr[t] = G[(size_t)i * cin + b * B + t];
    }
    __syncthreads();
    if (t < B) {
      float s1 = 0.f, s2 = 0.f;
      for (int j = 0; j < B; ++j) {
        s1 = fmaf(wr[j], pb[j][t], s1);
        s2 = fmaf(gr[j], pb[j][t], s2);
      }
      const uint32_t keep = (bits[(size_t)i * words + ((b * B + t) >> 5)] >> (t & 31)) & 1u;
      am[t] = keep ? s1 : 0.f;
      ym[t] = keep ? s2 : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = t + 256 * q;
      if (e < B * B) {
        const int j = e / B, k = e % B;
        acc[q] = fmaf(gr[j], am[k], fmaf(wr[j], ym[k], acc[q]));
      }
    }
  }
  float* dst = part + ((size_t)chunk * (cin / B) + b) * B * B;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int e = t + 256 * q;
    if (e < B * B) dst[e] = acc[q];
  }
}

int adjoint_chunks(int cout, int nb, int B) {
  int chunks = (1024 + nb - 1) / nb;
  const int rows_tile = 32 * (4 / (B / 32));
  const int max_chunks = (cout + rows_tile - 1) / rows_tile;
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  return chunks;
}

static int adjoint_chunk_rows(int cout, int chunks, int B) {
  const int rows_tile = 32 * (4 / (B / 32));
  int cr = (cout + chunks - 1) / chunks;
  return (cr + rows_tile - 1) / rows_tile * rows_tile;
}

hipError_t launch_adjoint_bf16(const uint16_t* G, const uint16_t* W, const float* P,
                               const uint32_t* bits, int cout, int cin, int B, int chunks,
                               float* part, hipStream_t s) {
  const int cr = adjoint_chunk_rows(cout, chunks, B);
  dim3 grid(cin / B, chunks);
  switch (B) {
    case 32: adjoint_bf16_kernel<32><<<grid, 256, 0, s>>>(G, W, P, bits, cout, cin, cr, part); break;
    case 64: adjoint_bf16_kernel<64><<<grid, 256, 0, s>>>(G, W, P, bits, cout, cin, cr, part); break;
    case 128: adjoint_bf16_kernel<128><<<grid, 256, 0, s>>>(G, W, P, bits, cout, cin, cr, part); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_adjoint_f32(const float* G, const float* W, const float* P,
                              const uint32_t* bits, int cout, int cin, int B, int chunks,
                              float* part, hipStream_t s) {
  const int cr = adjoint_chunk_rows(cout, chunks, B);
  dim3 grid(cin / B, chunks);
  switch (B) {
    case 32: adjoint_f32_kernel<32><<<grid, 256, 0, s>>>(G, W, P, bits, cout, cin, cr, part); break;
    case 64: adjoint_f32_kernel<64><<<grid, 256, 0, s>>>(G, W, P, bits, cout, cin, cr, part); break;
    case 128: adjoint_f32_kernel<128><<<grid, 256, 0, s>>>(G, W, P, bits, cout, cin, cr, part); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lcp
