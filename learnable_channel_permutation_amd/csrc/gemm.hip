// GEMMs of the LCP step: the output error R = D X^T (E = ||R||_F) and the
// backward product G = dL/dW_tilde = c A X (A = R with c = -1/E for the
// Frobenius objective, A = dL/dY~ with c = 1 for the cosine objective), both
// written as C[m][n] = sum_k A[m][k] B[n][k] with A and B row-major and K
// contiguous (the backward reads X transposed, prepared once per layer).
//
// bf16 kernels (gfx950): BM x BN x 64 tiles, 8 waves (two per SIMD) in a
// 4 x 2 layout, each wave owning (BM/4) x (BN/2) of the tile as MFMA blocks
// with fp32 accumulators. Operand tiles move global -> LDS with 16-byte
// direct-to-LDS loads (no register staging) into a ring of stages. Chunk c
// of row r is stored at position c ^ ((r >> 1) & 7): the 16-byte fragment
// reads of 16 consecutive rows then cover all 64 LDS banks. The MFMA A
// operand is taken from the B matrix, so each lane ends up holding
// consecutive output columns of one output row. Workgroups are ordered so
// that each XCD (workgroup id mod 8) works on a compact group of 4 row panels
// x N column panels, which keeps the panels shared inside that XCD's L2.
// Operands are loaded through buffer resources with per-lane offsets fixed
// per tile (a K step moves only the scalar offset). Out-of-range A rows are
// read from a clamped row (their outputs are never stored); out-of-range K
// chunks and B rows of the error product read zeros (offsets past the
// resource), so padded output columns come out exactly zero.
//  * gemm_dd_kernel (the backward product): a two-stage ring on 32x32x16
//    MFMAs, one barrier per K step after which the next tile's loads go out
//    one at a time between the MFMAs of the first sub-steps; each 16-wide
//    sub-step reads the next one's fragments before its MFMAs.
//  * gemm_err_kernel (the error product): a software-pipelined three-stage
//    ring on 16x16x32 MFMAs, described at the kernel.
//  * gemm_dd_kernel<..., ADJ = true>: the same backward product with the
//    block adjoint of the LCP forward (B = 64) taken from the accumulators in
//    the epilogue instead of storing G (dd_adjoint_epilogue).
//
// Epilogues: ERR stores C in bf16 and one sum of squares of the fp32
// accumulators per workgroup (reduced later in a fixed order); ERRCOS also
// writes one sum of Y . C per workgroup, Y a matrix of C's layout (the dense
// layer outputs of the cosine objective); DD scales by a factor read from
// device memory (written by the finalisation kernel) and stores bf16.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lcp {

enum { EPI_ERR = 0, EPI_DD = 1, EPI_ERRCOS = 2 };

constexpr int GBK = 64;
constexpr int GROUP_M = 4;
constexpr int GWM = 4, GWN = 2, GNW = GWM * GWN, GNT = 64 * GNW;   // wave layout, threads

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Operand loads go through buffer resources: the per-lane byte offset of each
// load is computed once per tile, and a K step only changes the scalar
// offset, so issuing a load costs no vector instruction. An offset at or past
// the resource's size reads zeros (used for rows past the matrix and the K
// tail). Word 3: 32-bit data format, the only format field raw loads need.
constexpr uint32_t kOOB = 0x80000000u;                     // an offset past every operand
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const uint16_t* p, size_t elems) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, (int)(uint32_t)(elems * 2),
                                           0x00020000);
}
// 16 bytes at byte offset voff + soff of r into LDS at ldst + 16 * lane
__device__ __forceinline__ void load16_lds(__amdgpu_buffer_rsrc_t r, uint16_t* ldst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)ldst, 16, (int)voff, (int)soff, 0, 0);
}

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

__device__ __forceinline__ int swz(int row, int ch) { return row * GBK + ((ch ^ ((row >> 1) & 7)) << 3); }

template <int BM, int BN, int S>
constexpr size_t gemm_lds_bytes() { return (size_t)S * (BM + BN) * GBK * 2; }

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited on)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Fused block adjoint of the dD GEMM (ADJ, B = 64): arguments of the epilogue.
struct DdAdj {
  const uint16_t* W;     // [M][N] bf16, the layer weights
  const u32x4* frag;     // [nb][FB entries] adjoint P fragments (frag.h)
  const uint32_t* bits;  // [nb][M][2] mask words, block-major
  float* part;           // [tiles_m][nb][64][64] partial dL/dP_b (row panel sums)
  int nb;
};
constexpr int ADJ_B = 64, ADJ_FRAG = (ADJ_B / 32) * (ADJ_B / 16) * 64;   // u32x4 entries per block


// Identity as an MFMA B operand for K step v of a 32-column group whose K
// slot (h, e) stands for column 16h + 8v + e: slot e of lane (h, n) is 1 when
// that column is n.
__device__ __forceinline__ u32x4 dd_identity(int v, int h, int n) {
  uint32_t r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e0 = 16 * h + 8 * v + 2 * q;
    r[q] = (e0 == n ? 0x3f80u : 0u) | ((e0 + 1 == n ? 0x3f80u : 0u) << 16);
  }
  return u32x4{r[0], r[1], r[2], r[3]};
}

// Block adjoint from the dD accumulators (256 x 256 tile, B = 64). Wave
// (wm, wn) holds G for rows m0 + 64wm + [0, 64) and the two whole blocks of
// columns n0 + 128wn + [0, 128): lane (h, ln) of accumulator (i, j) has row
// 32i + ln, columns 32j + 16h + r. Packed to bf16 (the values the unfused
// path stores), eight of them are exactly the K slots of one MFMA A operand
// whose slot (h, e) is column 32j + 16h + 8v + e: the channel order of the
// adjoint fragments (frag.h), so G P_b needs no data movement. W is loaded in
// the same layout. Per block and 32-row group:
//   W_hat = W P_b, Y = G P_b (MFMA), masked -> A = W_hat . M, Y . M in bf16,
//   G and W transposed per 32-column group by an MFMA against the identity,
//   dP^T[k][j] += sum_i A[i][k] G[i][j] + (Y . M)[i][k] W[i][j].
// The four row waves of a block are summed through LDS in wave order, and
// the tile writes one partial per (row panel, block), which the Sinkhorn
// adjoint adds in panel order. Rows past M contribute nothing (G zeroed, W
// and the mask read as zeros).
__device__ __forceinline__ void dd_adjoint_epilogue(floatx16 (&acc)[2][4], float scale, uint16_t* lds,
                                                    const uint16_t* frag_lds, const DdAdj& adj, int M, int m0,
                                                    int n0, int tm, int w, int l) {
  const int wm = w / GWN, wn = w % GWN, h = l >> 5, ln = l & 31;
  // G operands gA[i][j][v]: columns 32j + 16h + 8v + e of the wave's 128
  u32x4 gA[2][4][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const bool rv = m0 + 64 * wm + 32 * i + ln < M;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const floatx16& a = acc[i][j];
        uint32_t q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          q[e] = rv ? pack2(a[8 * v + 2 * e] * scale, a[8 * v + 2 * e + 1] * scale) : 0u;
        gA[i][j][v] = u32x4{q[0], q[1], q[2], q[3]};
      }
  }
  __syncthreads();                                         // the ring is no longer read
  // mask words of the wave's two blocks and 64 rows: [jb][row][2] in LDS
  uint32_t* mw = reinterpret_cast<uint32_t*>(lds) + w * 256;
  float* red = reinterpret_cast<float*>(lds) + 8 * 256;    // [wn][wm - 1][a, o][16][64]
  const int bw0 = n0 / ADJ_B + 2 * wn;                     // first block of this wave
  {
    const int jb = l >> 5, c = l & 31;
    const size_t rows = (size_t)adj.nb * M;                // words in bits: rows * 2
    const size_t wi = ((size_t)(bw0 + jb) * M + m0 + 64 * wm) * 2 + 4 * c;
    // one 8-byte load per row (a row's two words are 8-byte aligned, four of
    // them need not be 16); rows past the array read zeros
    uint2 v0 = uint2{0u, 0u}, v1 = uint2{0u, 0u};
    if (wi + 2 <= rows * 2) v0 = *reinterpret_cast<const uint2*>(adj.bits + wi);
    if (wi + 4 <= rows * 2) v1 = *reinterpret_cast<const uint2*>(adj.bits + wi + 2);
    *reinterpret_cast<u32x4*>(mw + jb * 128 + 4 * c) = u32x4{v0.x, v0.y, v1.x, v1.y};
  }
  const u32x4* F0 = reinterpret_cast<const u32x4*>(frag_lds);
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int bidx = bw0 + jb;
    const bool bvalid = bidx < adj.nb;                     // uniform over the wave
    floatx16 cacc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int o = 0; o < 2; ++o) cacc[a][o] = floatx16{};
    if (bvalid) {
      const u32x4* F = F0 + (2 * wn + jb) * ADJ_FRAG;      // [a][p][lane]
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = m0 + 64 * wm + 32 * i + ln;
        u32x4 wA[2][2];
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
          for (int v = 0; v < 2; ++v)
            wA[o][v] = row < M ? *reinterpret_cast<const u32x4*>(adj.W + (size_t)row * (adj.nb * ADJ_B) + bidx * ADJ_B +
                                                                 32 * o + 16 * h + 8 * v)
                               : u32x4{0u, 0u, 0u, 0u};
        // keep bits: bit r of km[a] for accumulator element r, row 32i + 8(r/4) + 4h + r%4, position 32a + ln
        uint32_t km[2] = {0u, 0u};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4* src = reinterpret_cast<const u32x4*>(mw + jb * 128 + (32 * i + 8 * q + 4 * h) * 2);
          const u32x4 x0 = src[0], x1 = src[1];            // rows +0, +1 | +2, +3, words (t = 0, 1)
          const uint32_t wd[4][2] = {{x0.x, x0.y}, {x0.z, x0.w}, {x1.x, x1.y}, {x1.z, x1.w}};
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int a = 0; a < 2; ++a) km[a] |= ((wd[b][a] >> ln) & 1u) << (4 * q + b);
        }
        u32x4 aop[2][2], yop[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          floatx16 wh = {}, yy = {};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const u32x4 fp = F[(a * 4 + p) * 64 + l];
            wh = mfma32(wA[p >> 1][p & 1], fp, wh);
            yy = mfma32(gA[i][2 * jb + (p >> 1)][p & 1], fp, yy);
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            float av[8], yv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const bool keep = (km[a] >> (8 * u + e)) & 1u;
              av[e] = keep ? wh[8 * u + e] : 0.f;
              yv[e] = keep ? yy[8 * u + e] : 0.f;
            }
            aop[a][u] = u32x4{pack2(av[0], av[1]), pack2(av[2], av[3]), pack2(av[4], av[5]), pack2(av[6], av[7])};
            yop[a][u] = u32x4{pack2(yv[0], yv[1]), pack2(yv[2], yv[3]), pack2(yv[4], yv[5]), pack2(yv[6], yv[7])};
          }
        }
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          floatx16 tg = {}, tw = {};
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const u32x4 id = dd_identity(v, h, ln);
            tg = mfma32(gA[i][2 * jb + o][v], id, tg);
            tw = mfma32(wA[o][v], id, tw);
          }
          u32x4 gT[2], wT[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            gT[u] = u32x4{pack2_exact(tg[8 * u], tg[8 * u + 1]), pack2_exact(tg[8 * u + 2], tg[8 * u + 3]),
                          pack2_exact(tg[8 * u + 4], tg[8 * u + 5]), pack2_exact(tg[8 * u + 6], tg[8 * u + 7])};
            wT[u] = u32x4{pack2_exact(tw[8 * u], tw[8 * u + 1]), pack2_exact(tw[8 * u + 2], tw[8 * u + 3]),
                          pack2_exact(tw[8 * u + 4], tw[8 * u + 5]), pack2_exact(tw[8 * u + 6], tw[8 * u + 7])};
          }
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              cacc[a][o] = mfma32(aop[a][u], gT[u], cacc[a][o]);
              cacc[a][o] = mfma32(yop[a][u], wT[u], cacc[a][o]);
            }
        }
      }
    }
    // the four row waves of this block, summed in wave order through LDS
    __syncthreads();                                       // red of the previous block consumed
    if (wm > 0) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((((wn * 3 + wm - 1) * 4 + 2 * a + o) * 16) + r) * 64 + l] = cacc[a][o][r];
    }
    __syncthreads();
    if (wm == 0 && bvalid) {
#pragma unroll
      for (int s2 = 0; s2 < 3; ++s2)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int o = 0; o < 2; ++o)
#pragma unroll
            for (int r = 0; r < 16; ++r) cacc[a][o][r] += red[((((wn * 3 + s2) * 4 + 2 * a + o) * 16) + r) * 64 + l];
      // lane (h, ln) of (a, o) holds dP^T[k = 32a + 8(r/4) + 4h + r%4][j = 32o + ln]; stored as dP[j][k]
      float* dst = adj.part + ((size_t)tm * adj.nb + bidx) * (ADJ_B * ADJ_B);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          const int j = 32 * o + ln;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = 32 * a + 8 * q + 4 * h;
            *reinterpret_cast<floatx4*>(dst + j * ADJ_B + k) =
                floatx4{cacc[a][o][4 * q], cacc[a][o][4 * q + 1], cacc[a][o][4 * q + 2], cacc[a][o][4 * q + 3]};
          }
        }
    }
  }
}

// The backward product C = coef[1] * A B^T (bf16 out), or with ADJ the block
// adjoint of the LCP forward taken straight from the accumulators (C unused).
template <int BM, int BN, int S, int LSP, bool ADJ = false>
__global__ __launch_bounds__(GNT, 1) void gemm_dd_kernel(
    const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ Bm, int ldb, int M,
    int N_valid, int N_store, int K, uint16_t* __restrict__ C, int ldc, const float* __restrict__ Eptr,
    DdAdj adj) {
  constexpr int WM = BM / GWM, WN = BN / GWN, FM = WM / 32, FN = WN / 32;
  constexpr int AI = BM * 8 / GNT, BI = BN * 8 / GNT;     // 16-byte loads per thread per tile
  constexpr int STAGE = (BM + BN) * GBK;                   // bf16 elements per ring stage
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N_store + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int wm = w / GWN, wn = w % GWN;
  const int h = l >> 5, ln = l & 31;

  if constexpr (ADJ) {
    // the adjoint P fragments of the tile's four blocks (8 KB each, block-major)
    // go to LDS above the ring now; the main loop's first wait covers them.
    // Chunks of blocks past nb take the per-lane offset past the resource and
    // read zeros (those blocks are never used).
    static_assert(BN == 4 * ADJ_B && S == 2, "fused adjoint: four blocks of 64 per tile, two stages");
    const __amdgpu_buffer_rsrc_t rF = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(adj.frag), (short)0, (int)(uint32_t)((size_t)adj.nb * ADJ_FRAG * 16), 0x00020000);
    const int wq = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int chunk = q * GNW + wq;                      // 1 KB chunks 0 .. 31, 8 per block
      const uint32_t vo = (n0 / ADJ_B + chunk / 8 < adj.nb) ? (uint32_t)(l * 16) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rF, (lds_ptr_t)(lds + S * STAGE + chunk * 512), 16, (int)vo,
                                               (int)((uint32_t)(n0 / ADJ_B) * ADJ_FRAG * 16 + chunk * 1024), 0, 0);
    }
  }

  // load q (< AI: A rows, else B rows) of wave w fills the 64 consecutive
  // 16-byte chunks (q' * GNW + w) * 64 + lane of its matrix in the stage.
  // K is a multiple of GBK here (the transposed activations and the residual
  // are padded to 64 tokens), so no K tail; rows past M or N_valid read a
  // clamped row (those outputs are never stored). Each load's byte offset
  // from the matrix origin is computed once; a K step only moves the uniform
  // base, so the load takes the scalar-base + 32-bit-offset address form.
  constexpr int NL = AI + BI;                              // load instructions per tile
  const __amdgpu_buffer_rsrc_t rA = operand_rsrc(A, (size_t)M * lda), rB = operand_rsrc(Bm, (size_t)N_valid * ldb);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t voff[NL];
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int qq = q < AI ? q : q - AI;
    const int c = (qq * GNW + w) * 64 + l, row = c >> 3, ch = (c & 7) ^ ((row >> 1) & 7);
    if (q < AI) voff[q] = (uint32_t)(((size_t)min(m0 + row, M - 1) * lda + ch * 8) * 2);
    else voff[q] = (uint32_t)(((size_t)min(n0 + row, N_valid - 1) * ldb + ch * 8) * 2);
  }
  auto issue_one = [&](int stage, int k0, int q) {
    const int qq = q < AI ? q : q - AI;
    uint16_t* dst = lds + stage * STAGE + (q < AI ? 0 : BM * GBK) + (qq * GNW + wu) * 64 * 8;
    load16_lds(q < AI ? rA : rB, dst, voff[q], (uint32_t)k0 * 2);
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * WM + i * 32 + ln;
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = wn * WN + j * 32 + remap_row(ln);

  // multiply the tile in `stage`; with `load` the tile at k0 goes to stage
  // `lstage`, one load between consecutive MFMAs of the first LSP sub-steps
  constexpr int NP = GBK / 16, NM = FM * FN, SLOTS = LSP * NM;
  auto compute = [&](int stage, int lstage, int k0, auto LOAD) {
    const uint16_t* As = lds + stage * STAGE;
    const uint16_t* Bs = As + BM * GBK;
    u32x4 fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = *reinterpret_cast<const u32x4*>(&As[swz(arow[i], h)]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = *reinterpret_cast<const u32x4*>(&Bs[swz(brow[j], h)]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int c = p & 1;
      __builtin_amdgcn_sched_barrier(0);
      if (p + 1 < NP) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[c ^ 1][i] = *reinterpret_cast<const u32x4*>(&As[swz(arow[i], 2 * (p + 1) + h)]);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[c ^ 1][j] = *reinterpret_cast<const u32x4*>(&Bs[swz(brow[j], 2 * (p + 1) + h)]);
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int o = 0; o < NL; ++o)
          if (decltype(LOAD)::value && p < LSP && o * SLOTS / NL == p * NM + m) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(lstage, k0, o);
            __builtin_amdgcn_sched_barrier(0);
          }
        const int i = m / FN, j = m % FN;
        acc[i][j] = mfma32(fb[c][j], fa[c][i], acc[i][j]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // two-stage ring: at step kt this thread waits for its loads of tile kt,
  // the barrier makes every thread's part visible and guarantees that the
  // stage of tile kt - 1 is no longer read; tile kt + 1 then goes there while
  // tile kt is multiplied.
  static_assert(S == 2, "two stages");
  const int nk = (K + GBK - 1) / GBK;
#pragma unroll
  for (int q = 0; q < NL; ++q) issue_one(0, 0, q);
  for (int kt = 0; kt + 1 < nk; ++kt) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    compute(kt & 1, (kt + 1) & 1, (kt + 1) * GBK, std::true_type{});
  }
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  compute((nk - 1) & 1, 0, 0, std::false_type{});

  // ---- epilogue: lane (h, ln) of block (i, j) holds row m0 + wm*WM + 32i + ln,
  // columns n0 + wn*WN + 32j + 16h + r, r < 16.
  const float scale = Eptr[1];
  if constexpr (ADJ) {
    dd_adjoint_epilogue(acc, scale, lds, lds + S * STAGE, adj, M, m0, n0, tm, w, l);
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WM + 32 * i + ln;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nb = n0 + wn * WN + 32 * j + 16 * h;
      const floatx16 a = acc[i][j];
      if (m < M && nb < N_store) {   // rows past M were read from a clamped row
        u32x4* dst = reinterpret_cast<u32x4*>(C + (size_t)m * ldc + nb);
        dst[0] = u32x4{pack2(a[0] * scale, a[1] * scale), pack2(a[2] * scale, a[3] * scale),
                       pack2(a[4] * scale, a[5] * scale), pack2(a[6] * scale, a[7] * scale)};
        dst[1] = u32x4{pack2(a[8] * scale, a[9] * scale), pack2(a[10] * scale, a[11] * scale),
                       pack2(a[12] * scale, a[13] * scale), pack2(a[14] * scale, a[15] * scale)};
      }
    }
  }
}

// ---- error GEMM: software-pipelined ring ---------------------------------------
// 256 x 128 tiles, 8 waves (4 x 2, each 64 x 64), three-stage direct-to-LDS
// ring of 64-wide K steps. Two things keep the MFMA arrays fed:
//  * the loads of tile kt + 2 are not issued in one burst after the barrier
//    (which stalls every wave on the vector-memory queue at the same time)
//    but one at a time between the MFMAs of step kt;
//  * the step's barrier sits before its last 16-wide sub-step: the wave
//    waits for its own loads of tile kt + 1, meets the others, issues the
//    first fragment reads of tile kt + 1 and only then runs the last
//    sub-step's MFMAs, whose operands are already in registers. The barrier
//    and the LDS latency hide under those MFMAs.
// The barrier of step kt also retires stage kt - 1 (every wave has read its
// last fragments of it), which step kt + 1 refills with tile kt + 3.
// MF selects the MFMA: 32 (32x32x16, lane holds 16 consecutive columns of a
// row) or 16 (16x16x32, lane holds 4 consecutive columns of a row).
constexpr int RS = 3;   // ring stages

template <int EPI, int MF>
__global__ __launch_bounds__(GNT, 1) void gemm_err_kernel(
    const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ Bm, int ldb, int M,
    int N_valid, int N_store, int K, uint16_t* __restrict__ C, int ldc, float* __restrict__ part,
    const uint16_t* __restrict__ Yc, float* __restrict__ part2) {
  constexpr int BM = 256, BN = 128;
  constexpr int WM = BM / GWM, WN = BN / GWN;
  constexpr int FM = WM / MF, FN = WN / MF, NM = FM * FN;
  constexpr int KS = MF == 32 ? 16 : 32;                   // K per MFMA
  constexpr int P = GBK / KS;                              // sub-steps per K step
  constexpr int AI = BM * 8 / GNT, BI = BN * 8 / GNT, NL = AI + BI;
  constexpr int STAGE = (BM + BN) * GBK;
  static_assert(P % 2 == 0, "fragment double buffer alternates within a step");
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N_store + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int wm = w / GWN, wn = w % GWN;
  // fragment lane roles: MF 32: K half h, row ln; MF 16: K quarter q, row l16
  const int kq = MF == 32 ? (l >> 5) : (l >> 4);
  const int lr = MF == 32 ? (l & 31) : (l & 15);

  // load q of this thread for the tile at k0 into stage `stage`. Rows past M
  // read a clamped row (never stored); B rows past N_valid read zeros, so the
  // padded output columns are exactly zero. In a step whose K chunks reach
  // past K (the last one when K % 64 != 0) those chunks read zeros too.
  const __amdgpu_buffer_rsrc_t rA = operand_rsrc(A, (size_t)M * lda), rB = operand_rsrc(Bm, (size_t)N_valid * ldb);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t voff[NL];
  int kch[NL];                                             // K element offset of each load's chunk
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int qq = q < AI ? q : q - AI;
    const int c = (qq * GNW + w) * 64 + l, row = c >> 3, ch = (c & 7) ^ ((row >> 1) & 7);
    kch[q] = ch * 8;
    if (q < AI) voff[q] = (uint32_t)(((size_t)min(m0 + row, M - 1) * lda + ch * 8) * 2);
    else voff[q] = (n0 + row < N_valid) ? (uint32_t)(((size_t)(n0 + row) * ldb + ch * 8) * 2) : kOOB;
  }
  // TAIL: the tile at k0 may be the last one (the main loop never loads it)
  auto issue_one = [&](int stage, int k0, int q, auto TAIL) {
    const int qq = q < AI ? q : q - AI;
    uint16_t* dst = lds + stage * STAGE + (q < AI ? 0 : BM * GBK) + (qq * GNW + wu) * 64 * 8;
    uint32_t vo = voff[q];
    if (decltype(TAIL)::value && k0 + GBK > K) vo = (k0 + kch[q] < K) ? vo : kOOB;
    load16_lds(q < AI ? rA : rB, dst, vo, (uint32_t)k0 * 2);
  };

  typedef typename std::conditional<MF == 32, floatx16, floatx4>::type acc_t;
  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = acc_t{};
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * WM + i * MF + lr;
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = wn * WN + j * MF + (MF == 32 ? remap_row(lr) : lr);

  u32x4 fa[2][FM], fb[2][FN];
  auto rd = [&](int stage, int p, int fs) {
    const uint16_t* As = lds + stage * STAGE;
    const uint16_t* Bs = As + BM * GBK;
    const int ch = (KS / 8) * p + kq;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[fs][i] = *reinterpret_cast<const u32x4*>(&As[swz(arow[i], ch)]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[fs][j] = *reinterpret_cast<const u32x4*>(&Bs[swz(brow[j], ch)]);
  };
  auto mma = [&](int fs, int m) {
    const int i = m / FN, j = m % FN;
    if constexpr (MF == 32) acc[i][j] = mfma32(fb[fs][j], fa[fs][i], acc[i][j]);
    else acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(fb[fs][j]), as_bf16x8(fa[fs][i]), acc[i][j], 0, 0, 0);
  };
  // step on stage `stage`: with LOAD the tile at k0 goes to stage `lstage`
  // between the MFMAs of sub-steps 0 .. P-2; with NEXT the first fragments of
  // stage `nstage` are read after the barrier. WAIT1: one tile's loads (the
  // ones just issued) may stay in flight at the barrier.
  auto step = [&](int stage, int lstage, int k0, int nstage, auto LOAD, auto NEXT, auto WAIT1, auto TAIL) {
    constexpr bool DL = decltype(LOAD)::value, DN = decltype(NEXT)::value;
    constexpr int SLOTS = (P - 1) * NM;
#pragma unroll
    for (int p = 0; p < P - 1; ++p) {
      __builtin_amdgcn_sched_barrier(0);
      rd(stage, p + 1, (p + 1) & 1);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int o = 0; o < (DL ? NL : 0); ++o)
          if (o * SLOTS / NL == p * NM + m) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(lstage, k0, o, TAIL);
            __builtin_amdgcn_sched_barrier(0);
          }
        mma(p & 1, m);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(WAIT1)::value) wait_vmcnt<NL>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DN) rd(nstage, 0, 0);
#pragma unroll
    for (int m = 0; m < NM; ++m) mma((P - 1) & 1, m);
    __builtin_amdgcn_sched_barrier(0);
  };
  typedef std::true_type Y_;
  typedef std::false_type N_;

  const int nk = (K + GBK - 1) / GBK;
  // tiles 0 and 1 (a tile past K reads zeros and is never multiplied)
#pragma unroll
  for (int q = 0; q < NL; ++q) issue_one(0, 0, q, Y_{});
#pragma unroll
  for (int q = 0; q < NL; ++q) issue_one(1, GBK, q, Y_{});
  wait_vmcnt<NL>();
  __builtin_amdgcn_s_barrier();
  rd(0, 0, 0);
  int kt = 0;
  for (; kt + 5 < nk; kt += 3) {                           // loads tiles kt + 2 .. kt + 4 < nk - 1
    step(0, 2, (kt + 2) * GBK, 1, Y_{}, Y_{}, Y_{}, N_{});
    step(1, 0, (kt + 3) * GBK, 2, Y_{}, Y_{}, Y_{}, N_{});
    step(2, 1, (kt + 4) * GBK, 0, Y_{}, Y_{}, Y_{}, N_{});
  }
  for (; kt < nk; ++kt) {                                  // the last 1 .. 5 tiles
    const int st = kt % RS;
    if (kt + 2 < nk) {
      if (st == 0) step(0, 2, (kt + 2) * GBK, 1, Y_{}, Y_{}, Y_{}, Y_{});
      else if (st == 1) step(1, 0, (kt + 2) * GBK, 2, Y_{}, Y_{}, Y_{}, Y_{});
      else step(2, 1, (kt + 2) * GBK, 0, Y_{}, Y_{}, Y_{}, Y_{});
    } else if (kt + 1 < nk) {
      if (st == 0) step(0, 0, 0, 1, N_{}, Y_{}, N_{}, N_{});
      else if (st == 1) step(1, 0, 0, 2, N_{}, Y_{}, N_{}, N_{});
      else step(2, 0, 0, 0, N_{}, Y_{}, N_{}, N_{});
    } else {
      if (st == 0) step(0, 0, 0, 0, N_{}, N_{}, N_{}, N_{});
      else if (st == 1) step(1, 0, 0, 0, N_{}, N_{}, N_{}, N_{});
      else step(2, 0, 0, 0, N_{}, N_{}, N_{}, N_{});
    }
  }
  wait_vmcnt<0>();                                         // the zero tile of a one-tile K

  // ---- epilogue. MF 32: lane (h, ln) of block (i, j) holds row
  // m0 + wm*WM + 32i + ln, columns n0 + wn*WN + 32j + 16h + r (r < 16).
  // MF 16: lane (q, l16) holds row m0 + wm*WM + 16i + l16, columns
  // n0 + wn*WN + 16j + 4q + r (r < 4).
  constexpr int CPL = MF == 32 ? 16 : 4;                   // consecutive columns per lane
  float ss = 0.f, sy = 0.f;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WM + MF * i + lr;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nb = n0 + wn * WN + MF * j + CPL * kq;
      const acc_t a = acc[i][j];
      if (m < M) {   // rows past M were read from a clamped row
#pragma unroll
        for (int r = 0; r < CPL; ++r) ss += a[r] * a[r];
      }
      if (m < M && nb < N_store) {
        if constexpr (MF == 32) {
          if (EPI == EPI_ERRCOS) {
            const u32x4* ys = reinterpret_cast<const u32x4*>(Yc + (size_t)m * ldc + nb);
            const u32x4 y0 = ys[0], y1 = ys[1];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              sy += lo_bf(y0[q]) * a[2 * q] + hi_bf(y0[q]) * a[2 * q + 1];
              sy += lo_bf(y1[q]) * a[8 + 2 * q] + hi_bf(y1[q]) * a[8 + 2 * q + 1];
            }
          }
          u32x4* dst = reinterpret_cast<u32x4*>(C + (size_t)m * ldc + nb);
          dst[0] = u32x4{pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(a[4], a[5]), pack2(a[6], a[7])};
          dst[1] = u32x4{pack2(a[8], a[9]), pack2(a[10], a[11]), pack2(a[12], a[13]), pack2(a[14], a[15])};
        } else {
          if (EPI == EPI_ERRCOS) {
            const uint2 y = *reinterpret_cast<const uint2*>(Yc + (size_t)m * ldc + nb);
            sy += lo_bf(y.x) * a[0] + hi_bf(y.x) * a[1] + lo_bf(y.y) * a[2] + hi_bf(y.y) * a[3];
          }
          *reinterpret_cast<uint2*>(C + (size_t)m * ldc + nb) = uint2{pack2(a[0], a[1]), pack2(a[2], a[3])};
        }
      }
    }
  }
  __syncthreads();                                         // the ring is no longer read
  float* wsum = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) ss += shfl_xor(ss, x);
  if (EPI == EPI_ERRCOS) {
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) sy += shfl_xor(sy, x);
  }
  if (l == 0) {
    wsum[w] = ss;
    wsum[GNW + w] = sy;
  }
  __syncthreads();
  if (t == 0) {
    float tot = 0.f, toty = 0.f;
    for (int i = 0; i < GNW; ++i) {
      tot += wsum[i];
      toty += wsum[GNW + i];
    }
    part[blockIdx.x] = tot;
    if (EPI == EPI_ERRCOS) part2[blockIdx.x] = toty;
  }
}

// ---- fp32 VALU GEMM ------------------------------------------------------------
// TS x TS tiles (TS = 64, or 32 for grids that would leave most CUs idle),
// 16 x 16 threads, RPT x RPT outputs per thread, K step 16. Each thread loads
// one VEC-float piece of the A tile and of the B tile per K step; the next
// step's pieces are loaded into registers before the current step's FMAs,
// so the global latency hides under them. B_NN = 0: B is [N][K] (ldb);
// B_NN = 1: B is [K][N] (ldb).
template <int EPI, int B_NN, int TS>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda,
                                                       const float* __restrict__ Bm, int ldb, int M,
                                                       int N_valid, int N_store, int K,
                                                       float* __restrict__ C, int ldc,
                                                       float* __restrict__ part,
                                                       const float* __restrict__ Eptr,
                                                       const float* __restrict__ Yc,
                                                       float* __restrict__ part2) {
  constexpr int KS = 16, RPT = TS / 16, VEC = TS * KS / 256;
  constexpr int PAD = TS + 4;                               // keeps 16-byte alignment of LDS rows
  __shared__ __attribute__((aligned(16))) float as[KS][PAD];
  __shared__ __attribute__((aligned(16))) float bs[KS][PAD];
  const int tiles_n = (N_store + TS - 1) / TS;
  const int m0 = (blockIdx.x / tiles_n) * TS, n0 = (blockIdx.x % tiles_n) * TS;
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;

  // this thread's pieces: K-contiguous (row lr, K offset lk) or, for a [K][N]
  // B, N-contiguous (K row bk, N offset bn)
  constexpr int KPR = KS / VEC;                             // pieces per K-contiguous row
  const int lr = t / KPR, lk = (t % KPR) * VEC;
  constexpr int NPR = TS / VEC;                             // pieces per N-contiguous row
  const int bk = t / NPR, bn = (t % NPR) * VEC;
  float ra[VEC], rb[VEC];
  auto load_k = [&](const float* base, int ld, int r, int rmax, int k0, float (&v)[VEC]) {
    const int gk = k0 + lk;
    if (r < rmax && gk + VEC <= K) {
      const float* src = base + (size_t)r * ld + gk;
      if constexpr (VEC == 4) {
        const floatx4 q = *reinterpret_cast<const floatx4*>(src);
        v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
      } else {
        const float2 q = *reinterpret_cast<const float2*>(src);
        v[0] = q.x; v[1] = q.y;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = (r < rmax && gk + e < K) ? base[(size_t)r * ld + gk + e] : 0.f;
    }
  };
  auto load = [&](int k0) {
    load_k(A, lda, m0 + lr, M, k0, ra);
    if constexpr (B_NN) {
      const int gk = k0 + bk, gn = n0 + bn;
      if (gk < K && gn + VEC <= N_valid) {
        const float* src = Bm + (size_t)gk * ldb + gn;
        if constexpr (VEC == 4) {
          const floatx4 q = *reinterpret_cast<const floatx4*>(src);
          rb[0] = q[0]; rb[1] = q[1]; rb[2] = q[2]; rb[3] = q[3];
        } else {
          const float2 q = *reinterpret_cast<const float2*>(src);
          rb[0] = q.x; rb[1] = q.y;
        }
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) rb[e] = (gk < K && gn + e < N_valid) ? Bm[(size_t)gk * ldb + gn + e] : 0.f;
      }
    } else {
      load_k(Bm, ldb, n0 + lr, N_valid, k0, rb);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int e = 0; e < VEC; ++e) as[lk + e][lr] = ra[e];
    if constexpr (B_NN) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) bs[bk][bn + e] = rb[e];
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) bs[lk + e][lr] = rb[e];
    }
  };

  float acc[RPT][RPT] = {};
  load(0);
  for (int k0 = 0; k0 < K; k0 += KS) {
    store();
    __syncthreads();
    if (k0 + KS < K) load(k0 + KS);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      float av[RPT], bv[RPT];
#pragma unroll
      for (int a = 0; a < RPT; ++a) av[a] = as[kk][ty * RPT + a];
#pragma unroll
      for (int c = 0; c < RPT; ++c) bv[c] = bs[kk][tx * RPT + c];
#pragma unroll
      for (int a = 0; a < RPT; ++a)
#pragma unroll
        for (int c = 0; c < RPT; ++c) acc[a][c] = fmaf(av[a], bv[c], acc[a][c]);
    }
    __syncthreads();
  }
  constexpr bool ERRS = EPI == EPI_ERR || EPI == EPI_ERRCOS;
  const float scale = (EPI == EPI_DD) ? Eptr[1] : 1.f;
  float ss = 0.f, sy = 0.f;
#pragma unroll
  for (int a = 0; a < RPT; ++a)
#pragma unroll
    for (int c = 0; c < RPT; ++c) {
      const int m = m0 + ty * RPT + a, n = n0 + tx * RPT + c;
      if (ERRS) ss += acc[a][c] * acc[a][c];
      if (m < M && n < N_store) {
        C[(size_t)m * ldc + n] = acc[a][c] * scale;
        if (EPI == EPI_ERRCOS) sy += Yc[(size_t)m * ldc + n] * acc[a][c];
      }
    }
  if (ERRS) {
    __shared__ float wsum[8];
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) ss += shfl_xor(ss, x);
    if (EPI == EPI_ERRCOS) {
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) sy += shfl_xor(sy, x);
    }
    if ((t & 63) == 0) {
      wsum[t >> 6] = ss;
      wsum[4 + (t >> 6)] = sy;
    }
    __syncthreads();
    if (t == 0) {
      part[blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
      if (EPI == EPI_ERRCOS) part2[blockIdx.x] = (wsum[4] + wsum[5]) + (wsum[6] + wsum[7]);
    }
  }
}

// E = sqrt(sum of partials), summed in a fixed order by one wave: lane l adds
// part[l], part[l + 64], ... in order, then the lanes are combined by a fixed
// butterfly. The partials were just written by workgroups on every XCD, so
// each read is a far-memory round trip: a lane issues eight of them before it
// adds any, in the same order (a slot past n adds +0, which leaves the sum
// unchanged). E_ws[0] = E and E_ws[1] = -1/E (0 when E == 0), the factor the
// dD epilogue applies (dE/dR = R / E, dE/dW_tilde = -(R / E) X). With
// sum_only the plain sum is written to err (E_ws unused).
__global__ __launch_bounds__(64) void error_finalize_kernel(const float* __restrict__ part, int n,
                                                            float* __restrict__ E_ws,
                                                            float* __restrict__ err, int sum_only) {
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += 512) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (i + 64 * q < n) ? part[i + 64 * q] : 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[q];
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) s += shfl_xor(s, x);
  if (threadIdx.x == 0) {
    if (sum_only) {
      *err = s;
      return;
    }
    const float E = sqrtf(s);
    if (E_ws) {
      E_ws[0] = E;
      E_ws[1] = (E > 0.f) ? -1.f / E : 0.f;
    }
    if (err) *err = E;
  }
}

// ---- launchers -------------------------------------------------------------------
// error GEMM: 256 x 128 tiles (the 4096 x 2048 residual is exactly 256 tiles)
// in the pipelined three-stage ring (144 KB of LDS); dD GEMM: 256 x 256
// tiles, two stages (128 KB).
constexpr int EBM = 256, EBN = 128, DBM = 256, DBN = 256, DS = 2;
constexpr int EMF = 16;   // MFMA of the error GEMM
constexpr int DLSP = 2;   // dD GEMM: sub-steps its loads are spread over

// fp32 tile size: 64, or 32 when 64-wide tiles would occupy fewer than 128
// of the 256 CUs
static int f32_tile(int M, int N) { return ((M + 63) / 64) * ((N + 63) / 64) < 128 ? 32 : 64; }

int gemm_error_parts(int M, int N, int bf16) {
  if (bf16) return ((M + EBM - 1) / EBM) * ((N + EBN - 1) / EBN);
  const int ts = f32_tile(M, N);
  return ((M + ts - 1) / ts) * ((N + ts - 1) / ts);
}

hipError_t launch_gemm_error_bf16(const uint16_t* A, int lda, const uint16_t* Bm, int ldb, int M,
                                  int N_valid, int N_store, int K, uint16_t* C, int ldc,
                                  float* part, const uint16_t* Y, float* party, hipStream_t s) {
  const int G = gemm_error_parts(M, N_store, 1);
  constexpr size_t lds = gemm_lds_bytes<EBM, EBN, RS>();
  if (Y)
    gemm_err_kernel<EPI_ERRCOS, EMF><<<G, GNT, lds, s>>>(A, lda, Bm, ldb, M, N_valid, N_store, K, C, ldc,
                                                         part, Y, party);
  else
    gemm_err_kernel<EPI_ERR, EMF><<<G, GNT, lds, s>>>(A, lda, Bm, ldb, M, N_valid, N_store, K, C, ldc,
                                                      part, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_dd_bf16(const uint16_t* A, int lda, const uint16_t* Bm, int ldb, int M,
                               int N, int K, const float* E, uint16_t* C, int ldc, hipStream_t s) {
  const int G = ((M + DBM - 1) / DBM) * ((N + DBN - 1) / DBN);
  gemm_dd_kernel<DBM, DBN, DS, DLSP><<<G, GNT, gemm_lds_bytes<DBM, DBN, DS>(), s>>>(A, lda, Bm, ldb, M, N, N, K, C,
                                                                           ldc, E, DdAdj{});
  return hipGetLastError();
}

int dd_adjoint_panels(int M) { return (M + DBM - 1) / DBM; }

hipError_t launch_gemm_dd_adjoint_bf16(const uint16_t* A, int lda, const uint16_t* Bm, int ldb, int M, int N, int K,
                                       const float* E, const uint16_t* W, const u32x4* frag, const uint32_t* bits,
                                       float* part, hipStream_t s) {
  if (N % ADJ_B != 0) return hipErrorInvalidValue;
  const int G = ((M + DBM - 1) / DBM) * ((N + DBN - 1) / DBN);
  constexpr size_t lds = gemm_lds_bytes<DBM, DBN, DS>() + 4 * ADJ_FRAG * 16;
  gemm_dd_kernel<DBM, DBN, DS, DLSP, true><<<G, GNT, lds, s>>>(A, lda, Bm, ldb, M, N, N, K, nullptr, N, E,
                                                             DdAdj{W, frag, bits, part, N / ADJ_B});
  return hipGetLastError();
}

hipError_t launch_gemm_error_f32(const float* A, int lda, const float* Bm, int ldb, int M,
                                 int N_valid, int N_store, int K, float* C, int ldc, float* part,
                                 const float* Y, float* party, hipStream_t s) {
  const int G = gemm_error_parts(M, N_store, 0);
  const bool t32 = f32_tile(M, N_store) == 32;
  if (Y)
    (t32 ? gemm_f32_kernel<EPI_ERRCOS, 0, 32> : gemm_f32_kernel<EPI_ERRCOS, 0, 64>)<<<G, 256, 0, s>>>(
        A, lda, Bm, ldb, M, N_valid, N_store, K, C, ldc, part, nullptr, Y, party);
  else
    (t32 ? gemm_f32_kernel<EPI_ERR, 0, 32> : gemm_f32_kernel<EPI_ERR, 0, 64>)<<<G, 256, 0, s>>>(
        A, lda, Bm, ldb, M, N_valid, N_store, K, C, ldc, part, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_dd_f32(const float* R, int ldr, const float* X, int ldx, int M, int N,
                              int K, const float* E, float* C, int ldc, hipStream_t s) {
  const int G = gemm_error_parts(M, N, 0);
  (f32_tile(M, N) == 32 ? gemm_f32_kernel<EPI_DD, 1, 32> : gemm_f32_kernel<EPI_DD, 1, 64>)<<<G, 256, 0, s>>>(
      R, ldr, X, ldx, M, N, N, K, C, ldc, nullptr, E, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_error_finalize(const float* part, int nparts, float* E_ws, float* err,
                                 hipStream_t s) {
  error_finalize_kernel<<<1, 64, 0, s>>>(part, nparts, E_ws, err, 0);
  return hipGetLastError();
}

hipError_t launch_sum_finalize(const float* part, int nparts, float* out, hipStream_t s) {
  error_finalize_kernel<<<1, 64, 0, s>>>(part, nparts, nullptr, out, 1);
  return hipGetLastError();
}

}  // namespace lcp
