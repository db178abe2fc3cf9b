// Block adjoint of the LCP forward (mask held constant unless the
// straight-through term below is on). The step uses these kernels for fp32
// layers, B = 32 and 128, and the straight-through term; for bf16 layers
// with B = 64 the dD GEMM computes the same sums in its epilogue (gemm.hip).
//
// Forward (per block b): W_hat_b = W_b P_b, A_b = W_hat_b . M_b,
// W_tilde_b = A_b P_b^T. Given G = dL/dW_tilde (= -dL/dD), the chain rule gives
//   dL/dP_b = G_b^T A_b + W_b^T ((G_b P_b) . M_b),
// a sum over the Cout rows. Each workgroup reduces one block over one chunk of
// rows and writes that partial B x B matrix; the Sinkhorn adjoint kernel adds
// the chunk partials in chunk order (deterministic, no atomics).
//
// bf16 kernel (B <= 64): each wave runs its own pipeline over 32-row tiles of
// W and G. Tiles move HBM -> LDS with 16-byte direct-to-LDS loads into a
// private two-stage ring (no register staging, no workgroup barriers in the loop);
// load instruction (matrix, K step p) of a tile has lane l fetch exactly the
// 16 bytes that lane l later feeds to the MFMA for that K step, so the LDS
// reads are linear and conflict-free. Rows are remapped so that MFMA outputs
// land with 16 consecutive rows per lane. Per tile:
//   1. W_hat = W P_b and Y = G P_b (MFMA, P_b fragments prepared in LDS),
//      giving, per lane, one permuted position k and 16 rows i;
//   2. the tile's mask words (loaded with the tile) turn them into
//      A = W_hat . M and Y . M, rounded to bf16;
//   3. G and W are transposed into the same "16 rows per lane" layout by an
//      MFMA against the identity (exact: bf16 x 1.0 in fp32);
//   4. dP^T[k][j] += sum_i A[i][k] G[i][j] + (Y . M)[i][k] W[i][j], MFMA with
//      the rows i in the K slots on both sides.
// With the straight-through mask term (STE) step 4 also adds
//   dP^T[k][j] += sum_i (W_hat . Y)[i][k] S[i][j],  S[i][j] = |W[i][j]| n_j,
// which is S_b^T ((G_b P_b) . (W_b P_b)): the gradient reaching the 0/1 mask,
// dE/dM = (G_b P_b) . W_hat_b, handed unchanged to S_hat_b = S_b P_b.
// For B = 128 a workgroup has eight waves in two slots; the four waves of a
// slot take the same 32-row tile, share one three-stage ring (each wave
// issues a quarter of the loads, a barrier per tile) and each owns one 32-wide
// block of positions k: it forms W_hat and Y for its own positions only and
// transposes all of G and W, one source column block at a time; for B <= 64
// every wave owns whole tiles and its own ring. Partial sums of waves owning
// the same entries are added through LDS in a fixed order.
#include "common.h"
#include "kernels.h"

namespace lcp {

typedef __attribute__((address_space(3))) void* adj_lds_t;
constexpr uint32_t kAdjOOB = 0x80000000u;   // a buffer offset past every operand (reads zeros)

template <int B>
struct AdjGeom {
  static constexpr int KS = B / 16;             // K steps over a block
  static constexpr int TT = B / 32;             // 32-wide column blocks
  static constexpr int WS = (B == 128) ? 4 : 1; // waves sharing one row tile
  static constexpr int NA = TT / WS;            // position blocks (a) owned per wave
  // B = 128: eight waves, two row tiles (slots) of four waves each, so every
  // SIMD runs two waves; B <= 64: four waves, one row tile each
  static constexpr int WAVES = (B == 128) ? 8 : 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int TILES = WAVES / WS;      // row tiles in flight per workgroup
  static constexpr int ROWS = 32 * TILES;       // rows per workgroup step
  static constexpr int FRAG = TT * KS * 64;     // u32x4 entries of the P fragments
  // ring stages: a shared B = 128 ring is one stage deeper
  static constexpr int S = (B == 128) ? 3 : 2;
  static constexpr int BI = (TT + 1) / 2;       // mask-word load instructions per tile
  static constexpr int STAGE = 2 * KS * 1024 + BI * 256;   // bytes per stage
  static constexpr int IPT = 2 * KS + BI;       // load instructions per tile
};

// s_waitcnt vmcnt(n) for the wave-uniform counts the ring can need
// (0 and up to two later tiles of 4 or 5 loads); any other count waits for
// everything, which is always safe.
__device__ __forceinline__ void adj_wait_vm(int n) {
  constexpr int E = (7 << 4) | (15 << 8);
  switch (n) {
    case 4: __builtin_amdgcn_s_waitcnt(4 | E); break;
    case 5: __builtin_amdgcn_s_waitcnt(5 | E); break;
    case 8: __builtin_amdgcn_s_waitcnt(8 | E); break;
    case 10: __builtin_amdgcn_s_waitcnt(10 | E); break;
    default: __builtin_amdgcn_s_waitcnt(0 | E); break;
  }
}

__device__ __forceinline__ u32x4 identity_slots(int v, int h, int n) {
  // MFMA B operand of the 32 x 32 identity, K step v of a 32-column group:
  // slot e of lane (h, n) stands for column 16h + 8v + e of the group and is
  // 1 when that equals n
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e0 = 16 * h + 8 * v + 2 * q;
    w[q] = (e0 == n ? 0x3f80u : 0u) | ((e0 + 1 == n ? 0x3f80u : 0u) << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Persistent grid: workgroup g takes the contiguous range [g*tpw, (g+1)*tpw)
// of the block-major sequence of 32-row tiles (tpb tiles per block), which
// spans at most `maxseg` blocks; it writes one partial B x B matrix per block
// segment to part[(g * maxseg + k) * B * B] (k = block - first block of g).
template <int B, bool STE>
__global__ __launch_bounds__(AdjGeom<B>::THREADS, (B == 128) ? 1 : 2) void adjoint_bf16_kernel(
    const uint16_t* __restrict__ G, const uint16_t* __restrict__ W, const u32x4* __restrict__ gfrag,
    const float* __restrict__ P, const uint32_t* __restrict__ bits, int cout, int cin, int tpw,
    int maxseg, const float* __restrict__ ste_norms, float* __restrict__ part) {
  using Gm = AdjGeom<B>;
  constexpr int KS = Gm::KS, TT = Gm::TT, WS = Gm::WS, NA = Gm::NA, TILES = Gm::TILES;
  constexpr int S = Gm::S, STAGE = Gm::STAGE;
  extern __shared__ __attribute__((aligned(16))) unsigned char adj_lds[];
  // layout: P fragments | rings (one per row-tile slot, S stages); after the
  // tile loop of a segment the rings hold the cross-wave sums
  uint16_t* fb = reinterpret_cast<uint16_t*>(adj_lds);
  unsigned char* rings = adj_lds + Gm::FRAG * 16;
  float* red = reinterpret_cast<float*>(rings);

  // the wave index as a uniform value: the slot, the ring address and the
  // loads' scalar offsets derived from it then stay in scalar registers
  const int t = threadIdx.x, l = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = l >> 5, n = l & 31;
  const int slot = w / WS;          // row tile slot of this wave
  const int half = w % WS;          // position blocks a = half * NA + ai
  unsigned char* ring = rings + slot * S * STAGE;
  const u32x4* F = reinterpret_cast<const u32x4*>(fb);
  const int lrow = remap_row(n);    // tile row whose operands this lane fetches

  const int tpb = (cout + 31) / 32;
  const int total = (cin / B) * tpb;
  const int t_begin = blockIdx.x * tpw;
  const int t_end = min(total, t_begin + tpw);
  const int first_b = t_begin / tpb;
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(W), (short)0,
                                                                    (int)(uint32_t)((size_t)cout * cin * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rG = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(G), (short)0,
                                                                    (int)(uint32_t)((size_t)cout * cin * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rBits = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(bits), (short)0, (int)(uint32_t)((size_t)(cin / B) * cout * TT * 4), 0x00020000);
  const uint32_t vw_lane = (uint32_t)(((size_t)lrow * cin + 16 * h) * 2);  // W / G element (lrow, 16h) of a tile
  const uint32_t vb_lane = (uint32_t)((n * TT + h) * 4);                    // mask word h of tile row n

  for (int seg = t_begin; seg < t_end;) {
    const int b = seg / tpb;
    const int seg_end = min(t_end, (b + 1) * tpb);
    __syncthreads();                       // fragments and sums of the previous block consumed
    // P fragments (MFMA B operand, K = source channel j, N = position k):
    // F[(t*KS + p)*64 + lane][e] = P_b[32(p/2) + 16h + 8(p%2) + e][32t + n]
    if (gfrag != nullptr) {
      // global -> LDS directly, all of a thread's copies in flight at once
      // (FRAG is a multiple of 64: each wave copies whole 1 KB rows or none)
      const u32x4* src = gfrag + (size_t)b * Gm::FRAG;
      constexpr int PER = (Gm::FRAG + Gm::THREADS - 1) / Gm::THREADS;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e0 = k * Gm::THREADS + 64 * w;
        if (e0 < Gm::FRAG) __builtin_amdgcn_global_load_lds(src + e0 + l, (adj_lds_t)(fb + (size_t)e0 * 8), 16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));   // vmcnt(0)
    } else {
      const float* src = P + (size_t)b * B * B;
      for (int e_idx = t; e_idx < B * B; e_idx += Gm::THREADS) {
        const int j = e_idx / B, k = e_idx % B;
        const int tt = k >> 5, nn = k & 31, p = 2 * (j >> 5) + ((j >> 3) & 1), hh = (j >> 4) & 1, e = j & 7;
        fb[(((tt * KS + p) * 64) + 32 * hh + nn) * 8 + e] = (uint16_t)f2bf(src[e_idx]);
      }
    }
    __syncthreads();

    floatx16 acc[NA][TT];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int o = 0; o < TT; ++o) acc[a][o] = floatx16{};
    // column norms n_j of this lane's source channels j = bB + 32 o + n
    float nrm[TT];
#pragma unroll
    for (int o = 0; o < TT; ++o) nrm[o] = STE ? ste_norms[b * B + 32 * o + n] : 0.f;

    // the load instructions of one tile into stage st (with WS waves sharing a
    // ring, wave `half` issues every WS-th of them)
    // loads through buffer resources: a lane's offset inside a tile is fixed
    // (row lrow, or n for the mask words), the tile and block move only the
    // scalar offset, rows past cout read zeros (offset past the resource)
    auto issue = [&](int st, int tile) {
      unsigned char* sb = ring + st * STAGE;
      const int i0 = (tile - b * tpb) * 32;
      const uint32_t vw = (i0 + lrow < cout) ? vw_lane : kAdjOOB;
      const uint32_t vb = (i0 + n < cout) ? vb_lane : kAdjOOB;
      const uint32_t sw0 = (uint32_t)(((size_t)i0 * cin + b * B) * 2);
#pragma unroll
      for (int p = 0; p < KS; ++p) {
        if (p % WS != half) continue;
        // K step p: channels 32(p/2) + 16h + 8(p%2) + e of the block
        const uint32_t sp = sw0 + 2 * (32 * (p >> 1) + 8 * (p & 1));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (adj_lds_t)(sb + p * 1024), 16, (int)vw, (int)sp, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rG, (adj_lds_t)(sb + (KS + p) * 1024), 16, (int)vw, (int)sp, 0, 0);
      }
      // mask words (block-major [block][row][TT]): instruction q, lane (h, n)
      // -> word 2q + h of row i0 + n, all inside the tile's 32 * TT words
      const uint32_t sb0 = (uint32_t)(((size_t)b * cout + i0) * TT * 4);
#pragma unroll
      for (int q = 0; q < Gm::BI; ++q) {
        if (q % WS != half) continue;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rBits, (adj_lds_t)(sb + 2 * KS * 1024 + q * 256), 4,
                                                 (int)(vb + 4 * ((2 * q + h) % TT - h)), (int)sb0, 0, 0);
      }
    };

    const int first = seg + slot;
    const int ntile = (first < seg_end) ? (seg_end - first + TILES - 1) / TILES : 0;
    // every wave runs the first slot's count of iterations (the barrier of a
    // shared ring needs all of them); a slot with one tile fewer idles
    // through its last one
    const int nit = (seg_end - seg + TILES - 1) / TILES;
    // loads this wave issues per tile (the waves of a shared ring split them)
    const int nload = 2 * (KS / WS) + (WS == 1 ? Gm::BI : (half < Gm::BI ? 1 : 0));
#pragma unroll
    for (int q = 0; q < S - 1; ++q)
      if (q < ntile) issue(q, first + q * TILES);
    for (int it = 0; it < (WS > 1 ? nit : ntile); ++it) {
      // this wave's loads of tile `it` have landed (only later tiles' loads,
      // issued after them, may still be in flight); the stage refilled below
      // was consumed in the previous iteration. A shared ring also needs every
      // wave's part and every wave done with that stage: one barrier.
      const int later = max(0, min(S - 2, ntile - 1 - it));
      if (S == 2) __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
      else adj_wait_vm(later * nload);
      if (WS > 1) __builtin_amdgcn_s_barrier();
      if (it >= ntile) continue;                     // idle slot (shared ring only)
      if (it + S - 1 < ntile) issue((it + S - 1) % S, first + (it + S - 1) * TILES);
      const unsigned char* sb = ring + (it % S) * STAGE;
      const u32x4* LW = reinterpret_cast<const u32x4*>(sb);
      const u32x4* LG = reinterpret_cast<const u32x4*>(sb + KS * 1024);
      const uint32_t* LB = reinterpret_cast<const uint32_t*>(sb + 2 * KS * 1024);

      // G and W (and S = |W| n_j) of source column block o transposed into
      // the "16 rows per lane" layout (MFMA against the identity, exact)
      auto transpose_block = [&](int o, u32x4 (&gT)[2], u32x4 (&wT)[2], u32x4 (&sT)[2]) {
        floatx16 tg = {}, tw = {};
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const u32x4 id = identity_slots(v, h, n);
          tg = mfma32(LG[(2 * o + v) * 64 + l], id, tg);
          tw = mfma32(LW[(2 * o + v) * 64 + l], id, tw);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          gT[u] = u32x4{pack2_exact(tg[8 * u], tg[8 * u + 1]), pack2_exact(tg[8 * u + 2], tg[8 * u + 3]),
                        pack2_exact(tg[8 * u + 4], tg[8 * u + 5]), pack2_exact(tg[8 * u + 6], tg[8 * u + 7])};
          wT[u] = u32x4{pack2_exact(tw[8 * u], tw[8 * u + 1]), pack2_exact(tw[8 * u + 2], tw[8 * u + 3]),
                        pack2_exact(tw[8 * u + 4], tw[8 * u + 5]), pack2_exact(tw[8 * u + 6], tw[8 * u + 7])};
          if (STE) {
            float sv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[e] = __builtin_fabsf(tw[8 * u + e]) * nrm[o];
            sT[u] = u32x4{pack2(sv[0], sv[1]), pack2(sv[2], sv[3]), pack2(sv[4], sv[5]), pack2(sv[6], sv[7])};
          }
        }
      };
      // W_hat = W P_b and Y = G P_b for positions 32a + n (rows 16h + r),
      // masked and packed as MFMA A operands (and W_hat . Y unmasked for STE)
      auto position_block = [&](int a, u32x4 (&aop)[2], u32x4 (&yop)[2], u32x4 (&qop)[2]) {
        floatx16 wh = {}, yy = {};
#pragma unroll
        for (int p = 0; p < KS; ++p) {
          const u32x4 fp = F[(a * KS + p) * 64 + l];
          wh = mfma32(LW[p * 64 + l], fp, wh);
          yy = mfma32(LG[p * 64 + l], fp, yy);
        }
        // mask words of rows 16h + r for column block a (instruction a/2, lane half a%2)
        const u32x4* mw = reinterpret_cast<const u32x4*>(LB + (a / 2) * 64 + (a % 2) * 32 + 16 * h);
        uint32_t m16[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 v4 = mw[q];
          m16[4 * q] = v4.x; m16[4 * q + 1] = v4.y; m16[4 * q + 2] = v4.z; m16[4 * q + 3] = v4.w;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float av[8], yv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool keep = (m16[8 * u + e] >> n) & 1u;
            av[e] = keep ? wh[8 * u + e] : 0.f;
            yv[e] = keep ? yy[8 * u + e] : 0.f;
          }
          aop[u] = u32x4{pack2(av[0], av[1]), pack2(av[2], av[3]), pack2(av[4], av[5]), pack2(av[6], av[7])};
          yop[u] = u32x4{pack2(yv[0], yv[1]), pack2(yv[2], yv[3]), pack2(yv[4], yv[5]), pack2(yv[6], yv[7])};
          if (STE) {
            float qv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[e] = wh[8 * u + e] * yy[8 * u + e];
            qop[u] = u32x4{pack2(qv[0], qv[1]), pack2(qv[2], qv[3]), pack2(qv[4], qv[5]), pack2(qv[6], qv[7])};
          }
        }
      };
      // dP^T[k][j] += sum_i A[i][k] G[i][j] + (Y . M)[i][k] W[i][j] (+ STE term)
      auto accumulate = [&](floatx16& c, const u32x4 (&aop)[2], const u32x4 (&yop)[2], const u32x4 (&qop)[2],
                            const u32x4 (&gT)[2], const u32x4 (&wT)[2], const u32x4 (&sT)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          c = mfma32(aop[u], gT[u], c);
          c = mfma32(yop[u], wT[u], c);
        }
        if (STE) {
#pragma unroll
          for (int u = 0; u < 2; ++u) c = mfma32(qop[u], sT[u], c);
        }
      };
      if constexpr (NA > 1) {
        // every wave owns all positions: transpose once, then each position block
        u32x4 gT[TT][2], wT[TT][2], sT[TT][2];
#pragma unroll
        for (int o = 0; o < TT; ++o) transpose_block(o, gT[o], wT[o], sT[o]);
#pragma unroll
        for (int ai = 0; ai < NA; ++ai) {
          u32x4 aop[2], yop[2], qop[2];
          position_block(half * NA + ai, aop, yop, qop);
#pragma unroll
          for (int o = 0; o < TT; ++o) accumulate(acc[ai][o], aop, yop, qop, gT[o], wT[o], sT[o]);
        }
      } else {
        // one position block per wave: its operands first, then each source
        // column block transposed just before its multiply-adds (fewer live
        // registers; no transpose is repeated)
        u32x4 aop[2], yop[2], qop[2];
        position_block(half, aop, yop, qop);
#pragma unroll
        for (int o = 0; o < TT; ++o) {
          u32x4 gT[2], wT[2], sT[2];
          transpose_block(o, gT, wT, sT);
          accumulate(acc[0][o], aop, yop, qop, gT, wT, sT);
        }
      }
    }

    // lane (h, n) of block (ai, o) holds dP^T[k = 32a + 8(r/4) + 4h + r%4][j = 32 o + n]
    // with a = half * NA + ai; the row-tile slots are added into slot 0, one
    // slot per round
    if (TILES > 1) {
      for (int s2 = 1; s2 < TILES; ++s2) {
        __syncthreads();
        if (slot == s2) {
#pragma unroll
          for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int o = 0; o < TT; ++o)
#pragma unroll
              for (int r = 0; r < 16; ++r) red[(((half * NA + a) * TT + o) * 16 + r) * 64 + l] = acc[a][o][r];
        }
        __syncthreads();
        if (slot == 0) {
#pragma unroll
          for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int o = 0; o < TT; ++o)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[a][o][r] += red[(((half * NA + a) * TT + o) * 16 + r) * 64 + l];
        }
      }
    }
    if (slot == 0) {
      float* dst = part + ((size_t)blockIdx.x * maxseg + (b - first_b)) * B * B;
#pragma unroll
      for (int ai = 0; ai < NA; ++ai)
#pragma unroll
        for (int o = 0; o < TT; ++o) {
          const int j = 32 * o + n;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = 32 * (half * NA + ai) + 8 * q + 4 * h;
            *reinterpret_cast<floatx4*>(dst + j * B + k) =
                floatx4{acc[ai][o][4 * q], acc[ai][o][4 * q + 1], acc[ai][o][4 * q + 2], acc[ai][o][4 * q + 3]};
          }
        }
    }
    seg = seg_end;
  }
}

template <int B>
constexpr size_t adj_lds_bytes() {
  using Gm = AdjGeom<B>;
  const size_t ring = (size_t)Gm::TILES * Gm::S * Gm::STAGE;
  const size_t red = Gm::TILES > 1 ? (size_t)Gm::WS * Gm::NA * Gm::TT * 16 * 64 * 4 : 0;
  return (size_t)Gm::FRAG * 16 + (ring > red ? ring : red);
}

// fp32 VALU version: one thread per group of (j, k) outputs, rows streamed
// through LDS one at a time; same persistent tile ranges and (workgroup,
// segment) partial layout as the bf16 kernel.
template <int B, bool STE>
__global__ __launch_bounds__(256) void adjoint_f32_kernel(const float* __restrict__ G,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ P,
                                                          const uint32_t* __restrict__ bits,
                                                          int cout, int cin, int tpw, int maxseg,
                                                          const float* __restrict__ ste_norms,
                                                          float* __restrict__ part) {
  constexpr int PER = (B * B + 255) / 256;
  __shared__ float pb[B][B + 1];
  __shared__ float wr[B], gr[B], am[B], ym[B], sw[B], qm[B];
  const int t = threadIdx.x;
  const int tpb = (cout + 31) / 32;
  const int total = (cin / B) * tpb;
  const int t_begin = blockIdx.x * tpw;
  const int t_end = min(total, t_begin + tpw);
  const int first_b = t_begin / tpb;
  for (int seg = t_begin; seg < t_end;) {
    const int b = seg / tpb;
    const int seg_end = min(t_end, (b + 1) * tpb);
    __syncthreads();
    const float* src = P + (size_t)b * B * B;
    for (int e = t; e < B * B; e += 256) pb[e / B][e % B] = src[e];
    float acc[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) acc[q] = 0.f;
    const int r0 = (seg - b * tpb) * 32;
    const int r1 = min(cout, (seg_end - b * tpb) * 32);
    for (int i = r0; i < r1; ++i) {
      __syncthreads();
      if (t < B) {
        const float wv = W[(size_t)i * cin + b * B + t];
        wr[t] = wv;
        gr[t] = G[(size_t)i * cin + b * B + t];
        if (STE) sw[t] = __builtin_fabsf(wv) * ste_norms[b * B + t];
      }
      __syncthreads();
      if (t < B) {
        float s1 = 0.f, s2 = 0.f;
        for (int j = 0; j < B; ++j) {
          s1 = fmaf(wr[j], pb[j][t], s1);
          s2 = fmaf(gr[j], pb[j][t], s2);
        }
        const uint32_t keep = (bits[((size_t)b * cout + i) * (B >> 5) + (t >> 5)] >> (t & 31)) & 1u;
        am[t] = keep ? s1 : 0.f;
        ym[t] = keep ? s2 : 0.f;
        if (STE) qm[t] = s1 * s2;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int e = t + 256 * q;
        if (e < B * B) {
          const int j = e / B, k = e % B;
          acc[q] = fmaf(gr[j], am[k], fmaf(wr[j], ym[k], acc[q]));
          if (STE) acc[q] = fmaf(sw[j], qm[k], acc[q]);
        }
      }
    }
    float* dst = part + ((size_t)blockIdx.x * maxseg + (b - first_b)) * B * B;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = t + 256 * q;
      if (e < B * B) dst[e] = acc[q];
    }
    seg = seg_end;
  }
}

// Fixed grids (two resident workgroups per CU on 256 CUs for B <= 64, one
// for B = 128), independent of the device, so the work split and every result
// are the same everywhere.
AdjSplit adjoint_split(int cout, int cin, int B) {
  AdjSplit sp{};
  const int tpb = (cout + 31) / 32;
  const int total = (cin / B) * tpb;
  int grid = (B == 128) ? 256 : 512;
  sp.tpw = (total + grid - 1) / grid;
  sp.grid = (total + sp.tpw - 1) / sp.tpw;
  sp.maxseg = (sp.tpw + tpb - 1) / tpb + 1;
  sp.tpb = tpb;
  return sp;
}

template <int B, bool STE>
static void adj_bf16(const uint16_t* G, const uint16_t* W, const u32x4* gfrag, const float* P, const uint32_t* bits,
                     int cout, int cin, const AdjSplit& sp, const float* nrm, float* part, hipStream_t s) {
  adjoint_bf16_kernel<B, STE><<<sp.grid, AdjGeom<B>::THREADS, adj_lds_bytes<B>(), s>>>(G, W, gfrag, P, bits, cout, cin, sp.tpw,
                                                                      sp.maxseg, nrm, part);
}

hipError_t launch_adjoint_bf16(const uint16_t* G, const uint16_t* W, const u32x4* gfrag, const float* P,
                               const uint32_t* bits, int cout, int cin, int B, const AdjSplit& sp,
                               const float* ste_norms, float* part, hipStream_t s) {
  const bool ste = ste_norms != nullptr;
  switch (B) {
    case 32: (ste ? adj_bf16<32, true> : adj_bf16<32, false>)(G, W, gfrag, P, bits, cout, cin, sp, ste_norms, part, s); break;
    case 64: (ste ? adj_bf16<64, true> : adj_bf16<64, false>)(G, W, gfrag, P, bits, cout, cin, sp, ste_norms, part, s); break;
    case 128: (ste ? adj_bf16<128, true> : adj_bf16<128, false>)(G, W, gfrag, P, bits, cout, cin, sp, ste_norms, part, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// fp32 kernel: one workgroup per (block, 32-row tile range of one segment),
// written in the same (workgroup, segment) partial layout as the bf16 kernel.
template <int B, bool STE>
static void adj_f32(const float* G, const float* W, const float* P, const uint32_t* bits, int cout, int cin,
                    const AdjSplit& sp, const float* nrm, float* part, hipStream_t s) {
  adjoint_f32_kernel<B, STE><<<sp.grid, 256, 0, s>>>(G, W, P, bits, cout, cin, sp.tpw, sp.maxseg, nrm, part);
}

hipError_t launch_adjoint_f32(const float* G, const float* W, const float* P,
                              const uint32_t* bits, int cout, int cin, int B, const AdjSplit& sp,
                              const float* ste_norms, float* part, hipStream_t s) {
  const bool ste = ste_norms != nullptr;
  switch (B) {
    case 32: (ste ? adj_f32<32, true> : adj_f32<32, false>)(G, W, P, bits, cout, cin, sp, ste_norms, part, s); break;
    case 64: (ste ? adj_f32<64, true> : adj_f32<64, false>)(G, W, P, bits, cout, cin, sp, ste_norms, part, s); break;
    case 128: (ste ? adj_f32<128, true> : adj_f32<128, false>)(G, W, P, bits, cout, cin, sp, ste_norms, part, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lcp
