// Deploy path of a trained layer ([PermLLM] inference acceleration): the
// activations are gathered into the learned permuted channel order and
// multiplied by the 2:4-sparse permuted weight on the sparse matrix cores,
//   Y = (X P_B) ((W P_B) . M)^T      (T x Cout, bf16).
//
// Packed weight format (written by sparse_pack_kernel, read by the GEMM):
// fragment (rg, kf) covers rows 32 rg .. 32 rg + 31 and dense K positions
// 32 kf .. 32 kf + 31. Its 64 lanes hold, in lane order, the operand of one
// v_smfmac_f32_32x32x32_bf16: lane l carries row 32 rg + remap_row(l % 32)
// and the K positions 32 kf + 16 (l / 32) + [0, 16), i.e. four groups of four
// positions, as 8 bf16 values (the two kept entries of each group, lower
// position first) and 16 bits of positions (group g: bits 4g, 4g+1 = first
// position, 4g+2, 4g+3 = second). vals: [cout/32][cin/32][64][8] bf16;
// meta: [cout/32][ceil(cin/64)][64] uint32 holding the 16-bit words of
// fragments 2q (low half) and 2q + 1 (high half, 0 past cin).
//
// Lane layout of v_smfmac_f32_32x32x32_bf16 (measured on gfx950 with
// integer operands): with the A lanes as above, the dense operand of lane
// (h, n) holds column n and the K positions 8h + [0, 8) in its first eight
// values and 16 + 8h + [0, 8) in the last eight; the accumulator layout is
// that of the dense 32x32 MFMA (lane (h, n), register r: row
// 8 (r/4) + 4h + r%4, column n). With remap_row on the A rows, register r of
// lane (h, n) is output row 16h + r of the fragment.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lcp {

typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* dep_lds_t;
__device__ const u32x4 g_dep_zero[1] = {{0u, 0u, 0u, 0u}};

// ---- packing -------------------------------------------------------------------
// One thread per (fragment, lane): 16 permuted positions of one row.
__global__ __launch_bounds__(256) void sparse_pack_kernel(const uint16_t* __restrict__ W, int cout, int cin, int B,
                                                          const int* __restrict__ perm,
                                                          const uint32_t* __restrict__ bits,
                                                          u32x4* __restrict__ vals,
                                                          uint32_t* __restrict__ meta) {
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  const int KF = cin / 32;
  if (id >= (long long)(cout / 32) * KF * 64) return;
  const int l = (int)(id & 63);
  const long long fr = id >> 6;
  const int rg = (int)(fr / KF), kf = (int)(fr % KF);
  const int h = l >> 5;
  const int o = 32 * rg + remap_row(l & 31);
  const int k0 = 32 * kf + 16 * h;                       // first of the 16 positions
  const uint32_t word = bits[(size_t)o * (cin / 32) + kf] >> (16 * h);
  uint32_t v[4];
  uint32_t m16 = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t kept = (word >> (4 * g)) & 0xFu;
    // the first two kept positions, completed by the lowest free positions
    int pos[2], n = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (((kept >> q) & 1u) && n < 2) pos[n++] = q;
    bool real[2] = {n > 0, n > 1};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (!((kept >> q) & 1u) && n < 2) pos[n++] = q;
    if (pos[0] > pos[1]) {                                // keep positions ascending
      const int tp = pos[0]; pos[0] = pos[1]; pos[1] = tp;
      const bool tr = real[0]; real[0] = real[1]; real[1] = tr;
    }
    uint32_t e[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k = k0 + 4 * g + pos[s];                 // permuted position
      const int b = k / B;
      const int src = b * B + (perm[k] & (B - 1));       // source channel of position k
      e[s] = real[s] ? (uint32_t)W[(size_t)o * cin + src] : 0u;
    }
    v[g] = e[0] | (e[1] << 16);
    m16 |= (uint32_t)(pos[0] | (pos[1] << 2)) << (4 * g);
  }
  vals[id] = u32x4{v[0], v[1], v[2], v[3]};
  // meta word of the 64-position step: fragment kf fills half kf & 1
  const int KT = (cin + 63) / 64;
  uint16_t* mh = reinterpret_cast<uint16_t*>(meta);
  mh[(((size_t)rg * KT + (kf >> 1)) * 64 + l) * 2 + (kf & 1)] = (uint16_t)m16;
  if ((KF & 1) && kf == KF - 1) mh[(((size_t)rg * KT + (kf >> 1)) * 64 + l) * 2 + 1] = 0;
}

// ---- channel gather --------------------------------------------------------------
// Xp[t][bB + k] = X[t][bB + perm[b][k]]: each thread owns 8 consecutive
// positions (its source indices stay in registers) and walks 16 tokens.
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ X, int T, int cin, int B,
                                                     const int* __restrict__ perm, uint16_t* __restrict__ Xp) {
  const int c = blockIdx.x * 256 + threadIdx.x;          // chunk of 8 positions
  if (c >= cin / 8) return;
  int src[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = 8 * c + e;
    src[e] = (k / B) * B + (perm[k] & (B - 1));
  }
  const int t0 = blockIdx.y * 16, t1 = min(T, t0 + 16);
  for (int t = t0; t < t1; ++t) {
    const uint16_t* row = X + (size_t)t * cin;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = (uint32_t)row[src[2 * q]] | ((uint32_t)row[src[2 * q + 1]] << 16);
    *reinterpret_cast<u32x4*>(Xp + (size_t)t * cin + 8 * c) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ---- 2:4 sparse GEMM ----------------------------------------------------------------
// Y[t][o] = sum_k Ws[o][k] Xp[t][k]. 256 (rows o) x 128 (tokens t) tiles, 8
// waves in a 4 x 2 layout (each wave 64 x 64: 2 x 2 sparse MFMA blocks), K
// steps of 64 positions. A ring stage holds the 16 weight fragments of one
// step (16 KB, lane order, linear LDS reads), their position words (2 KB)
// and the 128 x 64 activation tile (16 KB, rows swizzled as in the dense
// GEMM), all moved with direct-to-LDS loads; four stages (136 KB of LDS)
// keep three tiles in flight per CU. The ring is software-pipelined
// like the dense error GEMM: the five loads of tile kt + RS - 1 go out one at a
// time between the first sub-step's MFMAs of step kt (a burst right after the
// barrier stalls every wave on the vector-memory queue), and each step's
// barrier sits before its second 32-position sub-step, whose MFMAs run from
// registers while the first fragments of the next stage are read.
constexpr int SP_BM = 256, SP_BN = 128, SP_NT = 512, SP_RS = 4, SP_NL = 5;
constexpr int SP_A1 = (SP_BM / 32) * 2 * 1024, SP_M1 = (SP_BM / 32) * 256, SP_B1 = SP_BN * 64 * 2;
constexpr int SP_STAGE = SP_A1 + SP_M1 + SP_B1;
constexpr int SP_MOFF = SP_A1, SP_BOFF = SP_A1 + SP_M1;

__device__ __forceinline__ void sp_tile_coords(int g, int G, int tiles_m, int tiles_n, int& tm, int& tn) {
  // consecutive workgroups of one XCD (id mod 8) take a compact group of
  // 4 row panels x all token panels
  int logical = g;
  if ((G & 7) == 0) logical = (g & 7) * (G >> 3) + (g >> 3);
  const int in_group = 4 * tiles_n;
  const int gid = logical / in_group;
  const int first_m = gid * 4;
  const int gsm = min(tiles_m - first_m, 4);
  const int rem = logical - gid * in_group;
  tm = first_m + rem % gsm;
  tn = rem / gsm;
}

__device__ __forceinline__ int sp_swz(int row, int ch) { return row * 64 + ((ch ^ ((row >> 1) & 7)) << 3); }

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited on)
template <int N>
__device__ __forceinline__ void sp_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int RS>
__global__ __launch_bounds__(SP_NT, 1) void spgemm_kernel(const u32x4* __restrict__ vals,
                                                          const uint32_t* __restrict__ meta,
                                                          const uint16_t* __restrict__ Xp, int T, int cout,
                                                          int cin, uint16_t* __restrict__ Y) {
  constexpr int FM = 2, FN = 2, NM = FM * FN, WM = 64, WN = 64, NL = SP_NL;
  static_assert(RS >= 3 && (RS - 2) * NL < 64, "ring depth");
  extern __shared__ __attribute__((aligned(16))) unsigned char sp_lds[];
  const int tiles_m = (cout + SP_BM - 1) / SP_BM, tiles_n = (T + SP_BN - 1) / SP_BN;
  int tm, tn;
  sp_tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * SP_BM, n0 = tn * SP_BN;
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int h = l >> 5, ln = l & 31;
  const int KF = cin / 32, NK = (cin + 63) / 64, RG = cout / 32;

  // load o of this thread for K step ks into ring stage `stage`: o < 2 the
  // weight fragment f = 8 o + w (row group f / 2, 32-position half f % 2),
  // o = 2 the position words of row group w, o > 2 activation chunks
  auto issue_one = [&](int stage, int ks, int o) {
    unsigned char* sb = sp_lds + stage * SP_STAGE;
    if (o < 2) {
      const int f = 8 * o + w, rg = m0 / 32 + (f >> 1), kf = 2 * ks + (f & 1);
      const void* src = (rg < RG && kf < KF) ? (const void*)(vals + ((size_t)rg * KF + kf) * 64 + l)
                                             : (const void*)g_dep_zero;
      __builtin_amdgcn_global_load_lds(src, (dep_lds_t)(sb + f * 1024), 16, 0, 0);
    } else if (o == 2) {
      const int rg = m0 / 32 + w;
      const void* src = (rg < RG && ks < NK) ? (const void*)(meta + ((size_t)rg * NK + ks) * 64 + l)
                                             : (const void*)g_dep_zero;
      __builtin_amdgcn_global_load_lds(src, (dep_lds_t)(sb + SP_MOFF + w * 256), 4, 0, 0);
    } else {
      const int c = ((o - 3) * 8 + w) * 64 + l, row = c >> 3, ch = (c & 7) ^ ((row >> 1) & 7);
      const int gn = n0 + row, gk = ks * 64 + ch * 8;
      const void* src = (gn < T && gk < cin) ? (const void*)(Xp + (size_t)gn * cin + gk) : (const void*)g_dep_zero;
      __builtin_amdgcn_global_load_lds(src, (dep_lds_t)(sb + SP_BOFF + ((o - 3) * 8 + w) * 1024), 16, 0, 0);
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

  // fragments of 32-position sub-step p of a stage into register set p; the
  // position word is kept whole (sub-step p uses its half p)
  u32x4 fa[2][FM];
  bf16x16 fb[2][FN];
  uint32_t fm[2][FM];
  auto rd = [&](int stage, int p) {
    const unsigned char* sb = sp_lds + stage * SP_STAGE;
    const u32x4* LA = reinterpret_cast<const u32x4*>(sb);
    const uint32_t* LM = reinterpret_cast<const uint32_t*>(sb + SP_MOFF);
    const uint16_t* LB = reinterpret_cast<const uint16_t*>(sb + SP_BOFF);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      fa[p][i] = LA[((wm * FM + i) * 2 + p) * 64 + l];
      fm[p][i] = LM[(wm * FM + i) * 64 + l];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn * WN + 32 * j + ln;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(&LB[sp_swz(row, 4 * p + h)]);
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(&LB[sp_swz(row, 4 * p + 2 + h)]);
      typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
      fb[p][j] = __builtin_bit_cast(bf16x16, u32x8{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w});
    }
  };
  // the instruction's index-set field picks half p of the position word
  auto mma = [&](int p, int m) {
    const int i = m / FN, j = m % FN;
    const int idx = (int)fm[p][i];
    if (p == 0)
      acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(as_bf16x8(fa[p][i]), fb[p][j], acc[i][j], idx, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(as_bf16x8(fa[p][i]), fb[p][j], acc[i][j], idx, 0, 1);
  };
  // step on stage `stage` (sub-step 0 fragments already in registers): with `load`
  // the tile of K step ks goes to stage `lstage`; with `next` the first
  // fragments of stage `nstage` are read after the barrier. WAIT (steady
  // state): the loads of the RS - 2 tiles after the next one may stay in flight.
  auto step = [&](int stage, int lstage, int ks, int nstage, bool load, bool next, auto WAIT) {
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // sub-step 0's fragments are in
    __builtin_amdgcn_sched_barrier(0);
    rd(stage, 1);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int o = 0; o < NL; ++o)
        if (load && o * NM / NL == m) {
          __builtin_amdgcn_sched_barrier(0);
          issue_one(lstage, ks, o);
          __builtin_amdgcn_sched_barrier(0);
        }
      mma(0, m);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(WAIT)::value) sp_wait_vmcnt<(RS - 2) * NL>();
    else sp_wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (next) rd(nstage, 0);
    __builtin_amdgcn_sched_barrier(0);                     // nothing here waits for those reads
#pragma unroll
    for (int m = 0; m < NM; ++m) mma(1, m);
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: tiles 0 .. RS - 2 (a tile past K reads zeros and is never multiplied)
#pragma unroll
  for (int s = 0; s < RS - 1; ++s)
#pragma unroll
    for (int o = 0; o < NL; ++o) issue_one(s, s, o);
  sp_wait_vmcnt<(RS - 2) * NL>();
  __builtin_amdgcn_s_barrier();
  rd(0, 0);
  int kt = 0;
  for (; kt + 2 * RS - 2 < NK; kt += RS) {                 // RS steady-state steps
#pragma unroll
    for (int s = 0; s < RS; ++s)
      step(s, (s + RS - 1) % RS, kt + s + RS - 1, (s + 1) % RS, true, true, std::true_type{});
  }
  for (; kt < NK; ++kt)                                    // the last steps, all loads retired at each barrier
    step(kt % RS, (kt + RS - 1) % RS, kt + RS - 1, (kt + 1) % RS, kt + RS - 1 < NK, kt + 1 < NK,
         std::false_type{});
  sp_wait_vmcnt<0>();                                      // the zero tiles of a short K

  // lane (h, ln) of block (i, j): token n0 + wn*64 + 32j + ln, rows
  // m0 + wm*64 + 32i + 16h + r (r < 16)
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int o = m0 + wm * WM + 32 * i + 16 * h;
    if (o >= cout) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int tk = n0 + wn * WN + 32 * j + ln;
      if (tk >= T) continue;
      const floatx16 a = acc[i][j];
      u32x4* dst = reinterpret_cast<u32x4*>(Y + (size_t)tk * cout + o);
      dst[0] = u32x4{pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(a[4], a[5]), pack2(a[6], a[7])};
      dst[1] = u32x4{pack2(a[8], a[9]), pack2(a[10], a[11]), pack2(a[12], a[13]), pack2(a[14], a[15])};
    }
  }
}

// ---- launchers ----------------------------------------------------------------------
size_t sparse_vals_bytes(int cout, int cin) { return (size_t)(cout / 32) * (cin / 32) * 64 * 16; }
size_t sparse_meta_bytes(int cout, int cin) { return (size_t)(cout / 32) * ((cin + 63) / 64) * 64 * 4; }

hipError_t launch_sparse_pack(const uint16_t* W, int cout, int cin, int B, const int* perm, const uint32_t* bits,
                              u32x4* vals, uint32_t* meta, hipStream_t s) {
  const long long n = (long long)(cout / 32) * (cin / 32) * 64;
  if (n == 0) return hipSuccess;
  sparse_pack_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(W, cout, cin, B, perm, bits, vals, meta);
  return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* X, int T, int cin, int B, const int* perm, uint16_t* Xp, hipStream_t s) {
  const dim3 grid((cin / 8 + 255) / 256, (T + 15) / 16);
  gather_kernel<<<grid, 256, 0, s>>>(X, T, cin, B, perm, Xp);
  return hipGetLastError();
}

hipError_t launch_spgemm(const u32x4* vals, const uint32_t* meta, const uint16_t* Xp, int T, int cout, int cin,
                         uint16_t* Y, hipStream_t s) {
  const int G = ((cout + SP_BM - 1) / SP_BM) * ((T + SP_BN - 1) / SP_BN);
  spgemm_kernel<SP_RS><<<G, SP_NT, SP_RS * SP_STAGE, s>>>(vals, meta, Xp, T, cout, cin, Y);
  return hipGetLastError();
}

}  // namespace lcp
