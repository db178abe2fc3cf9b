// Device-side helpers shared by the gfx950 kernels of liblcp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- bfloat16 bit helpers -------------------------------------------------
// float -> bf16 bits, round-to-nearest-even (inputs are finite or inf; a NaN
// keeps a quiet NaN pattern).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (lo in bits 0..15), round-to-nearest-even;
// one v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
}
// two floats that are exactly representable in bf16 -> packed pair (upper
// halves, one v_perm_b32)
__device__ __forceinline__ uint32_t pack2_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 32x32x16 bf16 MFMA: acc[r] += sum_k A[l%32][k] B[k][l%32'] with lane l
// holding A row (l%32), K slots 8*(l/32)+e and B column (l%32), K slots
// 8*(l/32)+e; output register r of lane l is row 8*(r/4)+4*(l/32)+(r%4),
// column l%32.
__device__ __forceinline__ floatx16 mfma32(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Row remap used by the fused kernels: MFMA row rho = 8q + 4h + s (q < 4,
// h < 2, s < 4) is given the logical index 16h + 4q + s, so that output
// register r of a lane in half h holds logical row 16h + r (16 consecutive
// rows per lane). remap_row(rho) maps rho -> logical; remap_inv the reverse.
__device__ __host__ __forceinline__ int remap_row(int rho) {
  return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
}
__device__ __host__ __forceinline__ int remap_inv(int k) {
  return 8 * ((k >> 2) & 3) + 4 * (k >> 4) + (k & 3);
}

// ---- transcendental helpers (base 2, hardware v_exp_f32 / v_log_f32) --------
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_(float x) { return __builtin_amdgcn_logf(x); }

// ---- N:M keep decision ------------------------------------------------------
// Position k of a group is kept iff
//   #{j: v_j > v_k} + #{j < k: v_j == v_k} < N
// (ties to the lower position). NaN is read as -inf (IEEE max returns the
// non-NaN operand); IEEE compares treat -0 == +0. With NaN gone, for j < k
// the pair contributes [v_j >= v_k] to k's rank and the complement
// [v_k > v_j] to j's, so each pair is compared once. Returns an M-bit mask,
// bit k = kept.
__device__ __forceinline__ float nan_to_ninf(float v) { return __builtin_fmaxf(v, -__builtin_inff()); }

template <int M>
__device__ __forceinline__ uint32_t nm_keep(const float* v, int N) {
  int rank[M];
#pragma unroll
  for (int k = 0; k < M; ++k) rank[k] = 0;
#pragma unroll
  for (int k = 1; k < M; ++k)
#pragma unroll
    for (int j = 0; j < k; ++j) {
      const int c = v[j] >= v[k];
      rank[k] += c;
      rank[j] += 1 - c;
    }
  uint32_t bits = 0;
#pragma unroll
  for (int k = 0; k < M; ++k) bits |= (uint32_t)(rank[k] < N) << k;
  return bits;
}

// M = 4 with N fixed at compile time, for scores that cannot be -inf (sums
// of non-negative products: every value is in [+0, +inf] or NaN). Same rule
// as nm_keep with NaN read as -inf: for j < k, j outranks k iff
// v_j >= v_k or v_k is NaN (a NaN v_j cannot reach a finite v_k, and no
// v_k is -inf). The comparisons become wave-wide 64-bit ballots; beats[k]
// lists the three events "another position outranks k", k is kept iff fewer
// than N of them hold, evaluated with scalar 64-bit and/or/not, and
// inverse_ballot hands each lane its own bit back as a condition. Every lane
// of the wave must be active.
template <int N>
__device__ __forceinline__ void nm_keep4_nonneg(const float* v, bool* keep) {
  typedef unsigned long long u64;
  const u64 n1 = __builtin_amdgcn_ballot_w64(__builtin_isnan(v[1]));
  const u64 n2 = __builtin_amdgcn_ballot_w64(__builtin_isnan(v[2]));
  const u64 n3 = __builtin_amdgcn_ballot_w64(__builtin_isnan(v[3]));
  const u64 c01 = __builtin_amdgcn_ballot_w64(v[0] >= v[1]) | n1;
  const u64 c02 = __builtin_amdgcn_ballot_w64(v[0] >= v[2]) | n2;
  const u64 c03 = __builtin_amdgcn_ballot_w64(v[0] >= v[3]) | n3;
  const u64 c12 = __builtin_amdgcn_ballot_w64(v[1] >= v[2]) | n2;
  const u64 c13 = __builtin_amdgcn_ballot_w64(v[1] >= v[3]) | n3;
  const u64 c23 = __builtin_amdgcn_ballot_w64(v[2] >= v[3]) | n3;
  const u64 beats[4][3] = {{~c01, ~c02, ~c03}, {c01, ~c12, ~c13}, {c02, c12, ~c23}, {c03, c13, c23}};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u64 x = beats[k][0], y = beats[k][1], z = beats[k][2];
    u64 kept;
    if (N == 1) kept = ~(x | y | z);
    else if (N == 2) kept = ~((x & y) | (x & z) | (y & z));
    else kept = ~(x & y & z);
    keep[k] = __builtin_amdgcn_inverse_ballot_w64(kept);
  }
}

// ---- wave helpers -------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Lane moves inside a row of 16 lanes (DPP): CTRL 0xB1 / 0x4E swap lanes at
// distance 1 / 2 inside each quad, 0x141 mirrors each half row (i <-> 7 - i),
// 0x140 mirrors the row (i <-> 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum / max over the 16 lanes of each row. Every lane of the row ends with the
// same float: at each step the two lanes of a pair hold the same partials and
// add them in opposite order, which gives the same result.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v + dpp<0x140>(v);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  return fmaxf(v, dpp<0x140>(v));
}
// Pair lane l with l ^ 16 (permlane16 swap) or l ^ 32 (permlane32 swap) and
// combine as (lower lane) op (upper lane), so both lanes get the same value.
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace lcp
