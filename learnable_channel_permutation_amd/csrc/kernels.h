// Host-side launchers of the gfx950 kernels (internal to liblcp). Every
// launcher enqueues on `s` and returns hipGetLastError() after the launch;
// argument validation is done by the C ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "frag.h"

namespace lcp {

// Work split of the block adjoint (see below).
struct AdjSplit {
  int grid, tpw, tpb, maxseg;
};

// Sinkhorn (sinkhorn.hip). With fwd != nullptr the forward also writes the
// MFMA operand fragments of P (frag.h): fwd [nb][frag_fwd_entries(B)] from P
// and the column norms n, adj [nb][frag_adj_entries(B)].
hipError_t launch_sinkhorn_fwd(const float* logits, float* P, float* off, int nb, int B,
                               int iters, float tau, const float* n, u32x4* fwd, u32x4* adj,
                               hipStream_t s);
// AdamW update applied to the logits (state m, v in fp32); bc1 = 1 - b1^t,
// bc2 = 1 - b2^t for step t.
struct AdamW {
  float* param;
  float* m;
  float* v;
  float lr, b1, b2, eps, wd, bc1, bc2;
};
// dP is either dense [nb][B][B] (seg == nullptr), the block adjoint's
// (workgroup, segment) partials described by seg, summed in workgroup order,
// or, with seg->tpw < 0, seg->grid row-panel partials [panel][nb][B][B]
// summed in panel order (the fused dD adjoint).
// dlogits may be null when opt is given; with opt the kernel also applies
// AdamW to opt->param (the logits themselves, updated in place).
hipError_t launch_sinkhorn_bwd(const float* logits, const float* dP, const AdjSplit* seg,
                               const float* off, float* dlogits, int nb, int B, int iters,
                               float tau, const AdamW* opt, hipStream_t s);
// Standalone AdamW over n elements.
hipError_t launch_adamw(const float* grad, int n, const AdamW& opt, hipStream_t s);

// Hardening (harden.hip): per block the permutation maximising Tr(P^T P_hat).
// Any of P_hard ([nb][B][B] 0/1 fp32), perm ([nb][B]: source row of each
// position) and the fragment sets (with the norms n) may be null.
hipError_t launch_harden(const float* P, int nb, int B, float* P_hard, int* perm, const float* n, u32x4* fwd,
                         u32x4* adj, hipStream_t s);

// Per-layer setup (layer.hip): column norms, optional bf16 transpose.
hipError_t launch_colnorm_f32(const float* X, int T, int cin, float* norms, hipStream_t s);
hipError_t launch_layer_init_bf16(const uint16_t* X, int T, int cin, int pitch, float* norms,
                                  uint16_t* Xt, hipStream_t s);

// N:M mask from fp32 scores (mask.hip).
hipError_t launch_nm_mask(const float* scores, int rows, int cin, int N, int M, uint32_t* bits,
                          hipStream_t s);
// The step keeps its mask block-major, [nb][rows][B / 32] words, so that a
// 32-row tile's words are contiguous; this converts to [rows][cin / 32].
hipError_t launch_bits_rowmajor(const uint32_t* bm, int rows, int cin, int B, uint32_t* out, hipStream_t s);

// Block permutation kernels (permute.hip).
enum PermMode {
  PERM_PLAIN = 0,       // out = A P_B (or A P_B^T)
  PERM_IMPORTANCE = 1,  // out = (|A| colscale) P_B, fp32, float32-accurate
  PERM_FWD = 2          // D = W - ((W P_B) . M) P_B^T and mask bits from (|W| n) P_B
};
// gfrag (nullable, forward mode only): precomputed fragments (frag.h).
hipError_t launch_permute_bf16(const uint16_t* A, int rows, int cin, const float* colscale,
                               const float* P, int B, int transposeP, const u32x4* gfrag, int mode,
                               void* out, int out_f32, uint32_t* bits, int N, int M, hipStream_t s);

hipError_t launch_permute_f32(const float* A, int rows, int cin, const float* colscale,
                              const float* P, int B, int transposeP, int mode, float* out,
                              uint32_t* bits, int N, int M, hipStream_t s);
hipError_t launch_diff(const void* W, const void* Wt, int n, int bf16, void* D, hipStream_t s);

// GEMMs (gemm.hip). C[m][n] = sum_k A[m][k] B[n][k].
// Error epilogue: store C (bf16 or f32, ldc) for n < n_store and write one
// partial sum of squares per workgroup to part[] (gemm_error_parts of them).
// With Y non-null (a matrix of C's layout and ldc) it also writes one partial
// of sum Y . C per workgroup to party[].
int gemm_error_parts(int M, int N, int bf16);
hipError_t launch_gemm_error_bf16(const uint16_t* A, int lda, const uint16_t* Bm, int ldb, int M,
                                  int N_valid, int N_store, int K, uint16_t* C, int ldc,
                                  float* part, const uint16_t* Y, float* party, hipStream_t s);
hipError_t launch_gemm_error_f32(const float* A, int lda, const float* Bm, int ldb, int M,
                                 int N_valid, int N_store, int K, float* C, int ldc, float* part,
                                 const float* Y, float* party, hipStream_t s);
// dD epilogue: C = coef[1] * acc, coef in device memory (written by a
// finalisation kernel: -1/E for the Frobenius objective, 1 for the cosine).
hipError_t launch_gemm_dd_bf16(const uint16_t* A, int lda, const uint16_t* Bm, int ldb, int M,
                               int N, int K, const float* coef, uint16_t* C, int ldc, hipStream_t s);
// dD GEMM with the block adjoint fused into its epilogue (bf16, B = 64,
// N % 64 == 0): G = coef[1] A B^T is not stored; each 256-row panel tm writes
// part[(tm * (N / 64) + b) * 64 * 64] = sum over its rows of
// G_b^T A_b + W_b^T ((G_b P_b) . M_b) (row-major [j][k]), with frag the
// adjoint P fragments and bits the block-major mask words. dd_adjoint_panels
// gives the number of panels.
int dd_adjoint_panels(int M);
hipError_t launch_gemm_dd_adjoint_bf16(const uint16_t* A, int lda, const uint16_t* Bm, int ldb, int M, int N, int K,
                                       const float* coef, const uint16_t* W, const u32x4* frag, const uint32_t* bits,
                                       float* part, hipStream_t s);
// f32 dD: C[m][n] = coef[1] sum_t R[m][t] X[t][n]  (X row-major [K][N]).
hipError_t launch_gemm_dd_f32(const float* R, int ldr, const float* X, int ldx, int M, int N,
                              int K, const float* coef, float* C, int ldc, hipStream_t s);
// E = sqrt(sum part) to err and E_ws[0]; E_ws[1] = -1/E (0 when E == 0).
hipError_t launch_error_finalize(const float* part, int nparts, float* E_ws, float* err,
                                 hipStream_t s);
// out = sum part (fixed order).
hipError_t launch_sum_finalize(const float* part, int nparts, float* out, hipStream_t s);

// Cosine objective (cosine.hip). From r = sum part (||R||^2), a = sum party
// (<Y, R>) and y2 = ||Y||^2 with R = Y - Y~: err = 1 - <Y, Y~> / (|Y| |Y~|),
// coef[0] = sqrt(r), coef[1] = 1 (dD factor), coef[2], coef[3] = the
// coefficients of Y and R in dL/dY~ (all zero when |Y| |Y~| == 0).
hipError_t launch_cosine_finalize(const float* part, const float* party, int nparts, const float* y2,
                                  float* coef, float* err, hipStream_t s);
// dY~ = coef[2] Y + coef[3] R over n elements (n % 8 == 0, 16-byte aligned).
hipError_t launch_cosine_grad(const void* Y, const void* R, size_t n, int bf16, const float* coef, void* out,
                              hipStream_t s);

// Block adjoint (adjoint.hip). Workgroup g of the fixed grid takes tiles
// [g*tpw, (g+1)*tpw) of the block-major 32-row tile sequence (tpb per block)
// and writes one partial B x B matrix per block it touches to
// part[(g * maxseg + (block - first block of g)) * B * B].
AdjSplit adjoint_split(int cout, int cin, int B);
// ste_norms non-null adds the straight-through term of the mask,
// S_b^T ((G_b P_b) . (W_b P_b)) with S = |W| . ste_norms[col].
hipError_t launch_adjoint_bf16(const uint16_t* G, const uint16_t* W, const u32x4* gfrag, const float* P,
                               const uint32_t* bits, int cout, int cin, int B, const AdjSplit& sp,
                               const float* ste_norms, float* part, hipStream_t s);
hipError_t launch_adjoint_f32(const float* G, const float* W, const float* P,
                              const uint32_t* bits, int cout, int cin, int B, const AdjSplit& sp,
                              const float* ste_norms, float* part, hipStream_t s);

// Deploy path (deploy.hip), bf16: packed 2:4 weights in fragment order,
// channel gather, sparse GEMM Y[t][o] = sum_k Ws[o][k] Xp[t][k]. perm is
// [nb][B] (entries taken mod B, B a power of two); bits row-major
// [cout][cin/32]; cout % 32 == 0, cin % 32 == 0.
size_t sparse_vals_bytes(int cout, int cin);
size_t sparse_meta_bytes(int cout, int cin);
hipError_t launch_sparse_pack(const uint16_t* W, int cout, int cin, int B, const int* perm, const uint32_t* bits,
                              u32x4* vals, uint32_t* meta, hipStream_t s);
hipError_t launch_gather(const uint16_t* X, int T, int cin, int B, const int* perm, uint16_t* Xp, hipStream_t s);
hipError_t launch_spgemm(const u32x4* vals, const uint32_t* meta, const uint16_t* Xp, int T, int cout, int cin,
                         uint16_t* Y, hipStream_t s);

}  // namespace lcp
