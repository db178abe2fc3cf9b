/*
 * lcp.h - C ABI of the MI355X (gfx950) learnable-channel-permutation library.
 *
 * One LCP step on one linear layer, as defined on the pages "PermLLM: Learnable
 * Channel Permutation for N:M Sparse Large Language Models" (summary of arXiv
 * 2510.10136; cited below as [PermLLM]) and the blog post "PermLLM: 动态通道置换
 * 优化N:M稀疏大模型" (cited as [blog]):
 *
 *   logits L (nb x B x B, fp32) --Sinkhorn--> P (soft block permutations)
 *   W_hat = W P_B,  S_hat = S P_B with S = |W| . ||X_col||_2   (importance)
 *   M = N:M top-N of S_hat per row and group of M permuted positions
 *   W_tilde = (W_hat . M) P_B^T,  D = W - W_tilde,  R = D X^T,  E = ||R||_F
 *   backward: dE/dL through the block permutation and the unrolled Sinkhorn,
 *   with the mask held constant.
 * Options of the step (lcp_cfg): the hardened forward of [PermLLM] Method 2;
 * the cosine objective of [PermLLM] (optimisation objective) in place of E;
 * the straight-through gradient of the mask's argmax ([PermLLM] integration
 * with pruning methods).
 *
 * Conventions shared by every entry point:
 *   - Matrices are row-major. W is Cout x Cin (like a linear layer), X is
 *     T x Cin (tokens x channels). Block b covers channels [bB, (b+1)B).
 *   - P_b[j][k]: row j is source channel bB+j, column k is permuted position
 *     bB+k; so W_hat[:, bB+k] = sum_j W[:, bB+j] P_b[j][k].
 *   - Every pointer argument is a device pointer owned by the caller, except
 *     the lcp_layer / lcp_cfg / lcp_timing structs and size_t* outputs, which
 *     live in host memory. The library never allocates, frees or synchronises,
 *     holds no global mutable state and is reentrant (the one exception is the
 *     fixed device scratch of lcp_layer_outputs_noalloc, described there). Work is enqueued on the
 *     given HIP stream (a hipStream_t passed as void*; NULL = null stream) and
 *     runs asynchronously.
 *   - Inputs are never written. Outputs are fully overwritten.
 *   - All arguments are validated before the first launch: an error code means
 *     nothing was enqueued and nothing written. Results are deterministic
 *     (no atomics in reductions): equal inputs give bitwise-equal outputs.
 *   - Sizes are limited to what 32-bit element indices of one matrix hold
 *     (rows * cols < 2^31); for BF16 layers W and X (and every bf16 matrix a
 *     GEMM reads) must also stay below 2^30 elements (2 GB), else
 *     LCP_E_INVAL.
 */
#ifndef LCP_H
#define LCP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define LCP_OK             0
#define LCP_E_INVAL       -1  /* null pointer, non-positive size, Cin % B, B % M,
                                 N outside [1, M-1], iters < 1, tau not finite
                                 or <= 0, Cin % 32 for mask words            */
#define LCP_E_UNSUPPORTED -2  /* B not in {32, 64, 128}, M not in {4, 8},
                                 iters * B > LCP_MAX_ITERS_B, unknown dtype,
                                 or a dtype/mode combination the library
                                 does not implement                          */
#define LCP_E_WORKSPACE   -3  /* workspace smaller than the size query says,
                                 or not 256-byte aligned                      */
#define LCP_E_HIP         -4  /* a kernel launch reported a HIP error         */
#define LCP_E_SCRATCH     -5  /* the input needs more than the fixed scratch
                                 of an allocation-free entry point            */

/* Largest iters * B the Sinkhorn kernels accept: the reverse pass keeps the
 * 2 * iters * B fp32 row and column offsets of every iteration of one block in
 * LDS (64 KB at the limit), so B = 128 allows up to 64 iterations, B = 64 up
 * to 128 and B = 32 up to 256. Larger products return LCP_E_UNSUPPORTED from
 * lcp_sinkhorn, lcp_sinkhorn_bwd and every step entry point, before any
 * launch. */
#define LCP_MAX_ITERS_B 8192

typedef enum lcp_dtype {
  LCP_F32 = 0,   /* IEEE binary32 */
  LCP_BF16 = 1   /* bfloat16 (upper half of binary32), round-to-nearest-even */
} lcp_dtype;

/* One layer and its calibration data (host struct holding device pointers). */
typedef struct lcp_layer {
  const void*  W;      /* [cout][cin], dtype                                  */
  const void*  X;      /* [T][cin], dtype                                     */
  const void*  Xt;     /* BF16 layers: [cin][lcp_xt_pitch(T)] bf16, written by
                          lcp_layer_init (X transposed, zero beyond T); used
                          by the backward. May be NULL for F32 layers.        */
  const float* norms;  /* [cin] ||X[:, j]||_2, written by lcp_layer_init      */
  const void*  Y;      /* cosine objective only (else may be NULL): the dense
                          outputs W X^T, [cout][lcp_xt_pitch(T)] dtype, zero
                          beyond column T, written by lcp_layer_outputs      */
  const float* y2;     /* cosine objective only: 1 fp32, ||Y||_F^2, written by
                          lcp_layer_outputs                                   */
  lcp_dtype    dtype;
  int          cout, cin, T;
  int          B;      /* block size, 32, 64 or 128; cin % B == 0            */
} lcp_layer;

/* Objectives (lcp_cfg.loss). */
#define LCP_LOSS_FROBENIUS 0  /* E = ||(W - W_tilde) X^T||_F                  */
#define LCP_LOSS_COSINE    1  /* [PermLLM] optimisation objective
                                 1 - y.y~ / (||y|| ||y~||) with y = vec(W X^T),
                                 y~ = vec(W_tilde X^T): one cosine over the
                                 layer's whole output; 1 (gradient 0) when
                                 either norm is 0                            */

/* Hyper-parameters of one step. */
typedef struct lcp_cfg {
  int   iters;  /* Sinkhorn iterations L >= 1 (one = row step then column step),
                   iters * B <= LCP_MAX_ITERS_B                                 */
  float tau;    /* temperature > 0                                              */
  int   N, M;   /* keep N of every M; M in {4, 8}, 1 <= N < M, B % M == 0       */
  int   harden; /* 0: the step uses the soft P_hat. 1: the forward uses the
                   hardened P of lcp_harden ([PermLLM] Method 2) and the
                   backward is straight-through: dE/dP at the hard P is handed
                   unchanged to the adjoint of the soft Sinkhorn.              */
  int   loss;   /* LCP_LOSS_FROBENIUS or LCP_LOSS_COSINE (needs L->Y, L->y2)  */
  int   mask_ste; /* 0: the mask is constant in the backward. 1: the gradient
                   reaching the 0/1 mask, (G_b P_b) . W_hat_b with
                   G = dL/dW_tilde, is handed unchanged to the permuted scores
                   S_hat_b = S_b P_b (straight-through estimator for the
                   argmax), adding S_b^T ((G_b P_b) . (W_b P_b)) to dL/dP_b;
                   S = |W| . norms. Under harden every P here is the hard P. */
} lcp_cfg;

/* Optional per-kernel timing hooks: hipEvent_t handles (as void*) recorded on
 * the step's stream immediately before (start[i]) and after (stop[i]) kernel i
 * of the step. NULL entries are skipped; a NULL lcp_timing* records nothing.
 * Forward kernels: 0 Sinkhorn, 1 permute+mask+unpermute, 2 error GEMM,
 * 3 error (or cosine) finalisation, 4 hardening (harden = 1 only). Backward
 * kernels: 0 dD GEMM, 1 block adjoint, 2 Sinkhorn adjoint, 3 cosine
 * gradient dL/dY~ (cosine objective only). For BF16 layers with B = 64 and
 * mask_ste = 0 the block adjoint runs inside the dD GEMM's epilogue: kernel 0
 * is then both, and nothing runs between start[1] and stop[1]. */
typedef struct lcp_timing {
  void* start[8];
  void* stop[8];
} lcp_timing;

/* Static description of a status code. */
const char* lcp_status_string(int code);

/* Library version, major * 10000 + minor * 100 + patch. */
int lcp_version(void);

/* ---------------------------------------------------------------------------
 * lcp_sinkhorn - soft permutations P = S_L(L / tau), batched over nb blocks.
 * [PermLLM] Method 1: S_0(X) = exp(X), S_i(X) = T_c(T_r(S_{i-1}(X))), with the
 * log-domain form of [blog] section 2.2 (subtract the row log-sum-exp, then the
 * column log-sum-exp, each iteration; exp at the end).
 *   logits: [nb][B][B] fp32 in;  P: [nb][B][B] fp32 out (may alias logits).
 *   B in {32, 64, 128}; iters >= 1 and iters * B <= LCP_MAX_ITERS_B (else
 *   LCP_E_UNSUPPORTED); tau finite and > 0.
 */
int lcp_sinkhorn(const float* logits, float* P, int nb, int B, int iters,
                 float tau, void* stream);

/* lcp_sinkhorn_bwd - reverse pass of lcp_sinkhorn: given dE/dP (fp32
 * [nb][B][B]) returns dE/dlogits (fp32 [nb][B][B]). The forward iterations are
 * recomputed from the logits; the derivative of each normalisation follows
 * from [PermLLM] Method 1 by the chain rule. dlogits must not alias dP.
 * Same limits as lcp_sinkhorn (iters * B <= LCP_MAX_ITERS_B). */
int lcp_sinkhorn_bwd(const float* logits, const float* dP, int nb, int B,
                     int iters, float tau, float* dlogits, void* stream);

/* lcp_harden - per block, the permutation matrix P maximising Tr(P^T P_hat)
 * ([PermLLM] Method 2: the hard permutation used in the forward pass), i.e.
 * the maximum-weight assignment of source channels j (rows) to permuted
 * positions k (columns). Exact (shortest augmenting paths in double
 * precision); among equally good assignments the result is deterministic.
 *   P: [nb][B][B] fp32 in (finite entries);
 *   P_hard (nullable): [nb][B][B] fp32 out, 1 where assigned, else 0;
 *   perm (nullable): [nb][B] int32 out, perm[b][k] = the row j assigned to
 *   column k. At least one output; P_hard must not alias P; P and P_hard
 *   16-byte aligned. B in {32,64,128}.
 */
int lcp_harden(const float* P, int nb, int B, float* P_hard, int32_t* perm,
               void* stream);

/* ---------------------------------------------------------------------------
 * lcp_colnorm - norms[j] = ||X[:, j]||_2 over the T tokens, fp32 accumulation.
 * The column norm is the activation factor of Wanda's importance, the one-shot
 * method [PermLLM] integrates with (its formula is not printed there).
 *   X: [T][cin] in dtype dt;  norms: [cin] fp32 out.
 */
int lcp_colnorm(const void* X, lcp_dtype dt, int T, int cin, float* norms,
                void* stream);

/* Row pitch (elements) of the transposed activations Xt and of the internal
 * residual R: T rounded up to a multiple of 64. Returns -1 for T <= 0. */
int lcp_xt_pitch(int T);

/* lcp_layer_init - per-layer setup, constant across LCP steps on one layer:
 * column norms and, for BF16, Xt[c][t] = X[t][c] (t < T) and 0 for
 * T <= t < lcp_xt_pitch(T).
 *   X: [T][cin] dtype in; norms: [cin] fp32 out; Xt: bf16 [cin][pitch] out
 *   (required for BF16, ignored and may be NULL for F32). cin % 32 == 0. */
int lcp_layer_init(const void* X, lcp_dtype dt, int T, int cin, float* norms,
                   void* Xt, void* stream);

/* ---------------------------------------------------------------------------
 * lcp_permute - block-wise permutation of the columns of A ([PermLLM]
 * Method 3: P_B = diag(P_1 .. P_nb), W_hat_B = W P_B; and the permuted
 * importance S_hat = S P_B of the integration formula).
 *   out[:, bB+k] = sum_j At[:, bB+j] * Pb[j][k]   with Pb = P_b, or Pb = P_b^T
 *   when transposeP != 0; At = A, or At = |A| * colscale[col] when colscale is
 *   non-NULL (importance mode).
 *   A: [rows][cin] adt; P: [nb][B][B] fp32; out: [rows][cin] odt.
 *   Importance mode requires odt == LCP_F32 and computes with float32-accurate
 *   accumulation. BF16 A in plain mode rounds P to bf16 as the MFMA operand.
 */
int lcp_permute(const void* A, lcp_dtype adt, int rows, int cin,
                const float* colscale, const float* P, int B, int transposeP,
                void* out, lcp_dtype odt, void* stream);

/* lcp_nm_mask - N:M mask from scores ([PermLLM] integration formula:
 * argmax_M sum (M . S_hat)_{i, kM:(k+1)M}; [blog] 2.1: keep the N largest of
 * every M consecutive positions). For every row and group g of positions
 * gM .. gM+M-1, position k is kept iff
 *   #{j in g : s_j > s_k} + #{j in g, j < k : s_j == s_k} < N,
 * i.e. ties go to the lower position, NaN ranks as -inf and -0 == +0.
 *   scores: [rows][cin] fp32; bits: [rows][cin/32] uint32 out, bit (k mod 32)
 *   of word k/32 is position k, 1 = kept. cin % 32 == 0, M in {4, 8}. */
int lcp_nm_mask(const float* scores, int rows, int cin, int N, int M,
                uint32_t* bits, void* stream);

/* ---------------------------------------------------------------------------
 * lcp_error - output error of a pruned weight on the calibration tokens:
 *   *err = ||(W - Wt) X^T||_F   (fp32 scalar written to device memory).
 * The [PermLLM] task definition asks for the permuted, pruned weight whose
 * layer outputs stay closest to the dense layer's; this is that distance.
 *   W, Wt: [cout][cin] dt; X: [T][cin] dt; err: 1 fp32 out;
 *   R_out (nullable): the residual (W - Wt) X^T, [cout][lcp_xt_pitch(T)] in dt
 *   (columns T .. pitch-1 are zero). BF16 computes D = W - Wt in fp32, rounds
 *   it to bf16 and multiplies with bf16 MFMA and fp32 accumulation; the norm
 *   is taken over the fp32 accumulators. ws: lcp_error_workspace_bytes bytes. */
int lcp_error_workspace_bytes(int cout, int cin, int T, lcp_dtype dt,
                              size_t* bytes);
int lcp_error(const void* W, const void* Wt, const void* X, lcp_dtype dt,
              int cout, int cin, int T, float* err, void* R_out, void* ws,
              size_t ws_bytes, void* stream);

/* lcp_layer_outputs - per-layer constants of the cosine objective ([PermLLM]
 * optimisation objective compares the dense outputs y with the sparse ones):
 *   Y = W X^T, [cout][lcp_xt_pitch(T)] in dt (columns T .. pitch-1 written 0);
 *   *y2 = ||Y||_F^2 (fp32, device), summed over the fp32 accumulators.
 * BF16 multiplies with bf16 MFMA and fp32 accumulation and rounds Y to bf16.
 *   W: [cout][cin] dt; X: [T][cin] dt; all 16-byte aligned; cin % 32 == 0.
 *   ws: lcp_error_workspace_bytes(cout, cin, T, dt) bytes (256-aligned). */
int lcp_layer_outputs(const void* W, const void* X, lcp_dtype dt, int cout,
                      int cin, int T, void* Y, float* y2, void* ws,
                      size_t ws_bytes, void* stream);

/* lcp_layer_outputs_noalloc - lcp_layer_outputs without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments minus
 * ws / ws_bytes, same kernels, bit-identical Y and *y2.
 * The partial sums of ||Y||^2 (one fp32 per GEMM workgroup) live in a fixed
 * device array inside the library, LCP_NOALLOC_MAX_PARTS floats (64 KB),
 * which every GPU the library runs on holds until the process ends. The
 * partial count is ceil(cout / 256) * ceil(pitch / 128) for BF16 and
 * ceil(cout / ts) * ceil(pitch / ts) for F32 (ts = 64, or 32 when 64-wide
 * tiles would number fewer than 128), pitch = lcp_xt_pitch(T); a shape that
 * needs more returns LCP_E_SCRATCH before any launch (a 4096 x 11008 BF16
 * layer with 2048 tokens needs 256). The first call on a device looks the array's
 * address up with that device current (the current HIP device must be the
 * stream's). Nothing is allocated, freed or cleared: each workgroup
 * overwrites its own partial. All calls on one GPU share the array, so calls
 * that overlap on one GPU (other streams or threads) race; calls ordered on
 * one stream do not. */
#define LCP_NOALLOC_MAX_PARTS 16384
int lcp_layer_outputs_noalloc(const void* W, const void* X, lcp_dtype dt,
                              int cout, int cin, int T, void* Y, float* y2,
                              void* stream);

/* ---------------------------------------------------------------------------
 * Full step. The workspace carries the forward's saved state (P, Sinkhorn
 * offsets, mask bits, residual R, E) to the backward; it must not be touched
 * between lcp_step_fwd and the matching lcp_step_bwd, and one workspace
 * serves one step in flight at a time.
 */
int lcp_step_workspace_bytes(int cout, int cin, int T, int B, int iters,
                             lcp_dtype dt, size_t* bytes);

/* lcp_step_fwd - Sinkhorn, (hardening,) permute, importance, N:M mask,
 * un-permute, difference, error GEMM: *err = the objective of c->loss (E, or
 * the cosine loss). Optional copies: P_out
 * [nb][B][B] fp32 (the P the forward used: P_hat, or the hard P when
 * c->harden), bits_out [cout][cin/32] uint32 (the mask in permuted
 * positions). */
int lcp_step_fwd(const lcp_layer* L, const float* logits, const lcp_cfg* c,
                 void* ws, size_t ws_bytes, float* err, float* P_out,
                 uint32_t* bits_out, const lcp_timing* tm, void* stream);

/* lcp_step_bwd - dlogits = dL/dlogits ([nb][B][B] fp32) of the objective L of
 * c->loss, with the mask of the matching lcp_step_fwd held constant unless
 * c->mask_ste; zero when E == 0 (Frobenius) or when ||Y|| ||Y~|| == 0
 * (cosine). c must equal the forward's. Needs L->Xt for BF16 layers. */
int lcp_step_bwd(const lcp_layer* L, const float* logits, const lcp_cfg* c,
                 void* ws, size_t ws_bytes, float* dlogits,
                 const lcp_timing* tm, void* stream);

/* ---------------------------------------------------------------------------
 * Optimiser step on the logits: AdamW ([PermLLM] implementation details:
 * AdamW, learning rate 1e-3 or 5e-3, temperature annealed linearly from 1 to
 * 0.1 by the caller through lcp_cfg.tau). Decoupled weight decay (Loshchilov
 * and Hutter): for step t >= 1,
 *   m = b1 m + (1 - b1) g,  v = b2 v + (1 - b2) g^2,
 *   p = p (1 - lr wd) - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
 * m and v are fp32 state owned by the caller (zero before step 1).
 */
typedef struct lcp_adamw_cfg {
  float lr;            /* >= 0                                                  */
  float beta1, beta2;  /* in [0, 1)                                             */
  float eps;           /* > 0                                                   */
  float weight_decay;  /* >= 0                                                  */
} lcp_adamw_cfg;

/* lcp_adamw - one update of n fp32 parameters from the gradient grad; param,
 * m and v are updated in place (distinct buffers; grad may alias none). */
int lcp_adamw(float* param, const float* grad, float* m, float* v, int n,
              int t, const lcp_adamw_cfg* oc, void* stream);

/* lcp_step_bwd_adamw - lcp_step_bwd followed by the AdamW update of the
 * logits, fused into the Sinkhorn adjoint's last pass (the gradient is not
 * written to memory unless dlogits is non-NULL). logits ([nb][B][B] fp32) is
 * updated in place; m and v are [nb][B][B] fp32 state; all three 16-byte
 * aligned and distinct. */
int lcp_step_bwd_adamw(const lcp_layer* L, float* logits, const lcp_cfg* c,
                       void* ws, size_t ws_bytes, float* m, float* v, int t,
                       const lcp_adamw_cfg* oc, float* dlogits,
                       const lcp_timing* tm, void* stream);

/* lcp_train - `steps` optimisation steps of one layer's logits in place:
 * for t = 0 .. steps-1, tau_t = tau0 + (tau1 - tau0) t / (steps - 1), then
 * lcp_step_fwd (its objective written to errs[t], device fp32) and
 * lcp_step_bwd_adamw with AdamW step t + 1. c->iters, N, M, harden, loss and
 * mask_ste apply to every step (the
 * pages train with the hardened forward); c->tau is ignored. m, v: AdamW
 * state as for lcp_step_bwd_adamw. Arguments are validated before the first
 * step; a launch error stops the loop and is returned. */
int lcp_train(const lcp_layer* L, float* logits, const lcp_cfg* c, void* ws,
              size_t ws_bytes, float* m, float* v, int steps, float tau0,
              float tau1, const lcp_adamw_cfg* oc, float* errs, void* stream);

/* ---------------------------------------------------------------------------
 * Deploy path of a trained layer ([PermLLM] inference acceleration: a
 * channel-permutation kernel applied to the activations at inference time and
 * the N:M-sparse layer). With the hard permutation perm ([nb][B] int32,
 * perm[b][k] = source channel of position bB + k, as lcp_harden writes it)
 * and the 2:4 mask in permuted positions (bits, [cout][cin/32] uint32 as
 * lcp_step_fwd's bits_out), the deployed layer computes
 *   Y = Xp Ws^T,  Xp[t][bB+k] = X[t][bB+perm[b][k]],  Ws = (W P_B) . M,
 * which equals X W_tilde^T. BF16 only; 2:4 only (the sparse matrix cores'
 * format); cout % 32 == 0, cin % 32 == 0, cin % B == 0. perm entries are
 * read modulo B (B is a power of two), so every access stays inside its
 * block; an entry that is not a permutation gives a wrong but bounded result.
 *
 * Packed weights (opaque to callers; produced by lcp_sparse_pack): vals
 * holds, per 32-row x 32-position fragment, the 64 lane operands of the
 * gfx950 sparse MFMA (each lane: one row, 16 positions, the 2 kept values of
 * each group of 4, lower position first); meta holds the 2-bit positions,
 * 16 bits per lane and fragment, two fragments per uint32.
 */
int lcp_sparse_pack_bytes(int cout, int cin, size_t* vals_bytes,
                          size_t* meta_bytes);

/* lcp_sparse_pack - pack W (bf16 [cout][cin]) permuted by perm and masked by
 * bits into (vals, meta). Groups of 4 whose mask does not keep exactly 2
 * positions are packed with their first two kept positions, completed by
 * the lowest free positions with value 0. vals 16-byte aligned, meta 4-byte
 * aligned, sizes from lcp_sparse_pack_bytes. */
int lcp_sparse_pack(const void* W, int cout, int cin, int B,
                    const int32_t* perm, const uint32_t* bits, void* vals,
                    uint32_t* meta, void* stream);

/* lcp_gather_channels - Xp[t][bB+k] = X[t][bB+perm[b][k]] (bf16 [T][cin]
 * both; Xp 16-byte aligned, not aliasing X): the channel permutation of the
 * activations. */
int lcp_gather_channels(const void* X, int T, int cin, int B,
                        const int32_t* perm, void* Xp, void* stream);

/* lcp_sparse_gemm - Y[t][o] = sum_k Ws[o][k] Xp[t][k] on the 2:4 sparse
 * matrix cores: Xp bf16 [T][cin], Y bf16 [T][cout] (fp32 accumulation, one
 * rounding), vals/meta from lcp_sparse_pack. Y, Xp, vals 16-byte aligned. */
int lcp_sparse_gemm(const void* vals, const uint32_t* meta, const void* Xp,
                    int T, int cout, int cin, void* Y, void* stream);

/* lcp_deploy_forward - lcp_gather_channels into the caller's buffer Xp
 * (bf16 [T][cin]) followed by lcp_sparse_gemm: the deployed layer's output
 * Y (bf16 [T][cout]) for activations X (bf16 [T][cin]). */
int lcp_deploy_forward(const void* vals, const uint32_t* meta,
                       const int32_t* perm, int B, const void* X, int T,
                       int cout, int cin, void* Xp, void* Y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LCP_H */
