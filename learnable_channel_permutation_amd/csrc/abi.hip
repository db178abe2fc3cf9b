// C ABI of liblcp: argument validation, workspace layout and the order of the
// kernels of one LCP step. Every check runs before the first launch, so an
// error return means nothing was enqueued.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/lcp.h"
#include "kernels.h"

using namespace lcp;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxIterB = LCP_MAX_ITERS_B;   // iters * B bound (Sinkhorn offsets kept in LDS)

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool good_dtype(lcp_dtype d) { return d == LCP_F32 || d == LCP_BF16; }
inline size_t esize(lcp_dtype d) { return d == LCP_BF16 ? 2 : 4; }
inline bool good_B(int B) { return B == 32 || B == 64 || B == 128; }
inline bool fits_i32(long long a, long long b) { return a > 0 && b > 0 && a * b < (1LL << 31); }
// bf16 GEMM operands are read through buffer resources whose zero reads
// (K tail, rows past the matrix) use an offset of 2^31 bytes: every bf16
// matrix a GEMM reads must stay below 2^30 elements (2 GB)
inline bool fits_bf16_gemm(long long a, long long b) { return a > 0 && b > 0 && a * b < (1LL << 30); }
inline bool good_tau(float tau) { return isfinite(tau) && tau > 0.f; }
inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int pitch_of(int T) { return (T + 63) / 64 * 64; }

struct StepLayout {
  size_t P, Ph, off, bits, D, R, part, party, E, GY, adj, fragF, fragA, total;
  int nb, pitch, nparts;
  AdjSplit sp;
};

StepLayout step_layout(int cout, int cin, int T, int B, int iters, lcp_dtype dt) {
  StepLayout L{};
  L.nb = cin / B;
  L.pitch = pitch_of(T);
  L.nparts = gemm_error_parts(cout, L.pitch, dt == LCP_BF16);
  L.sp = adjoint_split(cout, cin, B);
  const bool bf = dt == LCP_BF16;
  size_t o = 0;
  L.P = o;     o += align_up((size_t)L.nb * B * B * 4);
  L.Ph = o;    o += align_up((size_t)L.nb * B * B * 4);
  L.off = o;   o += align_up((size_t)L.nb * iters * 2 * B * 4);
  L.bits = o;  o += align_up((size_t)cout * (cin / 32) * 4);
  L.D = o;     o += align_up((size_t)cout * cin * esize(dt));
  L.R = o;     o += align_up((size_t)cout * L.pitch * esize(dt));
  L.part = o;  o += align_up((size_t)L.nparts * 4);
  L.party = o; o += align_up((size_t)L.nparts * 4);
  L.E = o;     o += align_up(4 * 4);    // E, dD factor, cosine coefficients of Y and R
  L.GY = o;    o += align_up((size_t)cout * L.pitch * esize(dt));   // cosine dL/dY~
  // block adjoint partials: (workgroup, segment) slots, or one per (row panel,
  // block) when the adjoint is fused into the dD GEMM (bf16, B = 64)
  const size_t adj_slots = std::max((size_t)L.sp.grid * L.sp.maxseg,
                                    bf && B == 64 ? (size_t)dd_adjoint_panels(cout) * L.nb : (size_t)0);
  L.adj = o;   o += align_up(adj_slots * B * B * 4);
  L.fragF = o; o += bf ? align_up((size_t)L.nb * frag_fwd_entries(B) * 16) : 0;
  L.fragA = o; o += bf ? align_up((size_t)L.nb * frag_adj_entries(B) * 16) : 0;
  L.total = o;
  return L;
}

int check_step_args(const lcp_layer* L, const float* logits, const lcp_cfg* c) {
  if (!L || !logits || !c) return LCP_E_INVAL;
  if (!good_dtype(L->dtype)) return LCP_E_UNSUPPORTED;
  if (!L->W || !L->X || !L->norms) return LCP_E_INVAL;
  if (L->cout <= 0 || L->cin <= 0 || L->T <= 0 || L->B <= 0) return LCP_E_INVAL;
  if (c->iters < 1 || !good_tau(c->tau)) return LCP_E_INVAL;
  if (c->M <= 0 || c->N < 1 || c->N >= c->M) return LCP_E_INVAL;
  if (c->harden != 0 && c->harden != 1) return LCP_E_INVAL;
  if (c->mask_ste != 0 && c->mask_ste != 1) return LCP_E_INVAL;
  if (c->loss != LCP_LOSS_FROBENIUS && c->loss != LCP_LOSS_COSINE) return LCP_E_INVAL;
  if (c->loss == LCP_LOSS_COSINE && (!L->Y || !L->y2 || !aligned16(L->Y))) return LCP_E_INVAL;
  if (L->cin % L->B != 0 || L->B % c->M != 0) return LCP_E_INVAL;
  if (!good_B(L->B)) return LCP_E_UNSUPPORTED;
  if (c->M != 4 && c->M != 8) return LCP_E_UNSUPPORTED;
  if ((long long)c->iters * L->B > kMaxIterB) return LCP_E_UNSUPPORTED;
  if (!fits_i32(L->cout, L->cin) || !fits_i32(L->T, L->cin) || !fits_i32(L->cout, pitch_of(L->T)) ||
      !fits_i32(L->cin, pitch_of(L->T)))
    return LCP_E_INVAL;
  if (L->dtype == LCP_BF16 && (!fits_bf16_gemm(L->cout, L->cin) || !fits_bf16_gemm(L->T, L->cin))) return LCP_E_INVAL;
  if (!aligned16(L->W) || !aligned16(L->X) || !aligned16(logits)) return LCP_E_INVAL;
  return LCP_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return LCP_E_INVAL;
  if (((uintptr_t)ws % kAlign) != 0 || ws_bytes < need) return LCP_E_WORKSPACE;
  return LCP_OK;
}

struct Timer {
  const lcp_timing* tm;
  hipStream_t s;
  void start(int i) const { if (tm && tm->start[i]) (void)hipEventRecord((hipEvent_t)tm->start[i], s); }
  void stop(int i) const { if (tm && tm->stop[i]) (void)hipEventRecord((hipEvent_t)tm->stop[i], s); }
};

#define LCP_RUN(expr)                         \
  do {                                        \
    if ((expr) != hipSuccess) return LCP_E_HIP; \
  } while (0)

}  // namespace

// AdamW arguments -> kernel parameters (bias corrections computed here).
static int make_adamw(float* param, float* m, float* v, int t, const lcp_adamw_cfg* oc, AdamW* o) {
  if (!param || !m || !v || !oc || t < 1) return LCP_E_INVAL;
  if (param == m || param == v || m == v) return LCP_E_INVAL;
  const bool ok = isfinite(oc->lr) && oc->lr >= 0.f && oc->beta1 >= 0.f && oc->beta1 < 1.f &&
                  oc->beta2 >= 0.f && oc->beta2 < 1.f && isfinite(oc->eps) && oc->eps > 0.f &&
                  isfinite(oc->weight_decay) && oc->weight_decay >= 0.f;
  if (!ok) return LCP_E_INVAL;
  const double bc1 = 1.0 - pow((double)oc->beta1, (double)t), bc2 = 1.0 - pow((double)oc->beta2, (double)t);
  if (!(bc1 > 0.0) || !(bc2 > 0.0)) return LCP_E_INVAL;
  *o = AdamW{param, m, v, oc->lr, oc->beta1, oc->beta2, oc->eps, oc->weight_decay, (float)bc1, (float)bc2};
  return LCP_OK;
}

static int step_bwd_impl(const lcp_layer* L, const float* logits, const lcp_cfg* c, void* ws, size_t ws_bytes,
                         float* dlogits, const AdamW* opt, const lcp_timing* tm, void* stream) {
  int rc = check_step_args(L, logits, c);
  if (rc != LCP_OK) return rc;
  if (dlogits && !aligned16(dlogits)) return LCP_E_INVAL;
  const bool bf = L->dtype == LCP_BF16;
  if (bf && (!L->Xt || !aligned16(L->Xt))) return LCP_E_INVAL;
  const StepLayout Ly = step_layout(L->cout, L->cin, L->T, L->B, c->iters, L->dtype);
  rc = check_ws(ws, ws_bytes, Ly.total);
  if (rc != LCP_OK) return rc;

  char* base = (char*)ws;
  // the block adjoint is taken at the P the forward used (the hard P when
  // hardened: straight-through, the Sinkhorn adjoint below stays soft)
  const float* P = (const float*)(base + (c->harden ? Ly.Ph : Ly.P));
  const float* off = (const float*)(base + Ly.off);
  const uint32_t* bits = (const uint32_t*)(base + Ly.bits);
  void* Gd = base + Ly.D;           // G reuses the forward's D buffer
  const void* R = base + Ly.R;
  const float* Ews = (const float*)(base + Ly.E);
  float* adj = (float*)(base + Ly.adj);
  hipStream_t s = S(stream);
  const Timer tmr{tm, s};

  if (c->loss == LCP_LOSS_COSINE) {
    // dL/dY~ from Y and R with the forward's coefficients; the dD GEMM then
    // forms G = dL/dW_tilde = (dL/dY~) X (factor 1)
    void* GY = base + Ly.GY;
    tmr.start(3);
    LCP_RUN(launch_cosine_grad(L->Y, R, (size_t)L->cout * Ly.pitch, bf, Ews, GY, s));
    tmr.stop(3);
    R = GY;
  }
  const float* ste = c->mask_ste ? L->norms : nullptr;
  const u32x4* fragA = (const u32x4*)(base + Ly.fragA);
  if (bf && L->B == 64 && !c->mask_ste) {
    // the block adjoint taken in the dD GEMM's epilogue (G is never stored);
    // the Sinkhorn adjoint adds the row-panel partials in panel order
    tmr.start(0);
    LCP_RUN(launch_gemm_dd_adjoint_bf16((const uint16_t*)R, Ly.pitch, (const uint16_t*)L->Xt, Ly.pitch, L->cout,
                                        L->cin, Ly.pitch, Ews, (const uint16_t*)L->W, fragA, bits, adj, s));
    tmr.stop(0);
    tmr.start(1);
    tmr.stop(1);
    const AdjSplit panels{dd_adjoint_panels(L->cout), -1, 0, 0};
    tmr.start(2);
    LCP_RUN(launch_sinkhorn_bwd(logits, adj, &panels, off, dlogits, Ly.nb, L->B, c->iters, c->tau, opt, s));
    tmr.stop(2);
    return LCP_OK;
  }
  tmr.start(0);
  if (bf)
    LCP_RUN(launch_gemm_dd_bf16((const uint16_t*)R, Ly.pitch, (const uint16_t*)L->Xt, Ly.pitch, L->cout, L->cin,
                                Ly.pitch, Ews, (uint16_t*)Gd, L->cin, s));
  else
    LCP_RUN(launch_gemm_dd_f32((const float*)R, Ly.pitch, (const float*)L->X, L->cin, L->cout, L->cin, L->T, Ews,
                               (float*)Gd, L->cin, s));
  tmr.stop(0);
  tmr.start(1);
  if (bf)
    LCP_RUN(launch_adjoint_bf16((const uint16_t*)Gd, (const uint16_t*)L->W, fragA, P, bits, L->cout, L->cin,
                                L->B, Ly.sp, ste, adj, s));
  else
    LCP_RUN(launch_adjoint_f32((const float*)Gd, (const float*)L->W, P, bits, L->cout, L->cin, L->B, Ly.sp,
                               ste, adj, s));
  tmr.stop(1);
  tmr.start(2);
  LCP_RUN(launch_sinkhorn_bwd(logits, adj, &Ly.sp, off, dlogits, Ly.nb, L->B, c->iters, c->tau, opt, s));
  tmr.stop(2);
  return LCP_OK;
}


// ---- allocation-free variant of lcp_layer_outputs ----------------------------
// The error GEMM's per-workgroup partial sums of ||Y||^2 live in this fixed
// device array instead of a caller workspace. Every GPU the library runs on
// holds its own copy until the process ends. In host code `scratch` is only a
// host-side stand-in: kernels get the device address looked up once per
// device with hipGetSymbolAddress (kept in g_scratch_dev) and never the name.
__device__ __attribute__((aligned(256))) float scratch[LCP_NOALLOC_MAX_PARTS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices];   // device address of `scratch` per device, null until first use

// Address of `scratch` on the current device; looked up with that device
// current on the first call there.
int scratch_on_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LCP_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LCP_E_HIP;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return LCP_OK;
}
}  // namespace

extern "C" {

const char* lcp_status_string(int code) {
  switch (code) {
    case LCP_OK: return "ok";
    case LCP_E_INVAL: return "invalid argument";
    case LCP_E_UNSUPPORTED: return "unsupported configuration";
    case LCP_E_WORKSPACE: return "workspace too small or misaligned";
    case LCP_E_HIP: return "HIP launch error";
    case LCP_E_SCRATCH: return "input exceeds the fixed scratch of an allocation-free entry point";
  }
  return "unknown status";
}

int lcp_version(void) { return 100; }

int lcp_xt_pitch(int T) { return T > 0 ? pitch_of(T) : -1; }

int lcp_sinkhorn(const float* logits, float* P, int nb, int B, int iters, float tau, void* stream) {
  if (!logits || !P || nb <= 0 || B <= 0 || iters < 1 || !good_tau(tau)) return LCP_E_INVAL;
  if (!good_B(B)) return LCP_E_UNSUPPORTED;
  if ((long long)iters * B > kMaxIterB) return LCP_E_UNSUPPORTED;
  if (!fits_i32(nb, (long long)B * B) || !aligned16(logits) || !aligned16(P)) return LCP_E_INVAL;
  LCP_RUN(launch_sinkhorn_fwd(logits, P, nullptr, nb, B, iters, tau, nullptr, nullptr, nullptr, S(stream)));
  return LCP_OK;
}

int lcp_sinkhorn_bwd(const float* logits, const float* dP, int nb, int B, int iters, float tau,
                     float* dlogits, void* stream) {
  if (!logits || !dP || !dlogits || nb <= 0 || B <= 0 || iters < 1 || !good_tau(tau)) return LCP_E_INVAL;
  if (dlogits == dP) return LCP_E_INVAL;
  if (!good_B(B)) return LCP_E_UNSUPPORTED;
  if ((long long)iters * B > kMaxIterB) return LCP_E_UNSUPPORTED;
  if (!fits_i32(nb, (long long)B * B) || !aligned16(logits) || !aligned16(dP) || !aligned16(dlogits))
    return LCP_E_INVAL;
  LCP_RUN(launch_sinkhorn_bwd(logits, dP, nullptr, nullptr, dlogits, nb, B, iters, tau, nullptr, S(stream)));
  return LCP_OK;
}

int lcp_harden(const float* P, int nb, int B, float* P_hard, int32_t* perm, void* stream) {
  if (!P || nb <= 0 || B <= 0 || (!P_hard && !perm)) return LCP_E_INVAL;
  if (!good_B(B)) return LCP_E_UNSUPPORTED;
  if (!fits_i32(nb, (long long)B * B)) return LCP_E_INVAL;
  if (P_hard == P || !aligned16(P) || (P_hard && !aligned16(P_hard))) return LCP_E_INVAL;
  LCP_RUN(launch_harden(P, nb, B, P_hard, perm, nullptr, nullptr, nullptr, S(stream)));
  return LCP_OK;
}

int lcp_colnorm(const void* X, lcp_dtype dt, int T, int cin, float* norms, void* stream) {
  if (!X || !norms || T <= 0 || cin <= 0) return LCP_E_INVAL;
  if (!good_dtype(dt)) return LCP_E_UNSUPPORTED;
  if (!fits_i32(T, cin) || !aligned16(X)) return LCP_E_INVAL;
  if (dt == LCP_BF16) {
    if (cin % 8) return LCP_E_INVAL;
    LCP_RUN(launch_layer_init_bf16((const uint16_t*)X, T, cin, pitch_of(T), norms, nullptr, S(stream)));
  } else {
    LCP_RUN(launch_colnorm_f32((const float*)X, T, cin, norms, S(stream)));
  }
  return LCP_OK;
}

int lcp_layer_init(const void* X, lcp_dtype dt, int T, int cin, float* norms, void* Xt, void* stream) {
  if (!X || !norms || T <= 0 || cin <= 0) return LCP_E_INVAL;
  if (!good_dtype(dt)) return LCP_E_UNSUPPORTED;
  if (cin % 32 || !fits_i32(T, cin) || !fits_i32(cin, pitch_of(T)) || !aligned16(X)) return LCP_E_INVAL;
  if (dt == LCP_BF16) {
    if (!Xt || !aligned16(Xt)) return LCP_E_INVAL;
    LCP_RUN(launch_layer_init_bf16((const uint16_t*)X, T, cin, pitch_of(T), norms, (uint16_t*)Xt, S(stream)));
  } else {
    LCP_RUN(launch_colnorm_f32((const float*)X, T, cin, norms, S(stream)));
  }
  return LCP_OK;
}

int lcp_permute(const void* A, lcp_dtype adt, int rows, int cin, const float* colscale, const float* P,
                int B, int transposeP, void* out, lcp_dtype odt, void* stream) {
  if (!A || !P || !out || rows <= 0 || cin <= 0 || B <= 0) return LCP_E_INVAL;
  if (!good_dtype(adt) || !good_dtype(odt)) return LCP_E_UNSUPPORTED;
  if (cin % B) return LCP_E_INVAL;
  if (!good_B(B)) return LCP_E_UNSUPPORTED;
  if (!fits_i32(rows, cin) || !aligned16(A) || !aligned16(out) || !aligned16(P)) return LCP_E_INVAL;
  const int mode = colscale ? PERM_IMPORTANCE : PERM_PLAIN;
  if (mode == PERM_IMPORTANCE && odt != LCP_F32) return LCP_E_UNSUPPORTED;
  if (adt == LCP_F32 && odt != LCP_F32) return LCP_E_UNSUPPORTED;
  if (adt == LCP_BF16) {
    LCP_RUN(launch_permute_bf16((const uint16_t*)A, rows, cin, colscale, P, B, transposeP ? 1 : 0, nullptr,
                                mode, out, odt == LCP_F32, nullptr, 0, 4, S(stream)));
  } else {
    LCP_RUN(launch_permute_f32((const float*)A, rows, cin, colscale, P, B, transposeP ? 1 : 0, mode,
                               (float*)out, nullptr, 0, 4, S(stream)));
  }
  return LCP_OK;
}

int lcp_nm_mask(const float* scores, int rows, int cin, int N, int M, uint32_t* bits, void* stream) {
  if (!scores || !bits || rows <= 0 || cin <= 0 || M <= 0) return LCP_E_INVAL;
  if (N < 1 || N >= M || cin % 32) return LCP_E_INVAL;
  if (M != 4 && M != 8) return LCP_E_UNSUPPORTED;
  if (!fits_i32(rows, cin) || !aligned16(scores)) return LCP_E_INVAL;
  LCP_RUN(launch_nm_mask(scores, rows, cin, N, M, bits, S(stream)));
  return LCP_OK;
}

int lcp_error_workspace_bytes(int cout, int cin, int T, lcp_dtype dt, size_t* bytes) {
  if (!bytes || cout <= 0 || cin <= 0 || T <= 0) return LCP_E_INVAL;
  if (!good_dtype(dt)) return LCP_E_UNSUPPORTED;
  if (!fits_i32(cout, cin) || !fits_i32(cout, pitch_of(T))) return LCP_E_INVAL;
  const int pitch = pitch_of(T);
  *bytes = align_up((size_t)cout * cin * esize(dt)) + align_up((size_t)cout * pitch * esize(dt)) +
           align_up((size_t)gemm_error_parts(cout, pitch, dt == LCP_BF16) * 4) + align_up(4);
  return LCP_OK;
}

int lcp_error(const void* W, const void* Wt, const void* X, lcp_dtype dt, int cout, int cin, int T,
              float* err, void* R_out, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !Wt || !X || !err || cout <= 0 || cin <= 0 || T <= 0) return LCP_E_INVAL;
  if (!good_dtype(dt)) return LCP_E_UNSUPPORTED;
  if (cin % 32 || !fits_i32(cout, cin) || !fits_i32(T, cin) || !fits_i32(cout, pitch_of(T))) return LCP_E_INVAL;
  if (dt == LCP_BF16 && (!fits_bf16_gemm(cout, cin) || !fits_bf16_gemm(T, cin))) return LCP_E_INVAL;
  if (!aligned16(W) || !aligned16(Wt) || !aligned16(X) || (R_out && !aligned16(R_out))) return LCP_E_INVAL;
  size_t need = 0;
  int rc = lcp_error_workspace_bytes(cout, cin, T, dt, &need);
  if (rc != LCP_OK) return rc;
  rc = check_ws(ws, ws_bytes, need);
  if (rc != LCP_OK) return rc;
  const int pitch = pitch_of(T);
  char* base = (char*)ws;
  void* D = base;
  char* Rp = base + align_up((size_t)cout * cin * esize(dt));
  float* part = (float*)(Rp + align_up((size_t)cout * pitch * esize(dt)));
  const int nparts = gemm_error_parts(cout, pitch, dt == LCP_BF16);
  float* Ews = (float*)((char*)part + align_up((size_t)nparts * 4));
  void* R = R_out ? R_out : (void*)Rp;
  hipStream_t s = S(stream);
  LCP_RUN(launch_diff(W, Wt, cout * cin, dt == LCP_BF16, D, s));
  if (dt == LCP_BF16)
    LCP_RUN(launch_gemm_error_bf16((const uint16_t*)D, cin, (const uint16_t*)X, cin, cout, T, pitch, cin,
                                   (uint16_t*)R, pitch, part, nullptr, nullptr, s));
  else
    LCP_RUN(launch_gemm_error_f32((const float*)D, cin, (const float*)X, cin, cout, T, pitch, cin, (float*)R,
                                  pitch, part, nullptr, nullptr, s));
  LCP_RUN(launch_error_finalize(part, nparts, Ews, err, s));
  return LCP_OK;
}

int lcp_layer_outputs(const void* W, const void* X, lcp_dtype dt, int cout, int cin, int T, void* Y, float* y2,
                      void* ws, size_t ws_bytes, void* stream) {
  if (!W || !X || !Y || !y2 || cout <= 0 || cin <= 0 || T <= 0) return LCP_E_INVAL;
  if (!good_dtype(dt)) return LCP_E_UNSUPPORTED;
  if (cin % 32 || !fits_i32(cout, cin) || !fits_i32(T, cin) || !fits_i32(cout, pitch_of(T))) return LCP_E_INVAL;
  if (dt == LCP_BF16 && (!fits_bf16_gemm(cout, cin) || !fits_bf16_gemm(T, cin))) return LCP_E_INVAL;
  if (!aligned16(W) || !aligned16(X) || !aligned16(Y)) return LCP_E_INVAL;
  size_t need = 0;
  int rc = lcp_error_workspace_bytes(cout, cin, T, dt, &need);
  if (rc != LCP_OK) return rc;
  rc = check_ws(ws, ws_bytes, need);
  if (rc != LCP_OK) return rc;
  const int pitch = pitch_of(T);
  const int nparts = gemm_error_parts(cout, pitch, dt == LCP_BF16);
  float* part = (float*)ws;
  hipStream_t s = S(stream);
  if (dt == LCP_BF16)
    LCP_RUN(launch_gemm_error_bf16((const uint16_t*)W, cin, (const uint16_t*)X, cin, cout, T, pitch, cin,
                                   (uint16_t*)Y, pitch, part, nullptr, nullptr, s));
  else
    LCP_RUN(launch_gemm_error_f32((const float*)W, cin, (const float*)X, cin, cout, T, pitch, cin, (float*)Y,
                                  pitch, part, nullptr, nullptr, s));
  LCP_RUN(launch_sum_finalize(part, nparts, y2, s));
  return LCP_OK;
}

// Same kernels as lcp_layer_outputs, partial sums in the fixed scratch.
int lcp_layer_outputs_noalloc(const void* W, const void* X, lcp_dtype dt, int cout, int cin, int T, void* Y,
                              float* y2, void* stream) {
  if (!W || !X || !Y || !y2 || cout <= 0 || cin <= 0 || T <= 0) return LCP_E_INVAL;
  if (!good_dtype(dt)) return LCP_E_UNSUPPORTED;
  if (cin % 32 || !fits_i32(cout, cin) || !fits_i32(T, cin) || !fits_i32(cout, pitch_of(T))) return LCP_E_INVAL;
  if (dt == LCP_BF16 && (!fits_bf16_gemm(cout, cin) || !fits_bf16_gemm(T, cin))) return LCP_E_INVAL;
  if (!aligned16(W) || !aligned16(X) || !aligned16(Y)) return LCP_E_INVAL;
  const int pitch = pitch_of(T);
  const int nparts = gemm_error_parts(cout, pitch, dt == LCP_BF16);
  if (nparts > LCP_NOALLOC_MAX_PARTS) return LCP_E_SCRATCH;
  float* part = nullptr;
  const int rc = scratch_on_current_device(&part);
  if (rc != LCP_OK) return rc;
  hipStream_t s = S(stream);
  // the same kernels as lcp_layer_outputs; each workgroup overwrites its own
  // partial, so nothing needs clearing between calls
  if (dt == LCP_BF16)
    LCP_RUN(launch_gemm_error_bf16((const uint16_t*)W, cin, (const uint16_t*)X, cin, cout, T, pitch, cin,
                                   (uint16_t*)Y, pitch, part, nullptr, nullptr, s));
  else
    LCP_RUN(launch_gemm_error_f32((const float*)W, cin, (const float*)X, cin, cout, T, pitch, cin, (float*)Y,
                                  pitch, part, nullptr, nullptr, s));
  LCP_RUN(launch_sum_finalize(part, nparts, y2, s));
  return LCP_OK;
}

int lcp_sparse_pack_bytes(int cout, int cin, size_t* vals_bytes, size_t* meta_bytes) {
  if (!vals_bytes || !meta_bytes || cout <= 0 || cin <= 0 || cout % 32 || cin % 32) return LCP_E_INVAL;
  if (!fits_i32(cout, cin)) return LCP_E_INVAL;
  *vals_bytes = sparse_vals_bytes(cout, cin);
  *meta_bytes = sparse_meta_bytes(cout, cin);
  return LCP_OK;
}

int lcp_sparse_pack(const void* W, int cout, int cin, int B, const int32_t* perm, const uint32_t* bits, void* vals,
                    uint32_t* meta, void* stream) {
  if (!W || !perm || !bits || !vals || !meta) return LCP_E_INVAL;
  if (cout <= 0 || cin <= 0 || cout % 32 || cin % 32 || !fits_i32(cout, cin)) return LCP_E_INVAL;
  if (!good_B(B)) return LCP_E_UNSUPPORTED;
  if (cin % B) return LCP_E_INVAL;
  if (!aligned16(vals) || ((uintptr_t)meta & 3u)) return LCP_E_INVAL;
  LCP_RUN(launch_sparse_pack((const uint16_t*)W, cout, cin, B, perm, bits, (u32x4*)vals, meta, S(stream)));
  return LCP_OK;
}

static int check_gather(const void* X, int T, int cin, int B, const int32_t* perm, const void* Xp) {
  if (!X || !perm || !Xp || T <= 0 || cin <= 0 || !fits_i32(T, cin)) return LCP_E_INVAL;
  if (!good_B(B)) return LCP_E_UNSUPPORTED;
  if (cin % B) return LCP_E_INVAL;
  if (!aligned16(Xp) || X == Xp) return LCP_E_INVAL;
  return LCP_OK;
}

static int check_spgemm(const void* vals, const uint32_t* meta, const void* Xp, int T, int cout, int cin,
                        const void* Y) {
  if (!vals || !meta || !Xp || !Y || T <= 0 || cout <= 0 || cin <= 0) return LCP_E_INVAL;
  if (cout % 32 || cin % 32 || !fits_i32(cout, cin) || !fits_i32(T, cin) || !fits_i32(T, cout)) return LCP_E_INVAL;
  if (!fits_bf16_gemm(T, cin)) return LCP_E_INVAL;
  if (!aligned16(vals) || !aligned16(Xp) || !aligned16(Y) || ((uintptr_t)meta & 3u)) return LCP_E_INVAL;
  return LCP_OK;
}

int lcp_gather_channels(const void* X, int T, int cin, int B, const int32_t* perm, void* Xp, void* stream) {
  const int rc = check_gather(X, T, cin, B, perm, Xp);
  if (rc != LCP_OK) return rc;
  LCP_RUN(launch_gather((const uint16_t*)X, T, cin, B, perm, (uint16_t*)Xp, S(stream)));
  return LCP_OK;
}

int lcp_sparse_gemm(const void* vals, const uint32_t* meta, const void* Xp, int T, int cout, int cin, void* Y,
                    void* stream) {
  const int rc = check_spgemm(vals, meta, Xp, T, cout, cin, Y);
  if (rc != LCP_OK) return rc;
  LCP_RUN(launch_spgemm((const u32x4*)vals, meta, (const uint16_t*)Xp, T, cout, cin, (uint16_t*)Y, S(stream)));
  return LCP_OK;
}

int lcp_deploy_forward(const void* vals, const uint32_t* meta, const int32_t* perm, int B, const void* X, int T,
                       int cout, int cin, void* Xp, void* Y, void* stream) {
  int rc = check_gather(X, T, cin, B, perm, Xp);
  if (rc != LCP_OK) return rc;
  rc = check_spgemm(vals, meta, Xp, T, cout, cin, Y);
  if (rc != LCP_OK) return rc;
  if (Y == X || Y == Xp) return LCP_E_INVAL;
  LCP_RUN(launch_gather((const uint16_t*)X, T, cin, B, perm, (uint16_t*)Xp, S(stream)));
  LCP_RUN(launch_spgemm((const u32x4*)vals, meta, (const uint16_t*)Xp, T, cout, cin, (uint16_t*)Y, S(stream)));
  return LCP_OK;
}

int lcp_step_workspace_bytes(int cout, int cin, int T, int B, int iters, lcp_dtype dt, size_t* bytes) {
  if (!bytes || cout <= 0 || cin <= 0 || T <= 0 || B <= 0 || iters < 1) return LCP_E_INVAL;
  if (!good_dtype(dt)) return LCP_E_UNSUPPORTED;
  if (cin % B) return LCP_E_INVAL;
  if (!good_B(B)) return LCP_E_UNSUPPORTED;
  if (!fits_i32(cout, cin) || !fits_i32(cout, pitch_of(T))) return LCP_E_INVAL;
  *bytes = step_layout(cout, cin, T, B, iters, dt).total;
  return LCP_OK;
}

int lcp_step_fwd(const lcp_layer* L, const float* logits, const lcp_cfg* c, void* ws, size_t ws_bytes,
                 float* err, float* P_out, uint32_t* bits_out, const lcp_timing* tm, void* stream) {
  int rc = check_step_args(L, logits, c);
  if (rc != LCP_OK) return rc;
  if (!err) return LCP_E_INVAL;
  const StepLayout Ly = step_layout(L->cout, L->cin, L->T, L->B, c->iters, L->dtype);
  rc = check_ws(ws, ws_bytes, Ly.total);
  if (rc != LCP_OK) return rc;

  char* base = (char*)ws;
  float* P = (float*)(base + Ly.P);
  float* off = (float*)(base + Ly.off);
  uint32_t* bits = (uint32_t*)(base + Ly.bits);
  void* D = base + Ly.D;
  void* R = base + Ly.R;
  float* part = (float*)(base + Ly.part);
  float* party = (float*)(base + Ly.party);
  float* Ews = (float*)(base + Ly.E);
  hipStream_t s = S(stream);
  const Timer tmr{tm, s};
  const bool bf = L->dtype == LCP_BF16;
  const bool cosine = c->loss == LCP_LOSS_COSINE;

  u32x4* fragF = (u32x4*)(base + Ly.fragF);
  u32x4* fragA = (u32x4*)(base + Ly.fragA);
  const bool hard = c->harden != 0;
  tmr.start(0);
  LCP_RUN(launch_sinkhorn_fwd(logits, P, off, Ly.nb, L->B, c->iters, c->tau, L->norms,
                              (bf && !hard) ? fragF : nullptr, (bf && !hard) ? fragA : nullptr, s));
  tmr.stop(0);
  // hardened forward: the block permutation, mask and un-permute use the
  // per-block assignment of P_hat ([PermLLM] Method 2)
  float* Pu = P;
  if (hard) {
    Pu = (float*)(base + Ly.Ph);
    tmr.start(4);
    LCP_RUN(launch_harden(P, Ly.nb, L->B, Pu, nullptr, L->norms, bf ? fragF : nullptr, bf ? fragA : nullptr, s));
    tmr.stop(4);
  }
  tmr.start(1);
  if (bf)
    LCP_RUN(launch_permute_bf16((const uint16_t*)L->W, L->cout, L->cin, L->norms, Pu, L->B, 0, fragF, PERM_FWD,
                                D, 0, bits, c->N, c->M, s));
  else
    LCP_RUN(launch_permute_f32((const float*)L->W, L->cout, L->cin, L->norms, Pu, L->B, 0, PERM_FWD, (float*)D,
                               bits, c->N, c->M, s));
  tmr.stop(1);
  // the cosine objective also needs <Y, R> (second partial set)
  tmr.start(2);
  if (bf)
    LCP_RUN(launch_gemm_error_bf16((const uint16_t*)D, L->cin, (const uint16_t*)L->X, L->cin, L->cout, L->T,
                                   Ly.pitch, L->cin, (uint16_t*)R, Ly.pitch, part,
                                   cosine ? (const uint16_t*)L->Y : nullptr, party, s));
  else
    LCP_RUN(launch_gemm_error_f32((const float*)D, L->cin, (const float*)L->X, L->cin, L->cout, L->T, Ly.pitch,
                                  L->cin, (float*)R, Ly.pitch, part, cosine ? (const float*)L->Y : nullptr,
                                  party, s));
  tmr.stop(2);
  tmr.start(3);
  if (cosine) LCP_RUN(launch_cosine_finalize(part, party, Ly.nparts, L->y2, Ews, err, s));
  else LCP_RUN(launch_error_finalize(part, Ly.nparts, Ews, err, s));
  tmr.stop(3);
  if (P_out)
    LCP_RUN(hipMemcpyAsync(P_out, Pu, (size_t)Ly.nb * L->B * L->B * 4, hipMemcpyDeviceToDevice, s));
  if (bits_out) LCP_RUN(launch_bits_rowmajor(bits, L->cout, L->cin, L->B, bits_out, s));
  return LCP_OK;
}

int lcp_step_bwd(const lcp_layer* L, const float* logits, const lcp_cfg* c, void* ws, size_t ws_bytes,
                 float* dlogits, const lcp_timing* tm, void* stream) {
  if (!dlogits) return LCP_E_INVAL;
  return step_bwd_impl(L, logits, c, ws, ws_bytes, dlogits, nullptr, tm, stream);
}

int lcp_adamw(float* param, const float* grad, float* m, float* v, int n, int t, const lcp_adamw_cfg* oc,
              void* stream) {
  AdamW o;
  int rc = make_adamw(param, m, v, t, oc, &o);
  if (rc != LCP_OK) return rc;
  if (!grad || n <= 0) return LCP_E_INVAL;
  LCP_RUN(launch_adamw(grad, n, o, S(stream)));
  return LCP_OK;
}

int lcp_step_bwd_adamw(const lcp_layer* L, float* logits, const lcp_cfg* c, void* ws, size_t ws_bytes,
                       float* m, float* v, int t, const lcp_adamw_cfg* oc, float* dlogits,
                       const lcp_timing* tm, void* stream) {
  AdamW o;
  int rc = make_adamw(logits, m, v, t, oc, &o);
  if (rc != LCP_OK) return rc;
  if (!aligned16(logits) || !aligned16(m) || !aligned16(v)) return LCP_E_INVAL;
  if (dlogits == logits || dlogits == m || dlogits == v) return LCP_E_INVAL;
  return step_bwd_impl(L, logits, c, ws, ws_bytes, dlogits, &o, tm, stream);
}

int lcp_train(const lcp_layer* L, float* logits, const lcp_cfg* c, void* ws, size_t ws_bytes, float* m,
              float* v, int steps, float tau0, float tau1, const lcp_adamw_cfg* oc, float* errs,
              void* stream) {
  if (!c || steps < 1 || !good_tau(tau0) || !good_tau(tau1)) return LCP_E_INVAL;
  if (!errs) return LCP_E_INVAL;
  lcp_cfg cs = *c;
  // validate everything once with the first step's arguments (nothing is
  // enqueued on an error)
  cs.tau = tau0;
  int rc = check_step_args(L, logits, &cs);
  if (rc != LCP_OK) return rc;
  AdamW probe;
  rc = make_adamw(logits, m, v, steps, oc, &probe);
  if (rc != LCP_OK) return rc;
  rc = make_adamw(logits, m, v, 1, oc, &probe);
  if (rc != LCP_OK) return rc;
  const StepLayout Ly = step_layout(L->cout, L->cin, L->T, L->B, c->iters, L->dtype);
  rc = check_ws(ws, ws_bytes, Ly.total);
  if (rc != LCP_OK) return rc;
  if (L->dtype == LCP_BF16 && (!L->Xt || !aligned16(L->Xt))) return LCP_E_INVAL;
  if (!aligned16(m) || !aligned16(v)) return LCP_E_INVAL;
  for (int t = 0; t < steps; ++t) {
    // temperature linear from tau0 (first step) to tau1 (last step)
    cs.tau = (float)((double)tau0 + ((double)tau1 - tau0) * (steps > 1 ? (double)t / (steps - 1) : 0.0));
    rc = lcp_step_fwd(L, logits, &cs, ws, ws_bytes, errs + t, nullptr, nullptr, nullptr, stream);
    if (rc != LCP_OK) return rc;
    rc = lcp_step_bwd_adamw(L, logits, &cs, ws, ws_bytes, m, v, t + 1, oc, nullptr, nullptr, stream);
    if (rc != LCP_OK) return rc;
  }
  return LCP_OK;
}

}  // extern "C"
