/* Host-side argument validation of liblcp under AddressSanitizer (the ABI
 * layer built with host-only ASan). Every call below must be rejected by
 * the validation before any HIP call; device pointers are fake, aligned
 * addresses that are never dereferenced. Prints "ok <n>" with the number
 * of checks. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <stdlib.h>

#include "lcp.h"

static int n_checks = 0;
static int failed = 0;

#define EXPECT(call, want)                                                  \
  do {                                                                      \
    int got_ = (call);                                                      \
    ++n_checks;                                                             \
    if (got_ != (want)) {                                                   \
      printf("FAIL line %d: %s -> %d, want %d\n", __LINE__, #call, got_,    \
             (int)(want));                                                  \
      failed = 1;                                                           \
    }                                                                       \
  } while (0)

int main(void) {
  /* fake device addresses: 256-aligned and misaligned by 4 / 8 bytes */
  void* p = (void*)(uintptr_t)0x100000;
  void* p4 = (void*)(uintptr_t)0x100004;
  void* p8 = (void*)(uintptr_t)0x100008;
  float* fp = (float*)p;
  size_t big = (size_t)1 << 30, bytes = 0, vb = 0, mb = 0;

  /* status and sizes */
  EXPECT(lcp_status_string(LCP_OK) != NULL, 1);
  EXPECT(lcp_status_string(-12345) != NULL, 1);
  EXPECT(lcp_version() > 0, 1);
  EXPECT(lcp_xt_pitch(0), -1);
  EXPECT(lcp_xt_pitch(65), 128);
  EXPECT(lcp_error_workspace_bytes(64, 128, 32, LCP_BF16, &bytes), LCP_OK);
  EXPECT(bytes > 0, 1);
  EXPECT(lcp_error_workspace_bytes(64, 128, 32, LCP_BF16, NULL), LCP_E_INVAL);
  EXPECT(lcp_step_workspace_bytes(64, 128, 32, 64, 5, LCP_BF16, &bytes), LCP_OK);
  EXPECT(lcp_step_workspace_bytes(64, 128, 32, 48, 5, LCP_BF16, &bytes) != LCP_OK, 1);
  EXPECT(lcp_sparse_pack_bytes(64, 128, &vb, &mb), LCP_OK);
  EXPECT(lcp_sparse_pack_bytes(64, 100, &vb, &mb) != LCP_OK, 1);

  /* Sinkhorn */
  EXPECT(lcp_sinkhorn(NULL, fp, 4, 64, 5, 1.f, NULL), LCP_E_INVAL);
  EXPECT(lcp_sinkhorn(fp, fp, 4, 64, 0, 1.f, NULL), LCP_E_INVAL);
  EXPECT(lcp_sinkhorn(fp, fp, 4, 64, 5, 0.f, NULL), LCP_E_INVAL);
  EXPECT(lcp_sinkhorn(fp, fp, 4, 48, 5, 1.f, NULL), LCP_E_UNSUPPORTED);
  EXPECT(lcp_sinkhorn((float*)p4, fp, 4, 64, 5, 1.f, NULL), LCP_E_INVAL);
  EXPECT(lcp_sinkhorn_bwd(fp, fp, 4, 64, 5, 1.f, fp, NULL), LCP_E_INVAL);
  EXPECT(lcp_harden(NULL, 4, 64, fp, NULL, NULL), LCP_E_INVAL);

  /* per-layer setup, permute, mask */
  EXPECT(lcp_colnorm(p, LCP_BF16, 0, 64, fp, NULL), LCP_E_INVAL);
  EXPECT(lcp_layer_init(p, LCP_BF16, 16, 48, fp, p, NULL), LCP_E_INVAL);
  EXPECT(lcp_layer_init(p, LCP_BF16, 16, 64, fp, p8, NULL), LCP_E_INVAL);
  EXPECT(lcp_permute(p, LCP_BF16, 8, 100, NULL, fp, 64, 0, p, LCP_BF16, NULL), LCP_E_INVAL);
  EXPECT(lcp_permute(p, LCP_BF16, 8, 96, NULL, fp, 96, 0, p, LCP_BF16, NULL), LCP_E_UNSUPPORTED);
  EXPECT(lcp_nm_mask(fp, 8, 64, 0, 4, (uint32_t*)p, NULL), LCP_E_INVAL);
  EXPECT(lcp_nm_mask(fp, 8, 64, 2, 16, (uint32_t*)p, NULL), LCP_E_UNSUPPORTED);

  /* error GEMM and layer outputs */
  EXPECT(lcp_error(p, p, p, LCP_BF16, 8, 64, 16, NULL, NULL, p, big, NULL), LCP_E_INVAL);
  EXPECT(lcp_error(p, p, p, LCP_BF16, 8, 64, 16, fp, NULL, p, 16, NULL), LCP_E_WORKSPACE);
  EXPECT(lcp_layer_outputs(p, p, LCP_BF16, 8, 64, 16, p, fp, p, 16, NULL), LCP_E_WORKSPACE);

  /* full step: a valid-looking layer, then one defect at a time */
  {
    lcp_layer L;
    lcp_cfg c;
    size_t need = 0;
    memset(&L, 0, sizeof L);
    memset(&c, 0, sizeof c);
    L.W = p; L.X = p; L.Xt = p; L.norms = fp; L.dtype = LCP_BF16;
    L.cout = 64; L.cin = 128; L.T = 32; L.B = 64;
    c.iters = 5; c.tau = 1.f; c.N = 2; c.M = 4;
    EXPECT(lcp_step_workspace_bytes(64, 128, 32, 64, 5, LCP_BF16, &need), LCP_OK);
    EXPECT(lcp_step_fwd(&L, fp, &c, p, need - 1, fp, NULL, NULL, NULL, NULL), LCP_E_WORKSPACE);
    EXPECT(lcp_step_fwd(&L, fp, &c, p, need, NULL, NULL, NULL, NULL, NULL), LCP_E_INVAL);
    EXPECT(lcp_step_fwd(NULL, fp, &c, p, need, fp, NULL, NULL, NULL, NULL), LCP_E_INVAL);
    EXPECT(lcp_step_fwd(&L, fp, NULL, p, need, fp, NULL, NULL, NULL, NULL), LCP_E_INVAL);
    c.tau = 0.f;
    EXPECT(lcp_step_fwd(&L, fp, &c, p, need, fp, NULL, NULL, NULL, NULL), LCP_E_INVAL);
    c.tau = 1.f; c.M = 3;
    EXPECT(lcp_step_fwd(&L, fp, &c, p, need, fp, NULL, NULL, NULL, NULL), LCP_E_INVAL);
    c.M = 4; c.loss = 7;
    EXPECT(lcp_step_fwd(&L, fp, &c, p, need, fp, NULL, NULL, NULL, NULL), LCP_E_INVAL);
    c.loss = LCP_LOSS_COSINE;   /* needs Y and y2 */
    EXPECT(lcp_step_fwd(&L, fp, &c, p, need, fp, NULL, NULL, NULL, NULL), LCP_E_INVAL);
    c.loss = LCP_LOSS_FROBENIUS;
    L.cin = 96;
    EXPECT(lcp_step_fwd(&L, fp, &c, p, need, fp, NULL, NULL, NULL, NULL), LCP_E_INVAL);
    L.cin = 128; L.X = p8;
    EXPECT(lcp_step_bwd(&L, fp, &c, p, need, fp, NULL, NULL), LCP_E_INVAL);
    L.X = p;
    EXPECT(lcp_step_bwd(&L, fp, &c, p, need - 256, fp, NULL, NULL), LCP_E_WORKSPACE);
  }

  /* deploy path */
  EXPECT(lcp_sparse_pack(p, 64, 100, 64, (const int32_t*)p, (const uint32_t*)p, p, p, NULL), LCP_E_INVAL);
  EXPECT(lcp_gather_channels(p, 16, 128, 48, (const int32_t*)p, p, NULL), LCP_E_UNSUPPORTED);
  EXPECT(lcp_gather_channels(p, 16, 128, 64, (const int32_t*)p, p8, NULL), LCP_E_INVAL);

  if (failed) return 1;
  printf("ok %d\n", n_checks);
  return 0;
}
