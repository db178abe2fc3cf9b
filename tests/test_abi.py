"""Host-side contract of the C ABI (no GPU needed): the library loads, exports
every function include/lcp.h declares, and rejects bad arguments with the
documented status codes before touching the device."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcp.h")


def _lib():
    from learnable_channel_permutation_amd import _lib as L
    return L


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lcp_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_step_entry_points():
    names = _declared()
    for n in ("lcp_sinkhorn", "lcp_permute", "lcp_nm_mask", "lcp_error", "lcp_step_fwd", "lcp_step_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    lib = ctypes.CDLL(L._LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(L.EXPORTS) == _declared()


def test_status_strings_and_version():
    L = _lib()
    assert L.status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert L.status_string(code) not in ("ok", "unknown status")
    assert L.status_string(12345) == "unknown status"
    assert L.LIB.lcp_version() >= 100


def test_xt_pitch():
    L = _lib()
    assert L.lcp_xt_pitch(1) == 64
    assert L.lcp_xt_pitch(64) == 64
    assert L.lcp_xt_pitch(2048) == 2048
    assert L.lcp_xt_pitch(2049) == 2112
    assert L.lcp_xt_pitch(0) == -1


def test_workspace_queries():
    L = _lib()
    a = L.lcp_step_workspace_bytes(4096, 11008, 2048, 64, 5, L.LCP_BF16)
    # P + offsets + bits + D + R at least
    floor = 172 * 64 * 64 * 4 + 172 * 5 * 2 * 64 * 4 + 4096 * 344 * 4 + 4096 * 11008 * 2 + 4096 * 2048 * 2
    assert a >= floor and a % 256 == 0
    b = L.lcp_step_workspace_bytes(4096, 11008, 2048, 64, 5, L.LCP_F32)
    assert b > a
    with pytest.raises(L.LcpError) as e:
        L.lcp_step_workspace_bytes(4096, 11000, 2048, 64, 5, L.LCP_BF16)   # cin % B
    assert e.value.code == L.LCP_E_INVAL
    with pytest.raises(L.LcpError) as e:
        L.lcp_step_workspace_bytes(4096, 11008, 2048, 16 * 43, 5, L.LCP_BF16)   # B unsupported
    assert e.value.code in (L.LCP_E_UNSUPPORTED, L.LCP_E_INVAL)
    assert L.lcp_error_workspace_bytes(256, 256, 256, L.LCP_F32) > 256 * 256 * 4


def _fake(addr=0x100000):
    return ctypes.c_void_p(addr)


def test_invalid_arguments_return_codes_without_launching():
    """Every call below fails validation, so no HIP call is made (this runs
    on a machine without a GPU)."""
    L = _lib()
    lib = L.LIB
    p = _fake()
    s = None
    # sinkhorn
    assert lib.lcp_sinkhorn(None, p, 4, 64, 5, 1.0, s) == L.LCP_E_INVAL
    assert lib.lcp_sinkhorn(p, p, 4, 64, 0, 1.0, s) == L.LCP_E_INVAL
    assert lib.lcp_sinkhorn(p, p, 4, 64, 5, 0.0, s) == L.LCP_E_INVAL
    assert lib.lcp_sinkhorn(p, p, 4, 64, 5, -1.0, s) == L.LCP_E_INVAL
    assert lib.lcp_sinkhorn(p, p, 4, 64, 5, math.inf, s) == L.LCP_E_INVAL
    assert lib.lcp_sinkhorn(p, p, 4, 64, 5, math.nan, s) == L.LCP_E_INVAL
    assert lib.lcp_sinkhorn(p, p, 4, 48, 5, 1.0, s) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_sinkhorn(p, p, 4, 64, 1000, 1.0, s) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_sinkhorn(_fake(0x100004), p, 4, 64, 5, 1.0, s) == L.LCP_E_INVAL  # misaligned
    assert lib.lcp_sinkhorn_bwd(p, p, 4, 64, 5, 1.0, p, s) == L.LCP_E_INVAL        # dlogits aliases dP
    # mask
    assert lib.lcp_nm_mask(p, 8, 64, 0, 4, p, s) == L.LCP_E_INVAL
    assert lib.lcp_nm_mask(p, 8, 64, 4, 4, p, s) == L.LCP_E_INVAL
    assert lib.lcp_nm_mask(p, 8, 48, 2, 4, p, s) == L.LCP_E_INVAL
    assert lib.lcp_nm_mask(p, 8, 64, 2, 16, p, s) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_nm_mask(p, 0, 64, 2, 4, p, s) == L.LCP_E_INVAL
    # permute
    assert lib.lcp_permute(p, L.LCP_BF16, 8, 100, None, p, 64, 0, p, L.LCP_BF16, s) == L.LCP_E_INVAL
    assert lib.lcp_permute(p, L.LCP_BF16, 8, 96, None, p, 96, 0, p, L.LCP_BF16, s) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_permute(p, L.LCP_BF16, 8, 128, p, p, 64, 0, p, L.LCP_BF16, s) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_permute(p, 7, 8, 128, None, p, 64, 0, p, L.LCP_BF16, s) == L.LCP_E_UNSUPPORTED
    # colnorm / layer init
    assert lib.lcp_colnorm(p, L.LCP_BF16, 0, 64, p, s) == L.LCP_E_INVAL
    assert lib.lcp_layer_init(p, L.LCP_BF16, 16, 64, p, None, s) == L.LCP_E_INVAL    # bf16 needs Xt
    assert lib.lcp_layer_init(p, L.LCP_BF16, 16, 48, p, p, s) == L.LCP_E_INVAL      # cin % 32
    # error
    n = ctypes.c_size_t(1 << 20)
    assert lib.lcp_error(p, p, p, L.LCP_BF16, 8, 64, 16, None, None, p, n, s) == L.LCP_E_INVAL
    assert lib.lcp_error(p, p, p, L.LCP_BF16, 8, 64, 16, p, None, p, ctypes.c_size_t(16), s) == L.LCP_E_WORKSPACE
    assert lib.lcp_error(p, p, p, L.LCP_BF16, 8, 64, 16, p, None, _fake(0x100010), n, s) == L.LCP_E_WORKSPACE


def _lay(L, W, X, Xt, norms, dtype, cout, cin, T, B, Y=0, y2=0):
    return L.lcp_layer(W=W, X=X, Xt=Xt, norms=norms, Y=Y, y2=y2, dtype=dtype, cout=cout, cin=cin, T=T, B=B)


def test_step_argument_validation():
    L = _lib()
    lib = L.LIB
    p = 0x100000
    layer = _lay(L, p, p, p, p, L.LCP_BF16, 64, 128, 32, 64)
    cfg = L.lcp_cfg(5, 1.0, 2, 4)
    ws = ctypes.c_void_p(p)
    need = L.lcp_step_workspace_bytes(64, 128, 32, 64, 5, L.LCP_BF16)
    err = ctypes.c_void_p(p)

    def fwd(layer=layer, cfg=cfg, ws=ws, n=need, err=err):
        return lib.lcp_step_fwd(ctypes.byref(layer), ctypes.c_void_p(p), ctypes.byref(cfg), ws,
                                ctypes.c_size_t(n), err, None, None, None, None)

    def bwd(layer=layer, cfg=cfg, ws=ws, n=need):
        return lib.lcp_step_bwd(ctypes.byref(layer), ctypes.c_void_p(p), ctypes.byref(cfg), ws,
                                ctypes.c_size_t(n), ctypes.c_void_p(p), None, None)

    assert fwd(n=need - 1) == L.LCP_E_WORKSPACE
    assert fwd(ws=ctypes.c_void_p(p + 128)) == L.LCP_E_WORKSPACE
    assert fwd(err=None) == L.LCP_E_INVAL
    assert fwd(cfg=L.lcp_cfg(0, 1.0, 2, 4)) == L.LCP_E_INVAL
    assert fwd(cfg=L.lcp_cfg(5, 0.0, 2, 4)) == L.LCP_E_INVAL
    assert fwd(cfg=L.lcp_cfg(5, 1.0, 4, 4)) == L.LCP_E_INVAL
    assert fwd(cfg=L.lcp_cfg(5, 1.0, 0, 4)) == L.LCP_E_INVAL
    assert fwd(cfg=L.lcp_cfg(5, 1.0, 2, 16)) in (L.LCP_E_UNSUPPORTED, L.LCP_E_INVAL)
    assert fwd(cfg=L.lcp_cfg(5, 1.0, 2, 3)) == L.LCP_E_INVAL           # B % M
    assert fwd(layer=_lay(L, p, p, p, p, L.LCP_BF16, 64, 96, 32, 64)) == L.LCP_E_INVAL   # cin % B
    assert fwd(layer=_lay(L, p, p, p, p, L.LCP_BF16, 64, 96, 32, 96)) == L.LCP_E_UNSUPPORTED
    assert fwd(layer=_lay(L, p, p, p, p, 5, 64, 128, 32, 64)) == L.LCP_E_UNSUPPORTED
    assert fwd(layer=_lay(L, 0, p, p, p, L.LCP_BF16, 64, 128, 32, 64)) == L.LCP_E_INVAL
    assert fwd(layer=_lay(L, p, p, p, p, L.LCP_BF16, 0, 128, 32, 64)) == L.LCP_E_INVAL
    assert fwd(layer=_lay(L, p, p, p, p, L.LCP_BF16, 1 << 20, 1 << 12, 32, 64)) == L.LCP_E_INVAL
    assert fwd(layer=_lay(L, p, p, p, p, L.LCP_BF16, 1 << 18, 1 << 12, 32, 64)) == L.LCP_E_INVAL   # bf16 W of 2^30
    assert fwd(layer=_lay(L, p, p, p, p, L.LCP_BF16, 64, 1 << 12, 1 << 18, 64)) == L.LCP_E_INVAL   # bf16 X of 2^30
    assert bwd(layer=_lay(L, p, p, 0, p, L.LCP_BF16, 64, 128, 32, 64)) == L.LCP_E_INVAL   # bf16 needs Xt
    assert bwd(n=need - 256) == L.LCP_E_WORKSPACE
    # iters * B above LCP_MAX_ITERS_B (8192): unsupported, nothing enqueued
    assert L.LCP_MAX_ITERS_B == 8192
    assert fwd(cfg=L.lcp_cfg(129, 1.0, 2, 4)) == L.LCP_E_UNSUPPORTED          # 129 * 64 > 8192
    assert bwd(cfg=L.lcp_cfg(129, 1.0, 2, 4)) == L.LCP_E_UNSUPPORTED
    big = _lay(L, p, p, p, p, L.LCP_BF16, 64, 256, 32, 128)
    need128 = L.lcp_step_workspace_bytes(64, 256, 32, 128, 65, L.LCP_BF16)
    assert fwd(layer=big, cfg=L.lcp_cfg(65, 1.0, 4, 8), n=need128) == L.LCP_E_UNSUPPORTED   # 65 * 128
    assert bwd(layer=big, cfg=L.lcp_cfg(65, 1.0, 4, 8), n=need128) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_sinkhorn(ctypes.c_void_p(p), ctypes.c_void_p(p), 4, 128, 65, 1.0, None) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_sinkhorn_bwd(ctypes.c_void_p(p), ctypes.c_void_p(p + 4096), 4, 32, 257, 1.0,
                                ctypes.c_void_p(p + 8192), None) == L.LCP_E_UNSUPPORTED
    m, vv = ctypes.c_void_p(p + 4096), ctypes.c_void_p(p + 8192)
    ac = L.lcp_adamw_cfg(1e-3, 0.9, 0.999, 1e-8, 0.01)
    errs = ctypes.c_void_p(p + 16384)
    assert lib.lcp_train(ctypes.byref(big), ctypes.c_void_p(p), ctypes.byref(L.lcp_cfg(65, 1.0, 4, 8)), ws,
                         ctypes.c_size_t(need128), m, vv, 3, ctypes.c_float(1.0), ctypes.c_float(0.1),
                         ctypes.byref(ac), errs, None) == L.LCP_E_UNSUPPORTED
    # objective and straight-through options
    assert fwd(cfg=L.lcp_cfg(5, 1.0, 2, 4, 0, 2, 0)) == L.LCP_E_INVAL            # unknown loss
    assert fwd(cfg=L.lcp_cfg(5, 1.0, 2, 4, 0, 0, 2)) == L.LCP_E_INVAL            # mask_ste not 0/1
    cos = L.lcp_cfg(5, 1.0, 2, 4, 0, L.LCP_LOSS_COSINE, 1)
    assert fwd(cfg=cos) == L.LCP_E_INVAL                                         # cosine needs Y, y2
    assert fwd(cfg=cos, layer=_lay(L, p, p, p, p, L.LCP_BF16, 64, 128, 32, 64, Y=p)) == L.LCP_E_INVAL
    assert fwd(cfg=cos, layer=_lay(L, p, p, p, p, L.LCP_BF16, 64, 128, 32, 64, Y=p + 8, y2=p)) == L.LCP_E_INVAL
    assert bwd(cfg=cos) == L.LCP_E_INVAL
    # layer outputs of the cosine objective
    s = None
    en = ctypes.c_size_t(1 << 20)
    assert lib.lcp_layer_outputs(p, p, L.LCP_BF16, 8, 64, 16, None, p, p, en, s) == L.LCP_E_INVAL
    assert lib.lcp_layer_outputs(p, p, L.LCP_BF16, 8, 64, 16, p, None, p, en, s) == L.LCP_E_INVAL
    assert lib.lcp_layer_outputs(p, p, L.LCP_BF16, 8, 48, 16, p, p, p, en, s) == L.LCP_E_INVAL
    assert lib.lcp_layer_outputs(p, p, 9, 8, 64, 16, p, p, p, en, s) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_layer_outputs(p, p, L.LCP_BF16, 8, 64, 16, p, p, p, ctypes.c_size_t(16), s) == L.LCP_E_WORKSPACE


def test_noalloc_argument_validation():
    """lcp_layer_outputs_noalloc rejects bad arguments and shapes whose
    partial sums exceed its fixed scratch before any HIP call (this runs on a
    machine without a GPU)."""
    L = _lib()
    lib = L.LIB
    p = ctypes.c_void_p(0x100000)
    s = None
    assert L.LCP_NOALLOC_MAX_PARTS == 16384
    assert L.status_string(L.LCP_E_SCRATCH) not in ("ok", "unknown status")
    assert lib.lcp_layer_outputs_noalloc(None, p, L.LCP_BF16, 8, 64, 16, p, p, s) == L.LCP_E_INVAL
    assert lib.lcp_layer_outputs_noalloc(p, p, L.LCP_BF16, 8, 64, 16, None, p, s) == L.LCP_E_INVAL
    assert lib.lcp_layer_outputs_noalloc(p, p, L.LCP_BF16, 8, 48, 16, p, p, s) == L.LCP_E_INVAL     # cin % 32
    assert lib.lcp_layer_outputs_noalloc(p, p, 9, 8, 64, 16, p, p, s) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_layer_outputs_noalloc(ctypes.c_void_p(0x100008), p, L.LCP_BF16, 8, 64, 16, p, p,
                                         s) == L.LCP_E_INVAL                                      # alignment
    # bf16: ceil(cout / 256) * ceil(pitch / 128) partials; 128 * 129 > 16384
    assert lib.lcp_layer_outputs_noalloc(p, p, L.LCP_BF16, 128 * 256, 32, 129 * 128, p, p, s) == L.LCP_E_SCRATCH
    # f32: 64-wide tiles, 129 * 128 > 16384
    assert lib.lcp_layer_outputs_noalloc(p, p, L.LCP_F32, 129 * 64, 32, 128 * 64, p, p, s) == L.LCP_E_SCRATCH


def test_deploy_argument_validation():
    """Deploy entry points reject bad sizes, block sizes and alignment before
    any launch (no GPU needed: nothing is enqueued on an error)."""
    L = _lib()
    lib = L.LIB
    p = 0x100000
    s = None
    vb, mb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.lcp_sparse_pack_bytes(4096, 11008, ctypes.byref(vb), ctypes.byref(mb)) == L.LCP_OK
    assert vb.value == 4096 * 11008 and mb.value == (4096 // 32) * ((11008 + 63) // 64) * 64 * 4
    assert lib.lcp_sparse_pack_bytes(100, 64, ctypes.byref(vb), ctypes.byref(mb)) == L.LCP_E_INVAL
    assert lib.lcp_sparse_pack_bytes(64, 48, ctypes.byref(vb), ctypes.byref(mb)) == L.LCP_E_INVAL
    # pack
    assert lib.lcp_sparse_pack(None, 64, 128, 64, p, p, p, p, s) == L.LCP_E_INVAL
    assert lib.lcp_sparse_pack(p, 60, 128, 64, p, p, p, p, s) == L.LCP_E_INVAL
    assert lib.lcp_sparse_pack(p, 64, 128, 48, p, p, p, p, s) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_sparse_pack(p, 64, 96, 64, p, p, p, p, s) == L.LCP_E_INVAL       # cin % B
    assert lib.lcp_sparse_pack(p, 64, 128, 64, p, p, p + 8, p, s) == L.LCP_E_INVAL   # vals alignment
    assert lib.lcp_sparse_pack(p, 64, 128, 64, p, p, p, p + 2, s) == L.LCP_E_INVAL   # meta alignment
    # gather
    assert lib.lcp_gather_channels(p, 0, 128, 64, p, p + 4096, s) == L.LCP_E_INVAL
    assert lib.lcp_gather_channels(p, 8, 128, 96, p, p + 4096, s) == L.LCP_E_UNSUPPORTED
    assert lib.lcp_gather_channels(p, 8, 128, 64, p, p, s) == L.LCP_E_INVAL            # in place
    assert lib.lcp_gather_channels(p, 8, 128, 64, p, p + 8, s) == L.LCP_E_INVAL        # alignment
    # sparse GEMM and the combined call
    assert lib.lcp_sparse_gemm(p, p, p, 8, 60, 128, p, s) == L.LCP_E_INVAL
    assert lib.lcp_sparse_gemm(p, p, p, 8, 64, 80, p, s) == L.LCP_E_INVAL
    assert lib.lcp_sparse_gemm(p, p + 2, p, 8, 64, 128, p, s) == L.LCP_E_INVAL
    assert lib.lcp_sparse_gemm(p, p, p, 8, 64, 128, p + 8, s) == L.LCP_E_INVAL
    assert lib.lcp_deploy_forward(p, p, p, 64, p, 8, 64, 128, p + 4096, p, s) == L.LCP_E_INVAL   # Y aliases X
    assert lib.lcp_deploy_forward(p, p, p, 64, p, 8, 64, 128, p, p + 4096, s) == L.LCP_E_INVAL   # Xp aliases X
    assert lib.lcp_deploy_forward(p, p, p, 32, p, 8, 60, 128, p + 4096, p + 8192, s) == L.LCP_E_INVAL


def test_header_is_plain_c_and_links(tmp_path):
    """include/lcp.h compiles as C99 (gcc, warnings as errors), and a C
    program that takes the address of every declared entry point links
    against liblcp.so and runs its host-side checks (no GPU calls)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    L = _lib()
    names = _declared()
    src = ["#include <stdio.h>", "#include <string.h>", '#include "lcp.h"', "",
           "int main(void) {",
           "  void* fns[] = {" + ", ".join("(void*)&" + n for n in names) + "};",
           "  size_t i, n = sizeof fns / sizeof fns[0];",
           "  for (i = 0; i < n; ++i) if (!fns[i]) return 2;",
           "  if (lcp_version() <= 0) return 3;",
           "  if (strlen(lcp_status_string(LCP_E_INVAL)) == 0) return 4;",
           "  size_t bytes = 0;",
           "  if (lcp_step_workspace_bytes(4096, 11008, 2048, 64, 5, LCP_BF16, &bytes) != LCP_OK || bytes == 0) return 5;",
           "  if (lcp_sinkhorn(0, 0, 1, 64, 5, 1.0f, 0) != LCP_E_INVAL) return 6;",
           "  lcp_cfg c; memset(&c, 0, sizeof c); c.iters = 5; c.tau = 1.0f; c.N = 2; c.M = 4;",
           "  c.loss = LCP_LOSS_COSINE;",
           "  if (lcp_step_fwd(0, 0, &c, 0, 0, 0, 0, 0, 0, 0) != LCP_E_INVAL) return 7;",
           '  printf("ok %u\\n", (unsigned)n);',
           "  return 0;", "}"]
    cfile = tmp_path / "abi_check.c"
    cfile.write_text("\n".join(src) + "\n")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(L._LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(cfile),
           "-L", libdir, "-llcp", "-Wl,-rpath," + libdir, "-o", str(exe)]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.strip() == "ok %d" % len(names)
