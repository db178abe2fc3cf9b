"""ctypes binding of liblcp.so (the C ABI in include/lcp.h).

Argument marshalling only: tensors become device pointers, dtypes become
lcp_dtype codes, the current torch stream becomes the HIP stream; every step
of the computation runs in the library's kernels. A non-zero status raises
LcpError. If the shared library is missing this module raises at import:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblcp.so")

LCP_OK = 0
LCP_E_INVAL = -1
LCP_E_UNSUPPORTED = -2
LCP_E_WORKSPACE = -3
LCP_E_HIP = -4

LCP_E_SCRATCH = -5

LCP_MAX_ITERS_B = 8192   # largest iters * B the Sinkhorn kernels accept
LCP_NOALLOC_MAX_PARTS = 16384   # partial sums held by lcp_layer_outputs_noalloc's fixed scratch

LCP_F32 = 0
LCP_BF16 = 1

LCP_LOSS_FROBENIUS = 0
LCP_LOSS_COSINE = 1

EXPORTS = [
    "lcp_status_string", "lcp_version", "lcp_sinkhorn", "lcp_sinkhorn_bwd", "lcp_colnorm",
    "lcp_xt_pitch", "lcp_layer_init", "lcp_permute", "lcp_nm_mask",
    "lcp_error_workspace_bytes", "lcp_error", "lcp_step_workspace_bytes", "lcp_step_fwd",
    "lcp_step_bwd", "lcp_harden", "lcp_adamw", "lcp_step_bwd_adamw", "lcp_train",
    "lcp_layer_outputs", "lcp_layer_outputs_noalloc", "lcp_sparse_pack_bytes", "lcp_sparse_pack", "lcp_gather_channels",
    "lcp_sparse_gemm", "lcp_deploy_forward",
]


class lcp_layer(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("X", ctypes.c_void_p), ("Xt", ctypes.c_void_p),
                ("norms", ctypes.c_void_p), ("Y", ctypes.c_void_p), ("y2", ctypes.c_void_p),
                ("dtype", ctypes.c_int), ("cout", ctypes.c_int), ("cin", ctypes.c_int),
                ("T", ctypes.c_int), ("B", ctypes.c_int)]


class lcp_cfg(ctypes.Structure):
    _fields_ = [("iters", ctypes.c_int), ("tau", ctypes.c_float), ("N", ctypes.c_int),
                ("M", ctypes.c_int), ("harden", ctypes.c_int), ("loss", ctypes.c_int),
                ("mask_ste", ctypes.c_int)]


class lcp_adamw_cfg(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class lcp_timing(ctypes.Structure):
    _fields_ = [("start", ctypes.c_void_p * 8), ("stop", ctypes.c_void_p * 8)]


class LcpError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__("%s failed: %d (%s)" % (fn, code, status_string(code)))
        self.code = code


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError("liblcp.so not built (%s); run python "
                          "learnable_channel_permutation_amd/build.py" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    psz = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "lcp_status_string": (ctypes.c_char_p, [i]),
        "lcp_version": (i, []),
        "lcp_sinkhorn": (i, [vp, vp, i, i, i, f, vp]),
        "lcp_sinkhorn_bwd": (i, [vp, vp, i, i, i, f, vp, vp]),
        "lcp_harden": (i, [vp, i, i, vp, vp, vp]),
        "lcp_adamw": (i, [vp, vp, vp, vp, i, i, ctypes.POINTER(lcp_adamw_cfg), vp]),
        "lcp_step_bwd_adamw": (i, [ctypes.POINTER(lcp_layer), vp, ctypes.POINTER(lcp_cfg), vp, sz, vp, vp, i,
                                   ctypes.POINTER(lcp_adamw_cfg), vp, ctypes.POINTER(lcp_timing), vp]),
        "lcp_train": (i, [ctypes.POINTER(lcp_layer), vp, ctypes.POINTER(lcp_cfg), vp, sz, vp, vp, i, f, f,
                          ctypes.POINTER(lcp_adamw_cfg), vp, vp]),
        "lcp_colnorm": (i, [vp, i, i, i, vp, vp]),
        "lcp_xt_pitch": (i, [i]),
        "lcp_layer_init": (i, [vp, i, i, i, vp, vp, vp]),
        "lcp_permute": (i, [vp, i, i, i, vp, vp, i, i, vp, i, vp]),
        "lcp_nm_mask": (i, [vp, i, i, i, i, vp, vp]),
        "lcp_error_workspace_bytes": (i, [i, i, i, i, psz]),
        "lcp_error": (i, [vp, vp, vp, i, i, i, i, vp, vp, vp, sz, vp]),
        "lcp_layer_outputs": (i, [vp, vp, i, i, i, i, vp, vp, vp, sz, vp]),
        "lcp_layer_outputs_noalloc": (i, [vp, vp, i, i, i, i, vp, vp, vp]),
        "lcp_sparse_pack_bytes": (i, [i, i, psz, psz]),
        "lcp_sparse_pack": (i, [vp, i, i, i, vp, vp, vp, vp, vp]),
        "lcp_gather_channels": (i, [vp, i, i, i, vp, vp, vp]),
        "lcp_sparse_gemm": (i, [vp, vp, vp, i, i, i, vp, vp]),
        "lcp_deploy_forward": (i, [vp, vp, vp, i, vp, i, i, i, vp, vp, vp]),
        "lcp_step_workspace_bytes": (i, [i, i, i, i, i, i, psz]),
        "lcp_step_fwd": (i, [ctypes.POINTER(lcp_layer), vp, ctypes.POINTER(lcp_cfg), vp, sz, vp, vp, vp,
                             ctypes.POINTER(lcp_timing), vp]),
        "lcp_step_bwd": (i, [ctypes.POINTER(lcp_layer), vp, ctypes.POINTER(lcp_cfg), vp, sz, vp,
                             ctypes.POINTER(lcp_timing), vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def status_string(code):
    return LIB.lcp_status_string(int(code)).decode()


def _check(fn, code):
    if code != LCP_OK:
        raise LcpError(fn, code)
    return code


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_code(t):
    if t.dtype == torch.float32:
        return LCP_F32
    if t.dtype == torch.bfloat16:
        return LCP_BF16
    raise TypeError("unsupported dtype %s" % t.dtype)


# ---- entry points (same names as the C ABI) --------------------------------
def lcp_sinkhorn(logits, P, iters, tau, stream=None):
    nb, B, _ = logits.shape
    return _check("lcp_sinkhorn", LIB.lcp_sinkhorn(_p(logits), _p(P), nb, B, iters, tau, _stream(stream)))


def lcp_sinkhorn_bwd(logits, dP, iters, tau, dlogits, stream=None):
    nb, B, _ = logits.shape
    return _check("lcp_sinkhorn_bwd", LIB.lcp_sinkhorn_bwd(_p(logits), _p(dP), nb, B, iters, tau,
                                                           _p(dlogits), _stream(stream)))


def lcp_harden(P, P_hard=None, perm=None, stream=None):
    nb, B, _ = P.shape
    return _check("lcp_harden", LIB.lcp_harden(_p(P), nb, B, _p(P_hard), _p(perm), _stream(stream)))


def make_adamw_cfg(lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01):
    return lcp_adamw_cfg(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay))


def lcp_adamw(param, grad, m, v, t, cfg, stream=None):
    return _check("lcp_adamw", LIB.lcp_adamw(_p(param), _p(grad), _p(m), _p(v), param.numel(), int(t),
                                             ctypes.byref(cfg), _stream(stream)))


def lcp_colnorm(X, norms, stream=None):
    T, cin = X.shape
    return _check("lcp_colnorm", LIB.lcp_colnorm(_p(X), dtype_code(X), T, cin, _p(norms), _stream(stream)))


def lcp_xt_pitch(T):
    return LIB.lcp_xt_pitch(int(T))


def lcp_layer_init(X, norms, Xt, stream=None):
    T, cin = X.shape
    return _check("lcp_layer_init", LIB.lcp_layer_init(_p(X), dtype_code(X), T, cin, _p(norms), _p(Xt),
                                                       _stream(stream)))


def lcp_permute(A, P, B, out, colscale=None, transposeP=False, stream=None):
    rows, cin = A.shape
    return _check("lcp_permute", LIB.lcp_permute(_p(A), dtype_code(A), rows, cin, _p(colscale), _p(P), B,
                                                 1 if transposeP else 0, _p(out), dtype_code(out),
                                                 _stream(stream)))


def lcp_nm_mask(scores, N, M, bits, stream=None):
    rows, cin = scores.shape
    return _check("lcp_nm_mask", LIB.lcp_nm_mask(_p(scores), rows, cin, N, M, _p(bits), _stream(stream)))


def lcp_error_workspace_bytes(cout, cin, T, dtype):
    out = ctypes.c_size_t(0)
    _check("lcp_error_workspace_bytes", LIB.lcp_error_workspace_bytes(cout, cin, T, dtype, ctypes.byref(out)))
    return out.value


def lcp_error(W, Wt, X, err, ws, R_out=None, stream=None):
    cout, cin = W.shape
    T = X.shape[0]
    return _check("lcp_error", LIB.lcp_error(_p(W), _p(Wt), _p(X), dtype_code(W), cout, cin, T, _p(err),
                                             _p(R_out), _p(ws), ws.numel() * ws.element_size(),
                                             _stream(stream)))


def lcp_layer_outputs(W, X, Y, y2, ws, stream=None):
    cout, cin = W.shape
    T = X.shape[0]
    return _check("lcp_layer_outputs",
                  LIB.lcp_layer_outputs(_p(W), _p(X), dtype_code(W), cout, cin, T, _p(Y), _p(y2), _p(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))


def lcp_layer_outputs_noalloc(W, X, Y, y2, stream=None):
    cout, cin = W.shape
    T = X.shape[0]
    return _check("lcp_layer_outputs_noalloc",
                  LIB.lcp_layer_outputs_noalloc(_p(W), _p(X), dtype_code(W), cout, cin, T, _p(Y), _p(y2),
                                                _stream(stream)))


def lcp_step_workspace_bytes(cout, cin, T, B, iters, dtype):
    out = ctypes.c_size_t(0)
    _check("lcp_step_workspace_bytes",
           LIB.lcp_step_workspace_bytes(cout, cin, T, B, iters, dtype, ctypes.byref(out)))
    return out.value


def make_layer(W, X, norms, B, Xt=None, Y=None, y2=None):
    cout, cin = W.shape
    return lcp_layer(W.data_ptr(), X.data_ptr(), None if Xt is None else Xt.data_ptr(), norms.data_ptr(),
                     None if Y is None else Y.data_ptr(), None if y2 is None else y2.data_ptr(),
                     dtype_code(W), cout, cin, X.shape[0], B)


def make_cfg(iters, tau, N, M, harden=False, loss="frobenius", mask_ste=False):
    codes = {"frobenius": LCP_LOSS_FROBENIUS, "cosine": LCP_LOSS_COSINE}
    return lcp_cfg(int(iters), float(tau), int(N), int(M), 1 if harden else 0, codes[loss],
                   1 if mask_ste else 0)


def make_timing(starts=(), stops=()):
    tm = lcp_timing()
    for k, e in enumerate(starts):
        tm.start[k] = None if e is None else e.cuda_event
    for k, e in enumerate(stops):
        tm.stop[k] = None if e is None else e.cuda_event
    return tm


def lcp_step_fwd(layer, logits, cfg, ws, err, P_out=None, bits_out=None, timing=None, stream=None):
    return _check("lcp_step_fwd", LIB.lcp_step_fwd(ctypes.byref(layer), _p(logits), ctypes.byref(cfg), _p(ws),
                                                   ws.numel() * ws.element_size(), _p(err), _p(P_out),
                                                   _p(bits_out),
                                                   None if timing is None else ctypes.byref(timing),
                                                   _stream(stream)))


def lcp_step_bwd(layer, logits, cfg, ws, dlogits, timing=None, stream=None):
    return _check("lcp_step_bwd", LIB.lcp_step_bwd(ctypes.byref(layer), _p(logits), ctypes.byref(cfg), _p(ws),
                                                   ws.numel() * ws.element_size(), _p(dlogits),
                                                   None if timing is None else ctypes.byref(timing),
                                                   _stream(stream)))


def lcp_step_bwd_adamw(layer, logits, cfg, ws, m, v, t, acfg, dlogits=None, timing=None, stream=None):
    return _check("lcp_step_bwd_adamw",
                  LIB.lcp_step_bwd_adamw(ctypes.byref(layer), _p(logits), ctypes.byref(cfg), _p(ws),
                                         ws.numel() * ws.element_size(), _p(m), _p(v), int(t), ctypes.byref(acfg),
                                         _p(dlogits), None if timing is None else ctypes.byref(timing),
                                         _stream(stream)))


def lcp_train(layer, logits, cfg, ws, m, v, steps, tau0, tau1, acfg, errs, stream=None):
    return _check("lcp_train", LIB.lcp_train(ctypes.byref(layer), _p(logits), ctypes.byref(cfg), _p(ws),
                                             ws.numel() * ws.element_size(), _p(m), _p(v), int(steps),
                                             float(tau0), float(tau1), ctypes.byref(acfg), _p(errs),
                                             _stream(stream)))



# ---- deploy path ------------------------------------------------------------
def lcp_sparse_pack_bytes(cout, cin):
    vb, mb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("lcp_sparse_pack_bytes", LIB.lcp_sparse_pack_bytes(cout, cin, ctypes.byref(vb), ctypes.byref(mb)))
    return vb.value, mb.value


def lcp_sparse_pack(W, B, perm, bits, vals, meta, stream=None):
    cout, cin = W.shape
    return _check("lcp_sparse_pack", LIB.lcp_sparse_pack(_p(W), cout, cin, int(B), _p(perm), _p(bits), _p(vals),
                                                         _p(meta), _stream(stream)))


def lcp_gather_channels(X, B, perm, Xp, stream=None):
    T, cin = X.shape
    return _check("lcp_gather_channels", LIB.lcp_gather_channels(_p(X), T, cin, int(B), _p(perm), _p(Xp),
                                                                 _stream(stream)))


def lcp_sparse_gemm(vals, meta, Xp, cout, Y, stream=None):
    T, cin = Xp.shape
    return _check("lcp_sparse_gemm", LIB.lcp_sparse_gemm(_p(vals), _p(meta), _p(Xp), T, int(cout), cin, _p(Y),
                                                         _stream(stream)))


def lcp_deploy_forward(vals, meta, perm, B, X, cout, Xp, Y, stream=None):
    T, cin = X.shape
    return _check("lcp_deploy_forward", LIB.lcp_deploy_forward(_p(vals), _p(meta), _p(perm), int(B), _p(X), T,
                                                               int(cout), cin, _p(Xp), _p(Y), _stream(stream)))
