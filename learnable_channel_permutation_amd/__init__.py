"""MI355X (gfx950) learnable channel permutation (LCP) step.

The computation lives in liblcp.so (HIP kernels behind the C ABI of
include/lcp.h); this package only binds it (``_lib``) and wraps the
per-layer buffers in a small session object. Importing fails if the library
has not been built.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (LCP_BF16, LCP_F32, LcpError, lcp_colnorm, lcp_error,  # noqa: F401
                   lcp_error_workspace_bytes, lcp_harden, lcp_layer_init, lcp_nm_mask, lcp_permute,
                   lcp_sinkhorn, lcp_sinkhorn_bwd, lcp_step_bwd, lcp_step_fwd,
                   lcp_step_workspace_bytes, lcp_xt_pitch, make_cfg, make_layer, make_timing,
                   lcp_adamw, lcp_step_bwd_adamw, lcp_train, make_adamw_cfg, lcp_layer_outputs)

__all__ = ["LayerSession", "LcpError"] + [n for n in _lib.EXPORTS if n.startswith("lcp_")]


class LayerSession:
    """Device buffers for repeated LCP steps on one layer.

    Holds W and X (caller tensors on one GPU), the per-layer setup written by
    lcp_layer_init (column norms; X transposed for bf16 layers) and one step
    workspace sized by lcp_step_workspace_bytes. harden=True runs the
    hardened forward with the straight-through backward; loss="cosine"
    optimises the cosine objective (the dense outputs Y = W X^T and ||Y||^2
    are then computed once here by lcp_layer_outputs); mask_ste=True adds the
    straight-through gradient of the mask.
    """

    def __init__(self, W, X, B, iters, tau, N, M, stream=None, harden=False, loss="frobenius",
                 mask_ste=False):
        if W.device != X.device or W.dtype != X.dtype:
            raise ValueError("W and X must share device and dtype")
        self.W, self.X = W, X
        self.B, self.iters, self.tau, self.N, self.M = B, iters, tau, N, M
        cout, cin = W.shape
        T = X.shape[0]
        dev = W.device
        self.norms = torch.empty(cin, dtype=torch.float32, device=dev)
        self.Xt = None
        if W.dtype == torch.bfloat16:
            self.Xt = torch.empty((cin, lcp_xt_pitch(T)), dtype=torch.bfloat16, device=dev)
        nbytes = lcp_step_workspace_bytes(cout, cin, T, B, iters, _lib.dtype_code(W))
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.err = torch.empty(1, dtype=torch.float32, device=dev)
        self.Y = self.y2 = None
        if loss == "cosine":
            self.Y = torch.empty((cout, lcp_xt_pitch(T)), dtype=W.dtype, device=dev)
            self.y2 = torch.empty(1, dtype=torch.float32, device=dev)
        self.layer = make_layer(W, X, self.norms, B, self.Xt, self.Y, self.y2)
        self.cfg = make_cfg(iters, tau, N, M, harden, loss, mask_ste)
        self.init(stream)

    def init(self, stream=None):
        """Per-layer setup (column norms, transposed X; dense outputs and
        their squared norm for the cosine objective)."""
        lcp_layer_init(self.X, self.norms, self.Xt, stream=stream)
        if self.Y is not None:
            cout, cin = self.W.shape
            ebytes = lcp_error_workspace_bytes(cout, cin, self.X.shape[0], _lib.dtype_code(self.W))
            if ebytes > self.ws.numel():
                raise RuntimeError("step workspace smaller than the layer-output workspace")
            lcp_layer_outputs(self.W, self.X, self.Y, self.y2, self.ws, stream=stream)

    def forward(self, logits, P_out=None, bits_out=None, timing=None, stream=None):
        lcp_step_fwd(self.layer, logits, self.cfg, self.ws, self.err, P_out, bits_out, timing, stream)
        return self.err

    def backward(self, logits, dlogits=None, timing=None, stream=None):
        if dlogits is None:
            dlogits = torch.empty_like(logits)
        lcp_step_bwd(self.layer, logits, self.cfg, self.ws, dlogits, timing, stream)
        return dlogits

    def capture_step(self, logits, dlogits, setup=True):
        """Capture one step on fixed buffers into a HIP graph
        (torch.cuda.CUDAGraph): the per-layer setup (when `setup`), the
        forward (E into self.err) and the backward (into `dlogits`). The
        library allocates nothing, synchronises nothing and issues no memset
        inside a step, so the captured kernels are exactly the eager ones;
        graph.replay() reruns them on the current contents of the buffers."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):           # one eager run before capture
            if setup:
                self.init()
            self.forward(logits)
            self.backward(logits, dlogits)
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            if setup:
                self.init()
            self.forward(logits)
            self.backward(logits, dlogits)
        return g

    def train(self, logits, steps, lr, tau0=1.0, tau1=0.1, beta1=0.9, beta2=0.999, eps=1e-8,
              weight_decay=0.01, stream=None):
        """`steps` AdamW steps on `logits` (updated in place) with the
        temperature annealed linearly from tau0 to tau1 (lcp_train). Returns
        the per-step objective values as a device tensor."""
        m = torch.zeros_like(logits)
        v = torch.zeros_like(logits)
        errs = torch.empty(steps, dtype=torch.float32, device=logits.device)
        acfg = make_adamw_cfg(lr, beta1, beta2, eps, weight_decay)
        lcp_train(self.layer, logits, self.cfg, self.ws, m, v, steps, tau0, tau1, acfg, errs, stream)
        return errs

