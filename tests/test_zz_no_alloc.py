"""The allocation-free entry point lcp_layer_outputs_noalloc (fixed device
scratch inside the library, no workspace argument) against the workspace
entry point lcp_layer_outputs, through the C ABI: the same kernels, so Y and
||Y||^2 must agree bit for bit; two calls in a row on one GPU, the second on
a smaller input, each checked (the scratch keeps the previous call's
partials, which must not leak into the next result)."""
import numpy as np
import pytest
import torch

import lcp_synth
import oracle
from tests.gpu_util import DEV, down, rel_fro, say, up

pytestmark = pytest.mark.gpu

lcp = pytest.importorskip("learnable_channel_permutation_amd")
L = lcp._lib


def _inputs(cout, cin, T, dtype, seed):
    W = lcp_synth.random_matrix(seed, (cout, cin), std=0.02, dtype=dtype)
    X = lcp_synth.random_matrix(seed + 1, (T, cin), std=1.0, dtype=dtype)
    return W, X


def _both(W, X, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cout, cin = W.shape
    T = X.shape[0]
    pitch = L.lcp_xt_pitch(T)
    dW, dX = up(W, tdt), up(X, tdt)
    ws = torch.empty(L.lcp_error_workspace_bytes(cout, cin, T, L.dtype_code(dW)), dtype=torch.uint8, device=DEV)
    Y_ws = torch.full((cout, pitch), 7.0, dtype=tdt, device=DEV)
    y2_ws = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    Y_na = torch.full((cout, pitch), 9.0, dtype=tdt, device=DEV)
    y2_na = torch.full((1,), -2.0, dtype=torch.float32, device=DEV)
    L.lcp_layer_outputs(dW, dX, Y_ws, y2_ws, ws)
    L.lcp_layer_outputs_noalloc(dW, dX, Y_na, y2_na)
    torch.cuda.synchronize()
    return Y_ws, y2_ws, Y_na, y2_na


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point_two_calls(dtype):
    shapes = [(1100, 384, 700), (300, 160, 130)] if dtype == "bf16" else [(200, 192, 150), (70, 96, 33)]
    for k, (cout, cin, T) in enumerate(shapes):
        say("noalloc layer outputs", dtype, "call", k, cout, cin, T)
        W, X = _inputs(cout, cin, T, dtype, 50 + 7 * k)
        Y_ws, y2_ws, Y_na, y2_na = _both(W, X, dtype)
        assert torch.equal(Y_ws, Y_na)
        assert torch.equal(y2_ws, y2_na)
        # and the result is the layer's output (oracle, float64)
        ref = oracle.layer_output(W, X)
        tol = 1e-2 if dtype == "bf16" else 1e-5
        assert rel_fro(down(Y_na)[:, :T], ref) < tol
        assert np.all(down(Y_na)[:, T:] == 0)
        want = float(np.sum(ref * ref))
        assert abs(float(y2_na.item()) - want) / want < tol


def test_noalloc_rejects_oversized_input_before_launch():
    """A shape needing more partials than the fixed scratch holds returns
    LCP_E_SCRATCH and leaves the outputs untouched."""
    say("noalloc oversized")
    cout, cin, T = 129 * 256, 32, 128 * 128 + 1
    W = torch.zeros((1, 32), dtype=torch.bfloat16, device=DEV)
    Y = torch.full((4,), 3.0, dtype=torch.bfloat16, device=DEV)
    y2 = torch.full((1,), 5.0, dtype=torch.float32, device=DEV)
    rc = L.LIB.lcp_layer_outputs_noalloc(L._p(W), L._p(W), L.LCP_BF16, cout, cin, T, L._p(Y), L._p(y2), None)
    torch.cuda.synchronize()
    assert rc == L.LCP_E_SCRATCH
    assert float(y2.item()) == 5.0 and torch.all(Y == 3.0)
