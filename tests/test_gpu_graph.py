"""The LCP step captured into a HIP graph: every replay, with eager work and
synchronisations between replays, gives bit for bit the eager step's error
and gradient (the kernels are deterministic, and the step allocates and
clears nothing)."""
import numpy as np
import pytest
import torch

import lcp_synth
from tests.gpu_util import say, up

pytestmark = pytest.mark.gpu

lcp = pytest.importorskip("learnable_channel_permutation_amd")


@pytest.mark.parametrize("ci,harden,loss", [(2, False, "frobenius"), (2, True, "cosine"), (0, False, "frobenius")])
def test_graph_replays_match_eager(ci, harden, loss):
    spec = lcp_synth.CONFIGS[ci]
    lay = lcp_synth.make_layer(spec, cout=256, cin=256, T=128)
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    say("graph", spec.name, harden, loss)
    s = lcp.LayerSession(up(lay.W, tdt), up(lay.X, tdt), spec.B, spec.iters, spec.tau, spec.N, spec.M,
                         harden=harden, loss=loss)
    lg = up(lay.logits)
    dl = torch.empty_like(lg)
    # eager reference
    s.init()
    e_ref = s.forward(lg).clone()
    s.backward(lg, dl)
    d_ref = dl.clone()
    torch.cuda.synchronize()
    g = s.capture_step(lg, dl)
    other = up(lcp_synth.random_logits(5, lg.shape[0], spec.B))
    for r in range(3):
        dl.fill_(123.0)
        s.err.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(s.err, e_ref), (r, s.err.item(), e_ref.item())
        assert torch.equal(dl, d_ref), r
        # eager work between replays on the same session and buffers
        s.forward(other)
        s.backward(other, dl)
        torch.cuda.synchronize()
        assert not torch.equal(dl, d_ref)
    # the replay reads the logits' current contents
    lg.copy_(other)
    g.replay()
    torch.cuda.synchronize()
    dl2 = torch.empty_like(dl)
    e2 = s.forward(other).clone()
    s.backward(other, dl2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(s.err, e2) and torch.equal(dl, dl2)
