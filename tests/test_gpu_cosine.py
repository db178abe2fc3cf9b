"""GPU parity of the cosine objective ([PermLLM] optimisation objective) and
of the straight-through mask gradient ([PermLLM] integration with pruning
methods) against the float64 oracle, through the C ABI, on seeded inputs.
Tolerances: layer outputs and their squared norm 1e-2 relative (bf16) or
1e-5 (fp32); the cosine loss 1e-2 relative (1e-4 in fp32); masks >= 99.9 %;
gradients against the oracle's backward on the GPU's mask: 1e-2 relative in
the Frobenius norm over the whole tensor and 2e-2 for every B x B block."""
import numpy as np
import pytest
import torch

import lcp_synth
import oracle
from tests.grad_check import check_gradient, oracle_backward_on_mask
from tests.gpu_util import DEV, bit_agreement, bits_down, down, empty_bits, rel_fro, say, up

pytestmark = pytest.mark.gpu

lcp = pytest.importorskip("learnable_channel_permutation_amd")
L = lcp._lib


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cout,cin,T", [(300, 352, 200), (513, 128, 65), (256, 256, 256)])
def test_layer_outputs(dtype, cout, cin, T):
    """Y = W X^T with zero padding columns, and ||Y||^2."""
    W = lcp_synth.random_matrix(11 + cout, (cout, cin), std=0.02, dtype=dtype)
    X = lcp_synth.random_matrix(12 + cout, (T, cin), std=1.0, dtype=dtype)
    say("layer outputs", dtype, cout, cin, T)
    tdt = _tdt(dtype)
    pitch = L.lcp_xt_pitch(T)
    Y = torch.full((cout, pitch), 5.0, dtype=tdt, device=DEV)
    y2 = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(L.lcp_error_workspace_bytes(cout, cin, T, L.dtype_code(Y)), dtype=torch.uint8, device=DEV)
    L.lcp_layer_outputs(up(W, tdt), up(X, tdt), Y, y2, ws)
    torch.cuda.synchronize()
    ref = oracle.layer_output(W, X)
    tol = 1e-2 if dtype == "bf16" else 1e-5
    Yg = down(Y)
    assert rel_fro(Yg[:, :T], ref) < tol
    assert np.all(Yg[:, T:] == 0)
    want = float(np.sum(ref * ref))
    assert abs(float(y2.item()) - want) / want < tol


def _session(lay, spec, **kw):
    tdt = _tdt(spec.dtype)
    return lcp.LayerSession(up(lay.W, tdt), up(lay.X, tdt), spec.B, spec.iters, spec.tau, spec.N, spec.M, **kw)


def _check(lay, spec, lg, loss, mask_ste, harden, l_tol=1e-2, g_tol=1e-2):
    s = _session(lay, spec, harden=harden, loss=loss, mask_ste=mask_ste)
    d_lg = up(lg)
    bits = empty_bits(lay.cout, lay.cin)
    err = s.forward(d_lg, bits_out=bits)
    dl = s.backward(d_lg)
    torch.cuda.synchronize()
    fw = oracle.step_forward(lay.W, lay.X, lg, spec.tau, spec.iters, spec.N, spec.M, hard=harden, loss=loss)
    agree = bit_agreement(bits_down(bits), oracle.pack_bits(fw["mask"]), lay.cout * lay.cin)
    assert agree >= 0.999, agree
    got = float(err.item())
    assert abs(got - fw["L"]) / fw["L"] < l_tol, (got, fw["L"])
    # gradient: the oracle's backward on the GPU's mask, whole and per block
    fwm, bw = oracle_backward_on_mask(lay, spec, lg, bits_down(bits), hard=harden, loss=loss, mask_ste=mask_ste)
    check_gradient(down(dl), bw["dlogits"], tol=g_tol, block_tol=2e-2)
    return fwm, bw


SMALL = [
    # (config index, cout, cin, T): several tiles and ragged tails
    (0, 256, 256, 256),
    (1, 300, 512, 200),
    (2, 270, 640, 130),
    (3, 257, 512, 96),
]


@pytest.mark.parametrize("ci,cout,cin,T", SMALL)
@pytest.mark.parametrize("harden", [False, True])
def test_step_cosine(ci, cout, cin, T, harden):
    """Cosine objective, mask constant: the loss and its gradient."""
    spec = lcp_synth.CONFIGS[ci]
    lay = lcp_synth.make_layer(spec, cout=cout, cin=cin, T=T)
    lg = lay.logits
    if harden:
        lg, _ = lcp_synth.planted_logits(600 + ci, cin // spec.B, spec.B, peak=1.5, noise_std=0.3)
    say("step cosine", spec.name, cout, cin, T, harden)
    tight = spec.dtype == "f32"
    _check(lay, spec, lg, "cosine", False, harden, l_tol=1e-4 if tight else 1e-2)


@pytest.mark.parametrize("ci,cout,cin,T", SMALL)
@pytest.mark.parametrize("loss", ["frobenius", "cosine"])
@pytest.mark.parametrize("harden", [False, True])
def test_step_mask_ste(ci, cout, cin, T, loss, harden):
    """Straight-through gradient of the mask for both objectives, soft and
    hardened forward; the extra term changes the gradient visibly."""
    spec = lcp_synth.CONFIGS[ci]
    lay = lcp_synth.make_layer(spec, cout=cout, cin=cin, T=T)
    lg = lay.logits
    if harden:
        lg, _ = lcp_synth.planted_logits(700 + ci, cin // spec.B, spec.B, peak=1.5, noise_std=0.3)
    say("step mask ste", spec.name, cout, cin, T, loss, harden)
    fw, bw = _check(lay, spec, lg, loss, True, harden)
    plain = oracle.step_backward(fw, lay.X, lay.W)["dlogits"]
    assert rel_fro(plain, bw["dlogits"]) > 0.05


def test_cosine_zero_outputs():
    """X = 0: both output norms vanish, the loss is 1 and the gradient 0."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=64, cin=128, T=64)
    lay.X[:] = 0.0
    say("cosine zero X")
    s = _session(lay, spec, loss="cosine", mask_ste=True)
    d_lg = up(lay.logits)
    err = s.forward(d_lg)
    dl = s.backward(d_lg)
    torch.cuda.synchronize()
    assert float(err.item()) == 1.0
    assert torch.count_nonzero(dl).item() == 0


def test_cosine_scale_invariance():
    """Scaling X by a power of two scales Y and Y~ alike: the GPU's cosine
    loss is unchanged (within rounding)."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=256, cin=256, T=128)
    say("cosine scale invariance")
    vals = []
    for scale in (1.0, 4.0):
        X = lay.X * np.float32(scale)
        s = lcp.LayerSession(up(lay.W, torch.bfloat16), up(X, torch.bfloat16), spec.B, spec.iters, spec.tau,
                             spec.N, spec.M, loss="cosine")
        vals.append(float(s.forward(up(lay.logits)).item()))
    torch.cuda.synchronize()
    assert abs(vals[0] - vals[1]) <= 1e-4 * vals[0], vals


def test_step_cosine_full_size_bench_layer():
    """The 4096 x 11008 layer at full size with the cosine objective and the
    mask's straight-through term: loss, mask and gradient against the full
    float64 oracle."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec)
    say("step cosine full size", spec.name)
    _check(lay, spec, lay.logits, "cosine", True, False)


def test_step_cosine_ste_hardened_full_size_b128():
    """The 13824 x 5120 layer (B = 128, 4:8) at full size with every option:
    hardened forward, cosine objective, the mask's straight-through term."""
    spec = lcp_synth.UP_PROJ_13824x5120
    lay = lcp_synth.make_layer(spec)
    lg, _ = lcp_synth.planted_logits(650, lay.cin // spec.B, spec.B, peak=1.5, noise_std=0.3)
    say("step cosine ste hardened full size", spec.name)
    _check(lay, spec, lg, "cosine", True, True)


def test_training_cosine_beats_wanda():
    """lcp_train on the cosine objective (hardened forward, straight-through
    backward through P, mask constant): the first step is plain Wanda's
    cosine loss, the loop reaches hard permutations with a lower loss, and
    the GPU's loss of the final logits agrees with the oracle's."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=256, cin=512, T=256)
    nb = lay.cin // spec.B
    lg0 = lcp_synth.make_logits(np.random.Generator(np.random.PCG64(7)), nb, spec.B, diag=0.5)
    say("train cosine")
    s = _session(lay, spec, harden=True, loss="cosine")
    lg = up(lg0)
    errs = down(s.train(lg, 40, 1e-2))
    s.cfg.tau = 0.1
    final_gpu = float(s.forward(lg).item())
    torch.cuda.synchronize()
    eye = np.eye(spec.B)[None].repeat(nb, axis=0)
    wanda = oracle.step_forward(lay.W, lay.X, None, 1.0, spec.iters, spec.N, spec.M, P=eye, loss="cosine")["L"]
    final = oracle.step_forward(lay.W, lay.X, down(lg), 0.1, spec.iters, spec.N, spec.M, hard=True,
                                loss="cosine")["L"]
    assert abs(errs[0] - wanda) / wanda < 1e-2, (errs[0], wanda)
    assert np.min(errs) < 0.99 * wanda, (np.min(errs), wanda)
    assert abs(final_gpu - final) / final < 1e-2, (final_gpu, final)
    # as for the Frobenius loop on this slice, the last iterate is not
    # reliably below Wanda's loss; the final-vs-Wanda pin runs on the whole
    # layers (test_gpu_parity.py, test_training_beats_wanda_full_size)
