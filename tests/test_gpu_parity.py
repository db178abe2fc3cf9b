"""GPU parity: every kernel of the LCP step against the float64 oracle, through
the C ABI, on seeded inputs. Tolerances: Sinkhorn per entry 1e-5 relative +
1e-9; masks bit-exact on the oracle's scores and >= 99.9 % of bits end to end;
GEMM residual and error 1e-2 relative; gradients against the oracle's backward
taken on the GPU's mask (held constant): 1e-2 relative (Frobenius) over the
whole tensor and 2e-2 for every B x B block."""
import dataclasses

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


def _sink_tol(ref):
    return 1e-5 * np.abs(ref) + 1e-9


# ------------------------------------------------------------------ Sinkhorn --
@pytest.mark.parametrize("B,iters,tau,kind", [
    (32, 5, 1.0, "eye"), (64, 5, 1.0, "eye"), (128, 7, 1.0, "eye"),
    (32, 1, 1.0, "randn"), (64, 5, 0.5, "randn"), (128, 5, 1.0, "randn"),
    (64, 20, 1.0, "randn"), (64, 5, 0.1, "eye"), (32, 3, 2.0, "uniform"),
])
def test_sinkhorn_forward(B, iters, tau, kind):
    nb = 37
    if kind == "eye":
        lg = lcp_synth.make_logits(np.random.Generator(np.random.PCG64(B + iters)), nb, B)
    elif kind == "randn":
        lg = lcp_synth.random_logits(B * 7 + iters, nb, B)
    else:
        lg = np.full((nb, B, B), 0.25, dtype=np.float32)
    say("sinkhorn fwd", B, iters, tau, kind)
    d_lg = up(lg)
    d_P = torch.empty_like(d_lg)
    L.lcp_sinkhorn(d_lg, d_P, iters, tau)
    torch.cuda.synchronize()
    ref = oracle.sinkhorn(lg.astype(np.float64), np.float64(np.float32(tau)), iters)
    got = down(d_P)
    assert np.all(np.abs(got - ref) <= _sink_tol(ref)), np.max(np.abs(got - ref) / (np.abs(ref) + 1e-9))
    # in place
    L.lcp_sinkhorn(d_lg, d_lg, iters, tau)
    torch.cuda.synchronize()
    assert np.array_equal(down(d_lg), got)


@pytest.mark.parametrize("B", [32, 64, 128])
def test_sinkhorn_underflowing_columns(B):
    """Blocks with a column far below every row's maximum (its exponentials
    underflow in the row step) next to ordinary blocks: the forward, and the
    backward that recomputes the iterates, still follow the log-domain
    definition. Logits of magnitude 200 put |Z| near 290 (base 2), which
    float32 carries to about |Z| 2^-24 per operation; over the 2L
    subtractions of the iterates that bounds P's relative error by
    2L |Z| 2^-24 ln 2 (1.2e-4 here) on top of the usual 1e-5."""
    nb, iters, tau = 6, 5, 1.0
    lg = lcp_synth.random_logits(300 + B, nb, B, scale=0.5)
    lg[0, :, 3] = -200.0                  # one such column
    lg[1, :, :B // 2] -= 150.0            # half the columns of a block
    lg[2, 5, :] = 120.0                   # one dominant row
    lg[2, 5, 7] = 240.0
    say("sinkhorn underflowing columns", B)
    d_lg = up(lg)
    d_P = torch.empty_like(d_lg)
    L.lcp_sinkhorn(d_lg, d_P, iters, tau)
    torch.cuda.synchronize()
    ref = oracle.sinkhorn(lg.astype(np.float64), np.float64(tau), iters)
    got = down(d_P)
    assert np.all(np.isfinite(got))
    zmax = np.max(np.abs(lg)) / tau * np.log2(np.e)
    tol = _sink_tol(ref) + 2 * iters * zmax * 2.0 ** -24 * np.log(2) * np.abs(ref)
    assert np.all(np.abs(got - ref) <= tol), np.max(np.abs(got - ref) / (np.abs(ref) + 1e-9))
    dP = lcp_synth.random_matrix(400 + B, (nb, B, B))
    d_out = torch.empty((nb, B, B), dtype=torch.float32, device=DEV)
    L.lcp_sinkhorn_bwd(d_lg, up(dP), iters, tau, d_out)
    torch.cuda.synchronize()
    P, tr = oracle.sinkhorn(lg.astype(np.float64), np.float64(tau), iters, trace=True)
    want = oracle.sinkhorn_adjoint(dP.astype(np.float64), P, tr, np.float64(tau))
    assert rel_fro(down(d_out), want) < 1e-4


@pytest.mark.parametrize("B,iters,tau", [(32, 5, 1.0), (64, 5, 0.7), (128, 7, 1.0), (64, 1, 1.0)])
def test_sinkhorn_backward(B, iters, tau):
    nb = 19
    lg = lcp_synth.random_logits(100 + B, nb, B, scale=0.5)
    dP = lcp_synth.random_matrix(200 + B, (nb, B, B))
    say("sinkhorn bwd", B, iters, tau)
    d_out = torch.empty((nb, B, B), dtype=torch.float32, device=DEV)
    L.lcp_sinkhorn_bwd(up(lg), up(dP), iters, tau, d_out)
    torch.cuda.synchronize()
    tau64 = np.float64(np.float32(tau))
    P, tr = oracle.sinkhorn(lg.astype(np.float64), tau64, iters, trace=True)
    ref = oracle.sinkhorn_adjoint(dP.astype(np.float64), P, tr, tau64)
    assert rel_fro(down(d_out), ref) < 1e-4


@pytest.mark.parametrize("B", [32, 64, 128])
def test_sinkhorn_at_the_iteration_cap(B):
    """iters * B = LCP_MAX_ITERS_B, the largest count the kernels accept (the
    reverse pass keeps the offsets of every iteration of a block in LDS):
    the forward per entry and the backward against the oracle. The iterates
    are rebuilt from 2L offsets, each subtraction rounding by up to
    |Z| 2^-24 (base 2), which bounds the extra relative error by
    2L |Z| 2^-24 ln 2 (about 3e-5 at L = 256 here)."""
    iters, nb, tau = L.LCP_MAX_ITERS_B // B, 5, 1.0
    lg = lcp_synth.random_logits(500 + B, nb, B, scale=0.5)
    say("sinkhorn at the iteration cap", B, iters)
    d_lg = up(lg)
    d_P = torch.empty_like(d_lg)
    L.lcp_sinkhorn(d_lg, d_P, iters, tau)
    dP = lcp_synth.random_matrix(600 + B, (nb, B, B))
    d_out = torch.empty((nb, B, B), dtype=torch.float32, device=DEV)
    L.lcp_sinkhorn_bwd(d_lg, up(dP), iters, tau, d_out)
    torch.cuda.synchronize()
    P, tr = oracle.sinkhorn(lg.astype(np.float64), np.float64(tau), iters, trace=True)
    drift = 2 * iters * (np.max(np.abs(lg)) / tau * np.log2(np.e)) * 2.0 ** -24 * np.log(2)
    got = down(d_P)
    assert np.all(np.abs(got - P) <= _sink_tol(P) + drift * np.abs(P)), np.max(np.abs(got - P) / (np.abs(P) + 1e-9))
    want = oracle.sinkhorn_adjoint(dP.astype(np.float64), P, tr, np.float64(tau))
    assert rel_fro(down(d_out), want) < 1e-4 + drift


def test_step_at_the_iteration_cap():
    """A whole bf16 step (B = 64) with iters * B = LCP_MAX_ITERS_B: the
    forward's offsets and the backward's LDS copy of them at their largest,
    against the float64 oracle with the same tolerances as every step."""
    spec = dataclasses.replace(lcp_synth.CONFIGS[2], iters=L.LCP_MAX_ITERS_B // 64)
    lay = lcp_synth.make_layer(spec, cout=96, cin=128, T=64)
    say("step at the iteration cap", spec.iters)
    got = _run_step(lay, spec)
    _check_step(lay, spec, got)


# ---------------------------------------------------------------- N:M mask --
def _mask_scores(rows, cin, seed):
    lay = lcp_synth.make_layer(lcp_synth.DOWN_PROJ_4096x11008, seed=seed, cout=rows, cin=cin, T=64)
    fw = oracle.step_forward(lay.W, lay.X, lay.logits, 1.0, 5, 2, 4)
    S = fw["S_hat"].astype(np.float32)
    rng = np.random.Generator(np.random.PCG64(seed))
    S[0, :] = 1.0                                          # all ties
    S[1, :] = rng.integers(0, 3, size=cin).astype(np.float32)  # many ties
    S[2, ::5] = np.nan
    S[3, ::7] = np.inf
    S[3, 1::7] = -np.inf
    S[4, ::2] = -0.0
    S[4, 1::2] = 0.0
    return S


@pytest.mark.parametrize("N,M", [(1, 4), (2, 4), (3, 4), (1, 8), (2, 8), (4, 8), (7, 8)])
def test_nm_mask_bit_exact(N, M):
    rows, cin = 67, 256
    S = _mask_scores(rows, cin, 31 + N + M)
    say("nm_mask", N, M)
    bits = empty_bits(rows, cin)
    L.lcp_nm_mask(up(S), N, M, bits)
    torch.cuda.synchronize()
    want = oracle.pack_bits(oracle.nm_mask(S, N, M))
    got = bits_down(bits)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("rows,cin", [(1, 32), (5, 96), (300, 1056)])
@pytest.mark.parametrize("N,M", [(2, 4), (4, 8)])
def test_nm_mask_shapes(rows, cin, N, M):
    """Partial workgroups and partial waves: the last thread's words and
    the words past the end (which must not be written)."""
    S = np.ascontiguousarray(_mask_scores(max(rows, 8), (cin + 63) // 64 * 64, 7 + rows)[:rows, :cin])
    say("nm_mask shapes", rows, cin, N, M)
    flat = torch.full((rows * (cin // 32) + 16,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    L.lcp_nm_mask(up(S), N, M, flat)
    torch.cuda.synchronize()
    want = oracle.pack_bits(oracle.nm_mask(S, N, M))
    got = flat.cpu().numpy()
    assert np.array_equal(got[: rows * (cin // 32)].view(np.uint32).reshape(rows, cin // 32), want)
    assert np.all(got[rows * (cin // 32):] == 0x5A5A5A5A)


# ------------------------------------------------------------ layer setup --
@pytest.mark.parametrize("T,cin", [(100, 96), (2048, 256), (64, 32)])
def test_layer_init_bf16(T, cin):
    lay = lcp_synth.make_layer(lcp_synth.F32_256x256, seed=5, cout=32, cin=cin, T=T, dtype="bf16")
    say("layer_init bf16", T, cin)
    X = up(lay.X, torch.bfloat16)
    norms = torch.empty(cin, dtype=torch.float32, device=DEV)
    pitch = L.lcp_xt_pitch(T)
    Xt = torch.full((cin, pitch), 7.0, dtype=torch.bfloat16, device=DEV)
    L.lcp_layer_init(X, norms, Xt)
    n2 = torch.empty_like(norms)
    L.lcp_colnorm(X, n2)
    torch.cuda.synchronize()
    ref = oracle.colnorm(lay.X)
    assert np.max(np.abs(down(norms) - ref) / ref) < 1e-5
    assert np.array_equal(down(norms), down(n2))
    xt = down(Xt)
    assert np.array_equal(xt[:, :T], lay.X.T.astype(np.float64))
    assert np.all(xt[:, T:] == 0)


def test_colnorm_f32():
    lay = lcp_synth.make_layer(lcp_synth.F32_256x256, seed=6, cout=32, cin=96, T=77)
    say("colnorm f32")
    norms = torch.empty(96, dtype=torch.float32, device=DEV)
    L.lcp_colnorm(up(lay.X), norms)
    torch.cuda.synchronize()
    ref = oracle.colnorm(lay.X)
    assert np.max(np.abs(down(norms) - ref) / ref) < 1e-5


# ------------------------------------------------------------------ permute --
def _perm_case(rows, cin, B, seed, dtype="bf16"):
    W = lcp_synth.random_matrix(seed, (rows, cin), std=0.02, dtype=dtype)
    lg = lcp_synth.random_logits(seed + 1, cin // B, B, scale=1.0)
    P = oracle.sinkhorn(lg.astype(np.float64), 1.0, 5).astype(np.float32)
    return W, P


@pytest.mark.parametrize("rows,cin,B", [(100, 192, 64), (300, 256, 128), (77, 96, 32), (256, 512, 64)])
@pytest.mark.parametrize("transposeP", [False, True])
def test_permute_plain_bf16(rows, cin, B, transposeP):
    W, P = _perm_case(rows, cin, B, rows + cin + B)
    say("permute plain bf16", rows, cin, B, transposeP)
    dW = up(W, torch.bfloat16)
    out32 = torch.empty((rows, cin), dtype=torch.float32, device=DEV)
    out16 = torch.empty((rows, cin), dtype=torch.bfloat16, device=DEV)
    L.lcp_permute(dW, up(P), B, out32, transposeP=transposeP)
    L.lcp_permute(dW, up(P), B, out16, transposeP=transposeP)
    torch.cuda.synchronize()
    ref = oracle.block_permute(W, P, transpose=transposeP)
    # P enters the MFMA as bf16 (relative rounding <= 2^-9 per entry), products
    # are exact and accumulate in fp32; bf16 output adds 2^-9 relative.
    bound = oracle.block_permute(np.abs(W), np.abs(P), transpose=transposeP) * 2.0 ** -8 + 1e-12
    assert np.all(np.abs(down(out32) - ref) <= bound)
    assert np.all(np.abs(down(out16) - ref) <= bound + np.abs(ref) * 2.0 ** -8)


@pytest.mark.parametrize("rows,cin,B", [(100, 192, 64), (300, 256, 128), (77, 96, 32)])
def test_permute_importance_bf16(rows, cin, B):
    W, P = _perm_case(rows, cin, B, 3 * rows + B)
    n = (np.random.Generator(np.random.PCG64(rows)).lognormal(0, 1, cin) * 40).astype(np.float32)
    say("permute importance bf16", rows, cin, B)
    out = torch.empty((rows, cin), dtype=torch.float32, device=DEV)
    L.lcp_permute(up(W, torch.bfloat16), up(P), B, out, colscale=up(n))
    torch.cuda.synchronize()
    ref = oracle.block_permute(oracle.importance(W, n), P)
    # float32-accurate: n_j P_jk rounds once to fp32, its bf16 split is exact
    # (B = 128 keeps two terms: 2^-17), products exact, fp32 accumulation
    rel = np.abs(down(out) - ref) / np.maximum(ref, 1e-30)
    assert np.max(rel) < (2e-5 if B == 128 else 5e-6), np.max(rel)


@pytest.mark.parametrize("B", [32, 64, 128])
def test_permute_f32(B):
    rows, cin = 45, 2 * B
    W, P = _perm_case(rows, cin, B, 11 * B, dtype="f32")
    n = np.abs(lcp_synth.random_matrix(5, (cin,))) + 0.5
    say("permute f32", B)
    out = torch.empty((rows, cin), dtype=torch.float32, device=DEV)
    L.lcp_permute(up(W), up(P), B, out)
    imp = torch.empty_like(out)
    L.lcp_permute(up(W), up(P), B, imp, colscale=up(n))
    torch.cuda.synchronize()
    assert rel_fro(down(out), oracle.block_permute(W, P)) < 1e-6
    assert rel_fro(down(imp), oracle.block_permute(oracle.importance(W, n), P)) < 1e-6


# -------------------------------------------------------------------- error --
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cout,cin,T", [(300, 352, 200), (256, 256, 256), (513, 128, 65)])
def test_error_gemm(dtype, cout, cin, T):
    W = lcp_synth.random_matrix(1 + cout, (cout, cin), std=0.02, dtype=dtype)
    Wt = lcp_synth.random_matrix(2 + cout, (cout, cin), std=0.02, dtype=dtype)
    X = lcp_synth.random_matrix(3 + cout, (T, cin), std=1.0, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    say("error gemm", dtype, cout, cin, T)
    ws = torch.empty(L.lcp_error_workspace_bytes(cout, cin, T, L.LCP_BF16 if dtype == "bf16" else L.LCP_F32),
                     dtype=torch.uint8, device=DEV)
    err = torch.empty(1, dtype=torch.float32, device=DEV)
    pitch = L.lcp_xt_pitch(T)
    R = torch.full((cout, pitch), 3.0, dtype=tdt, device=DEV)
    L.lcp_error(up(W, tdt), up(Wt, tdt), up(X, tdt), err, ws, R_out=R)
    torch.cuda.synchronize()
    Rref, Eref = oracle.pruning_error(W.astype(np.float64) - Wt, X)
    Rg = down(R)
    tol = 1e-2 if dtype == "bf16" else 1e-5
    assert abs(float(err.item()) - Eref) / Eref < tol
    assert rel_fro(Rg[:, :T], Rref) < tol
    assert np.all(Rg[:, T:] == 0)


@pytest.mark.parametrize("cin", list(range(32, 545, 32)))
def test_error_gemm_k_tails(cin):
    """bf16 error GEMM over every count of 64-wide K steps from 1 to 9 (the
    software-pipelined ring has separate paths for the last 1 .. 5 steps),
    whole and half last steps, with ragged rows (257) and tokens (130)."""
    cout, T = 257, 130
    W = lcp_synth.random_matrix(40 + cin, (cout, cin), std=0.02, dtype="bf16")
    Wt = lcp_synth.random_matrix(41 + cin, (cout, cin), std=0.02, dtype="bf16")
    X = lcp_synth.random_matrix(42 + cin, (T, cin), std=1.0, dtype="bf16")
    say("error gemm k tails", cin)
    ws = torch.empty(L.lcp_error_workspace_bytes(cout, cin, T, L.LCP_BF16), dtype=torch.uint8, device=DEV)
    err = torch.empty(1, dtype=torch.float32, device=DEV)
    pitch = L.lcp_xt_pitch(T)
    R = torch.full((cout, pitch), 3.0, dtype=torch.bfloat16, device=DEV)
    L.lcp_error(up(W, torch.bfloat16), up(Wt, torch.bfloat16), up(X, torch.bfloat16), err, ws, R_out=R)
    torch.cuda.synchronize()
    Rref, Eref = oracle.pruning_error(W.astype(np.float64) - Wt, X)
    Rg = down(R)
    assert abs(float(err.item()) - Eref) / Eref < 1e-2
    assert rel_fro(Rg[:, :T], Rref) < 1e-2
    assert np.all(Rg[:, T:] == 0)


# --------------------------------------------------------------- full step --
def _run_step(lay, spec, backward=True, dtype=None):
    dtype = dtype or spec.dtype
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    W, X = up(lay.W, tdt), up(lay.X, tdt)
    lg = up(lay.logits)
    s = lcp.LayerSession(W, X, spec.B, spec.iters, spec.tau, spec.N, spec.M)
    P = torch.empty_like(lg)
    bits = empty_bits(lay.cout, lay.cin)
    err = s.forward(lg, P_out=P, bits_out=bits)
    dl = s.backward(lg) if backward else None
    torch.cuda.synchronize()
    return float(err.item()), down(P), bits_down(bits), (down(dl) if dl is not None else None)


def _check_step(lay, spec, got, backward=True, e_tol=1e-2):
    E, P, bits, dl = got
    fw = oracle.step_forward(lay.W, lay.X, lay.logits, spec.tau, spec.iters, spec.N, spec.M)
    assert np.all(np.abs(P - fw["P"]) <= _sink_tol(fw["P"]))
    agree = bit_agreement(bits, oracle.pack_bits(fw["mask"]), lay.cout * lay.cin)
    assert agree >= 0.999, agree
    assert abs(E - fw["E"]) / fw["E"] < e_tol, (E, fw["E"])
    if backward:
        # the oracle's backward on the GPU's mask (held constant), whole
        # tensor and every block
        _, bw = oracle_backward_on_mask(lay, spec, lay.logits, bits)
        check_gradient(dl, bw["dlogits"])
    return fw


SMALL = [
    # (config index, cout, cin, T): shapes with several tiles and ragged tails
    (1, 300, 512, 200),
    (2, 520, 640, 130),
    (3, 270, 512, 160),
    (4, 257, 384, 96),
    (2, 64, 64, 64),
]


MASK_CASES = [
    # (config index, cout, cin, T, N, M): every N:M selection path of the
    # fused permute (M = 4 with N compiled in, M = 8 at run time, the fp32
    # kernel) at B = 32, 64 and 128, ragged row counts
    (0, 70, 256, 64, 2, 4),
    (2, 300, 512, 130, 2, 4),
    (2, 257, 384, 96, 1, 4),
    (2, 257, 384, 96, 3, 4),
    (2, 257, 384, 96, 4, 8),
    (3, 270, 512, 160, 4, 8),
    (3, 100, 256, 64, 2, 4),
]


@pytest.mark.parametrize("ci,cout,cin,T,N,M", MASK_CASES)
def test_step_mask_is_nm_rule_of_its_scores(ci, cout, cin, T, N, M):
    """The fused permute's keep decision, bit for bit: the step's mask is the
    oracle's N:M rule (PermLLM blog 2.1, ties to the lower position) applied
    to the importance scores S_hat = (|W| n) P that the same MFMA (or fp32
    FMA) sequence produces, taken from the importance-only permute on the
    step's own P and column norms. The step tests compare the mask with the
    oracle's float64 scores; this one isolates the selection itself."""
    spec = lcp_synth.CONFIGS[ci]
    lay = lcp_synth.make_layer(spec, cout=cout, cin=cin, T=T)
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    W, X = up(lay.W, tdt), up(lay.X, tdt)
    lg = up(lay.logits)
    say("step mask vs its scores", spec.name, cout, cin, T, N, M)
    s = lcp.LayerSession(W, X, spec.B, spec.iters, spec.tau, N, M)
    P = torch.empty_like(lg)
    bits = empty_bits(cout, cin)
    s.forward(lg, P_out=P, bits_out=bits)
    S = torch.empty((cout, cin), dtype=torch.float32, device=DEV)
    L.lcp_permute(W, P, spec.B, S, colscale=s.norms)
    torch.cuda.synchronize()
    want = oracle.pack_bits(oracle.nm_mask(down(S), N, M))
    got = bits_down(bits)
    assert np.array_equal(got, want), bit_agreement(got, want, cout * cin)


@pytest.mark.parametrize("ci,cout,cin,T", SMALL)
def test_step_small(ci, cout, cin, T):
    spec = lcp_synth.CONFIGS[ci]
    lay = lcp_synth.make_layer(spec, cout=cout, cin=cin, T=T)
    say("step", spec.name, cout, cin, T)
    got = _run_step(lay, spec)
    _check_step(lay, spec, got)


FUSED = [
    # (cout, cin, T) of the 4096 x 11008 layer's kind (bf16, B = 64): the dD
    # GEMM takes the block adjoint in its epilogue, 256 x 256 tiles of four
    # blocks. Exactly one tile; rows one short of a panel with a last column
    # tile holding one valid block (of four); three valid blocks in the last
    # tile; a last panel of one row with wave-half blocks past Cin; a single
    # K step (T = 1); four panels by four column tiles.
    (256, 256, 64),
    (255, 320, 96),
    (511, 448, 130),
    (769, 192, 70),
    (300, 256, 1),
    (1024, 1024, 128),
]


@pytest.mark.parametrize("cout,cin,T", FUSED)
def test_step_fused_adjoint_tiling(cout, cin, T):
    """Tilings of the dD GEMM with the fused block adjoint: ragged row
    panels, column tiles with fewer than four valid blocks, one K step."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=cout, cin=cin, T=T)
    say("step fused adjoint tiling", cout, cin, T)
    got = _run_step(lay, spec)
    _check_step(lay, spec, got)


TINY = [
    # (config index, cout, cin, T): one output row, one token, one block,
    # sizes one past a tile boundary
    (2, 1, 64, 1),
    (2, 3, 128, 7),
    (2, 33, 64, 65),
    (0, 1, 32, 1),
    (0, 5, 64, 3),
    (3, 2, 128, 2),
]


@pytest.mark.parametrize("ci,cout,cin,T", TINY)
def test_step_tiny_shapes(ci, cout, cin, T):
    """Degenerate sizes: the guards and clamps of every kernel of the step."""
    spec = lcp_synth.CONFIGS[ci]
    lay = lcp_synth.make_layer(spec, cout=cout, cin=cin, T=T)
    say("step tiny", spec.name, cout, cin, T)
    got = _run_step(lay, spec)
    _check_step(lay, spec, got, e_tol=1e-2 if spec.dtype == "bf16" else 1e-4)


def test_step_c1_fp32_full_size():
    """The 256 x 256 float32 layer at its full size, forward and backward."""
    spec = lcp_synth.F32_256x256
    lay = lcp_synth.make_layer(spec)
    say("step C1 f32 full")
    got = _run_step(lay, spec, backward=True)
    _check_step(lay, spec, got, backward=True, e_tol=1e-4)


def test_step_random_logits_and_harder_tau():
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=200, cin=256, T=100)
    lay.logits[:] = lcp_synth.random_logits(77, 4, 64, scale=1.0)
    spec2 = lcp_synth.LayerSpec(**{**spec.__dict__, "tau": 0.5, "iters": 7})
    say("step random logits tau 0.5")
    got = _run_step(lay, spec2)
    _check_step(lay, spec2, got)


def test_step_zero_error_gives_zero_gradient():
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=64, cin=128, T=64)
    lay.X[:] = 0.0
    say("step zero X")
    E, P, bits, dl = _run_step(lay, spec)
    assert E == 0.0
    assert np.all(dl == 0.0)


def test_step_peaked_logits_is_hard_pruning():
    """Sharply peaked logits make P a hard permutation: D = W with the pruned
    entries only, so E equals the error of plain N:M pruning of the gathered
    channels (oracle with the hard P)."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=128, cin=128, T=64)
    rng = np.random.Generator(np.random.PCG64(9))
    Pi = np.zeros((2, 64, 64))
    for b in range(2):
        Pi[b, rng.permutation(64), np.arange(64)] = 1.0
    lay.logits[:] = (60.0 * Pi).astype(np.float32)
    say("step peaked logits")
    E, P, bits, dl = _run_step(lay, spec, backward=False)
    fw = oracle.step_forward(lay.W, lay.X, None, 1.0, 1, 2, 4, P=Pi)
    assert abs(E - fw["E"]) / fw["E"] < 1e-2
    assert bit_agreement(bits, oracle.pack_bits(fw["mask"]), 128 * 128) == 1.0


def test_step_deterministic():
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=384, cin=256, T=128)
    say("step determinism")
    a = _run_step(lay, spec)
    b = _run_step(lay, spec)
    assert a[0] == b[0]
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])


def test_step_full_size_bench_layer():
    """The 4096 x 11008 layer at full size, in the launch configuration the
    benchmark times: P, every mask bit, E and the gradient against the full
    float64 oracle."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec)
    say("step full size", spec.name)
    got = _run_step(lay, spec)
    _check_step(lay, spec, got)


@pytest.mark.parametrize("ci", [1, 3, 4])
def test_step_full_size_other_layers(ci):
    """The other seeded layers at their full sizes, through the same session
    path the benchmark uses: 4096 x 4096 (forward only), 13824 x 5120 (B = 128,
    4:8) and 28672 x 8192, each against the full float64 oracle."""
    spec = lcp_synth.CONFIGS[ci]
    lay = lcp_synth.make_layer(spec)
    say("step full size", spec.name)
    got = _run_step(lay, spec, backward=spec.backward)
    _check_step(lay, spec, got, backward=spec.backward)


# -------------------------------------------------------------- hardening --
def _assignment_value(P, perm):
    nb, B, _ = P.shape
    return np.array([P[b, perm[b], np.arange(B)].sum() for b in range(nb)])


@pytest.mark.parametrize("B", [32, 64, 128])
@pytest.mark.parametrize("kind", ["sinkhorn", "planted", "ties"])
def test_harden_assignment(B, kind):
    """lcp_harden against the oracle's assignment of the same fp32 P_hat:
    identical permutations where the optimum is unique, and an optimal,
    valid permutation when every assignment ties."""
    nb = 9
    if kind == "sinkhorn":
        P = oracle.sinkhorn(lcp_synth.random_logits(300 + B, nb, B).astype(np.float64), 1.0, 5).astype(np.float32)
    elif kind == "planted":
        lg, _ = lcp_synth.planted_logits(400 + B, nb, B)
        P = oracle.sinkhorn(lg.astype(np.float64), 1.0, 5).astype(np.float32)
    else:
        P = np.full((nb, B, B), 1.0 / B, dtype=np.float32)
    say("harden", B, kind)
    d_P = up(P)
    d_hard = torch.full((nb, B, B), 5.0, dtype=torch.float32, device=DEV)
    d_perm = torch.full((nb, B), -7, dtype=torch.int32, device=DEV)
    L.lcp_harden(d_P, d_hard, d_perm)
    torch.cuda.synchronize()
    perm = d_perm.cpu().numpy()
    hard = down(d_hard)
    for b in range(nb):
        assert sorted(perm[b].tolist()) == list(range(B))
    want_hard = np.zeros((nb, B, B), dtype=np.float32)
    for b in range(nb):
        want_hard[b, perm[b], np.arange(B)] = 1.0
    assert np.array_equal(hard, want_hard)
    ref = oracle.harden(P.astype(np.float64))
    ref_perm = np.argmax(ref, axis=1)                  # row assigned to each column
    P64 = P.astype(np.float64)
    if kind == "ties":
        assert np.allclose(_assignment_value(P64, perm), _assignment_value(P64, ref_perm), rtol=0, atol=1e-12)
    else:
        assert np.array_equal(perm, ref_perm)


SMALL_HARD = [
    # (config index, cout, cin, T)
    (0, 256, 256, 256),
    (1, 300, 512, 200),
    (2, 270, 640, 130),
    (3, 257, 512, 96),
]


@pytest.mark.parametrize("ci,cout,cin,T", SMALL_HARD)
def test_step_hardened(ci, cout, cin, T):
    """Hardened forward (Method 2) and straight-through backward against the
    oracle: the hard P exactly, the mask, E and the gradient."""
    spec = lcp_synth.CONFIGS[ci]
    say("step hardened", spec.name, cout, cin, T)
    _check_hardened(spec, cout, cin, T, 500 + ci)


def _check_hardened(spec, cout, cin, T, seed):
    lay = lcp_synth.make_layer(spec, cout=cout, cin=cin, T=T)
    lg, Pi = lcp_synth.planted_logits(seed, cin // spec.B, spec.B, peak=1.5, noise_std=0.3)
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    s = lcp.LayerSession(up(lay.W, tdt), up(lay.X, tdt), spec.B, spec.iters, spec.tau, spec.N, spec.M,
                         harden=True)
    d_lg = up(lg)
    P = torch.empty_like(d_lg)
    bits = empty_bits(lay.cout, lay.cin)
    err = s.forward(d_lg, P_out=P, bits_out=bits)
    dl = s.backward(d_lg)
    torch.cuda.synchronize()
    fw = oracle.step_forward(lay.W, lay.X, lg, spec.tau, spec.iters, spec.N, spec.M, hard=True)
    assert np.array_equal(down(P), fw["P"])
    assert np.max(np.abs(fw["P_soft"] - fw["P"])) > 0.05          # the soft P_hat is not hard
    agree = bit_agreement(bits_down(bits), oracle.pack_bits(fw["mask"]), lay.cout * lay.cin)
    assert agree >= 0.999, agree
    assert abs(float(err.item()) - fw["E"]) / fw["E"] < 1e-2
    _, bw = oracle_backward_on_mask(lay, spec, lg, bits_down(bits), hard=True)
    check_gradient(down(dl), bw["dlogits"])


@pytest.mark.parametrize("cout,cin,T", [(300, 256, 130), (33, 96, 65)])
def test_step_bf16_block32(cout, cin, T):
    """bf16 layers with B = 32 (the bench layer's distributions, 2:4): the
    B = 32 Sinkhorn, permute and separate adjoint of a bf16 step, soft and
    hardened, against the oracle with the same tolerances as every step."""
    spec = dataclasses.replace(lcp_synth.CONFIGS[2], B=32)
    lay = lcp_synth.make_layer(spec, cout=cout, cin=cin, T=T)
    say("step bf16 B = 32", cout, cin, T)
    got = _run_step(lay, spec)
    _check_step(lay, spec, got)
    _check_hardened(spec, cout, cin, T, 700 + cout)


def test_step_hardened_full_size_bench_layer():
    """The hardened step (Method 2 forward, straight-through backward) on the
    full 4096 x 11008 layer against the full float64 oracle: the hard P
    exactly, the mask, E and the gradient."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec)
    lg, _ = lcp_synth.planted_logits(550, lay.cin // spec.B, spec.B, peak=1.5, noise_std=0.3)
    say("step hardened full size", spec.name)
    s = lcp.LayerSession(up(lay.W, torch.bfloat16), up(lay.X, torch.bfloat16), spec.B, spec.iters, spec.tau,
                         spec.N, spec.M, harden=True)
    d_lg = up(lg)
    P = torch.empty_like(d_lg)
    bits = empty_bits(lay.cout, lay.cin)
    err = s.forward(d_lg, P_out=P, bits_out=bits)
    dl = s.backward(d_lg)
    torch.cuda.synchronize()
    fw = oracle.step_forward(lay.W, lay.X, lg, spec.tau, spec.iters, spec.N, spec.M, hard=True)
    assert np.array_equal(down(P), fw["P"])
    agree = bit_agreement(bits_down(bits), oracle.pack_bits(fw["mask"]), lay.cout * lay.cin)
    assert agree >= 0.999, agree
    assert abs(float(err.item()) - fw["E"]) / fw["E"] < 1e-2
    _, bw = oracle_backward_on_mask(lay, spec, lg, bits_down(bits), hard=True)
    check_gradient(down(dl), bw["dlogits"])


# ------------------------------------------------------------ optimiser --
def test_adamw_kernel():
    """lcp_adamw against the oracle's AdamW (float64) after three steps."""
    rng = np.random.Generator(np.random.PCG64(31))
    n = 70001
    p0 = rng.standard_normal(n).astype(np.float32)
    grads = [rng.standard_normal(n).astype(np.float32) for _ in range(3)]
    say("adamw")
    d_p, d_m, d_v = up(p0), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    acfg = lcp.make_adamw_cfg(5e-3, weight_decay=0.1)
    # the oracle gets the hyper-parameters as the kernel receives them (fp32)
    f = lambda x: float(np.float32(x))  # noqa: E731
    hp = dict(beta1=f(0.9), beta2=f(0.999), eps=f(1e-8), weight_decay=f(0.1))
    p, m, v = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads):
        L.lcp_adamw(d_p, up(g), d_m, d_v, t + 1, acfg)
        p, m, v = oracle.adamw(p, g, m, v, t + 1, f(5e-3), **hp)
    torch.cuda.synchronize()
    assert np.max(np.abs(down(d_p) - p) / (np.abs(p) + 1e-3)) < 1e-5
    assert np.max(np.abs(down(d_v) - v) / (np.abs(v) + 1e-12)) < 1e-5


@pytest.mark.parametrize("harden", [False, True])
def test_step_bwd_adamw_fused(harden):
    """The AdamW update fused into the Sinkhorn adjoint equals the plain
    backward followed by the standalone AdamW kernel, bit for bit."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=300, cin=512, T=160)
    say("step bwd adamw", harden)
    s = lcp.LayerSession(up(lay.W, torch.bfloat16), up(lay.X, torch.bfloat16), spec.B, spec.iters, spec.tau,
                         spec.N, spec.M, harden=harden)
    lg0 = up(lay.logits)
    rng = np.random.Generator(np.random.PCG64(32))
    m0 = up(rng.standard_normal(lay.logits.shape).astype(np.float32) * 1e-3)
    v0 = up(np.abs(rng.standard_normal(lay.logits.shape)).astype(np.float32) * 1e-6)
    acfg = lcp.make_adamw_cfg(1e-3)
    # separate: backward, then the standalone kernel
    lg_a, m_a, v_a = lg0.clone(), m0.clone(), v0.clone()
    s.forward(lg_a)
    g = s.backward(lg_a)
    L.lcp_adamw(lg_a, g, m_a, v_a, 4, acfg)
    # fused
    lg_b, m_b, v_b = lg0.clone(), m0.clone(), v0.clone()
    s.forward(lg_b)
    L.lcp_step_bwd_adamw(s.layer, lg_b, s.cfg, s.ws, m_b, v_b, 4, acfg)
    torch.cuda.synchronize()
    assert torch.equal(lg_a, lg_b) and torch.equal(m_a, m_b) and torch.equal(v_a, v_b)
    assert not torch.equal(lg_a, lg0)


def test_training_beats_wanda():
    """lcp_train (hardened forward, straight-through backward, AdamW,
    temperature 1 -> 0.1) on a seeded layer from a weak identity prior: the
    first step is plain Wanda (identity permutation), the loop reaches hard
    permutations with lower output error, and the GPU's error of the final
    logits agrees with the oracle's."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=256, cin=512, T=256)
    nb = lay.cin // spec.B
    lg0 = lcp_synth.make_logits(np.random.Generator(np.random.PCG64(7)), nb, spec.B, diag=0.5)
    say("train")
    s = lcp.LayerSession(up(lay.W, torch.bfloat16), up(lay.X, torch.bfloat16), spec.B, spec.iters, spec.tau,
                         spec.N, spec.M, harden=True)
    lg = up(lg0)
    errs = down(s.train(lg, 40, 1e-2))
    s.cfg.tau = 0.1
    e_final = float(s.forward(lg).item())
    torch.cuda.synchronize()
    eye = np.eye(spec.B)[None].repeat(nb, axis=0)
    wanda = oracle.step_forward(lay.W, lay.X, None, 1.0, spec.iters, spec.N, spec.M, P=eye)["E"]
    final = oracle.step_forward(lay.W, lay.X, down(lg), 0.1, spec.iters, spec.N, spec.M, hard=True)["E"]
    assert abs(errs[0] - wanda) / wanda < 1e-2
    assert np.min(errs) < 0.99 * wanda, (np.min(errs), wanda)
    assert abs(e_final - final) / final < 1e-2, (e_final, final)
    # No final-vs-Wanda assertion on this 8-block slice: the last iterate of
    # the hardened straight-through loop is noisy here. The oracle's own loop
    # with gradient noise at the GPU's rounding level (3e-3 relative) ends at
    # 0.97 .. 1.02 of Wanda's error over six seeds, while min(errs) stays near
    # 0.95 (gradient ascent reaches only 0.996, which the check above
    # rejects). test_training_beats_wanda_full_size pins the final hard
    # permutation on the whole layers.


@pytest.mark.parametrize("ci", [1, 2])
def test_training_beats_wanda_full_size(ci):
    """The optimiser-loop pin at full size: lcp_train on the whole 4096 x 4096
    and 4096 x 11008 layers with the pages' schedule (AdamW, learning rate
    5e-3, temperature linear from 1 to 0.1, hardened forward with the
    straight-through backward; PermLLM summary, implementation details),
    100 steps from a weak identity prior (0.5 I per block, so the first
    hardened step is plain Wanda). The oracle's error of the final hard
    permutation is below Wanda's, and the GPU's error of the final logits
    agrees with the oracle's."""
    spec = lcp_synth.CONFIGS[ci]
    lay = lcp_synth.make_layer(spec)
    nb = lay.cin // spec.B
    lg0 = lcp_synth.make_logits(np.random.Generator(np.random.PCG64(70 + ci)), nb, spec.B, diag=0.5)
    say("train full size", spec.name)
    s = lcp.LayerSession(up(lay.W, torch.bfloat16), up(lay.X, torch.bfloat16), spec.B, spec.iters, 1.0,
                         spec.N, spec.M, harden=True)
    lg = up(lg0)
    errs = down(s.train(lg, 100, 5e-3))
    s.cfg.tau = 0.1
    e_final = float(s.forward(lg).item())
    torch.cuda.synchronize()
    eye = np.eye(spec.B)[None].repeat(nb, axis=0)
    wanda = oracle.step_forward(lay.W, lay.X, None, 1.0, spec.iters, spec.N, spec.M, P=eye)["E"]
    final = oracle.step_forward(lay.W, lay.X, down(lg), 0.1, spec.iters, spec.N, spec.M, hard=True)["E"]
    say("train full size %s: wanda %.6f first %.6f min %.6f last %.6f final oracle %.6f gpu %.6f"
        % (spec.name, wanda, errs[0], np.min(errs), errs[-1], final, e_final))
    assert abs(errs[0] - wanda) / wanda < 1e-2, (errs[0], wanda)
    assert abs(e_final - final) / final < 1e-2, (e_final, final)
    assert final < wanda, (final, wanda)
    assert e_final < wanda, (e_final, wanda)
