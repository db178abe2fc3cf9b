"""GPU parity of the deploy path ([PermLLM] inference acceleration): the
channel gather, the 2:4 weight packing and the sparse-matrix-core GEMM,
against the float64 oracle, through the C ABI. Bars: gather and packing
bit-exact (they move bf16 values); layer outputs within 1e-2 relative in
the Frobenius norm and elementwise within the bf16 output rounding plus the
fp32 accumulation bound."""
import numpy as np
import pytest
import torch

import lcp_synth
import oracle
from tests.gpu_util import DEV, bits_down, down, say, up

pytestmark = pytest.mark.gpu

lcp = pytest.importorskip("learnable_channel_permutation_amd")
L = lcp._lib


def _remap_row(rho):
    return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3)


def decode_packed(vals, meta, cout, cin):
    """Host decoder of the packed fragment format documented in lcp.h:
    returns the dense permuted sparse weight and the positions per group."""
    RG, KF, KT = cout // 32, cin // 32, (cin + 63) // 64
    v = vals.view(np.uint16).reshape(RG, KF, 64, 8)
    m = meta.view(np.uint32).reshape(RG, KT, 64)
    vf = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Ws = np.zeros((cout, cin))
    pos = np.zeros((cout, cin // 4, 2), dtype=np.int64)
    lanes = np.arange(64)
    rows_of_lane = np.array([_remap_row(x % 32) for x in lanes])
    for kf in range(KF):
        m16 = (m[:, kf // 2, :] >> (16 * (kf % 2))) & 0xFFFF            # [RG, 64]
        for g in range(4):
            p0 = (m16 >> (4 * g)) & 3
            p1 = (m16 >> (4 * g + 2)) & 3
            for rg in range(RG):
                o = 32 * rg + rows_of_lane
                k = 32 * kf + 16 * (lanes // 32) + 4 * g
                Ws[o, k + p0[rg]] += vf[rg, kf, :, 2 * g]
                Ws[o, k + p1[rg]] += vf[rg, kf, :, 2 * g + 1]
                grp = k // 4
                pos[o, grp, 0] = p0[rg]
                pos[o, grp, 1] = p1[rg]
    return Ws, pos


def _case(seed, cout, cin, T, B):
    rng = np.random.Generator(np.random.PCG64(seed))
    W = lcp_synth.random_matrix(seed + 1, (cout, cin), std=0.02, dtype="bf16")
    X = lcp_synth.random_matrix(seed + 2, (T, cin), std=1.0, dtype="bf16")
    nb = cin // B
    perm = np.stack([rng.permutation(B) for _ in range(nb)]).astype(np.int32)
    P = np.zeros((nb, B, B))
    for b in range(nb):
        P[b, perm[b], np.arange(B)] = 1.0
    fw = oracle.step_forward(W, X, None, 1.0, 1, 2, 4, P=P)
    return W, X, P, perm, fw["mask"]


SHAPES = [
    # (cout, cin, T, B): ragged token tail, a partial 256-row tile, an odd
    # number of 32-position fragments (cin % 64 == 32), B = 32 / 64 / 128
    (256, 512, 200, 64),
    (288, 352, 77, 32),
    (512, 1024, 256, 128),
    (64, 64, 1, 64),
]


@pytest.mark.parametrize("cout,cin,T,B", SHAPES)
def test_gather_channels(cout, cin, T, B):
    W, X, P, perm, mask = _case(50 + cin, cout, cin, T, B)
    say("gather", cin, T, B)
    d_X = up(X, torch.bfloat16)
    d_Xp = torch.full_like(d_X, 7.0)
    L.lcp_gather_channels(d_X, B, torch.from_numpy(perm).to(DEV), d_Xp)
    torch.cuda.synchronize()
    assert np.array_equal(down(d_Xp), oracle.gather_channels(X, P))


@pytest.mark.parametrize("cout,cin,T,B", SHAPES)
def test_sparse_pack(cout, cin, T, B):
    W, X, P, perm, mask = _case(60 + cin, cout, cin, T, B)
    say("sparse pack", cout, cin, B)
    vb, mb = L.lcp_sparse_pack_bytes(cout, cin)
    vals = torch.empty(vb, dtype=torch.uint8, device=DEV)
    meta = torch.empty(mb, dtype=torch.uint8, device=DEV)
    bits = torch.from_numpy(oracle.pack_bits(mask).view(np.int32)).to(DEV)
    d_perm = torch.from_numpy(perm).to(DEV)
    L.lcp_sparse_pack(up(W, torch.bfloat16), B, d_perm, bits, vals, meta)
    torch.cuda.synchronize()
    Ws, pos = decode_packed(vals.cpu().numpy(), meta.cpu().numpy(), cout, cin)
    want = oracle.block_permute(W, P) * mask
    assert np.array_equal(Ws, want)
    _, opos = oracle.sparse_pack(want, 2, 4)
    # every kept entry of these random bf16 weights is nonzero, so the
    # oracle's positions are the mask's
    assert np.array_equal(pos, opos)


def _deploy(W, X, perm, bits, B):
    cout, cin = W.shape
    T = X.shape[0]
    vb, mb = L.lcp_sparse_pack_bytes(cout, cin)
    vals = torch.empty(vb, dtype=torch.uint8, device=DEV)
    meta = torch.empty(mb, dtype=torch.uint8, device=DEV)
    d_perm = torch.from_numpy(np.ascontiguousarray(perm, dtype=np.int32)).to(DEV)
    L.lcp_sparse_pack(up(W, torch.bfloat16), B, d_perm, bits, vals, meta)
    d_X = up(X, torch.bfloat16)
    Xp = torch.empty_like(d_X)
    Y = torch.full((T, cout), 3.0, dtype=torch.bfloat16, device=DEV)
    L.lcp_deploy_forward(vals, meta, d_perm, B, d_X, cout, Xp, Y)
    torch.cuda.synchronize()
    return down(Y)


def _check_y(Yg, ref, absW, absX):
    assert np.all(np.isfinite(Yg))
    assert np.linalg.norm(Yg - ref) / np.linalg.norm(ref) < 1e-2
    # elementwise: bf16 output rounding (2^-8 relative) + fp32 accumulation
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * (absX @ absW.T) + 1e-30
    assert np.all(np.abs(Yg - ref) <= bound), float(np.max(np.abs(Yg - ref) / bound))


@pytest.mark.parametrize("cout,cin,T,B", SHAPES)
def test_deploy_forward(cout, cin, T, B):
    """Gather + 2:4 sparse GEMM against the oracle's dense X W_tilde^T."""
    W, X, P, perm, mask = _case(70 + cin, cout, cin, T, B)
    say("deploy forward", cout, cin, T, B)
    bits = torch.from_numpy(oracle.pack_bits(mask).view(np.int32)).to(DEV)
    Yg = _deploy(W, X, perm, bits, B)
    ref = oracle.deploy_forward(W, X, P, mask)
    _check_y(Yg, ref, np.abs(W), np.abs(X))


def test_deploy_after_hardened_step():
    """End to end on a seeded layer: the hardened step's P and mask (through
    lcp_step_fwd and lcp_harden) are packed and deployed; the output equals
    the oracle's X W_tilde^T for the oracle's own hard P and mask."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    lay = lcp_synth.make_layer(spec, cout=512, cin=1024, T=320)
    lg, _ = lcp_synth.planted_logits(800, lay.cin // spec.B, spec.B, peak=1.5, noise_std=0.3)
    say("deploy after hardened step")
    s = lcp.LayerSession(up(lay.W, torch.bfloat16), up(lay.X, torch.bfloat16), spec.B, spec.iters, spec.tau,
                         spec.N, spec.M, harden=True)
    d_lg = up(lg)
    P = torch.empty_like(d_lg)
    bits = torch.empty((lay.cout, lay.cin // 32), dtype=torch.int32, device=DEV)
    s.forward(d_lg, P_out=P, bits_out=bits)
    perm = torch.empty((lay.cin // spec.B, spec.B), dtype=torch.int32, device=DEV)
    L.lcp_harden(P, None, perm)                       # the permutation of the hard P itself
    torch.cuda.synchronize()
    Yg = _deploy(lay.W, lay.X, perm.cpu().numpy(), bits, spec.B)
    fw = oracle.step_forward(lay.W, lay.X, lg, spec.tau, spec.iters, spec.N, spec.M, hard=True)
    assert np.array_equal(down(P), fw["P"])
    ref = oracle.deploy_forward(lay.W, lay.X, fw["P"], fw["mask"])
    # the GPU mask may differ from the oracle's in a few near-tied groups
    # (>= 99.9 % agreement is the step's bar): output channels whose mask
    # rows agree are checked elementwise, all of them in norm
    same = np.all(oracle.unpack_bits(bits_down(bits), lay.cin) == fw["mask"], axis=1)
    assert same.mean() >= 0.9, same.mean()
    assert np.linalg.norm(Yg - ref) / np.linalg.norm(ref) < 1e-2
    _check_y(Yg[:, same], ref[:, same], np.abs(lay.W[same]), np.abs(lay.X))


def test_deploy_full_size_bench_layer():
    """The 4096 x 11008 layer with 2048 tokens, the benchmark's deploy
    configuration, against the full float64 oracle."""
    spec = lcp_synth.DOWN_PROJ_4096x11008
    cout, cin, T, B = spec.cout, spec.cin, spec.T, spec.B
    W, X, P, perm, mask = _case(90, cout, cin, T, B)
    say("deploy full size", cout, cin, T)
    bits = torch.from_numpy(oracle.pack_bits(mask).view(np.int32)).to(DEV)
    Yg = _deploy(W, X, perm, bits, B)
    ref = oracle.deploy_forward(W, X, P, mask)
    _check_y(Yg, ref, np.abs(W), np.abs(X))


@pytest.mark.parametrize("cin", [32, 96, 224, 416, 480, 736, 992])
def test_deploy_forward_k_tails(cin):
    """Every count of 64-position steps modulo the ring depth, short K
    (fewer steps than the ring holds) and odd fragment counts (cin % 64 ==
    32), with a ragged token tail and a partial row tile."""
    cout, T, B = 288, 130, 32
    W, X, P, perm, mask = _case(90 + cin, cout, cin, T, B)
    say("deploy forward k tails", cout, cin, T, B)
    bits = torch.from_numpy(oracle.pack_bits(mask).view(np.int32)).to(DEV)
    Yg = _deploy(W, X, perm, bits, B)
    ref = oracle.deploy_forward(W, X, P, mask)
    _check_y(Yg, ref, np.abs(W), np.abs(X))
