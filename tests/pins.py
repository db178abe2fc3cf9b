"""Pins for the float64 oracle: checks against facts that do not come from the
oracle itself (hand-worked examples, closed forms, textbook routines, brute
force, finite differences).

Every pin is a function of the oracle module, so the mutation tests can run the
same pins against an oracle with a planted mistake and confirm they fail.
"""
from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------- Sinkhorn --
def pin_sinkhorn_2x2_golden(o):
    """Hand-worked rationals (golden/sinkhorn_2x2_ln3.txt), for two tau."""
    rows = []
    with open(os.path.join(GOLDEN, "sinkhorn_2x2_ln3.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(t) for t in line.split()])
    for tau in (1.0, 0.5, 3.0):
        logits = np.array([[[math.log(3.0) * tau, 0.0], [0.0, 0.0]]])
        for r in rows:
            L = r[0]
            want = np.array([float(Fraction(r[1 + 2 * i], r[2 + 2 * i])) for i in range(4)])
            got = o.sinkhorn(logits, tau, L)[0].reshape(-1)
            assert np.allclose(got, want, rtol=0, atol=1e-14), (tau, L, got, want)


def pin_sinkhorn_uniform(o):
    """Uniform logits give exactly 1/B for every L >= 1 and tau."""
    for B in (4, 32, 64):
        for tau in (0.1, 1.0, 2.5):
            for L in (1, 5):
                P = o.sinkhorn(np.full((2, B, B), 0.7), tau, L)
                assert np.allclose(P, 1.0 / B, rtol=1e-13, atol=0), (B, tau, L)


def pin_sinkhorn_closed_form(o):
    """a*I (or a*Pi) logits: diagonal e^{a/tau}/(e^{a/tau}+B-1), off-diagonal
    1/(e^{a/tau}+B-1) for every L >= 1 (the matrix is already balanced after
    one row step, since every row and column holds the same multiset)."""
    rng = _rng(1)
    for B in (8, 32, 64, 128):
        for a, tau in ((3.0, 1.0), (3.0, 0.5), (1.0, 0.3)):
            e = math.exp(a / tau)
            diag = e / (e + B - 1)
            off = 1.0 / (e + B - 1)
            pi = rng.permutation(B)
            Pi = np.zeros((B, B))
            Pi[np.arange(B), pi] = 1.0
            for L in (1, 4):
                P = o.sinkhorn((a * Pi)[None], tau, L)[0]
                want = np.where(Pi > 0, diag, off)
                assert np.allclose(P, want, rtol=1e-12, atol=0), (B, a, tau, L)


def pin_sinkhorn_closed_form_values(o):
    """The three block sizes at a = 3, tau = 1, printed to 7 digits."""
    for B, d, f in ((32, 0.3931746, 0.0195750), (64, 0.2417453, 0.0120358),
                    (128, 0.1365568, 0.0067988)):
        P = o.sinkhorn((3.0 * np.eye(B))[None], 1.0, 5)[0]
        assert abs(P[0, 0] - d) < 6e-8 and abs(P[0, 1] - f) < 6e-8, (B, P[0, 0], P[0, 1])


def pin_sinkhorn_doubly_stochastic(o):
    """Columns sum to 1 after every iteration (the column step is last);
    rows approach 1 as L grows."""
    rng = _rng(2)
    lg = rng.standard_normal((3, 16, 16))
    for L in (1, 3, 5):
        P = o.sinkhorn(lg, 1.0, L)
        assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    P = o.sinkhorn(lg, 1.0, 300)
    assert np.allclose(P.sum(axis=2), 1.0, rtol=0, atol=1e-10)
    assert np.all(P > 0)


def pin_sinkhorn_knopp(o):
    """Agrees with the multiplicative Sinkhorn-Knopp iteration (a different
    formula: divide by row sums, then column sums, in the linear domain)."""
    rng = _rng(3)
    for tau in (1.0, 0.5):
        lg = rng.standard_normal((4, 12, 12))
        for L in range(1, 7):
            K = np.exp(lg / tau)
            for _ in range(L):
                K = K / K.sum(axis=2, keepdims=True)
                K = K / K.sum(axis=1, keepdims=True)
            P = o.sinkhorn(lg, tau, L)
            assert np.allclose(P, K, rtol=1e-12, atol=1e-15), (tau, L)


def pin_sinkhorn_equivariance(o):
    """Sinkhorn(Pi1 Lambda Pi2) = Pi1 Sinkhorn(Lambda) Pi2."""
    rng = _rng(4)
    B = 10
    lg = rng.standard_normal((1, B, B))
    P1 = np.eye(B)[rng.permutation(B)]
    P2 = np.eye(B)[rng.permutation(B)]
    a = o.sinkhorn((P1 @ lg[0] @ P2)[None], 0.7, 5)[0]
    b = P1 @ o.sinkhorn(lg, 0.7, 5)[0] @ P2
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)


def pin_sinkhorn_peaked(o):
    """s*Pi + small noise with s/tau >= 30 gives Pi within B e^{-s/tau}, and
    hardening recovers Pi."""
    rng = _rng(5)
    B = 16
    pi = rng.permutation(B)
    Pi = np.zeros((B, B))
    Pi[np.arange(B), pi] = 1.0
    for s, tau in ((3.0, 0.1), (40.0, 1.0)):
        lg = s * Pi + 1e-3 * rng.standard_normal((B, B))
        P = o.sinkhorn(lg[None], tau, 5)
        assert np.max(np.abs(P[0] - Pi)) <= B * math.exp(-s / tau) * 1.5
        assert np.array_equal(o.harden(P)[0], Pi)


def pin_sinkhorn_small_tau_assignment(o):
    """As tau -> 0 (with enough iterations) the Sinkhorn output hardens to the
    maximum-weight assignment of the logits (Gumbel-Sinkhorn, Mena et al.,
    ICLR 2018); the assignment is computed independently by SciPy."""
    from scipy.optimize import linear_sum_assignment
    rng = _rng(6)
    for trial in range(4):
        B = 7
        lg = rng.standard_normal((B, B))
        r, c = linear_sum_assignment(lg, maximize=True)
        want = np.zeros((B, B))
        want[r, c] = 1.0
        P = o.sinkhorn(lg[None], 0.02, 2000)
        assert np.array_equal(o.harden(P)[0], want), trial
        # entropic bound: <P, Lambda> >= max - tau * B log B at the limit
        opt = float(lg[r, c].sum())
        assert float(np.sum(P[0] * lg)) >= opt - 0.02 * B * math.log(B) - 1e-6, trial


def pin_sinkhorn_adjoint_fd(o):
    """Reverse pass of the Sinkhorn checked by central differences of the
    linear functional <C, P_hat(Lambda)>."""
    rng = _rng(7)
    nb, B, tau, L = 2, 5, 0.7, 4
    lg = rng.standard_normal((nb, B, B))
    C = rng.standard_normal((nb, B, B))
    P, tr = o.sinkhorn(lg, tau, L, trace=True)
    g = o.sinkhorn_adjoint(C, P, tr, tau)
    h = 1e-6
    fd = np.zeros_like(lg)
    for idx in np.ndindex(lg.shape):
        lp = lg.copy(); lp[idx] += h
        lm = lg.copy(); lm[idx] -= h
        fd[idx] = (np.sum(C * o.sinkhorn(lp, tau, L)) - np.sum(C * o.sinkhorn(lm, tau, L))) / (2 * h)
    err = np.linalg.norm(g - fd) / np.linalg.norm(fd)
    assert err < 1e-7, err


# ------------------------------------------------------- permute and mask --
def pin_block_permute_gather(o):
    """A hard P (P_b[j, k] = 1 iff j = pi_b(k)) reduces A P_B to the column
    gather out[:, bB+k] = A[:, bB+pi_b(k)], and A P_B^T to its inverse."""
    rng = _rng(8)
    rows, B, nb = 5, 8, 3
    A = rng.standard_normal((rows, nb * B))
    P = np.zeros((nb, B, B))
    src = np.zeros(nb * B, dtype=int)
    for b in range(nb):
        pi = rng.permutation(B)
        P[b, pi, np.arange(B)] = 1.0
        src[b * B:(b + 1) * B] = b * B + pi
    out = o.block_permute(A, P)
    assert np.array_equal(out, A[:, src])
    back = o.block_permute(out, P, transpose=True)
    assert np.array_equal(back, A)


def pin_block_permute_dense(o):
    """A P_B equals the product with the dense block-diagonal matrix."""
    rng = _rng(9)
    rows, B, nb = 4, 4, 3
    A = rng.standard_normal((rows, nb * B))
    P = rng.random((nb, B, B))
    dense = np.zeros((nb * B, nb * B))
    for b in range(nb):
        dense[b * B:(b + 1) * B, b * B:(b + 1) * B] = P[b]
    assert np.allclose(o.block_permute(A, P), A @ dense, rtol=1e-14, atol=1e-14)
    assert np.allclose(o.block_permute(A, P, transpose=True), A @ dense.T, rtol=1e-14, atol=1e-14)


def _read_mask_golden():
    out = []
    with open(os.path.join(GOLDEN, "nm_mask_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            nm, s, k = [t.strip() for t in line.split("|")]
            N, M = (int(t) for t in nm.split())
            scores = np.array([float(t) for t in s.split()], dtype=np.float32)
            keep = np.array([int(t) for t in k.split()], dtype=bool)
            out.append((N, M, scores, keep))
    return out


def pin_nm_mask_golden(o):
    for N, M, scores, keep in _read_mask_golden():
        got = o.nm_mask(scores[None, :], N, M)[0]
        assert np.array_equal(got, keep), (N, M, scores, got, keep)


def pin_nm_mask_bruteforce(o):
    """Brute force over all N-subsets of each group: the mask is the subset
    with the largest score sum; among equal sums, the lexicographically
    smallest positions (equal scores go to the lower position). Small integer
    scores make ties frequent."""
    rng = _rng(10)
    for N, M in ((1, 4), (2, 4), (3, 4), (2, 8), (4, 8), (6, 8)):
        S = rng.integers(0, 4, size=(40, 2 * M)).astype(np.float32)
        got = o.nm_mask(S, N, M)
        for i in range(S.shape[0]):
            for g in range(2):
                v = S[i, g * M:(g + 1) * M]
                best, best_sub = None, None
                for sub in itertools.combinations(range(M), N):
                    tot = sum(float(v[t]) for t in sub)
                    if best is None or tot > best:
                        best, best_sub = tot, sub
                want = np.zeros(M, dtype=bool)
                want[list(best_sub)] = True
                assert np.array_equal(got[i, g * M:(g + 1) * M], want), (N, M, v)


def pin_nm_mask_counts(o):
    """Every group keeps exactly N positions, NaN and infinities included."""
    rng = _rng(11)
    S = rng.standard_normal((30, 64)).astype(np.float32)
    S[rng.random(S.shape) < 0.05] = np.nan
    S[rng.random(S.shape) < 0.05] = np.inf
    S[rng.random(S.shape) < 0.05] = -np.inf
    for N, M in ((2, 4), (4, 8), (1, 8)):
        m = o.nm_mask(S, N, M)
        assert np.all(m.reshape(30, -1, M).sum(axis=2) == N)


def pin_pack_bits(o):
    rng = _rng(12)
    m = rng.random((3, 96)) < 0.5
    bits = o.pack_bits(m)
    for i in range(3):
        for k in range(96):
            assert bool((int(bits[i, k // 32]) >> (k % 32)) & 1) == bool(m[i, k])
    assert np.array_equal(o.unpack_bits(bits, 96), m)


def pin_identity_is_wanda(o):
    """With the identity permutation the method reduces to plain Wanda N:M
    pruning: keep the top-N of |W_ij| ||X_j|| in each group of M source
    channels (computed here by an explicit per-group loop)."""
    rng = _rng(13)
    cout, cin, T, B = 6, 32, 20, 8
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin)) * rng.lognormal(0, 1, cin)
    P = np.tile(np.eye(B), (cin // B, 1, 1))
    fw = o.step_forward(W, X, None, 1.0, 1, 2, 4, P=P)
    n = np.sqrt((X ** 2).sum(axis=0))
    keep = np.zeros((cout, cin), dtype=bool)
    for i in range(cout):
        for g in range(cin // 4):
            s = [abs(W[i, 4 * g + t]) * n[4 * g + t] for t in range(4)]
            top = sorted(range(4), key=lambda t: (-s[t], t))[:2]
            for t in top:
                keep[i, 4 * g + t] = True
    assert np.array_equal(fw["mask"], keep)
    D = np.where(keep, 0.0, W)
    assert np.allclose(fw["D"], D, rtol=0, atol=1e-15)
    # the same via sharply peaked logits through the Sinkhorn
    fw2 = o.step_forward(W, X, np.tile(60.0 * np.eye(B), (cin // B, 1, 1)), 1.0, 5, 2, 4)
    assert np.array_equal(fw2["mask"], keep)
    assert abs(fw2["E"] - fw["E"]) <= 1e-9 * fw["E"]


# ------------------------------------------------------------------ error --
def _pruned_error_direct(W, X, S, perm, N, M):
    """Error of a hard permutation by explicit loops: permuted position k holds
    source channel perm[k]; in each group of M positions the N highest
    importances survive (equal -> lower position); the rest are zeroed."""
    cout, cin = W.shape
    D = np.zeros_like(W)
    for i in range(cout):
        for g in range(cin // M):
            pos = list(range(g * M, (g + 1) * M))
            order = sorted(pos, key=lambda k: (-np.float32(S[i, perm[k]]), k))
            for k in order[N:]:
                D[i, perm[k]] = W[i, perm[k]]
    R = D @ X.T
    return math.sqrt(float(np.sum(R * R)))


def pin_hard_perm_error(o):
    """Hard P: E = ||(W . not M_orig) X^T||_F, computed by explicit loops."""
    rng = _rng(14)
    cout, cin, T, B = 5, 24, 9, 8
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin))
    P = np.zeros((cin // B, B, B))
    perm = np.zeros(cin, dtype=int)
    for b in range(cin // B):
        pi = rng.permutation(B)
        P[b, pi, np.arange(B)] = 1.0
        perm[b * B:(b + 1) * B] = b * B + pi
    fw = o.step_forward(W, X, None, 1.0, 1, 2, 4, P=P)
    S = np.abs(W) * np.sqrt((X ** 2).sum(axis=0))
    want = _pruned_error_direct(W, X, S, perm, 2, 4)
    assert abs(fw["E"] - want) <= 1e-12 * want, (fw["E"], want)


def pin_gram_identity(o):
    """E^2 = tr(D (X^T X) D^T) for soft permutations too."""
    rng = _rng(15)
    cout, cin, T, B = 7, 32, 11, 16
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin))
    lg = rng.standard_normal((cin // B, B, B))
    fw = o.step_forward(W, X, lg, 0.8, 5, 2, 4)
    H = X.T @ X
    D = fw["D"]
    e2 = sum(float(D[i] @ H @ D[i]) for i in range(cout))
    assert abs(fw["E"] ** 2 - e2) <= 1e-10 * e2
    # W_tilde returns to the source order: for the same soft P, W_tilde P_B
    # equals (W_hat . M) P_B^T P_B
    dense = np.zeros((cin, cin))
    for b in range(cin // B):
        dense[b * B:(b + 1) * B, b * B:(b + 1) * B] = fw["P"][b]
    A = (W @ dense) * fw["mask"]
    assert np.allclose(fw["W_tilde"], A @ dense.T, rtol=1e-12, atol=1e-14)


def enumerate_cin8(o, seed, T=12, classes_only=False):
    """All 8! hard permutations of one 8-channel block, 2:4 (or, with
    classes_only, one permutation per partition of the 8 channels into two
    groups of 4, which fixes both the error and the retained importance).
    Returns the step's E per permutation, the explicit-loop E, and the
    retained importance per permutation."""
    rng = _rng(seed)
    cout, cin = 6, 8
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin)) * rng.lognormal(0, 1, cin)
    S = np.abs(W) * np.sqrt((X ** 2).sum(axis=0))
    if classes_only:
        perms = [tuple(c) + tuple(t for t in range(8) if t not in c)
                 for c in itertools.combinations(range(8), 4) if 0 in c]
    else:
        perms = list(itertools.permutations(range(8)))
    E_step = np.zeros(len(perms))
    E_dir = np.zeros(len(perms))
    kept = np.zeros(len(perms))
    for t, perm in enumerate(perms):
        P = np.zeros((1, 8, 8))
        P[0, list(perm), np.arange(8)] = 1.0
        fw = o.step_forward(W, X, None, 1.0, 1, 2, 4, P=P)
        E_step[t] = fw["E"]
        kept[t] = float(np.sum(fw["S_hat"] * fw["mask"]))
    # explicit loops only on one representative per partition class
    classes = {}
    for t, perm in enumerate(perms):
        key = (frozenset(perm[:4]), frozenset(perm[4:]))
        key = min(key, key[::-1], key=lambda k: sorted(k[0]))
        if key not in classes:
            classes[key] = _pruned_error_direct(W, X, S, perm, 2, 4)
        E_dir[t] = classes[key]
    return perms, E_step, E_dir, kept, (W, X)


def pin_cin8_enumeration(o):
    perms, E_step, E_dir, kept, (W, X) = enumerate_cin8(o, 16)
    assert np.allclose(E_step, E_dir, rtol=1e-12, atol=0)
    assert len(np.unique(np.round(E_step, 10))) <= 35
    assert abs(E_step.min() - E_dir.min()) <= 1e-12 * E_dir.min()
    # the same permutations reached through sharply peaked logits
    rng = _rng(17)
    for t in rng.choice(len(perms), size=40, replace=False):
        Pi = np.zeros((8, 8))
        Pi[list(perms[t]), np.arange(8)] = 1.0
        fw = o.step_forward(W, X, (60.0 * Pi)[None], 1.0, 5, 2, 4)
        assert abs(fw["E"] - E_step[t]) <= 1e-9 * E_step[t]


# -------------------------------------------------------------- gradients --
def _fd_case(seed, cout=6, cin=16, T=10, B=8, L=5, tau=0.7, N=2, M=4):
    rng = _rng(seed)
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin))
    lg = rng.standard_normal((cin // B, B, B))
    return W, X, lg, tau, L, N, M


def pin_step_gradient_fd(o):
    """d E / d logits against central differences with the mask frozen at
    the base point (the mask is held constant in the backward pass)."""
    for seed, kw in ((18, {}), (19, {"B": 8, "N": 4, "M": 8, "L": 3, "tau": 1.3})):
        W, X, lg, tau, L, N, M = _fd_case(seed, **kw)
        fw = o.step_forward(W, X, lg, tau, L, N, M)
        g = o.step_backward(fw, X, W)["dlogits"]
        mask = fw["mask"]
        h = 1e-6
        fd = np.zeros_like(lg)
        for idx in np.ndindex(lg.shape):
            lp = lg.copy(); lp[idx] += h
            lm = lg.copy(); lm[idx] -= h
            ep = o.step_forward(W, X, lp, tau, L, N, M, mask=mask)["E"]
            em = o.step_forward(W, X, lm, tau, L, N, M, mask=mask)["E"]
            fd[idx] = (ep - em) / (2 * h)
        err = np.linalg.norm(g - fd) / np.linalg.norm(fd)
        assert err < 1e-6, (seed, err)


def pin_block_adjoint_fd(o):
    """d E / d P (before the Sinkhorn adjoint) against central differences in
    P itself, mask frozen."""
    rng = _rng(20)
    cout, cin, T, B = 5, 8, 7, 4
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin))
    P = rng.random((cin // B, B, B))
    fw = o.step_forward(W, X, None, 1.0, 1, 2, 4, P=P)
    dR = fw["R"] / fw["E"]
    G = -(dR @ X)
    dP = o.block_adjoint(G, fw["A"], W, P, fw["mask"])
    h = 1e-6
    fd = np.zeros_like(P)
    for idx in np.ndindex(P.shape):
        pp = P.copy(); pp[idx] += h
        pm = P.copy(); pm[idx] -= h
        ep = o.step_forward(W, X, None, 1.0, 1, 2, 4, P=pp, mask=fw["mask"])["E"]
        em = o.step_forward(W, X, None, 1.0, 1, 2, 4, P=pm, mask=fw["mask"])["E"]
        fd[idx] = (ep - em) / (2 * h)
    err = np.linalg.norm(dP - fd) / np.linalg.norm(fd)
    assert err < 1e-7, err


def pin_zero_error_gradient(o):
    """E = 0 (nothing pruned: X is zero) gives a zero gradient, not NaN."""
    rng = _rng(21)
    W = rng.standard_normal((3, 8))
    X = np.zeros((4, 8))
    lg = rng.standard_normal((1, 8, 8))
    fw = o.step_forward(W, X, lg, 1.0, 2, 2, 4)
    assert fw["E"] == 0.0
    g = o.step_backward(fw, X, W)["dlogits"]
    assert np.all(g == 0.0)


def pin_colnorm(o):
    rng = _rng(22)
    X = rng.standard_normal((13, 5))
    want = np.array([math.sqrt(sum(float(X[t, j]) ** 2 for t in range(13))) for j in range(5)])
    assert np.allclose(o.colnorm(X), want, rtol=1e-14, atol=0)


def pin_harden_bruteforce(o):
    """Hardening (PermLLM summary, Method 2: the permutation matrix P that
    maximises Tr(P^T P_hat)) against brute force over all B! permutations."""
    rng = _rng(23)
    for B in (3, 4, 5, 6):
        for trial in range(3):
            Ph = rng.random((1, B, B))
            best, arg = -math.inf, None
            for perm in itertools.permutations(range(B)):
                val = sum(Ph[0, j, perm[j]] for j in range(B))     # row j -> column perm[j]
                if val > best:
                    best, arg = val, perm
            want = np.zeros((B, B))
            want[np.arange(B), list(arg)] = 1.0
            assert np.array_equal(o.harden(Ph)[0], want), (B, trial)


def pin_hard_forward_planted(o):
    """Logits peaked around a planted block permutation: the hardened forward
    is exactly the forward of the planted hard P (same P, mask and E), while
    the soft Sinkhorn output is still visibly soft."""
    rng = _rng(24)
    cout, cin, T, B = 6, 16, 9, 8
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin))
    nb = cin // B
    Pi = np.zeros((nb, B, B))
    for b in range(nb):
        Pi[b, np.arange(B), rng.permutation(B)] = 1.0
    lg = 2.0 * Pi + 0.05 * rng.standard_normal((nb, B, B))
    fh = o.step_forward(W, X, lg, 1.0, 3, 2, 4, hard=True)
    fp = o.step_forward(W, X, None, 1.0, 3, 2, 4, P=Pi)
    assert np.array_equal(fh["P"], Pi)
    assert np.max(np.abs(fh["P_soft"] - Pi)) > 0.1
    assert np.array_equal(fh["mask"], fp["mask"])
    assert abs(fh["E"] - fp["E"]) <= 1e-12 * fp["E"]


def pin_straight_through_gradient_fd(o):
    """Hardened step: the gradient is the straight-through estimate
    dE/dLambda = J^T g, with g = dE/dP at the hard P (mask frozen) and J the
    Jacobian of the soft Sinkhorn output. Both g and J^T g are taken by
    central differences here, independently of the adjoint formulas."""
    rng = _rng(25)
    cout, cin, T, B, tau, L = 5, 8, 7, 4, 0.8, 3
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin))
    lg = rng.standard_normal((cin // B, B, B))
    fw = o.step_forward(W, X, lg, tau, L, 2, 4, hard=True)
    got = o.step_backward(fw, X, W)["dlogits"]
    Ph, mask = fw["P"], fw["mask"]
    h = 1e-6
    gP = np.zeros_like(Ph)
    for idx in np.ndindex(Ph.shape):
        pp = Ph.copy(); pp[idx] += h
        pm = Ph.copy(); pm[idx] -= h
        ep = o.step_forward(W, X, None, tau, L, 2, 4, P=pp, mask=mask)["E"]
        em = o.step_forward(W, X, None, tau, L, 2, 4, P=pm, mask=mask)["E"]
        gP[idx] = (ep - em) / (2 * h)
    fd = np.zeros_like(lg)
    for idx in np.ndindex(lg.shape):
        lp = lg.copy(); lp[idx] += h
        lm = lg.copy(); lm[idx] -= h
        fd[idx] = (np.sum(gP * o.sinkhorn(lp, tau, L)) - np.sum(gP * o.sinkhorn(lm, tau, L))) / (2 * h)
    err = np.linalg.norm(got - fd) / np.linalg.norm(fd)
    assert err < 1e-6, err


def pin_adamw_torch(o):
    """AdamW against torch.optim.AdamW (CPU, float64) over several steps with
    changing gradients."""
    import torch
    rng = _rng(26)
    p0 = rng.standard_normal((3, 4, 4))
    grads = [rng.standard_normal(p0.shape) for _ in range(5)]
    for lr, wd in ((1e-3, 0.01), (5e-3, 0.1)):
        tp = torch.tensor(p0.copy(), dtype=torch.float64, requires_grad=True)
        opt = torch.optim.AdamW([tp], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd)
        p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
        for t, g in enumerate(grads):
            tp.grad = torch.tensor(g, dtype=torch.float64)
            opt.step()
            p, m, v = o.adamw(p, g, m, v, t + 1, lr, weight_decay=wd)
        assert np.allclose(p, tp.detach().numpy(), rtol=1e-12, atol=1e-15), (lr, wd)


def pin_tau_schedule(o):
    """Linear temperature from 1 to 0.1 (PermLLM summary, implementation
    details): endpoints and constant steps."""
    assert o.tau_schedule(0, 11) == 1.0
    assert abs(o.tau_schedule(10, 11) - 0.1) < 1e-15
    steps = [o.tau_schedule(t, 11) for t in range(11)]
    assert np.allclose(np.diff(steps), -0.09, rtol=0, atol=1e-15)


def pin_training_beats_wanda(o):
    """The method's claim on a seeded layer with an outlier-scaled X: after
    AdamW training of the logits (hardened forward, straight-through
    backward), the hard permutation prunes with less output error than plain
    Wanda (identity permutation), and the loss has come down."""
    rng = _rng(27)
    cout, cin, T, B = 16, 32, 24, 8
    W = rng.standard_normal((cout, cin)) * 0.02
    X = rng.standard_normal((T, cin)) * np.exp(rng.standard_normal(cin))[None, :]
    nb = cin // B
    lg0 = 3.0 * np.eye(B)[None].repeat(nb, axis=0) + 1e-3 * rng.standard_normal((nb, B, B))
    wanda = o.step_forward(W, X, None, 1.0, 5, 2, 4, P=np.eye(B)[None].repeat(nb, axis=0))["E"]
    lg, errs = o.train(W, X, lg0, 60, 5e-2, 2, 4, 5, hard=True)
    final = o.step_forward(W, X, lg, 0.1, 5, 2, 4, hard=True)["E"]
    assert final < wanda, (final, wanda)
    assert min(errs[-10:]) < errs[0], (errs[0], errs[-10:])


# ------------------------------------------------- cosine objective, mask STE --
def pin_cosine_closed_forms(o):
    """Cosine loss (PermLLM summary, optimisation objective) on vectors whose
    angle is known, its invariance to scaling y~, the zero-norm convention,
    and scipy's cosine distance (a library routine of the same definition)
    on flattened random matrices."""
    from scipy.spatial.distance import cosine
    assert abs(o.cosine_loss([[1.0, 0.0]], [[1.0, 1.0]]) - (1 - 1 / math.sqrt(2))) < 1e-15
    assert abs(o.cosine_loss([[3.0, 4.0]], [[4.0, -3.0]]) - 1.0) < 1e-15
    assert abs(o.cosine_loss([[1.0, 2.0]], [[-2.0, -4.0]]) - 2.0) < 1e-15
    assert abs(o.cosine_loss([[1.0, 2.0]], [[2.0, 4.0]])) < 1e-15
    rng = _rng(28)
    Y = rng.standard_normal((5, 7))
    Yt = Y + 0.3 * rng.standard_normal((5, 7))
    want = cosine(Y.ravel(), Yt.ravel())
    assert abs(o.cosine_loss(Y, Yt) - want) < 1e-14
    assert abs(o.cosine_loss(Y, 2.5 * Yt) - want) < 1e-14
    assert abs(o.cosine_loss(Y.T, Yt.T) - want) < 1e-14
    assert o.cosine_loss(Y, np.zeros_like(Y)) == 1.0


def pin_cosine_dense_is_zero(o):
    """All-ones mask and a hard P: the sparse layer is the dense one, so the
    cosine loss is 0; with the N:M mask it is positive."""
    rng = _rng(29)
    cout, cin, T, B = 6, 16, 9, 8
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin))
    nb = cin // B
    Pi = np.zeros((nb, B, B))
    for b in range(nb):
        Pi[b, np.arange(B), rng.permutation(B)] = 1.0
    lg = 2.0 * Pi + 0.05 * rng.standard_normal((nb, B, B))
    ones = np.ones((cout, cin))
    fw = o.step_forward(W, X, lg, 1.0, 3, 2, 4, hard=True, mask=ones, loss="cosine")
    assert abs(fw["L"]) < 1e-14, fw["L"]
    fs = o.step_forward(W, X, lg, 1.0, 3, 2, 4, hard=True, loss="cosine")
    assert fs["L"] > 1e-3, fs["L"]


def pin_cosine_gradient_fd(o):
    """d L_cos / d logits against central differences with the mask frozen."""
    for seed, kw in ((30, {}), (31, {"B": 8, "N": 4, "M": 8, "L": 3, "tau": 1.3})):
        W, X, lg, tau, L, N, M = _fd_case(seed, **kw)
        fw = o.step_forward(W, X, lg, tau, L, N, M, loss="cosine")
        g = o.step_backward(fw, X, W)["dlogits"]
        mask = fw["mask"]
        h = 1e-6
        fd = np.zeros_like(lg)
        for idx in np.ndindex(lg.shape):
            lp = lg.copy(); lp[idx] += h
            lm = lg.copy(); lm[idx] -= h
            ep = o.step_forward(W, X, lp, tau, L, N, M, mask=mask, loss="cosine")["L"]
            em = o.step_forward(W, X, lm, tau, L, N, M, mask=mask, loss="cosine")["L"]
            fd[idx] = (ep - em) / (2 * h)
        err = np.linalg.norm(g - fd) / np.linalg.norm(fd)
        assert err < 1e-6, (seed, err)


def pin_cosine_grad_geometry(o):
    """Scale invariance of the cosine makes its gradient orthogonal to y~,
    and by Cauchy-Schwarz it never points along y: <dL/dy~, y~> = 0 and
    <dL/dy~, y> <= 0."""
    W, X, lg, tau, L, N, M = _fd_case(32)
    fw = o.step_forward(W, X, lg, tau, L, N, M, loss="cosine")
    d = o.step_backward(fw, X, W)["dYt"]
    Yt, Y = fw["Y_tilde"], fw["Y"]
    assert abs(np.sum(d * Yt)) <= 1e-12 * np.linalg.norm(d) * np.linalg.norm(Yt)
    assert np.sum(d * Y) < 0


def _surrogate_loss(o, W, X, S, P, P0, M0, tau, L, N, M, loss):
    """Objective with the mask replaced by M0 + S_hat(P) - S_hat(P0): equal to
    the real objective at P0, with the identity as d mask / d S_hat."""
    mask = M0 + o.block_permute(S, P) - o.block_permute(S, P0)
    return o.step_forward(W, X, None, tau, L, N, M, P=P, mask=mask, loss=loss)["L"]


def pin_mask_ste_fd(o):
    """Straight-through gradient of the mask (soft P): step_backward with
    mask_ste equals central differences of the surrogate objective whose mask
    moves one for one with the permuted scores, for both objectives."""
    for seed, loss in ((33, "frobenius"), (34, "cosine")):
        W, X, lg, tau, L, N, M = _fd_case(seed, cout=5, cin=8, T=7, B=4, L=3)
        fw = o.step_forward(W, X, lg, tau, L, N, M, loss=loss)
        g = o.step_backward(fw, X, W, mask_ste=True)["dlogits"]
        g0 = o.step_backward(fw, X, W)["dlogits"]
        S, P0, M0 = fw["S"], fw["P"], fw["mask"].astype(np.float64)
        h = 1e-6
        fd = np.zeros_like(lg)
        for idx in np.ndindex(lg.shape):
            lp = lg.copy(); lp[idx] += h
            lm = lg.copy(); lm[idx] -= h
            ep = _surrogate_loss(o, W, X, S, o.sinkhorn(lp, tau, L), P0, M0, tau, L, N, M, loss)
            em = _surrogate_loss(o, W, X, S, o.sinkhorn(lm, tau, L), P0, M0, tau, L, N, M, loss)
            fd[idx] = (ep - em) / (2 * h)
        err = np.linalg.norm(g - fd) / np.linalg.norm(fd)
        assert err < 1e-6, (seed, loss, err)
        assert np.linalg.norm(g - g0) > 1e-2 * np.linalg.norm(g0), (seed, loss)


def pin_mask_ste_hard_dP_fd(o):
    """Hardened step with the mask's straight-through term: d L / d P at the
    hard P (block adjoint plus mask term) equals central differences in P of
    the surrogate objective, for both objectives."""
    rng = _rng(35)
    cout, cin, T, B, tau, L = 5, 8, 7, 4, 0.8, 3
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin))
    lg = rng.standard_normal((cin // B, B, B))
    for loss in ("frobenius", "cosine"):
        fw = o.step_forward(W, X, lg, tau, L, 2, 4, hard=True, loss=loss)
        dP = o.step_backward(fw, X, W, mask_ste=True)["dP"]
        S, P0, M0 = fw["S"], fw["P"], fw["mask"].astype(np.float64)
        h = 1e-6
        fd = np.zeros_like(P0)
        for idx in np.ndindex(P0.shape):
            pp = P0.copy(); pp[idx] += h
            pm = P0.copy(); pm[idx] -= h
            fd[idx] = (_surrogate_loss(o, W, X, S, pp, P0, M0, tau, L, 2, 4, loss)
                       - _surrogate_loss(o, W, X, S, pm, P0, M0, tau, L, 2, 4, loss)) / (2 * h)
        err = np.linalg.norm(dP - fd) / np.linalg.norm(fd)
        assert err < 1e-7, (loss, err)


def pin_training_cosine(o):
    """Training on the cosine objective (hardened forward, straight-through
    backward through P and the mask) on the outlier-scaled layer: the learned
    hard permutation has a lower cosine loss than plain Wanda (identity
    permutation)."""
    rng = _rng(27)
    cout, cin, T, B = 16, 32, 24, 8
    W = rng.standard_normal((cout, cin)) * 0.02
    X = rng.standard_normal((T, cin)) * np.exp(rng.standard_normal(cin))[None, :]
    nb = cin // B
    lg0 = 3.0 * np.eye(B)[None].repeat(nb, axis=0) + 1e-3 * rng.standard_normal((nb, B, B))
    eye = np.eye(B)[None].repeat(nb, axis=0)
    wanda = o.step_forward(W, X, None, 1.0, 5, 2, 4, P=eye, loss="cosine")["L"]
    lg, errs = o.train(W, X, lg0, 60, 5e-2, 2, 4, 5, hard=True, loss="cosine", mask_ste=True)
    final = o.step_forward(W, X, lg, 0.1, 5, 2, 4, hard=True, loss="cosine")["L"]
    assert abs(errs[0] - wanda) < 1e-12, (errs[0], wanda)
    assert final < wanda, (final, wanda)


# ------------------------------------------------------------------- deploy --
def _hard_case(seed, cout=6, cin=16, T=5, B=8):
    rng = _rng(seed)
    W = rng.standard_normal((cout, cin))
    X = rng.standard_normal((T, cin))
    nb = cin // B
    perm = np.stack([rng.permutation(B) for _ in range(nb)])
    P = np.zeros((nb, B, B))
    for b in range(nb):
        P[b, perm[b], np.arange(B)] = 1.0          # position k takes source row perm[b][k]
    return W, X, P, perm


def pin_deploy_forms(o):
    """The deployed layer three ways, for a hard P and its N:M mask: the
    definition X W_tilde^T; permuted activations times the N:M-sparse
    permuted weight (the inference form); and X times W with the mask moved
    back to source positions by explicit loops."""
    for seed, (N, M) in ((40, (2, 4)), (41, (4, 8)), (42, (1, 4))):
        W, X, P, perm = _hard_case(seed)
        cout, cin = W.shape
        B = P.shape[1]
        fw = o.step_forward(W, X, None, 1.0, 1, N, M, P=P)
        mask = fw["mask"]
        Y = o.deploy_forward(W, X, P, mask)
        Ws = o.block_permute(W, P) * mask
        Y2 = o.gather_channels(X, P) @ Ws.T
        Morig = np.zeros((cout, cin))
        for i in range(cout):
            for b in range(cin // B):
                for k in range(B):
                    Morig[i, b * B + perm[b][k]] = mask[i, b * B + k]
        Y3 = X @ (W * Morig).T
        assert np.allclose(Y, Y2, rtol=1e-13, atol=1e-13)
        assert np.allclose(Y, Y3, rtol=1e-13, atol=1e-13)
        assert np.sum(Morig) == cout * cin * N // M


def pin_gather_is_index_select(o):
    """gather_channels equals numpy fancy indexing with the global source
    index of every position; perm_from_hard recovers the permutation."""
    W, X, P, perm = _hard_case(43, cin=24, B=8)
    B = P.shape[1]
    g = np.concatenate([b * B + perm[b] for b in range(perm.shape[0])])
    assert np.array_equal(o.perm_from_hard(P), perm)
    assert np.array_equal(o.gather_channels(X, P), X[:, g])


def pin_sparse_pack(o):
    """Compressed N:M storage: decoding vals and positions gives the matrix
    back exactly, positions ascend inside each group, and groups with fewer
    nonzeros are completed with zeros at the lowest free positions."""
    rng = _rng(44)
    for N, M in ((2, 4), (4, 8), (1, 4)):
        A = rng.standard_normal((5, 32))
        keep = o.nm_mask(np.abs(A), N, M)
        A = A * keep
        vals, pos = o.sparse_pack(A, N, M)
        back = np.zeros_like(A)
        for i in range(A.shape[0]):
            for g in range(A.shape[1] // M):
                assert list(pos[i, g]) == sorted(pos[i, g]) and len(set(pos[i, g])) == N
                for s in range(N):
                    back[i, g * M + pos[i, g, s]] += vals[i, g * N + s]
        assert np.array_equal(back, A)
    Z = np.zeros((1, 4))
    Z[0, 2] = 5.0
    vals, pos = o.sparse_pack(Z, 2, 4)
    assert list(pos[0, 0]) == [0, 2] and list(vals[0]) == [0.0, 5.0]


ALL_PINS = [
    pin_sinkhorn_2x2_golden, pin_sinkhorn_uniform, pin_sinkhorn_closed_form,
    pin_sinkhorn_closed_form_values, pin_sinkhorn_doubly_stochastic,
    pin_sinkhorn_knopp, pin_sinkhorn_equivariance, pin_sinkhorn_peaked,
    pin_sinkhorn_small_tau_assignment, pin_sinkhorn_adjoint_fd,
    pin_block_permute_gather, pin_block_permute_dense, pin_nm_mask_golden,
    pin_nm_mask_bruteforce, pin_nm_mask_counts, pin_pack_bits,
    pin_identity_is_wanda, pin_hard_perm_error, pin_gram_identity,
    pin_cin8_enumeration, pin_step_gradient_fd, pin_block_adjoint_fd,
    pin_zero_error_gradient, pin_colnorm, pin_harden_bruteforce,
    pin_hard_forward_planted, pin_straight_through_gradient_fd, pin_adamw_torch,
    pin_tau_schedule, pin_training_beats_wanda, pin_cosine_closed_forms,
    pin_cosine_dense_is_zero, pin_cosine_gradient_fd, pin_cosine_grad_geometry,
    pin_mask_ste_fd, pin_mask_ste_hard_dP_fd, pin_training_cosine, pin_deploy_forms,
    pin_gather_is_index_select, pin_sparse_pack,
]
