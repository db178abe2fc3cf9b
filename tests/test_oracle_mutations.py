"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them. A pin set that lets a dropped term, a wrong sign, a
swapped order or a transposed operand through would not be evidence."""
import numpy as np
import pytest

import oracle.lcp as olcp
from tests import pins

_orig = {name: getattr(olcp, name) for name in olcp.__all__}


def _sinkhorn_cols_first(logits, tau, iters, trace=False):
    lg = np.transpose(np.asarray(logits, dtype=np.float64), (0, 2, 1))
    out = _orig["sinkhorn"](lg, tau, iters, trace=trace)
    if trace:
        P, tr = out
        return np.transpose(P, (0, 2, 1)), tr
    return np.transpose(out, (0, 2, 1))


def _sinkhorn_times_tau(logits, tau, iters, trace=False):
    return _orig["sinkhorn"](np.asarray(logits, dtype=np.float64) * tau * tau, tau, iters, trace)


def _sinkhorn_rows_only(logits, tau, iters, trace=False):
    Z = np.asarray(logits, dtype=np.float64) / tau
    for _ in range(iters):
        Z = Z - olcp.logsumexp(Z, axis=2)
    return np.exp(Z)


def _sinkhorn_one_iter_short(logits, tau, iters, trace=False):
    return _orig["sinkhorn"](logits, tau, max(1, iters - 1), trace)


def _permute_transposed(A, P, transpose=False):
    return _orig["block_permute"](A, P, transpose=not transpose)


def _mask_ties_high(S_hat, N, M, decision_dtype=np.float32):
    S = np.asarray(S_hat)
    return _orig["nm_mask"](S[:, ::-1], N, M, decision_dtype)[:, ::-1]


def _mask_smallest(S_hat, N, M, decision_dtype=np.float32):
    return _orig["nm_mask"](-np.asarray(S_hat, dtype=np.float64), N, M, decision_dtype)


def _mask_unstable(S_hat, N, M, decision_dtype=np.float32):
    # descending order taken as a reversed ascending sort: equal scores then
    # come out highest position first
    S = np.asarray(S_hat).astype(decision_dtype).astype(np.float64)
    rows, cin = S.shape
    g = np.where(np.isnan(S), -np.inf, S).reshape(rows, cin // M, M)
    order = np.flip(np.argsort(g, axis=2, kind="stable"), axis=2)
    keep = np.zeros(g.shape, dtype=bool)
    np.put_along_axis(keep, order[:, :, :N], True, axis=2)
    return keep.reshape(rows, cin)


def _mask_negzero_below(S_hat, N, M, decision_dtype=np.float32):
    S = np.asarray(S_hat).astype(np.float32)
    S = np.where((S == 0) & np.signbit(S), np.float32(-1e-30), S)
    return _orig["nm_mask"](S, N, M, decision_dtype)


def _pack_bits_msb(mask):
    m = np.asarray(mask, dtype=bool)
    rows, cin = m.shape
    return _orig["pack_bits"](m.reshape(rows, cin // 32, 32)[:, :, ::-1].reshape(rows, cin))


def _unpermute_no_transpose(W, W_hat, mask, P):
    A = np.asarray(W_hat, dtype=np.float64) * np.asarray(mask, dtype=np.float64)
    Wt = _orig["block_permute"](A, P)
    return A, Wt, np.asarray(W, dtype=np.float64) - Wt


def _unpermute_no_mask(W, W_hat, mask, P):
    return _orig["unpermute_diff"](W, W_hat, np.ones_like(np.asarray(mask, dtype=bool)), P)


def _error_squared(D, X):
    R, E = _orig["pruning_error"](D, X)
    return R, E * E


def _colnorm_l1(X):
    return np.sum(np.abs(np.asarray(X, dtype=np.float64)), axis=0)


def _importance_signed(W, n):
    return np.asarray(W, dtype=np.float64) * np.asarray(n, dtype=np.float64)[None, :]


def _importance_unscaled(W, n):
    return np.abs(np.asarray(W, dtype=np.float64))


def _block_adjoint_one_term(G, A, W, P, mask):
    P = np.asarray(P, dtype=np.float64)
    nb, B, _ = P.shape
    rows = G.shape[0]
    Gb = np.asarray(G).reshape(rows, nb, B).transpose(1, 0, 2)
    Ab = np.asarray(A).reshape(rows, nb, B).transpose(1, 0, 2)
    return np.matmul(Gb.transpose(0, 2, 1), Ab)


def _block_adjoint_unmasked(G, A, W, P, mask):
    return _orig["block_adjoint"](G, A, W, P, np.ones_like(np.asarray(mask, dtype=bool)))


def _block_adjoint_sign(G, A, W, P, mask):
    return _orig["block_adjoint"](-np.asarray(G), A, W, P, mask)


def _adjoint_no_row_step(dP, P, trace, tau):
    G = np.asarray(dP) * np.asarray(P)
    for i in range(len(trace["Z"]) - 1, -1, -1):
        G = G - np.exp(trace["Z"][i]) * np.sum(G, axis=1, keepdims=True)
    return G / tau


def _adjoint_swapped_steps(dP, P, trace, tau):
    G = np.asarray(dP) * np.asarray(P)
    for i in range(len(trace["Z"]) - 1, -1, -1):
        G = G - np.exp(trace["U"][i]) * np.sum(G, axis=2, keepdims=True)
        G = G - np.exp(trace["Z"][i]) * np.sum(G, axis=1, keepdims=True)
    return G / tau


def _adjoint_no_tau(dP, P, trace, tau):
    return _orig["sinkhorn_adjoint"](dP, P, trace, tau) * tau


def _adjoint_forward_order(dP, P, trace, tau):
    G = np.asarray(dP) * np.asarray(P)
    for i in range(len(trace["Z"])):
        G = G - np.exp(trace["Z"][i]) * np.sum(G, axis=1, keepdims=True)
        G = G - np.exp(trace["U"][i]) * np.sum(G, axis=2, keepdims=True)
    return G / tau


def _backward_unscaled(fw, X, W):
    fw2 = dict(fw)
    fw2["E"] = 1.0
    return _orig["step_backward"](fw2, X, W)


def _harden_minimise(P):
    return _orig["harden"](-np.asarray(P, dtype=np.float64))


def _harden_transposed(P):
    return np.transpose(_orig["harden"](P), (0, 2, 1))


def _ste_hard_in_sinkhorn_adjoint(fw, X, W):
    fw2 = dict(fw)
    fw2["P_soft"] = fw["P"]
    return _orig["step_backward"](fw2, X, W)


def _ste_soft_in_block_adjoint(fw, X, W):
    fw2 = dict(fw)
    fw2["P"] = fw["P_soft"]
    return _orig["step_backward"](fw2, X, W)


def _adamw_no_bias_correction(param, grad, m, v, t, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01):
    g = np.asarray(grad, dtype=np.float64)
    m = beta1 * np.asarray(m) + (1 - beta1) * g
    v = beta2 * np.asarray(v) + (1 - beta2) * g * g
    return np.asarray(param) * (1 - lr * weight_decay) - lr * m / (np.sqrt(v) + eps), m, v


def _adamw_coupled_decay(param, grad, m, v, t, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01):
    g = np.asarray(grad, dtype=np.float64) + weight_decay * np.asarray(param, dtype=np.float64)
    return _orig["adamw"](param, g, m, v, t, lr, beta1, beta2, eps, 0.0)


def _tau_reversed(t, steps, tau0=1.0, tau1=0.1):
    return _orig["tau_schedule"](t, steps, tau1, tau0)


def _train_soft(W, X, logits, steps, lr, N, M, iters, hard=True, **kw):
    return _orig["train"](W, X, logits, steps, lr, N, M, iters, hard=False, **kw)


MUTATIONS = [
    ("sinkhorn", _sinkhorn_cols_first),
    ("sinkhorn", _sinkhorn_times_tau),
    ("sinkhorn", _sinkhorn_rows_only),
    ("sinkhorn", _sinkhorn_one_iter_short),
    ("block_permute", _permute_transposed),
    ("nm_mask", _mask_ties_high),
    ("nm_mask", _mask_smallest),
    ("nm_mask", _mask_unstable),
    ("nm_mask", _mask_negzero_below),
    ("pack_bits", _pack_bits_msb),
    ("unpermute_diff", _unpermute_no_transpose),
    ("unpermute_diff", _unpermute_no_mask),
    ("pruning_error", _error_squared),
    ("colnorm", _colnorm_l1),
    ("importance", _importance_signed),
    ("importance", _importance_unscaled),
    ("block_adjoint", _block_adjoint_one_term),
    ("block_adjoint", _block_adjoint_unmasked),
    ("block_adjoint", _block_adjoint_sign),
    ("sinkhorn_adjoint", _adjoint_no_row_step),
    ("sinkhorn_adjoint", _adjoint_swapped_steps),
    ("sinkhorn_adjoint", _adjoint_no_tau),
    ("sinkhorn_adjoint", _adjoint_forward_order),
    ("step_backward", _backward_unscaled),
    ("harden", _harden_minimise),
    ("harden", _harden_transposed),
    ("step_backward", _ste_hard_in_sinkhorn_adjoint),
    ("step_backward", _ste_soft_in_block_adjoint),
    ("adamw", _adamw_no_bias_correction),
    ("adamw", _adamw_coupled_decay),
    ("tau_schedule", _tau_reversed),
    ("train", _train_soft),
]

# the full 8! enumeration is covered by the plain pin run; the rest are fast
FAST_PINS = [p for p in pins.ALL_PINS if p is not pins.pin_cin8_enumeration]


@pytest.mark.parametrize("name,bad", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(olcp, name, bad)
    caught = []
    for pin in FAST_PINS:
        try:
            pin(olcp)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, "mutation %s of %s passed every pin" % (bad.__name__, name)
