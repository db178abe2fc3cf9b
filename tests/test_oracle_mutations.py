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


def _backward_unscaled(fw, X, W, mask_ste=False):
    fw2 = dict(fw)
    fw2["E"] = 1.0
    return _orig["step_backward"](fw2, X, W, mask_ste)


def _harden_minimise(P):
    return _orig["harden"](-np.asarray(P, dtype=np.float64))


def _harden_transposed(P):
    return np.transpose(_orig["harden"](P), (0, 2, 1))


def _ste_hard_in_sinkhorn_adjoint(fw, X, W, mask_ste=False):
    fw2 = dict(fw)
    fw2["P_soft"] = fw["P"]
    return _orig["step_backward"](fw2, X, W, mask_ste)


def _ste_soft_in_block_adjoint(fw, X, W, mask_ste=False):
    fw2 = dict(fw)
    fw2["P"] = fw["P_soft"]
    return _orig["step_backward"](fw2, X, W, mask_ste)


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


def _cosine_norm_y_squared(Y, Yt):
    y = np.asarray(Y, dtype=np.float64).ravel()
    yt = np.asarray(Yt, dtype=np.float64).ravel()
    return float(1.0 - np.dot(y, yt) / np.dot(y, y))


def _cosine_similarity_not_loss(Y, Yt):
    return 1.0 - _orig["cosine_loss"](Y, Yt)


def _cosine_grad_cube_dropped(Y, Yt):
    Y = np.asarray(Y, dtype=np.float64)
    Yt = np.asarray(Yt, dtype=np.float64)
    ny, nt = np.linalg.norm(Y), np.linalg.norm(Yt)
    return -Y / (ny * nt) + np.sum(Y * Yt) * Yt / (ny * nt ** 2)


def _cosine_grad_first_term(Y, Yt):
    Y = np.asarray(Y, dtype=np.float64)
    return -Y / (np.linalg.norm(Y) * np.linalg.norm(np.asarray(Yt, dtype=np.float64)))


def _cosine_of_residual(W, X, logits, tau, iters, N, M, P=None, mask=None, hard=False,
                        loss="frobenius"):
    fw = _orig["step_forward"](W, X, logits, tau, iters, N, M, P, mask, hard, loss)
    if loss == "cosine":
        fw["L"] = olcp.cosine_loss(fw["Y"], fw["R"])
    return fw


def _ste_without_weight(G, W, S, P):
    return _orig["mask_ste_adjoint"](G, np.ones_like(np.asarray(W, dtype=np.float64)), S, P)


def _ste_unscaled_importance(G, W, S, P):
    return _orig["mask_ste_adjoint"](G, W, np.abs(np.asarray(W, dtype=np.float64)), P)


def _ste_sign(G, W, S, P):
    return -_orig["mask_ste_adjoint"](G, W, S, P)


def _ste_unpermuted_weight(G, W, S, P):
    P = np.asarray(P, dtype=np.float64)
    nb, B, _ = P.shape
    rows = G.shape[0]
    Gb = np.asarray(G, dtype=np.float64).reshape(rows, nb, B).transpose(1, 0, 2)
    Wb = np.asarray(W, dtype=np.float64).reshape(rows, nb, B).transpose(1, 0, 2)
    Sb = np.asarray(S, dtype=np.float64).reshape(rows, nb, B).transpose(1, 0, 2)
    return np.matmul(Sb.transpose(0, 2, 1), np.matmul(Gb, P) * Wb)


def _ste_mask_term_at_soft_P(fw, X, W, mask_ste=False):
    out = _orig["step_backward"](fw, X, W)
    if mask_ste:
        dP = out["dP"] + olcp.mask_ste_adjoint(out["G"], W, fw["S"], fw["P_soft"])
        out["dP"] = dP
        out["dlogits"] = olcp.sinkhorn_adjoint(dP, fw["P_soft"], fw["trace"], fw["tau"])
    return out


def _train_ignores_loss(W, X, logits, steps, lr, N, M, iters, hard=True, loss="frobenius",
                        mask_ste=False, **kw):
    return _orig["train"](W, X, logits, steps, lr, N, M, iters, hard=hard, mask_ste=mask_ste, **kw)


def _gather_inverse(X, P):
    return _orig["gather_channels"](X, np.transpose(np.asarray(P, dtype=np.float64), (0, 2, 1)))


def _pack_descending(A, N, M):
    vals, pos = _orig["sparse_pack"](A, N, M)
    rows, G = pos.shape[0], pos.shape[1]
    return vals.reshape(rows, G, N)[:, :, ::-1].reshape(rows, G * N), pos[:, :, ::-1]


def _deploy_unmasked(W, X, P, mask):
    return _orig["deploy_forward"](W, X, P, np.ones_like(np.asarray(mask, dtype=np.float64)))


def _deploy_permuted_order(W, X, P, mask):
    Ws = olcp.block_permute(W, P) * np.asarray(mask, dtype=np.float64)
    return np.asarray(X, dtype=np.float64) @ Ws.T


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
    ("cosine_loss", _cosine_norm_y_squared),
    ("cosine_loss", _cosine_similarity_not_loss),
    ("cosine_grad", _cosine_grad_cube_dropped),
    ("cosine_grad", _cosine_grad_first_term),
    ("step_forward", _cosine_of_residual),
    ("mask_ste_adjoint", _ste_without_weight),
    ("mask_ste_adjoint", _ste_unscaled_importance),
    ("mask_ste_adjoint", _ste_sign),
    ("mask_ste_adjoint", _ste_unpermuted_weight),
    ("step_backward", _ste_mask_term_at_soft_P),
    ("train", _train_ignores_loss),
    ("gather_channels", _gather_inverse),
    ("sparse_pack", _pack_descending),
    ("deploy_forward", _deploy_unmasked),
    ("deploy_forward", _deploy_permuted_order),
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
