"""Float64 oracle for one LCP step: O1 .. O11 (test infrastructure only).

Notation follows the PermLLM summary page:

* W in R^{Cout x Cin}  weight (row-major, like a linear layer); X in R^{T x Cin}
  calibration activations (tokens x channels); the layer output is X W^T.
* Logits Lambda: nb x B x B, one B x B matrix per channel block (Method 3).
* P_b[j, k]: row j is source channel b*B + j, column k is permuted position
  b*B + k, so W_hat = W P_B gives W_hat[:, bB+k] = sum_j W[:, bB+j] P_b[j, k]
  (task definition: W_hat = W P; Method 3: P_B = diag(P_1 .. P_nb)).

Readings taken where the pages leave a step open (each is also listed in the
design notes):

* Importance is Wanda's |W_ij| * ||X[:, j]||_2. The pages name Wanda as the
  one-shot method LCP plugs into but do not print its formula.
* Under a soft P the sparse weight is returned to the original channel order
  as W_tilde = (W_hat . M) P_B^T, and the loss is the output error
  E = ||(W - W_tilde) X^T||_F (not squared, not normalised). The task
  definition asks for the permuted, pruned weight closest to the dense one on
  the layer's outputs; this is that distance.
* By default the mask is held constant in the backward pass. With mask_ste
  the gradient that reaches the 0/1 mask is handed unchanged to the permuted
  scores S_hat = S P_B (straight-through estimator for the argmax that picks
  the mask, PermLLM summary, integration with pruning methods), which adds
  S_b^T ((G_b P_b) . (W_b P_b)) to d/dP_b.
* The cosine objective (PermLLM summary, optimisation objective) compares the
  dense outputs y = W X^T with the sparse outputs y~ = W_tilde X^T over the
  whole output tensor, flattened into one vector per layer:
  L = 1 - <y, y~> / (||y|| ||y~||). When either norm is zero the loss is 1
  and its gradient zero.
* Hardening (Method 2) is optional: the forward may replace P_hat by the
  permutation maximising Tr(P^T P_hat) per block; the backward then takes the
  block adjoint at the hard P and passes it unchanged to the adjoint of the
  soft Sinkhorn (straight-through estimator).
* Ties inside an N:M group go to the lower permuted position; NaN scores rank
  as -inf; -0 ties with +0. The keep decision is taken on float32 scores, the
  precision the GPU kernel decides in.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "colnorm", "importance", "logsumexp", "sinkhorn", "block_permute",
    "nm_mask", "pack_bits", "unpack_bits", "unpermute_diff", "pruning_error",
    "step_forward", "step_backward", "sinkhorn_adjoint", "block_adjoint",
    "harden", "adamw", "tau_schedule", "train", "layer_output", "cosine_loss",
    "cosine_grad", "mask_ste_adjoint", "perm_from_hard", "gather_channels", "sparse_pack",
    "deploy_forward",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# O1 -------------------------------------------------------------------------
def colnorm(X):
    """n_j = ||X[:, j]||_2 over the T calibration tokens (float64)."""
    X = _f64(X)
    return np.sqrt(np.sum(X * X, axis=0))


# O2 -------------------------------------------------------------------------
def importance(W, n):
    """Wanda importance S_ij = |W_ij| * n_j (PermLLM summary, integration with
    one-shot pruning: S is the pruning method's importance matrix)."""
    return np.abs(_f64(W)) * _f64(n)[None, :]


# O3 -------------------------------------------------------------------------
def logsumexp(Z, axis):
    """Max-shifted log(sum(exp(Z))) along one axis, keeping that axis."""
    m = np.max(Z, axis=axis, keepdims=True)
    return m + np.log(np.sum(np.exp(Z - m), axis=axis, keepdims=True))


def sinkhorn(logits, tau, iters, trace=False):
    """Soft permutation P_hat = S_L(Lambda / tau), batched over blocks.

    PermLLM summary, Method 1: S_0(X) = exp(X), S_i(X) = T_c(T_r(S_{i-1}(X)))
    with T_r / T_c normalising rows / columns, and P_hat = S_L(W_P / tau).
    PermLLM blog, section 2.2, gives the log-domain form: subtract the
    row-wise log-sum-exp, then the column-wise one, per iteration, and take exp
    at the end. One iteration = one row step then one column step.

    logits: [nb, B, B]. Returns P_hat [nb, B, B]; with trace=True also a dict
    holding, for i = 1..L, U^i (after the row step), Z^i (after the column
    step) and the offsets r^i (row lse, [nb, B]) and c^i (column lse, [nb, B]).
    """
    if iters < 1 or not (tau > 0):
        raise ValueError("iters >= 1 and tau > 0 required")
    Z = _f64(logits) / float(tau)
    U_list, Z_list, r_list, c_list = [], [], [], []
    for _ in range(iters):
        r = logsumexp(Z, axis=2)          # [nb, B, 1]: one value per row j
        U = Z - r                         # T_r in the log domain
        c = logsumexp(U, axis=1)          # [nb, 1, B]: one value per column k
        Z = U - c                         # T_c in the log domain
        if trace:
            U_list.append(U)
            Z_list.append(Z)
            r_list.append(r[:, :, 0])
            c_list.append(c[:, 0, :])
    P = np.exp(Z)
    if trace:
        return P, {"Z0": _f64(logits) / float(tau), "U": U_list, "Z": Z_list,
                   "r": r_list, "c": c_list}
    return P


# O4 -------------------------------------------------------------------------
def block_permute(A, P, transpose=False):
    """A P_B with P_B = diag(P_1 .. P_nb) (PermLLM summary, Method 3).

    out[:, bB+k] = sum_j A[:, bB+j] P_b[j, k]; with transpose=True the block
    matrices are transposed (A P_B^T), which maps permuted positions back to
    source channels.
    """
    A = _f64(A)
    P = _f64(P)
    nb, B, _ = P.shape
    rows, cin = A.shape
    if cin != nb * B:
        raise ValueError("A has %d columns, blocks cover %d" % (cin, nb * B))
    Pb = np.transpose(P, (0, 2, 1)) if transpose else P
    Ab = A.reshape(rows, nb, B).transpose(1, 0, 2)        # [nb, rows, B]
    out = np.matmul(Ab, Pb)                               # [nb, rows, B]
    return out.transpose(1, 0, 2).reshape(rows, cin)


# O5 -------------------------------------------------------------------------
def nm_mask(S_hat, N, M, decision_dtype=np.float32):
    """Importance-based N:M mask (PermLLM summary, integration formula:
    argmax over M of sum (M . S_hat)_{i, kM:(k+1)M}; PermLLM blog 2.1: keep
    the N largest of every M consecutive weights, zero the rest).

    Per output row i and group g (permuted positions gM .. gM+M-1) the N
    positions with the largest score survive; among equal scores the lower
    position wins. Scores are first rounded to `decision_dtype` (float32: the
    precision the keep decision is taken in), NaN is read as -inf.
    Returns a bool array of S_hat's shape, True = kept.
    """
    if not (1 <= N < M):
        raise ValueError("need 1 <= N < M")
    S = np.asarray(S_hat)
    rows, cin = S.shape
    if cin % M:
        raise ValueError("columns must be a multiple of M")
    v = S.astype(decision_dtype).astype(np.float64)
    v = np.where(np.isnan(v), -np.inf, v)
    g = v.reshape(rows, cin // M, M)
    # stable sort of -score: equal scores keep ascending position order
    order = np.argsort(-g, axis=2, kind="stable")
    keep = np.zeros(g.shape, dtype=bool)
    np.put_along_axis(keep, order[:, :, :N], True, axis=2)
    return keep.reshape(rows, cin)


def pack_bits(mask):
    """bool [rows, cin] -> uint32 [rows, cin/32]; bit (k mod 32) of word k/32
    is position k, 1 = kept."""
    mask = np.asarray(mask, dtype=bool)
    rows, cin = mask.shape
    if cin % 32:
        raise ValueError("cin must be a multiple of 32")
    b = mask.reshape(rows, cin // 32, 32).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (b * weights).sum(axis=2).astype(np.uint32)


def unpack_bits(bits, cin):
    bits = np.asarray(bits, dtype=np.uint32)
    rows = bits.shape[0]
    shifts = np.arange(32, dtype=np.uint32)
    m = (bits[:, :, None] >> shifts[None, None, :]) & np.uint32(1)
    return m.reshape(rows, cin).astype(bool)[:, :cin]


# O6 -------------------------------------------------------------------------
def unpermute_diff(W, W_hat, mask, P):
    """A = W_hat . M;  W_tilde = A P_B^T;  D = W - W_tilde.

    W_tilde is the pruned, permuted weight returned to the source channel
    order (for a hard P this is W with the pruned entries zeroed)."""
    A = _f64(W_hat) * np.asarray(mask, dtype=np.float64)
    W_tilde = block_permute(A, P, transpose=True)
    return A, W_tilde, _f64(W) - W_tilde


# O7 -------------------------------------------------------------------------
def pruning_error(D, X):
    """R = D X^T (Cout x T), E = ||R||_F."""
    R = _f64(D) @ _f64(X).T
    return R, float(np.sqrt(np.sum(R * R)))


# forward step ---------------------------------------------------------------
def step_forward(W, X, logits, tau, iters, N, M, P=None, mask=None, hard=False,
                 loss="frobenius"):
    """One LCP forward step (O1 .. O7). Returns a dict of every intermediate.

    P overrides the Sinkhorn output (used to feed hard permutations); mask
    overrides the N:M selection (used to freeze the mask for finite
    differences; any real array is accepted). hard=True replaces the soft
    P_hat by its hardened permutation before the block permutation (PermLLM
    summary, Method 2); the dict then holds the hard matrix as "P" and the
    Sinkhorn output as "P_soft". "L" is the objective named by `loss`:
    "frobenius" (L = E) or "cosine" (L = cosine_loss of the dense and sparse
    outputs, which are then returned as "Y" and "Y_tilde")."""
    if loss not in ("frobenius", "cosine"):
        raise ValueError("unknown loss %r" % (loss,))
    W = _f64(W)
    X = _f64(X)
    n = colnorm(X)
    S = importance(W, n)
    tr = None
    if P is None:
        P, tr = sinkhorn(logits, tau, iters, trace=True)
    P = _f64(P)
    P_soft = P
    if hard:
        P = harden(P_soft)
    W_hat = block_permute(W, P)
    S_hat = block_permute(S, P)
    if mask is None:
        mask = nm_mask(S_hat, N, M)
    A, W_tilde, D = unpermute_diff(W, W_hat, mask, P)
    R, E = pruning_error(D, X)
    out = {"n": n, "S": S, "P": P, "P_soft": P_soft, "hard": bool(hard), "trace": tr,
           "W_hat": W_hat, "S_hat": S_hat, "mask": mask, "A": A, "W_tilde": W_tilde,
           "D": D, "R": R, "E": E, "tau": float(tau), "iters": int(iters), "loss": loss,
           "L": E}
    if loss == "cosine":
        Y = layer_output(W, X)
        Yt = layer_output(W_tilde, X)
        out.update(Y=Y, Y_tilde=Yt, L=cosine_loss(Y, Yt))
    return out


# O8 .. O10 ------------------------------------------------------------------
def block_adjoint(G, A, W, P, mask):
    """dE/dP_b with the mask held constant, given G = dE/dW_tilde.

    W_tilde_b = A_b P_b^T contributes G_b^T A_b; A_b = (W_b P_b) . M_b
    contributes W_b^T ((G_b P_b) . M_b). Both sum over the Cout rows."""
    P = _f64(P)
    nb, B, _ = P.shape
    rows = G.shape[0]
    Gb = _f64(G).reshape(rows, nb, B).transpose(1, 0, 2)     # [nb, rows, B]
    Ab = _f64(A).reshape(rows, nb, B).transpose(1, 0, 2)
    Wb = _f64(W).reshape(rows, nb, B).transpose(1, 0, 2)
    Mb = np.asarray(mask, dtype=np.float64).reshape(rows, nb, B).transpose(1, 0, 2)
    GP = np.matmul(Gb, P) * Mb                                # dE/dW_hat
    return (np.matmul(Gb.transpose(0, 2, 1), Ab)
            + np.matmul(Wb.transpose(0, 2, 1), GP))


# O11 ------------------------------------------------------------------------
def sinkhorn_adjoint(dP, P, trace, tau):
    """Reverse pass through the unrolled log-domain Sinkhorn iterations.

    Gamma = dE/dZ^L = dP . P. A column step Z = U - 1 lse_col(U)^T has
    Jacobian-transpose Gamma -> Gamma - exp(Z) . (1 1^T Gamma) (column sums
    broadcast down each column); a row step U = Z' - lse_row(Z') 1^T has
    Gamma -> Gamma - exp(U) . (Gamma 1 1^T) (row sums broadcast along each
    row). Iterations are undone from L to 1, then d Lambda = Gamma / tau."""
    G = _f64(dP) * _f64(P)
    for i in range(len(trace["Z"]) - 1, -1, -1):
        Zi = trace["Z"][i]
        Ui = trace["U"][i]
        G = G - np.exp(Zi) * np.sum(G, axis=1, keepdims=True)
        G = G - np.exp(Ui) * np.sum(G, axis=2, keepdims=True)
    return G / float(tau)


def step_backward(fw, X, W, mask_ste=False):
    """Gradient of the forward's objective L with respect to the logits
    (O8 .. O11).

    Frobenius: dR = R / E (zero when E = 0) and G = dL/dW_tilde = -dR X.
    Cosine: G = (dL/dY~) X with dL/dY~ from cosine_grad. Then the block
    adjoint (mask constant), plus the mask's straight-through term when
    mask_ste, and the Sinkhorn adjoint. Requires a forward dict whose P came
    from the Sinkhorn (trace present). For a hardened forward the block
    adjoint is taken at the hard P and its result is handed unchanged to the
    Sinkhorn adjoint of the soft P_hat (straight-through estimator, PermLLM
    summary, Method 2)."""
    if fw["trace"] is None:
        raise ValueError("forward step must come from logits")
    out = {}
    if fw["loss"] == "cosine":
        dYt = cosine_grad(fw["Y"], fw["Y_tilde"])
        G = dYt @ _f64(X)
        out["dYt"] = dYt
    else:
        E = fw["E"]
        R = fw["R"]
        dR = R / E if E > 0 else np.zeros_like(R)
        G = -(dR @ _f64(X))
        out["dR"] = dR
    dP = block_adjoint(G, fw["A"], W, fw["P"], fw["mask"])
    if mask_ste:
        dP = dP + mask_ste_adjoint(G, W, fw["S"], fw["P"])
    dL = sinkhorn_adjoint(dP, fw["P_soft"], fw["trace"], fw["tau"])
    out.update(G=G, dP=dP, dlogits=dL)
    return out


# cosine objective and the mask's straight-through term ----------------------
def layer_output(W, X):
    """Y = W X^T (Cout x T): the layer's outputs on the T calibration tokens,
    one column per token."""
    return _f64(W) @ _f64(X).T


def cosine_loss(Y, Yt):
    """L = 1 - <y, y~> / (||y|| ||y~||) (PermLLM summary, optimisation
    objective) with y, y~ the flattened arrays; 1 when either norm is 0."""
    y = _f64(Y).ravel()
    yt = _f64(Yt).ravel()
    ny = np.sqrt(np.dot(y, y))
    nt = np.sqrt(np.dot(yt, yt))
    if ny == 0.0 or nt == 0.0:
        return 1.0
    return float(1.0 - np.dot(y, yt) / (ny * nt))


def cosine_grad(Y, Yt):
    """dL/dY~ of cosine_loss: -Y / (|Y| |Y~|) + <Y, Y~> Y~ / (|Y| |Y~|^3)
    (the quotient rule on the definition); zero when either norm is 0."""
    Y = _f64(Y)
    Yt = _f64(Yt)
    ny = np.sqrt(np.sum(Y * Y))
    nt = np.sqrt(np.sum(Yt * Yt))
    if ny == 0.0 or nt == 0.0:
        return np.zeros_like(Yt)
    p = np.sum(Y * Yt)
    return -Y / (ny * nt) + p * Yt / (ny * nt ** 3)


def mask_ste_adjoint(G, W, S, P):
    """Straight-through term of the N:M mask (PermLLM summary, integration
    with pruning methods: the argmax that picks the mask is passed through by
    the STE). A = W_hat . M gives dL/dM = dL/dA . W_hat = (G_b P_b) . W_hat_b;
    passed unchanged to S_hat_b = S_b P_b it contributes S_b^T dL/dM_b to
    dL/dP_b. G = dL/dW_tilde, S the unpermuted importance."""
    P = _f64(P)
    nb, B, _ = P.shape
    rows = G.shape[0]
    Gb = _f64(G).reshape(rows, nb, B).transpose(1, 0, 2)
    Wb = _f64(W).reshape(rows, nb, B).transpose(1, 0, 2)
    Sb = _f64(S).reshape(rows, nb, B).transpose(1, 0, 2)
    dM = np.matmul(Gb, P) * np.matmul(Wb, P)
    return np.matmul(Sb.transpose(0, 2, 1), dM)


# hardening (Method 2) -------------------------------------------------------
def harden(P):
    """Hard permutation per block: argmax over permutation matrices of
    Tr(P^T P_hat) (PermLLM summary, Method 2), via the Hungarian-type solver
    of scipy (a library linear-assignment routine). Returns [nb, B, B] 0/1."""
    from scipy.optimize import linear_sum_assignment
    P = _f64(P)
    out = np.zeros_like(P)
    for b in range(P.shape[0]):
        rows, cols = linear_sum_assignment(P[b], maximize=True)
        out[b, rows, cols] = 1.0
    return out


# optimiser loop (implementation details of the PermLLM summary) -------------
def adamw(param, grad, m, v, t, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01):
    """One AdamW update (Loshchilov and Hutter: Adam with decoupled weight
    decay) of step t >= 1. Returns (param, m, v):
    m = b1 m + (1 - b1) g; v = b2 v + (1 - b2) g^2;
    param <- param (1 - lr wd) - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)."""
    g = _f64(grad)
    m = beta1 * _f64(m) + (1.0 - beta1) * g
    v = beta2 * _f64(v) + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    p = _f64(param) * (1.0 - lr * weight_decay) - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v


def tau_schedule(t, steps, tau0=1.0, tau1=0.1):
    """Temperature of step t (0-based) of `steps`: linear from tau0 to tau1."""
    if steps <= 1:
        return float(tau0)
    return float(tau0 + (tau1 - tau0) * t / (steps - 1))


def train(W, X, logits, steps, lr, N, M, iters, hard=True, tau0=1.0, tau1=0.1,
          loss="frobenius", mask_ste=False, **adam):
    """`steps` LCP steps on one layer: forward (hardened when `hard`), the
    backward of the objective `loss` (with the mask's straight-through term
    when `mask_ste`), one AdamW update of the logits, tau annealed linearly.
    Returns (logits, list of the objective per step)."""
    lg = _f64(logits).copy()
    m = np.zeros_like(lg)
    v = np.zeros_like(lg)
    errs = []
    for t in range(steps):
        tau = tau_schedule(t, steps, tau0, tau1)
        fw = step_forward(W, X, lg, tau, iters, N, M, hard=hard, loss=loss)
        g = step_backward(fw, X, W, mask_ste=mask_ste)["dlogits"]
        errs.append(fw["L"])
        lg, m, v = adamw(lg, g, m, v, t + 1, lr, **adam)
    return lg, errs



# deploy: inference with the learned permutation ------------------------------
def perm_from_hard(P):
    """perm[b][k] = the source row j with P_b[j, k] = 1, for a hard P
    ([nb, B, B] 0/1 with one 1 per row and column). int64 [nb, B]."""
    P = _f64(P)
    if not np.all((P == 0.0) | (P == 1.0)) or not np.all(P.sum(axis=1) == 1.0) \
            or not np.all(P.sum(axis=2) == 1.0):
        raise ValueError("P is not a block permutation")
    return np.argmax(P, axis=1)


def gather_channels(X, P):
    """Activations in permuted channel order for a hard P: X P_B, so column
    bB + k holds X[:, bB + perm[b][k]] (PermLLM summary, inference
    acceleration: the channel permutation applied at inference time)."""
    perm_from_hard(P)
    return block_permute(X, P)


def sparse_pack(A, N, M):
    """Compressed form of a matrix with at most N nonzeros in every group of
    M consecutive columns: vals [rows, cin/M*N] holds each group's kept
    entries in ascending position, pos [rows, cin/M, N] their positions in
    the group. Groups with fewer than N nonzeros are completed with zero
    entries at the lowest free positions. Here "kept" means nonzero."""
    A = _f64(A)
    rows, cin = A.shape
    if cin % M:
        raise ValueError("columns must be a multiple of M")
    G = cin // M
    vals = np.zeros((rows, G * N))
    pos = np.zeros((rows, G, N), dtype=np.int64)
    for i in range(rows):
        for g in range(G):
            seg = A[i, g * M:(g + 1) * M]
            nz = [k for k in range(M) if seg[k] != 0.0]
            if len(nz) > N:
                raise ValueError("group with more than N nonzeros")
            free = [k for k in range(M) if k not in nz]
            chosen = sorted(nz + free[:N - len(nz)])
            for s, k in enumerate(chosen):
                pos[i, g, s] = k
                vals[i, g * N + s] = seg[k]
    return vals, pos


def deploy_forward(W, X, P, mask):
    """Layer outputs of the deployed sparse layer, Y = X W_tilde^T (T x Cout)
    with W_tilde = ((W P_B) . M) P_B^T the pruned weight in source order."""
    W_hat = block_permute(W, P)
    _, W_tilde, _ = unpermute_diff(W, W_hat, mask, P)
    return _f64(X) @ W_tilde.T
