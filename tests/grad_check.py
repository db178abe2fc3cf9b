"""Gradient parity helpers for the GPU tests: the oracle's backward taken on
the mask the GPU's forward chose (the mask is held constant in the backward,
so a flip near a tie would otherwise add noise unrelated to kernel error),
compared as a whole and block by block."""
import numpy as np

import oracle
from tests.gpu_util import rel_fro, say


def oracle_backward_on_mask(lay, spec, logits, bits_rowmajor, hard=False, loss="frobenius", mask_ste=False):
    """Oracle forward (its own P, or its hard P) with the given row-major mask
    words, then its backward. Returns (forward dict, backward dict)."""
    mask = oracle.unpack_bits(np.asarray(bits_rowmajor, dtype=np.uint32), lay.cin)
    fw = oracle.step_forward(lay.W, lay.X, logits, spec.tau, spec.iters, spec.N, spec.M, mask=mask,
                             hard=hard, loss=loss)
    bw = oracle.step_backward(fw, lay.X, lay.W, mask_ste=mask_ste)
    return fw, bw


def check_gradient(got, want, tol=1e-2, block_tol=2e-2, what="dlogits"):
    """Relative Frobenius error of the whole gradient (<= tol) and of every
    B x B block (<= block_tol). A block's error is taken relative to the
    larger of its own norm and the RMS block norm ||want|| / sqrt(nb): a block
    whose gradient nearly cancels (its terms large, their sum small) carries
    the rounding of its terms, not of its sum, while an error confined to a
    few row tiles of one block still shows against a typical block's norm."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    r = rel_fro(got, want)
    norms = np.sqrt(np.sum(want * want, axis=(1, 2)))
    errs = np.sqrt(np.sum((got - want) ** 2, axis=(1, 2)))
    scale = np.maximum(norms, np.linalg.norm(want) / np.sqrt(len(norms)))
    per = errs / scale
    worst = int(np.argmax(per))
    order = np.argsort(per)[::-1][:3]
    say("%s rel %.3e, worst blocks %s (norm / max block norm %s)"
        % (what, r, ", ".join("%d: %.3e" % (b, per[b]) for b in order),
           ", ".join("%.3f" % (norms[b] / norms.max()) for b in order)))
    assert r < tol, (what, r)
    assert per[worst] < block_tol, (what, worst, per[worst])
    return r, float(per[worst])
