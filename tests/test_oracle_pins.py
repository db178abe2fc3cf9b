"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.lcp)


def test_fig1_importance_vs_error():
    """The PermLLM summary's motivation (Figure 1): a channel permutation with
    more retained importance can have a larger output error. Over 20 seeded
    8-channel layers, the permutation that retains the most importance is
    usually not among the minimum-error ones."""
    differ = 0
    for seed in range(100, 120):
        perms, E_step, E_dir, kept, _ = pins.enumerate_cin8(oracle.lcp, seed, classes_only=True)
        assert len(perms) == 35
        best_kept = np.flatnonzero(kept >= kept.max() - 1e-12)
        if E_step[best_kept].min() > E_step.min() * (1 + 1e-9):
            differ += 1
    assert differ >= 5, differ
