"""The GPU tests' comparison (tests/gpu_helpers.compare_out) on the CPU: the
2e-3 bar after bf16 rounding of the oracle, and its one exception - an output
whose exact value lies within BF16_TIE_BAND of the midpoint between two bf16
values may be either neighbour (a float32 computation that correct to ~1e-6
may round either way there).  Pinned on hand-built values: no GPU involved."""
import numpy as np
import torch

import gpu_helpers as G

MID = 0.75 + 2.0 ** -9          # midpoint of the bf16 neighbours 0.75 and 0.75390625 (one step 2^-8)


def _bf(vals):
    return torch.tensor(vals, dtype=torch.bfloat16)


def test_plain_agreement_and_bar():
    ref = np.array([0.1234567, -0.0312, 1.9])
    G.compare_out(_bf(ref.tolist()), ref, "bf16", "rounded alike")


def test_tie_either_way():
    for d in (1e-7, -1e-7, G.BF16_TIE_BAND * 0.99, -G.BF16_TIE_BAND * 0.99):
        ref = np.array([MID + d])
        for got in (0.75, 0.75390625):          # both neighbours accepted
            assert G.compare_out(_bf([got]), ref, "bf16", "tie") == 0.0


def test_not_a_tie_still_fails():
    import pytest
    for d in (G.BF16_TIE_BAND * 1.5, 1e-3):
        ref = np.array([MID + d])                # rounds up to 0.75390625
        with pytest.raises(AssertionError):
            G.compare_out(_bf([0.75]), ref, "bf16", "one step off, away from the midpoint")
    # two steps off is never a tie
    with pytest.raises(AssertionError):
        G.compare_out(_bf([0.7578125]), np.array([MID]), "bf16", "two steps")


def test_small_outputs_keep_the_plain_bar():
    # below |O| = 0.25 one bf16 step is under the bar: no tie handling needed
    ref = np.array([0.2 + 1e-7])
    G.compare_out(_bf([0.2]), ref, "bf16", "small")
