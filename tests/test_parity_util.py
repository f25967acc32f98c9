"""The end-to-end keep-set comparison used by the GPU parity tests accepts
what it should and rejects planted mistakes (CPU only)."""
import numpy as np
import pytest

import oracle as O
from tests.parity_util import keep_swap_gap


def _row(seed, n=200):
    rng = np.random.default_rng(seed)
    return rng.random(n)


def test_equal_sets_have_no_gap():
    s = _row(1)
    want = O.select_keep(s, 200, 4, 16, 60)
    assert keep_swap_gap(want, want, s, 200, 4, 16) == 0.0


def test_near_tie_swap_is_accepted_and_reported():
    s = _row(2)
    want = O.select_keep(s, 200, 4, 16, 60)
    mid = [j for j in want if 4 <= j < 184]
    tau_j = min(mid, key=lambda j: s[j])
    out_j = max((j for j in range(4, 184) if j not in set(want)), key=lambda j: s[j])
    s2 = s.copy()
    s2[out_j] = s[tau_j] - 3e-7          # the best excluded score, just below the cut
    want2 = O.select_keep(s2, 200, 4, 16, 60)
    got = sorted((set(want2.tolist()) - {tau_j}) | {out_j})
    gap = keep_swap_gap(got, want2, s2, 200, 4, 16)
    assert 0 < gap <= 1e-6


def test_far_swap_is_rejected():
    s = _row(3)
    want = O.select_keep(s, 200, 4, 16, 60)
    mid = sorted(j for j in want if 4 <= j < 184)
    worst_out = min((j for j in range(4, 184) if j not in set(want)), key=lambda j: s[j])
    got = sorted((set(want.tolist()) - {mid[0]}) | {worst_out})
    with pytest.raises(AssertionError):
        keep_swap_gap(got, want, s, 200, 4, 16)


def test_size_or_forced_difference_is_rejected():
    s = _row(4)
    want = O.select_keep(s, 200, 4, 16, 60)
    with pytest.raises(AssertionError):
        keep_swap_gap(want[:-1], want, s, 200, 4, 16)
    # dropping a sink for a middle position
    got = sorted((set(want.tolist()) - {0}) | {next(j for j in range(4, 184) if j not in set(want))})
    with pytest.raises(AssertionError):
        keep_swap_gap(got, want, s, 200, 4, 16)
