"""CPU pins of the GPU acceptance rule (tests/checker.py): exact rows pass,
each plausible GPU mistake fails, ties inside the band are accepted."""
import numpy as np
import pytest

from tests.checker import check_row

TOL = 1e-3


def _exact(s, k):
    order = np.lexsort((np.arange(s.shape[0]), -s))[:k]
    idx = np.full(k, -1, np.int64)
    val = np.full(k, -np.inf)
    idx[:order.shape[0]] = order
    val[:order.shape[0]] = s[order]
    return idx, val


def _scores(seed=0, n=50):
    return np.random.default_rng(seed).standard_normal(n) * 4


def test_exact_row_passes():
    s = _scores()
    idx, val = _exact(s, 10)
    check_row(idx, val, s, 10, TOL)


def test_short_row_returns_every_key():
    s = _scores(n=6)
    idx, val = _exact(s, 10)
    check_row(idx, val, s, 10, TOL)
    bad = idx.copy()
    bad[5] = -1
    with pytest.raises(AssertionError):
        check_row(bad, None, s, 10, TOL)


@pytest.mark.parametrize("mistake", ["swap_in_loser", "duplicate", "bad_tail", "out_of_range",
                                     "value_off", "order", "value_tail"])
def test_mistakes_fail(mistake):
    s = _scores(1)
    idx, val = _exact(s, 10)
    order = np.lexsort((np.arange(s.shape[0]), -s))
    if mistake == "swap_in_loser":
        idx[9] = order[30]
        val[9] = s[order[30]]
    elif mistake == "duplicate":
        idx[9] = idx[8]
    elif mistake == "bad_tail":
        idx, val = _exact(s[:8], 10)
        idx[9] = 3
    elif mistake == "out_of_range":
        idx[0] = 50
    elif mistake == "value_off":
        val[3] *= 1.01
    elif mistake == "order":
        idx[[0, 5]] = idx[[5, 0]]
        val[[0, 5]] = val[[5, 0]]
    elif mistake == "value_tail":
        idx, val = _exact(s[:8], 10)
        val[9] = 0.0
    n = 8 if mistake in ("bad_tail", "value_tail") else 50
    with pytest.raises(AssertionError):
        check_row(idx, val, s[:n], 10, TOL)


def test_tie_inside_band_is_accepted():
    s = np.array([5.0, 4.0, 3.0, 3.0 + 1e-7, 1.0])
    # the exact answer for k = 3 keeps key 3 (3 + 1e-7); key 2 is within the band
    check_row(np.array([0, 1, 2]), np.array([5.0, 4.0, 3.0]), s, 3, TOL)
    with pytest.raises(AssertionError):   # key 4 is far below the k-th score
        check_row(np.array([0, 1, 4]), np.array([5.0, 4.0, 1.0]), s, 3, TOL)


def test_floor_follows_the_largest_magnitude():
    """A row whose scores are all <= 0 (a single negative-weight head): values
    near zero get the floor of the largest magnitude, as float32 sums do."""
    s = np.array([0.0, 0.0, -0.002, -8.0, -16.0])
    idx = np.array([0, 1, 2])
    val = np.array([0.0, 0.0, -0.002 + 1e-4])   # 5% off a near-zero score, 6e-6 of M
    check_row(idx, val, s, 3, 2e-2)
    with pytest.raises(AssertionError):       # an error well above the floor still fails
        check_row(idx, np.array([0.0, 0.0, -0.002 + 0.01]), s, 3, 2e-2)


def test_float32_error_budget():
    """Values within budget * 2^-24 * P_j of the exact score pass; a value off
    by more fails although it is well inside the tolerance; the largest error
    is recorded in units of 2^-24 P_j."""
    from tests.checker import U32, RowStats
    s = _scores(3)
    p = np.abs(s) * 3 + 1.0
    idx, val = _exact(s, 10)
    head = idx[:10]
    st = RowStats()
    ok = val.copy()
    ok[:10] = s[head] + 100 * U32 * p[head]
    check_row(idx, ok, s, 10, TOL, mag=p, budget=392, stats=st)
    assert 99 < st.max_err_u < 101
    bad = val.copy()
    bad[3] = s[head[3]] + 500 * U32 * p[head[3]]
    assert abs(bad[3] - s[head[3]]) < TOL * abs(s[head[3]])
    with pytest.raises(AssertionError):
        check_row(idx, bad, s, 10, TOL, mag=p, budget=392)


def test_cancellation_residue_row_uses_the_budget():
    """A row whose every score is a residue of cancelling terms (largest
    magnitude 4e-5 from terms summing to 49 in magnitude; float32 resolves
    49 * 2^-24 = 2.9e-6 there): a value off by 6.7e-8 fails the relative band
    with its floor (1e-3 * max(|s|, 2^-6 M) = 3.9e-8) but lies within 0.03 units
    of 2^-24 P_j and passes; off by more than the budget it still fails."""
    from tests.checker import U32, RowStats
    s = np.array([0.0, -3.889e-5, -3.95e-5, -4.0e-5])
    p = np.full(4, 49.0)
    idx = np.array([0, 1, 2, 3])
    val = s.copy()
    val[1] += 6.7e-8
    st = RowStats()
    check_row(idx, val, s, 4, TOL, mag=p, budget=266, stats=st)
    assert st.budget_val == 1
    with pytest.raises(AssertionError):   # without the budget the band alone rejects it
        check_row(idx, val, s, 4, TOL)
    bad = s.copy()
    bad[3] -= 300 * U32 * 49.0            # still the smallest value: only the budget fails
    with pytest.raises(AssertionError, match="budget|values off"):
        check_row(idx, bad, s, 4, TOL, mag=p, budget=266)
