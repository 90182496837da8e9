"""The plain C++17 fp64 oracle (oracle/li_oracle.cpp) against the numpy oracle.

The two are written independently (decoders, gathers, visibility, selection)
and check each other: every hand-worked example and seeded random problems
spanning every layout, dtype, mask mode, compressed keys, index offsets, TND
padding, key blocks and kept blocks must give the same indices, and values
that agree to the last float32 bit (both sum in float64; only the order of the
sums differs). The thread count does not change the result.
"""
import numpy as np
import pytest

from oracle import li_oracle as O
from oracle import liref
from sparse_attention_top_amd import synth
from tests import test_oracle as PINS


@pytest.fixture(scope="module", autouse=True)
def _built():
    liref.build()


def _compare(wl, rows=None, exact_values=False):
    o = O.run(wl, rows=rows)
    ci, cv, used = liref.run(wl, rows=rows)
    assert used >= 1
    assert np.array_equal(ci, o["indices"]), "indices differ between the two oracles"
    ov = o["values"]
    assert np.array_equal(np.isneginf(cv), np.isneginf(ov))
    fin = np.isfinite(ov)
    if exact_values:
        assert np.array_equal(cv[fin], ov[fin])
    else:
        # float64 sums in another order: at most one float32 ulp apart
        ulp = np.spacing(np.abs(ov[fin]).astype(np.float32))
        assert (np.abs(cv[fin].astype(np.float64) - ov[fin]) <= ulp).all()
    return ci


@pytest.mark.parametrize("case", PINS._CASES, ids=[c["name"] for c in PINS._CASES])
def test_hand_examples_agree(case):
    wl = PINS._hand_workload(case)
    ci = _compare(wl, exact_values=True)
    assert ci[:, 0, :].tolist() == case["expected_indices"]


def _random_problem(seed):
    rng = np.random.default_rng(500 + seed)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    layout = pick(["BSND", "TND", "PA", "TNDPAD", "TND_PA"])
    B = int(rng.integers(1, 4))
    sk = [int(x) for x in rng.integers(0, 300, B)]
    sq = [int(rng.integers(0, 40)) for _ in range(B)]
    if sum(sq) == 0:
        sq[0] = 3
    if sum(sk) == 0:
        sk[0] = 9
    mode = pick([0, 3])
    kw = dict(qk_dtype=pick(["f16", "bf16", "e4m3fn", "i8"]), w_dtype=pick(["f16", "bf16", "f32"]),
              N1=pick([1, 4, 16]), D=pick([8, 32]), seqlens_q=sq, seqlens_k=sk,
              sparse_count=pick([1, 5, 40, 300]), sparse_mode=mode)
    if layout == "BSND":
        kw.update(layout_q="BSND", layout_k="BSND", S1=max(sq) + 2, S2=max(sk) + 3)
    elif layout == "TND":
        kw.update(layout_q="TND", layout_k="TND")
    elif layout == "TNDPAD":
        kw.update(layout_q="TND", layout_k="TND",
                  padded_q=[s + int(rng.integers(0, 4)) for s in sq],
                  padded_k=[s + int(rng.integers(0, 4)) for s in sk])
    else:
        kw.update(layout_q="TND" if layout == "TND_PA" else "BSND", layout_k="PA_BSND",
                  block_size=pick([16, 32, 48]))
    if rng.random() < 0.3:
        r = pick([2, 4])
        kw["cmp_ratio"] = r
        if mode == 3:
            kw["cmp_residual_k"] = [int(x) for x in rng.integers(0, r, B)]
    if rng.random() < 0.3:
        kw["output_idx_offset"] = [int(x) for x in rng.integers(0, 1000, B)]
    if rng.random() < 0.3:
        kw["block_len"] = pick([2, 4, 16])
    if rng.random() < 0.3:
        kw["init_num"], kw["local_num"] = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        kw["sparse_count"] = max(kw["sparse_count"], kw["init_num"] + kw["local_num"])
    return synth.build(f"cpp{seed}", seed=seed, **kw)


@pytest.mark.parametrize("seed", range(40))
def test_random_problems_agree(seed):
    _compare(_random_problem(seed))


def test_row_subset_and_thread_count():
    """A subset of rows gives the rows of the full run; 1 thread and many agree."""
    wl = synth.build("sub", layout_q="TND", layout_k="TND", qk_dtype="bf16", w_dtype="bf16",
                     N1=8, D=32, seqlens_q=[30, 5, 50], seqlens_k=[30, 40, 50],
                     sparse_count=16, sparse_mode=3, seed=3)
    full_i, full_v, _ = liref.run(wl)
    one_i, one_v, used = liref.run(wl, nthreads=1)
    assert used == 1 and np.array_equal(full_i, one_i) and np.array_equal(full_v, one_v)
    rows = [(2, 49), (0, 0), (1, 4), (2, 7)]
    si, sv, _ = liref.run(wl, rows=rows)
    for r, (b, i) in enumerate(rows):
        assert np.array_equal(si[r], full_i[wl.row_of(b, i)])
        assert np.array_equal(sv[r], full_v[wl.row_of(b, i)])
    _compare(wl, rows=rows)
