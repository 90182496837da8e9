"""GPU-vs-oracle acceptance rule for one indexer output row.

Let s be the oracle's float64 scores of the row's visible keys (n of them),
m = min(k, n), s_(k) the k-th largest score, M = max_j |s_j| the row's
largest score magnitude, and tau = tol * max(|s_(k)|, 2^-6 * M) (tol = 1e-3
for fp16/bf16 inputs, 2e-2 for fp8/int8). The floor 2^-6 * M keeps the band
from vanishing near zero: the GPU sums the head dot products in float32, so
its error scales with the row's magnitudes, not with a score that cancels to
about zero (a row whose weights are all negative has every score <= 0, its
largest score is 0, and only M gives the scale). The GPU row G is accepted iff
  1. its first m entries are distinct visible keys and the rest are -1;
  2. every j in G has s_j >= s_(k) - tau;
  3. every visible j with s_j > s_(k) + tau is in G;
  4. consecutive entries are ordered by score within tau;
  5. returned values v_j satisfy |v_j - s_j| <= tol * max(|s_j|, 2^-6 M),
     are non-increasing, and the tail holds -inf.
Rules 2-3 make G equal the oracle's set whenever s_(k) and s_(k+1) are more
than tau apart; inside that band any choice whose oracle score is within tau
of the k-th is accepted. Rows that see at most k keys must return all of them.

Beside the tolerance, when the oracle's per-key magnitudes P_j (the sum of the
absolute values of the products in s_j) and an error budget c are given, every
returned value must also satisfy |v_j - s_j| <= c * 2^-24 * P_j: the forward
error bound of float32 dot products and sums, whatever their order. A GPU whose
values meet it computes the formula to float32 accuracy, so neither the
tolerance nor its floor is doing the work for the values.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

TOL = {"f16": 1e-3, "bf16": 1e-3, "e4m3fn": 2e-2, "i8": 2e-2}


def visible(wl, b: int, i: int) -> int:
    """Visible keys of row i of batch b, by the oracle's rule (0 past S_q)."""
    from oracle import li_oracle as O
    sq, sk = O.batch_lengths(wl)[b]
    return O.visible_count(i, sq, sk, wl.sparse_mode, *O.compression(wl, b))


def visible_pairs(wl) -> int:
    """Sum of the visible keys over all rows, by the oracle's rule."""
    from oracle import li_oracle as O
    tot = 0
    for b, (sq, sk) in enumerate(O.batch_lengths(wl)):
        cr, res = O.compression(wl, b)
        tot += sum(O.visible_count(i, sq, sk, wl.sparse_mode, cr, res) for i in range(sq))
    return tot


U32 = 2.0 ** -24   # float32 unit roundoff


def err_budget(wl) -> float:
    """Error budget c (in units of 2^-24 * P_j) of a float32 evaluation of the
    formula: D-term dot products, an N1-term head sum and a few scale and
    output roundings, doubled to cover any rounding mode of the accumulators.
    For e4m3fn the dot-product term is 8 D: the fp8 matrix instruction sums
    each step's 64 products in one fused operation that keeps fewer low bits of
    the smaller products than a float32 sum would (measured on the GPU: up to
    368 * 2^-24 P_j for D = 64 and one head, against 0.5 for the 16-bit types;
    exact on inputs whose products share a narrow exponent range, e4m3fn
    subnormal codes included)."""
    a = 8 if wl.qk_dtype == "e4m3fn" else 1
    return 2.0 * (a * wl.D + wl.N1 // wl.N2 + 4)


class RowStats:
    """Counts over the checked rows, plus two guards on the band floor:
    max_err_u, the largest |v_j - s_j| / (2^-24 P_j) over every returned value
    (bounded by the error budget when one is given), max_err_m, the same error
    over the row's largest score magnitude M, and the rows that would fail if
    the floor 2^-6 M were dropped (tau = tol * |s_(k)|): floor_sel for the
    selection (rules 2-4), floor_val for the values (rule 5; a value near zero
    whose terms cancel has a large error relative to itself, which the float32
    budget above bounds instead), and budget_val: values outside even the
    floored relative band but inside the float32 budget, i.e. scores that are
    cancellation residues finer than float32 resolves at the size of their own
    terms (a row whose largest magnitude M is itself such a residue)."""

    def __init__(self):
        self.rows = 0
        self.exact_set = 0
        self.in_band = 0
        self.all_keys = 0
        self.max_err_u = 0.0
        self.max_err_m = 0.0
        self.floor_sel = 0
        self.floor_val = 0
        self.budget_val = 0

    def __repr__(self):
        return (f"rows={self.rows} exact_set={self.exact_set} tie_band={self.in_band} "
                f"all_keys={self.all_keys} max_err/(u*P)={self.max_err_u:.3g} "
                f"max_err/M={self.max_err_m:.3g} floor_sel={self.floor_sel} "
                f"floor_val={self.floor_val} budget_val={self.budget_val}")


def check_row(gidx: np.ndarray, gval: Optional[np.ndarray], s: np.ndarray, k: int,
              tol: float, oidx: Optional[np.ndarray] = None,
              stats: Optional[RowStats] = None, where: str = "",
              mag: Optional[np.ndarray] = None, budget: Optional[float] = None) -> None:
    n = s.shape[0]
    m = min(k, n)
    gidx = np.asarray(gidx).astype(np.int64)
    assert gidx.shape == (k,), f"{where}: bad row shape {gidx.shape}"
    head, tail = gidx[:m], gidx[m:]
    assert (tail == -1).all(), f"{where}: tail must be -1 (m={m}), got {tail[:8]}"
    assert ((head >= 0) & (head < n)).all(), \
        f"{where}: index outside [0,{n}): {head[(head < 0) | (head >= n)][:8]}"
    assert np.unique(head).shape[0] == m, f"{where}: duplicate indices"
    if stats is not None:
        stats.rows += 1
    if m == 0:
        if gval is not None:
            assert np.isneginf(gval).all(), f"{where}: values of an empty row must be -inf"
        return
    srt = np.sort(s)[::-1]
    s1 = np.abs(s).max()
    floor = 2.0 ** -6 * s1
    needs_sel = needs_val = False
    if n <= k:
        assert np.array_equal(np.sort(head), np.arange(n)), f"{where}: must return every key"
        tau = tol * max(abs(srt[-1]), floor)
        if stats is not None:
            stats.all_keys += 1
    else:
        sk = srt[k - 1]
        tau = tol * max(abs(sk), floor)
        sel = s[head]
        bad = sel < sk - tau
        assert not bad.any(), f"{where}: picked keys below the k-th score band: " \
                              f"{head[bad][:5]} s={sel[bad][:5]} kth={sk} tau={tau}"
        must = np.nonzero(s > sk + tau)[0]
        missing = np.setdiff1d(must, head)
        assert missing.size == 0, f"{where}: missing clear winners {missing[:5]}"
        tau0 = tol * abs(sk)
        needs_sel |= bool((sel < sk - tau0).any())
        needs_sel |= np.setdiff1d(np.nonzero(s > sk + tau0)[0], head).size > 0
        if stats is not None:
            if oidx is not None and np.array_equal(np.sort(head), np.sort(oidx[:m])):
                stats.exact_set += 1
            else:
                stats.in_band += 1
    # ordering by score (within the band width)
    sh = s[head]
    band = tol * np.maximum(np.abs(sh), floor)
    assert (sh[1:] <= sh[:-1] + band[:-1] + band[1:]).all(), f"{where}: not sorted by score"
    band0 = tol * np.abs(sh)
    needs_sel |= not (sh[1:] <= sh[:-1] + band0[:-1] + band0[1:]).all()
    if gval is not None:
        gval = np.asarray(gval, dtype=np.float64)
        v, vt = gval[:m], gval[m:]
        assert np.isneginf(vt).all(), f"{where}: value tail must be -inf"
        err = np.abs(v - sh)
        lim = tol * np.maximum(np.abs(sh), floor)
        if mag is not None and budget is not None:
            # A value within the float32 error bound of its own terms is accepted
            # where the relative band is finer than float32 resolves.
            blim = budget * U32 * np.asarray(mag, np.float64)[head]
            if stats is not None and ((err > lim) & (err <= blim)).any():
                stats.budget_val += 1
            lim = np.maximum(lim, blim)
        assert (err <= lim).all(), f"{where}: values off by up to {err.max():.3g} " \
                                   f"(limit {lim[np.argmax(err - lim)]:.3g})"
        assert (np.diff(v) <= 0).all(), f"{where}: values not non-increasing"
        needs_val |= bool((err > tol * np.abs(sh)).any())
        if mag is not None:
            pm = np.asarray(mag, np.float64)[head]
            eu = np.where(pm > 0, err / (U32 * np.where(pm > 0, pm, 1.0)),
                          np.where(err > 0, np.inf, 0.0))
            if budget is not None:
                bad = eu > budget
                assert not bad.any(), f"{where}: values off by {eu.max():.3g} * 2^-24 P_j " \
                                      f"(budget {budget}) at keys {head[bad][:5]}"
            if stats is not None:
                stats.max_err_u = max(stats.max_err_u, float(eu.max()))
        if stats is not None and s1 > 0:
            stats.max_err_m = max(stats.max_err_m, float(err.max() / s1))
    if stats is not None:
        stats.floor_sel += int(needs_sel)
        stats.floor_val += int(needs_val)


def check_rows(gidx_rows: np.ndarray, gval_rows: Optional[np.ndarray], oracle_out: dict,
               k: int, tol: float, label: str = "", offsets=None,
               budget: Optional[float] = None) -> RowStats:
    """gidx_rows / gval_rows: (R, N2, k) arrays aligned with oracle_out['rows'].

    offsets: per-batch output_idx_offset (or None); returned indices must be the
    key index plus the offset, -1 slots stay -1, and the rule is then applied to
    the key indices. budget: the float32 error budget (err_budget) the values
    are held to against the oracle's magnitudes, when it returned them."""
    st = RowStats()
    for r, (b, i) in enumerate(oracle_out["rows"]):
        for h in range(gidx_rows.shape[1]):
            g = np.asarray(gidx_rows[r, h]).astype(np.int64)
            o = np.asarray(oracle_out["indices"][r, h]).astype(np.int64)
            if offsets is not None:
                off = int(offsets[b])
                valid = g >= 0
                assert (g[valid] >= off).all(), f"{label} row (b={b}, i={i}): offset not applied"
                assert (g[~valid] == -1).all()
                g = np.where(valid, g - off, g)
                o = np.where(o >= 0, o - off, o)
            gv = None if gval_rows is None else np.asarray(gval_rows[r, h], np.float64)
            sc = oracle_out["scores"][r][h]
            mg = oracle_out["mags"][r][h] if "mags" in oracle_out else None
            where = f"{label} row (b={b}, i={i})"
            f = int(oracle_out["kept"][r, h]) if "kept" in oracle_out else 0
            if f:
                g, gv, sc, o, k_rest, mg = _split_kept(g, gv, sc, o, f, k, tol, where, mg, budget)
            else:
                k_rest = k
            check_row(g, gv, sc, k_rest, tol, oidx=o, stats=st, where=where, mag=mg,
                      budget=budget)
    return st


def _split_kept(g, gv, s, o, f, k, tol, where, mag=None, budget=None):
    """Rows with blocks that are always kept: the first f slots must equal the
    oracle's (an index rule, no scores involved), their values within the
    tolerance; the remaining slots are then checked by the rule above over the
    other blocks, renumbered."""
    assert np.array_equal(g[:f], o[:f]), f"{where}: kept blocks {g[:f]} != {o[:f]}"
    floor = 2.0 ** -6 * np.abs(s).max()
    if gv is not None:
        err = np.abs(gv[:f] - s[g[:f]])
        lim = tol * np.maximum(np.abs(s[g[:f]]), floor)
        if mag is not None and budget is not None:   # as in check_row
            lim = np.maximum(lim, budget * U32 * np.asarray(mag, np.float64)[g[:f]])
        assert (err <= lim).all(), f"{where}: kept block values off by {err.max():.3g}"
        if mag is not None and budget is not None:
            assert (err <= budget * U32 * np.asarray(mag)[g[:f]]).all(), \
                f"{where}: kept block values outside the float32 error budget"
    rest = np.setdiff1d(np.arange(s.shape[0]), g[:f])
    pos = np.full(s.shape[0], -2, np.int64)
    pos[rest] = np.arange(rest.shape[0])
    def renum(x):
        x = x[f:]
        return np.where(x >= 0, pos[np.clip(x, 0, s.shape[0] - 1)], x)
    gr = renum(g)
    assert (gr != -2).all(), f"{where}: a kept block is returned twice"
    return (gr, (None if gv is None else gv[f:]), s[rest], renum(o), k - f,
            None if mag is None else np.asarray(mag)[rest])
