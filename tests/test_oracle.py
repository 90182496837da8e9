"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself.

Each test names what it pins: the IEEE/OCP field decoders (exhaustive against
library routines and closed forms), hand-worked examples of the formula
(tests/golden/hand_examples.json), brute force over all key subsets,
closed forms for special shapes, and invariants the formula implies.
"""
import itertools
import json
import math
import os
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import li_oracle as O
from sparse_attention_top_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")

# e4m3fn codes of the small integers used by the hand examples, written out
# from the field layout (sign | 4-bit exponent, bias 7 | 3-bit fraction).
_E4M3_CODE = {0.0: 0x00, 1.0: 0x38, 2.0: 0x40, 3.0: 0x44, -1.0: 0xB8, -2.0: 0xC0,
              30.0: 0x5F}


# ---------------------------------------------------------------------------
# decoders
# ---------------------------------------------------------------------------
def test_decode_f16_exhaustive_matches_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.decode_f16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_decode_f16_closed_forms():
    cases = {0x3C00: 1.0, 0x0001: 2.0 ** -24, 0x0400: 2.0 ** -14, 0x7BFF: 65504.0,
             0xC000: -2.0, 0x3555: 0.25 * (1 + 0x155 / 1024),
             0x7C00: math.inf, 0xFC00: -math.inf}
    for b, v in cases.items():
        assert O.decode_f16(np.array([b], np.uint16))[0] == v, hex(b)
    assert math.isnan(O.decode_f16(np.array([0x7E00], np.uint16))[0])
    z = O.decode_f16(np.array([0x8000], np.uint16))[0]
    assert z == 0.0 and math.copysign(1.0, z) < 0


def test_decode_bf16_exhaustive_matches_binary32_top_half():
    bits = np.arange(1 << 16, dtype=np.uint32)
    ours = O.decode_bf16(bits.astype(np.uint16))
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    tref = torch.from_numpy(bits.astype(np.int32).astype(np.int16)).view(torch.bfloat16)
    tref = tref.double().numpy()
    assert np.array_equal(ours[ok], tref[ok])


def test_decode_e4m3fn_exhaustive_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.isnan(ours).sum() == 2                     # S.1111.111 only
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_decode_e4m3fn_closed_forms():
    cases = {0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x38: 1.0, 0x44: 3.0, 0xC0: -2.0, 0x5F: 30.0, 0xFE: -448.0}
    for c, v in cases.items():
        assert O.decode_e4m3fn(np.array([c], np.uint8))[0] == v, hex(c)
    assert math.isnan(O.decode_e4m3fn(np.array([0x7F], np.uint8))[0])
    assert math.isnan(O.decode_e4m3fn(np.array([0xFF], np.uint8))[0])
    assert np.isfinite(O.decode_e4m3fn(np.arange(256, dtype=np.uint8))).sum() == 254


def test_decode_i8():
    c = np.arange(-128, 128, dtype=np.int8)
    assert np.array_equal(O.decode_i8(c), np.arange(-128, 128, dtype=np.float64))


# ---------------------------------------------------------------------------
# visibility rule
# ---------------------------------------------------------------------------
def test_visible_count_rules():
    # mode 0: every key of the sequence
    assert [O.visible_count(i, 3, 7, 0) for i in range(4)] == [7, 7, 7, 0]
    # mode 3, S_k >= S_q: j <= i + S_k - S_q  -> i + 1 + (S_k - S_q) keys
    assert [O.visible_count(i, 3, 7, 3) for i in range(3)] == [5, 6, 7]
    # square causal: row i sees i + 1 keys
    assert [O.visible_count(i, 4, 4, 3) for i in range(4)] == [1, 2, 3, 4]
    # S_q > S_k: the first S_q - S_k rows see nothing
    assert [O.visible_count(i, 5, 2, 3) for i in range(5)] == [0, 0, 0, 1, 2]
    with pytest.raises(ValueError):
        O.visible_count(0, 1, 1, 1)


def _visible_by_tokens(i, sq, sk, r, res):
    """Compressed visibility counted from its definition: compressed key j
    stands for original tokens j*r .. j*r + r - 1 of a sequence of sk*r + res
    tokens, and is visible when every one of them is visible to row i under the
    plain right-down rule t <= i + L - S_q."""
    L = sk * r + res
    return sum(all(t <= i + L - sq for t in range(j * r, j * r + r)) for j in range(sk))


def test_visible_count_compressed_matches_token_definition():
    for r in (1, 2, 3, 4, 8):
        for res in range(r):
            for sk in (0, 1, 2, 5, 9):
                for sq in (1, 2, 4, 7, 20, 45):
                    for i in range(sq):
                        assert O.visible_count(i, sq, sk, 3, r, res) == \
                            _visible_by_tokens(i, sq, sk, r, res), (i, sq, sk, r, res)
                        assert O.visible_count(i, sq, sk, 0, r, res) == sk


def test_visible_count_compressed_pages_example():
    """The V2 guide's example: S2 = 130 original keys, cmp_ratio 4, so 32
    compressed keys and residual 2, with S1 = 64 queries in mask mode 3. The
    last query row stands at the last original token and sees every compressed
    key; counts never decrease down the rows."""
    counts = [O.visible_count(i, 64, 130 // 4, 3, 4, 130 % 4) for i in range(64)]
    assert counts[-1] == 32
    assert all(a <= b for a, b in zip(counts, counts[1:]))
    # row 0 stands at original position 66: tokens 0..63 are complete keys 0..15
    assert counts[0] == 16


def test_output_offset_shifts_valid_indices_only():
    case = dict(next(c for c in _CASES if c["name"] == "C_causal"))
    base = O.run(_hand_workload(case))
    wl = _hand_workload(case)
    wl.output_idx_offset = np.array([7], np.int32)
    shifted = O.run(wl)
    bi, si = base["indices"], shifted["indices"]
    assert (si[bi < 0] == -1).all() and (bi < 0).any()
    assert np.array_equal(si[bi >= 0], bi[bi >= 0] + 7)
    assert np.array_equal(base["values"], shifted["values"])


# ---------------------------------------------------------------------------
# hand-worked examples
# ---------------------------------------------------------------------------
def _enc(vals, dtype):
    a = np.asarray(vals, np.float64)
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    if dtype == "e4m3fn":
        return np.vectorize(lambda v: _E4M3_CODE[float(v)], otypes=[np.uint8])(a)
    if dtype == "i8":
        return a.astype(np.int8)
    raise ValueError(dtype)


def _hand_workload(case):
    dt = case["dtype"]
    rows = case["rows"]
    G = len(rows[0]["q"])
    D = len(rows[0]["q"][0])
    quant = dt in ("e4m3fn", "i8")
    ns = SimpleNamespace(N1=G, N2=1, D=D, qk_dtype=dt, w_dtype="f32",
                         sparse_count=case["k"], sparse_mode=case["mode"],
                         q_scale=None, k_scale=None, cu_seqlens_q=None, cu_seqlens_k=None,
                         seqused_q=None, seqused_k=None, block_table=None)
    qv = np.array([r["q"] for r in rows], np.float64)
    wv = np.array([r["w"] for r in rows], np.float32)
    if case["layout"] == "TND":
        ns.B = len(case["cu_seqlens_q"]) - 1
        ns.layout_q = ns.layout_k = "TND"
        ns.cu_seqlens_q = np.array(case["cu_seqlens_q"], np.int32)
        ns.cu_seqlens_k = np.array(case["cu_seqlens_k"], np.int32)
        for f in ("seqused_q", "seqused_k"):   # TND padding
            if f in case:
                setattr(ns, f, np.array(case[f], np.int32))
        ns.q = _enc(qv, dt)
        ns.w = wv
        ns.k = _enc(np.array(case["keys"])[:, None, :], dt)
        return ns
    ns.cmp_ratio = case.get("cmp_ratio", 1)
    ns.cmp_residual_k = (np.array(case["cmp_residual_k"], np.int32)
                         if "cmp_residual_k" in case else None)
    ns.output_idx_offset = (np.array(case["output_idx_offset"], np.int32)
                            if "output_idx_offset" in case else None)
    ns.block_len = case.get("block_len", 1)
    ns.init_num = case.get("init_num", 0)
    ns.local_num = case.get("local_num", 0)
    ns.B = 1
    ns.layout_q = "BSND"
    ns.q = _enc(qv[None], dt)
    ns.w = wv[None]
    if quant:
        ns.q_scale = np.array([[r["q_scale"] for r in rows]], np.float32)
    if case["layout"] == "PA":
        ns.layout_k = "PA_BSND"
        ns.k = _enc(np.array(case["key_cache"])[:, :, None, :], dt)
        ns.block_table = np.array(case["block_table"], np.int32)
        ns.seqused_k = np.array([case["S_k"]], np.int32)
    else:
        ns.layout_k = "BSND"
        ns.k = _enc(np.array(case["keys"])[None, :, None, :], dt)
        if quant:
            ns.k_scale = np.array(case["key_scale"], np.float32)[None, :, None]
    return ns


def _expected(vals):
    return np.array([[-np.inf if v == "-inf" else v for v in r] for r in vals], np.float32)


with open(GOLDEN) as _f:
    _CASES = json.load(_f)["cases"]


@pytest.mark.parametrize("case", _CASES, ids=[c["name"] for c in _CASES])
def test_hand_examples(case):
    wl = _hand_workload(case)
    o = O.run(wl)
    idx = o["indices"][:, 0, :]
    val = o["values"][:, 0, :]
    assert idx.tolist() == case["expected_indices"]
    assert np.array_equal(val, _expected(case["expected_values"]))


def test_hand_example_scores_without_scales_differ():
    """Dropping the dequant scales changes example E's order: the scales are live."""
    case = dict(next(c for c in _CASES if c["name"] == "E_fp8_scales"))
    wl = _hand_workload(case)
    wl.q_scale = np.ones_like(wl.q_scale)
    wl.k_scale = np.ones_like(wl.k_scale)
    assert O.run(wl)["indices"][0, 0].tolist() == [1, 0, 2, 3]


# ---------------------------------------------------------------------------
# brute force over key subsets (selection and ordering)
# ---------------------------------------------------------------------------
def _brute_force(scores, k):
    """Best subset of size m = min(k, n): the one whose descending score list is
    lexicographically largest; among equals, whose ascending index list is
    lexicographically smallest. Returned in (score desc, index asc) order."""
    n = len(scores)
    m = min(k, n)
    best_key, best = None, None
    for sub in itertools.combinations(range(n), m):
        vals = sorted((scores[j] for j in sub), reverse=True)
        key = (tuple(vals), tuple(-j for j in sub))
        if best_key is None or key > best_key:
            best_key, best = key, sub
    return sorted(best, key=lambda j: (-scores[j], j))


def _py_scores(q, w, keys):
    """Row scores with explicit Python loops over heads and the head dim."""
    out = []
    for kv in keys:
        s = 0.0
        for g in range(len(q)):
            dot = sum(float(a) * float(b) for a, b in zip(q[g], kv))
            s += float(w[g]) * max(dot, 0.0)
        out.append(s)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_small(seed):
    rng = np.random.default_rng(1000 + seed)
    G, D, n = int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 10))
    k = int(rng.integers(1, 6))
    integer = seed % 2 == 0                       # integer data makes exact ties
    if integer:
        q = rng.integers(-2, 3, (G, D)).astype(np.float64)
        keys = rng.integers(-2, 3, (n, D)).astype(np.float64)
        w = rng.integers(-2, 3, G).astype(np.float64)
    else:
        q = rng.standard_normal((G, D))
        keys = rng.standard_normal((n, D))
        w = rng.standard_normal(G)
    s = O.row_scores(q, w, keys)
    assert np.allclose(s, _py_scores(q, w, keys), rtol=0, atol=1e-12)
    order = O.topk_order(s, k)
    assert list(order) == _brute_force(list(s), k)


@pytest.mark.parametrize("seed", range(16))
def test_block_selection_brute_force(seed):
    """Key blocks with kept sink / local blocks, against independent forms: block
    scores by numpy's reduceat (max over each block's keys), the kept blocks as a
    set membership test, and the rest by brute force over block subsets."""
    rng = np.random.default_rng(2000 + seed)
    n = int(rng.integers(1, 13))
    L = int(rng.integers(1, 5))
    s = rng.integers(-3, 4, n).astype(np.float64) if seed % 2 == 0 else rng.standard_normal(n)
    sb = O.block_scores(s, L)
    assert np.array_equal(sb, np.maximum.reduceat(s, np.arange(0, n, L)))
    nb = sb.shape[0]
    init_num, local_num = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    k = int(rng.integers(max(1, init_num + local_num), nb + 3))
    order, kept = O.select_blocks(sb, k, init_num, local_num)
    must = [c for c in range(nb) if c < init_num or c >= nb - local_num]
    assert kept == len(must) and list(order[:kept]) == must
    rest = [c for c in range(nb) if c not in must]
    best = _brute_force([sb[c] for c in rest], k - kept)
    assert list(order[kept:]) == [rest[t] for t in best]
    assert len(set(order.tolist())) == order.shape[0] == min(k, nb)


def test_blocks_of_one_reduce_to_the_plain_selection():
    """block_len 1 without kept blocks is the token top-k itself."""
    rng = np.random.default_rng(21)
    s = rng.integers(-4, 5, 60).astype(np.float64)
    assert np.array_equal(O.block_scores(s, 1), s)
    order, kept = O.select_blocks(s, 17, 0, 0)
    assert kept == 0 and np.array_equal(order, O.topk_order(s, 17))


def test_kept_blocks_win_over_higher_scores():
    """Kept blocks are returned even when every other block scores higher."""
    sb = np.array([-5.0, 9, 8, 7, 6, -4])
    order, kept = O.select_blocks(sb, 3, 1, 1)
    assert kept == 2 and order.tolist() == [0, 5, 1]


# ---------------------------------------------------------------------------
# closed forms and library special cases
# ---------------------------------------------------------------------------
def test_single_positive_head_is_topk_of_matvec():
    """G=1, W=1, q and keys entrywise positive: every dot is positive, so the
    score is the mat-vec K.q and the result is torch.topk of it."""
    rng = np.random.default_rng(7)
    q = rng.uniform(0.1, 1.0, (1, 16))
    keys = rng.uniform(0.1, 1.0, (300, 16))
    s = O.row_scores(q, np.ones(1), keys)
    tv, ti = torch.topk(torch.from_numpy(keys @ q[0]), 37, largest=True, sorted=True)
    order = O.topk_order(s, 37)
    assert order.tolist() == ti.tolist()
    assert np.allclose(s[order], tv.numpy(), rtol=1e-15)


def test_head_dim_one_closed_form():
    """D=1: s_j = k_j * sum_g W_g max(q_g,0) for k_j>0, |k_j| * sum_g W_g max(-q_g,0) for k_j<0."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((6, 1))
    w = rng.standard_normal(6)
    keys = rng.standard_normal((50, 1))
    s = O.row_scores(q, w, keys)
    pos = (w * np.maximum(q[:, 0], 0)).sum()
    neg = (w * np.maximum(-q[:, 0], 0)).sum()
    kj = keys[:, 0]
    closed = np.where(kj > 0, kj * pos, -kj * neg)
    assert np.allclose(s, closed, rtol=1e-13, atol=1e-15)


def test_exact_on_integer_inputs():
    """Small integers and power-of-two weights: float64 scores are exact, so they
    equal exact rational arithmetic."""
    rng = np.random.default_rng(9)
    G, D, n = 5, 9, 40
    q = rng.integers(-3, 4, (G, D))
    keys = rng.integers(-3, 4, (n, D))
    w = rng.integers(-8, 9, G) / 4.0
    s = O.row_scores(q.astype(float), w, keys.astype(float))
    for j in range(n):
        exact = sum(Fraction(w[g]) * max(0, int(q[g] @ keys[j])) for g in range(G))
        assert Fraction(s[j]) == exact


def test_matches_tensor_formulation_with_torch():
    """The same result from a whole-tensor formulation (batched einsum over
    b,s,g,d / b,t,d, ReLU, weight, sum over g, torch.topk sorted) in float64."""
    wl = synth.build("t", layout_q="BSND", layout_k="BSND", qk_dtype="f16", w_dtype="f32",
                     N1=4, D=8, seqlens_q=[6, 6], seqlens_k=[23, 23], sparse_count=5,
                     sparse_mode=0, seed=11)
    q = torch.from_numpy(O.decode(wl.q, "f16"))[:, :, :, :]        # b s g d
    k = torch.from_numpy(O.decode(wl.k, "f16"))[:, :, 0, :]        # b t d
    w = torch.from_numpy(wl.w.astype(np.float64))                  # b s g
    x = torch.einsum("bsgd,btd->bsgt", q, k).relu()
    s = (x * w[..., None]).sum(dim=2)                               # b s t
    tv, _ = torch.topk(s, 5, dim=-1, largest=True, sorted=True)
    o = O.run(wl)
    val = o["values"].reshape(2, 6, 5)
    assert np.allclose(val, tv.numpy().astype(np.float32), rtol=0, atol=0)
    idx = o["indices"].reshape(2, 6, 5)
    got = np.take_along_axis(s.numpy(), idx.astype(np.int64), axis=-1)
    assert np.array_equal(got.astype(np.float32), tv.numpy().astype(np.float32))


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def _small(seed, **kw):
    base = dict(layout_q="BSND", layout_k="BSND", qk_dtype="bf16", w_dtype="f32", N1=8, D=16,
                seqlens_q=[40], seqlens_k=[70], sparse_count=9, sparse_mode=3, seed=seed)
    base.update(kw)
    return synth.build("small", **base)


def _check_structure(wl, o):
    lengths = O.batch_lengths(wl)
    for r, (b, i) in enumerate(o["rows"]):
        sq, sk = lengths[b]
        n = O.visible_count(i, sq, sk, wl.sparse_mode)
        m = min(n, wl.sparse_count)
        row = o["indices"][r, 0]
        vals = o["values"][r, 0]
        assert (row[:m] >= 0).all() and (row[:m] < n).all()
        assert len(set(row[:m].tolist())) == m
        assert (row[m:] == -1).all()
        assert np.isneginf(vals[m:]).all() and np.isfinite(vals[:m]).all()
        assert (np.diff(vals[:m]) <= 0).all()


@pytest.mark.parametrize("mode", [0, 3])
def test_structure_and_mask(mode):
    wl = _small(21, sparse_mode=mode, seqlens_q=[40, 33], seqlens_k=[70, 20], S1=40, S2=70)
    _check_structure(wl, O.run(wl))


def test_weight_scaling_invariance():
    wl = _small(22)
    o1 = O.run(wl)
    wl.w = (wl.w * np.float32(4.0)).astype(np.float32)
    o2 = O.run(wl)
    assert np.array_equal(o1["indices"], o2["indices"])
    fin = np.isfinite(o1["values"])
    assert np.array_equal(o1["values"][fin] * 4, o2["values"][fin])


def test_head_permutation_invariance():
    wl = _small(23)
    o1 = O.run(wl)
    perm = np.random.default_rng(0).permutation(wl.N1)
    wl.q = wl.q[:, :, perm]
    wl.w = wl.w[:, :, perm]
    o2 = O.run(wl)
    assert np.array_equal(o1["indices"], o2["indices"])
    assert np.allclose(o1["values"], o2["values"], rtol=1e-6)


def test_paged_equals_contiguous():
    """PA_BSND with a permuted block pool gives what BSND gives on the gathered keys."""
    pa = synth.build("pa", layout_q="BSND", layout_k="PA_BSND", qk_dtype="bf16", w_dtype="f32",
                     N1=8, D=16, seqlens_q=[3, 3, 3], seqlens_k=[50, 17, 64], sparse_count=12,
                     sparse_mode=3, block_size=16, seed=24)
    S2 = int(pa.seqlens_k.max())
    kc = np.full((pa.B, S2, 1, pa.D), 0, np.uint16)
    for b in range(pa.B):
        for j in range(int(pa.seqlens_k[b])):
            kc[b, j] = pa.k[pa.block_table[b, j // 16], j % 16]
    flat = SimpleNamespace(**{**pa.__dict__})
    flat.layout_k, flat.k, flat.block_table = "BSND", kc, None
    flat.seqused_k = pa.seqlens_k.copy()
    a, b = O.run(pa), O.run(flat)
    assert np.array_equal(a["indices"], b["indices"])
    assert np.array_equal(a["values"], b["values"])
    _check_structure(pa, a)


def test_varlen_equals_per_sequence():
    """TND output rows are the per-sequence BSND outputs, concatenated."""
    tnd = synth.build("tnd", layout_q="TND", layout_k="TND", qk_dtype="e4m3fn", w_dtype="f32",
                      N1=8, D=32, seqlens_q=[5, 30, 12], seqlens_k=[5, 30, 12],
                      sparse_count=7, sparse_mode=3, seed=25)
    o = O.run(tnd)
    for b in range(tnd.B):
        q0, q1 = tnd.cu_seqlens_q[b], tnd.cu_seqlens_q[b + 1]
        k0, k1 = tnd.cu_seqlens_k[b], tnd.cu_seqlens_k[b + 1]
        one = SimpleNamespace(B=1, layout_q="BSND", layout_k="BSND", qk_dtype=tnd.qk_dtype,
                              w_dtype="f32", N1=8, N2=1, D=32, sparse_count=7, sparse_mode=3,
                              q=tnd.q[None, q0:q1], k=tnd.k[None, k0:k1], w=tnd.w[None, q0:q1],
                              q_scale=tnd.q_scale[None, q0:q1], k_scale=tnd.k_scale[None, k0:k1],
                              cu_seqlens_q=None, cu_seqlens_k=None, seqused_q=None,
                              seqused_k=None, block_table=None)
        ob = O.run(one)
        assert np.array_equal(o["indices"][q0:q1], ob["indices"])
        assert np.array_equal(o["values"][q0:q1], ob["values"])
    _check_structure(tnd, o)


def test_short_rows_return_every_visible_key():
    """Rows with n_valid <= k involve no selection: every visible key, sorted."""
    wl = _small(26, sparse_count=64)
    o = O.run(wl, want_scores=True)
    checked = 0
    for r, (b, i) in enumerate(o["rows"]):
        n = O.visible_count(i, 40, 70, 3)
        if n > 64:
            continue
        checked += 1
        assert sorted(o["indices"][r, 0, :n].tolist()) == list(range(n))
        s = o["scores"][r][0]
        assert np.array_equal(o["values"][r, 0, :n], np.sort(s)[::-1].astype(np.float32))
    assert checked == 34


def test_padding_rows_past_seqused_q():
    wl = _small(27, seqlens_q=[10, 40], seqlens_k=[70, 70], S1=40)
    o = O.run(wl)
    idx = o["indices"].reshape(2, 40, 1, -1)
    assert (idx[0, 10:] == -1).all()
    assert (idx[0, :10, :, 0] >= 0).all()


def test_poisoned_padding_never_selected():
    """BSND keys past seqused_k hold +30 poison; they must never be chosen."""
    wl = _small(28, seqlens_q=[40], seqlens_k=[50], S2=70, sparse_mode=0)
    o = O.run(wl)
    assert o["indices"].max() < 50


@pytest.mark.parametrize("mode", [0, 3])
def test_tnd_padding_equals_unpadded(mode):
    """TND padding (V2 guide, constraint list): rows past seqused_q inside a
    sequence's cu_seqlens_q range come out all -1 / -inf, and the used rows
    equal the same problem packed without the padding (the causal rule takes
    the used lengths). Keys past seqused_k hold the +30 poison and are never
    chosen."""
    kw = dict(layout_q="TND", layout_k="TND", qk_dtype="bf16", w_dtype="f32", N1=8, D=32,
              seqlens_q=[12, 0, 7], seqlens_k=[30, 9, 7], sparse_count=6, sparse_mode=mode,
              seed=29)
    pad = synth.build("pad", padded_q=[20, 3, 7], padded_k=[40, 9, 11], **kw)
    o = O.run(pad)
    rows = 0
    for b in range(pad.B):
        q0 = int(pad.cu_seqlens_q[b])
        used, allotted = int(pad.seqused_q[b]), int(pad.cu_seqlens_q[b + 1]) - q0
        k0, sk = int(pad.cu_seqlens_k[b]), int(pad.seqused_k[b])
        assert (o["indices"][q0 + used:q0 + allotted] == -1).all()
        assert np.isneginf(o["values"][q0 + used:q0 + allotted]).all()
        if used == 0:
            continue
        one = SimpleNamespace(B=1, layout_q="TND", layout_k="TND", qk_dtype="bf16",
                              w_dtype="f32", N1=8, N2=1, D=32, sparse_count=6, sparse_mode=mode,
                              q=pad.q[q0:q0 + used], k=pad.k[k0:k0 + sk],
                              w=pad.w[q0:q0 + used], q_scale=None, k_scale=None,
                              cu_seqlens_q=np.array([0, used], np.int32),
                              cu_seqlens_k=np.array([0, sk], np.int32), seqused_q=None,
                              seqused_k=None, block_table=None)
        ob = O.run(one)
        assert np.array_equal(o["indices"][q0:q0 + used], ob["indices"])
        assert np.array_equal(o["values"][q0:q0 + used], ob["values"])
        assert o["indices"][q0:q0 + used].max() < sk
        rows += used
    assert rows == 19
    _check_structure(pad, o)


def test_row_magnitudes_hand_values():
    """P_j = sum_g |w_g| sum_d |q_gd k_jd| on the shared hand data: with Q = I
    the per-head absolute dots of K = [[1,1],[2,-1],[-1,3],[-2,-2]] are
    (1,2,1,2) and (1,1,3,2); W = (1, 0.5) gives (1.5, 2.5, 2.5, 3) and
    W = (1, -1) gives (2, 3, 4, 4). With scales Sq = (2, 1), Sk = (1, 0.5, 2, 1)
    and W = (1, 0.5): (2*1 + 0.5*1, 0.5*(2*2 + 0.5*1), 2*(2*1 + 0.5*3),
    2*2 + 0.5*2) = (2.5, 2.25, 7, 5)."""
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    k = np.array([[1.0, 1.0], [2.0, -1.0], [-1.0, 3.0], [-2.0, -2.0]])
    assert O.row_magnitudes(q, np.array([1.0, 0.5]), k).tolist() == [1.5, 2.5, 2.5, 3.0]
    assert O.row_magnitudes(q, np.array([1.0, -1.0]), k).tolist() == [2.0, 3.0, 4.0, 4.0]
    p = O.row_magnitudes(q, np.array([1.0, 0.5]), k, np.array([2.0, 1.0]),
                         np.array([1.0, 0.5, 2.0, 1.0]))
    assert p.tolist() == [2.5, 2.25, 7.0, 5.0]
    # terms that cancel inside a dot still count: Q = [[1,1],[1,-1]] against
    # keys (1,1) and (2,-1) has dots (2,1) and (0,3) but term sums (2,3), (2,3)
    q2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    assert O.row_magnitudes(q2, np.array([1.0, 1.0]), k[:2]).tolist() == [4.0, 6.0]


def test_row_magnitudes_bound_and_equality():
    """P_j >= |s_j| always (triangle inequality, and ReLU(x) <= |x|), with
    equality when every q, k and w is non-negative (no term cancels and the
    ReLU is the identity)."""
    rng = np.random.default_rng(41)
    q, k, w = rng.normal(size=(16, 32)), rng.normal(size=(50, 32)), rng.normal(size=16)
    qs, ks = rng.random(16), rng.random(50)
    s = O.row_scores(q, w, k, qs, ks)
    p = O.row_magnitudes(q, w, k, qs, ks)
    assert (p >= np.abs(s) * (1 - 1e-12)).all() and (p > np.abs(s) * 1.01).any()
    qa, ka, wa = np.abs(q), np.abs(k), np.abs(w)
    np.testing.assert_allclose(O.row_magnitudes(qa, wa, ka, qs, ks),
                               O.row_scores(qa, wa, ka, qs, ks), rtol=1e-13)
