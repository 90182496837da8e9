"""The split-row top-k is exact: a CPU model of it against a direct top-k.

For few rows and k <= 2048 the task table cuts each long row into chunks (the
chunk records of li_metadata, read back from the table here). The library then
takes every chunk's sorted top k (score descending, key index ascending), lays
the lists side by side in chunk order and selects the row's top k over the list
*positions* (score descending, position ascending), mapping each position back
to its key. This file models those two passes with numpy on rows full of equal
scores and checks the result against a direct top-k of the whole row: equal
scores must keep key order across chunk boundaries. CPU only; the GPU tests
compare the kernels' split and unsplit results bit for bit.
"""
import numpy as np
import pytest

from sparse_attention_top_amd import binding as B
from sparse_attention_top_amd import indexer as I
from sparse_attention_top_amd import synth


def _topk(scores, keys, k):
    """k best (score desc, key asc); returns positions into the arrays."""
    order = np.lexsort((keys, -scores))
    return order[:k]


def _split_plan(n, k):
    """Chunk starts of one row of n keys, read from li_metadata's table."""
    wl = synth.build("split_model", layout_q="TND", layout_k="TND", qk_dtype="bf16",
                     w_dtype="bf16", N1=8, D=64, seqlens_q=[1], seqlens_k=[n], sparse_count=k,
                     sparse_mode=0, seed=1)
    L = B.make_lengths(wl.cu_seqlens_q, wl.cu_seqlens_k)
    meta = B.li_metadata(I.problem_of(wl), L, 256)
    rows, _ = B.parse_row_table(meta)
    chunks = sorted(int(r["idx_offset"]) for r in rows if int(r["kind"]) == B.ROW_CHUNK)
    merges = [r for r in rows if int(r["kind"]) == B.ROW_MERGE]
    assert len(merges) == 1 and int(merges[0]["n"]) == len(chunks) * k
    return chunks + [n]


@pytest.mark.parametrize("n,k,levels,seed", [
    (8193, 2048, 3, 0), (16377, 2048, 5, 1), (40000, 512, 2, 2), (70000, 2048, 40, 3),
    (30000, 1, 1, 4), (20000, 300, 7, 5),
])
def test_split_selection_equals_whole_row(n, k, levels, seed):
    edges = _split_plan(n, k)
    assert all(e % 4 == 0 for e in edges[:-1])
    lens = np.diff(edges)
    assert (lens > k).all() and (lens <= 8192).all()
    rng = np.random.default_rng(seed)
    scores = rng.integers(0, levels, n).astype(np.float64)   # heavy ties
    keys = np.arange(n)
    # first pass: each chunk's sorted top k, lists side by side in chunk order
    cand_s, cand_k = [], []
    for a, b in zip(edges[:-1], edges[1:]):
        sel = _topk(scores[a:b], keys[a:b], k)
        cand_s.append(scores[a:b][sel])
        cand_k.append(keys[a:b][sel])
    cs, ck = np.concatenate(cand_s), np.concatenate(cand_k)
    # second pass: top k over list positions, mapped back to keys
    pos = _topk(cs, np.arange(cs.shape[0]), k)
    got = ck[pos]
    want = keys[_topk(scores, keys, k)]
    assert np.array_equal(got, want)
    assert np.array_equal(cs[pos], scores[want])


def test_model_is_sensitive_to_list_order():
    """The position tie-break is only right because the lists stand in key order:
    with the chunk lists reversed the same model picks other keys."""
    n, k = 16377, 2048
    edges = _split_plan(n, k)
    scores = np.zeros(n)
    keys = np.arange(n)
    lists = [(scores[a:b][_topk(scores[a:b], keys[a:b], k)], keys[a:b][_topk(scores[a:b], keys[a:b], k)])
             for a, b in zip(edges[:-1], edges[1:])]
    cs = np.concatenate([s for s, _ in lists[::-1]])
    ck = np.concatenate([c for _, c in lists[::-1]])
    got = ck[_topk(cs, np.arange(cs.shape[0]), k)]
    assert not np.array_equal(got, np.arange(k))
