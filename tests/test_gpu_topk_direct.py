"""The top-k step alone, on crafted score rows.

The score step's output is replaced: rows of chosen float32 scores are written
into the workspace where li_score puts them (the batch record's ws_off, row
stride ld), then li_topk runs and every row is compared with the oracle's order
(score descending, lower key index first on equal scores; output slots past
the visible keys hold -1 / -inf). Indices and values must match exactly.

The rows aim at the selection's own edges, independent of the score arithmetic:
exact ties across the k-th place, scores bunched far from zero, a bucket segment
of exactly the longest length the in-bucket rank takes and one key more, infinite
scores, all-equal rows, subnormal scores, rows shorter than k, each row-length
class, k = 8192, and split rows (few rows, so the host cuts long rows into chunks)
beside the same rows unsplit. Scores are canonical as the score kernel stores
them (no -0, no NaN).
"""
import numpy as np
import pytest
import torch

from oracle import li_oracle as O
from sparse_attention_top_amd import binding as B
from sparse_attention_top_amd import indexer as I
from sparse_attention_top_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _canonical(s):
    s = np.asarray(s, dtype=np.float32) + np.float32(0.0)   # -0 -> +0
    assert not np.isnan(s).any()
    return s


def run_topk_rows(rows, k, num_cus=256, label=""):
    """One query row per sequence, sequence b with len(rows[b]) visible keys
    (no causal mask); returns (idx, val) as (rows, k) numpy arrays and the
    header of the task table."""
    lens = [len(r) for r in rows]
    print(f"[gpu] topk direct {label}: k={k} num_cus={num_cus} lens={lens[:8]}"
          f"{'...' if len(lens) > 8 else ''}", flush=True)
    wl = synth.build(f"topk_{label}", layout_q="TND", layout_k="TND", qk_dtype="bf16",
                     w_dtype="f32", N1=8, D=64, seqlens_q=[1] * len(rows), seqlens_k=lens,
                     sparse_count=k, sparse_mode=0, return_value=True, seed=3)
    dw = I.upload(wl, DEV, return_value=True)
    plan = I.make_plan(dw.problem, dw.lengths, DEV, num_cus)
    hdr, recs, _ = B.parse_metadata(plan.meta_host)
    for b, s in enumerate(rows):
        off, ld = int(recs[b]["ws_off"]), int(recs[b]["ld"])
        assert int(recs[b]["s_q"]) == 1 and int(recs[b]["s_k"]) == len(s) <= ld
        if len(s):
            plan.ws[off:off + len(s)] = torch.from_numpy(_canonical(s)).to(DEV)
    idx = torch.full((len(rows), k), 7, dtype=torch.int32, device=DEV)
    val = torch.zeros((len(rows), k), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    B.li_topk(dw.problem, plan.meta_host, int(plan.meta_dev.data_ptr()), int(plan.ws.data_ptr()),
              plan.ws_bytes, int(idx.data_ptr()), int(val.data_ptr()),
              int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy(), hdr


def check_rows(rows, k, gi, gv, label):
    for r, s in enumerate(rows):
        s = _canonical(s)
        order = O.topk_order(s.astype(np.float64), k)
        m = order.shape[0]
        assert gi[r, :m].tolist() == order.tolist(), f"{label}: row {r} (n={len(s)}) indices"
        assert np.array_equal(gv[r, :m].view(np.uint32), s[order].view(np.uint32)), \
            f"{label}: row {r} values"
        assert (gi[r, m:] == -1).all() and (gv[r, m:] == -np.inf).all(), f"{label}: row {r} tail"


def _segment_rows(seg_len):
    """n = 8000 keys (4096 buckets) spanning exactly [0, 4095.5], so a key's
    bucket is floor(score): 51 keys in the top bucket, seg_len keys (with ties)
    in bucket 4090 holding the 100th largest, the rest in buckets 0..2000."""
    rng = np.random.default_rng(seg_len)
    n = 8000
    top = np.concatenate([[4095.5], 4095.0 + np.arange(50) / 128.0])
    seg = 4090.0 + (1 + rng.integers(0, seg_len // 2, seg_len)) / 128.0
    rest = np.concatenate([[0.0], rng.uniform(0.0, 2000.0, n - 1 - top.size - seg.size)])
    s = np.concatenate([top, seg, rest]).astype(np.float32)
    return s[rng.permutation(n)]


def _cases():
    rng = np.random.default_rng(20261203)
    randn = lambda n, sc=3.0: (rng.standard_normal(n) * sc).astype(np.float32)
    c = {}
    c["spread_lengths"] = ([randn(n) for n in (1, 5, 100, 1500, 2047, 2048, 2049, 3000, 6000,
                                               8191, 8192)], 2048)
    c["class_lengths"] = ([randn(n) for n in (8193, 12000, 16384, 16385, 30000, 32768, 40000)],
                          2048)
    c["ties_at_kth"] = ([rng.integers(0, 50, n).astype(np.float32) for n in (3000, 6000, 20000)],
                        2048)
    c["narrow_offset"] = ([(1000.0 + 1e-3 * rng.standard_normal(n)).astype(np.float32)
                           for n in (4000, 9000)], 1024)
    c["far_offset_ulps"] = ([np.float32(1.0e7) + rng.integers(0, 3000, 5000).astype(np.float32),
                             np.float32(-1.0e7) - rng.integers(0, 3000, 5000).astype(np.float32)],
                            700)
    c["segment_64"] = ([_segment_rows(64)], 100)
    c["segment_65"] = ([_segment_rows(65)], 100)
    inf_row = randn(5000)
    inf_row[rng.choice(5000, 6, replace=False)] = np.inf
    inf_row[rng.choice(5000, 6, replace=False)] = -np.inf
    c["infinities"] = ([inf_row, np.full(3000, -np.inf, np.float32)], 512)
    few = np.zeros(6000, np.float32)
    few[[17, 4000, 5999]] = [1.0, 2.0, 0.5]
    c["zeros"] = ([np.zeros(6000, np.float32), few, -np.abs(randn(6000))], 2048)
    c["subnormal"] = ([(rng.standard_normal(5000) * 1e-41).astype(np.float32),
                       (rng.standard_normal(5000) * 1e-38).astype(np.float32)], 1000)
    c["k8192"] = ([randn(n) for n in (100, 8192, 9000, 12000, 20000)], 8192)
    c["k1"] = ([randn(n) for n in (1, 7, 5000, 17000)], 1)
    return c


CASES = _cases()


@pytest.mark.parametrize("num_cus", [256, 1])
@pytest.mark.parametrize("name", list(CASES))
def test_topk_direct_rows(name, num_cus):
    """num_cus = 256: problems this small split their rows over 8192 keys (k <= 2048);
    num_cus = 1: no row is split, so the long-row classes run on whole rows."""
    rows, k = CASES[name]
    gi, gv, _ = run_topk_rows(rows, k, num_cus=num_cus, label=name)
    check_rows(rows, k, gi, gv, name)


def test_topk_direct_split_equals_unsplit():
    """Few long rows: with 256 CUs the host splits rows over 8192 keys into chunk
    lists and a merge; with one CU it never splits. Both equal the oracle."""
    rng = np.random.default_rng(7)
    rows = [(rng.standard_normal(n) * 2).astype(np.float32) for n in (9000, 20000, 65000)]
    rows.append(rng.integers(0, 40, 30000).astype(np.float32))   # ties across chunk edges
    gi, gv, hdr = run_topk_rows(rows, 2048, num_cus=256, label="split")
    assert int(hdr["split_rows"]) == 4
    check_rows(rows, 2048, gi, gv, "split")
    gi1, gv1, hdr1 = run_topk_rows(rows, 2048, num_cus=1, label="unsplit")
    assert int(hdr1["split_rows"]) == 0
    assert np.array_equal(gi, gi1) and np.array_equal(gv.view(np.uint32), gv1.view(np.uint32))
