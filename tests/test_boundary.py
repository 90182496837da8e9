"""CPU tests of the C-ABI boundary: exported symbols, argument checks, the
metadata partitioner and workspace sizing. No compute call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_attention_top_amd import binding as B
from sparse_attention_top_amd import indexer as I
from sparse_attention_top_amd import synth
from tests.checker import visible, visible_pairs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from sparse_attention_top_amd import build
        build.build(verbose=False)
    return B.lib()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "li.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:li_status|const char\*|int32_t|size_t)\s+(li_\w+)\s*\(",
                                  hdr, re.M)))
    assert {"li_metadata", "li_workspace_size", "li_score", "li_topk", "li_indexer",
            "li_last_error", "li_api_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in li.h but not exported"
    assert B.li_api_version() == B.API_VERSION


def _prob(**kw):
    base = dict(layout_q="BSND", layout_k="BSND", dtype_qk="bf16", dtype_w="bf16", batch=2,
                s1=16, s2=64, n1=64, n2=1, d=128, sparse_count=32, sparse_mode=3)
    base.update(kw)
    return B.make_problem(**base)


def _status(p, lengths=None):
    L = lengths if lengths is not None else B.make_lengths()
    try:
        B.li_metadata(p, L)
        return B.OK
    except B.LIError as e:
        return e.status


BAD = [
    ("empty batch", dict(batch=0), B.ERR_EMPTY_TENSOR),
    ("empty heads", dict(n1=0), B.ERR_EMPTY_TENSOR),
    ("empty dim", dict(d=0), B.ERR_EMPTY_TENSOR),
    ("empty s1", dict(s1=0), B.ERR_EMPTY_TENSOR),
    ("empty s2", dict(s2=0), B.ERR_EMPTY_TENSOR),
    ("negative batch", dict(batch=-1), B.ERR_INVALID_ARGUMENT),
    ("layout pairing", dict(layout_k="TND", t2=64), B.ERR_INVALID_ARGUMENT),
    ("bad layout", dict(layout_q=7), B.ERR_INVALID_ARGUMENT),
    ("w dtype", dict(dtype_w="e4m3fn"), B.ERR_INVALID_ARGUMENT),
    ("qk dtype", dict(dtype_qk="f32"), B.ERR_INVALID_ARGUMENT),
    ("k zero", dict(sparse_count=0), B.ERR_INVALID_ARGUMENT),
    ("k too big", dict(sparse_count=8193), B.ERR_INVALID_ARGUMENT),
    ("cmp ratio negative", dict(cmp_ratio=-1), B.ERR_INVALID_ARGUMENT),
    ("cmp ratio too big", dict(cmp_ratio=129), B.ERR_INVALID_ARGUMENT),
    ("block_len 3", dict(block_len=3), B.ERR_INVALID_ARGUMENT),
    ("block_len 32", dict(block_len=32), B.ERR_INVALID_ARGUMENT),
    ("block_len negative", dict(block_len=-2), B.ERR_INVALID_ARGUMENT),
    ("init_num negative", dict(init_num=-1), B.ERR_INVALID_ARGUMENT),
    ("local_num negative", dict(local_num=-1), B.ERR_INVALID_ARGUMENT),
    ("kept blocks above k", dict(sparse_count=8, init_num=5, local_num=4), B.ERR_INVALID_ARGUMENT),
    ("mode 1", dict(sparse_mode=1), B.ERR_INVALID_ARGUMENT),
    ("mode 2", dict(sparse_mode=2), B.ERR_INVALID_ARGUMENT),
    ("pre_tokens", dict(pre_tokens=100), B.ERR_UNSUPPORTED),
    ("next_tokens", dict(next_tokens=0), B.ERR_UNSUPPORTED),
    ("n2 > 1", dict(n2=2), B.ERR_UNSUPPORTED),
    ("n1 > 64", dict(n1=65), B.ERR_UNSUPPORTED),
    ("d = 96", dict(d=96), B.ERR_UNSUPPORTED),
    ("pa block 8", dict(layout_k="PA_BSND", block_size=8, num_blocks=4, max_blocks_per_seq=4),
     B.ERR_INVALID_ARGUMENT),
    ("pa block 24", dict(layout_k="PA_BSND", block_size=24, num_blocks=4, max_blocks_per_seq=4),
     B.ERR_INVALID_ARGUMENT),
    ("pa block 2048", dict(layout_k="PA_BSND", block_size=2048, num_blocks=4,
                           max_blocks_per_seq=4), B.ERR_INVALID_ARGUMENT),
    ("pa no blocks", dict(layout_k="PA_BSND", block_size=16, num_blocks=0, max_blocks_per_seq=4),
     B.ERR_EMPTY_TENSOR),
    ("pa small stride", dict(layout_k="PA_BSND", block_size=16, num_blocks=4,
                             max_blocks_per_seq=4, k_block_stride=16), B.ERR_INVALID_ARGUMENT),
    ("quant scale dtype", dict(dtype_qk="e4m3fn", dtype_scale="f16"), B.ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,kw,status", BAD, ids=[b[0] for b in BAD])
def test_problem_checks(lib, name, kw, status):
    assert _status(_prob(**kw)) == status
    assert B.li_last_error()


def test_reserved_and_version(lib):
    p = _prob()
    p.reserved[2] = 1
    assert _status(p) == B.ERR_INVALID_ARGUMENT
    p = _prob()
    p.api_version = 99
    assert _status(p) == B.ERR_INVALID_ARGUMENT
    p = _prob()
    p.return_value = 2
    assert _status(p) == B.ERR_INVALID_ARGUMENT


LEN_BAD = [
    ("tnd without cu_seqlens_q", dict(layout_q="TND", layout_k="TND", t1=8, t2=8, batch=1),
     dict(cu_seqlens_k=[0, 8])),
    ("bsnd with cu_seqlens_q", dict(), dict(cu_seqlens_q=[0, 8, 16])),
    ("bsnd with cu_seqlens_k", dict(), dict(cu_seqlens_k=[0, 8, 16])),
    ("cu_seqlens first not 0", dict(layout_q="TND", layout_k="TND", t1=8, t2=8, batch=1),
     dict(cu_seqlens_q=[1, 8], cu_seqlens_k=[0, 8])),
    ("cu_seqlens decreasing", dict(layout_q="TND", layout_k="TND", t1=8, t2=8, batch=2),
     dict(cu_seqlens_q=[0, 9, 8], cu_seqlens_k=[0, 4, 8])),
    ("cu_seqlens negative entry", dict(layout_q="TND", layout_k="TND", t1=8, t2=8, batch=2),
     dict(cu_seqlens_q=[0, -2**31, 8], cu_seqlens_k=[0, 4, 8])),
    ("cu_seqlens total", dict(layout_q="TND", layout_k="TND", t1=8, t2=8, batch=1),
     dict(cu_seqlens_q=[0, 7], cu_seqlens_k=[0, 8])),
    ("seqused_q above s1", dict(), dict(seqused_q=[17, 3])),
    ("seqused_k above s2", dict(), dict(seqused_k=[3, 65])),
    ("seqused_k negative", dict(), dict(seqused_k=[-1, 3])),
    ("pa without seqused_k", dict(layout_k="PA_BSND", block_size=16, num_blocks=8,
                                  max_blocks_per_seq=4), dict()),
    ("pa block_table too short", dict(layout_k="PA_BSND", block_size=16, num_blocks=8,
                                      max_blocks_per_seq=4), dict(seqused_k=[65, 3])),
    ("tnd seqused_k beyond cu", dict(layout_q="TND", layout_k="TND", t1=8, t2=8, batch=1),
     dict(cu_seqlens_q=[0, 8], cu_seqlens_k=[0, 8], seqused_k=[9])),
    ("cmp without residual", dict(cmp_ratio=4), dict()),
    ("cmp residual >= ratio", dict(cmp_ratio=4), dict(cmp_residual_k=[0, 4])),
    ("cmp residual negative", dict(cmp_ratio=4), dict(cmp_residual_k=[-1, 0])),
    ("residual without cmp", dict(), dict(cmp_residual_k=[0, 0])),
    ("residual with ratio 1", dict(cmp_ratio=1), dict(cmp_residual_k=[0, 0])),
    ("residual in mode 0", dict(cmp_ratio=4, sparse_mode=0), dict(cmp_residual_k=[1, 1])),
    ("negative index offset", dict(), dict(output_idx_offset=[0, -1])),
    ("index offset overflows", dict(), dict(output_idx_offset=[0, 2**31 - 63])),
]


@pytest.mark.parametrize("name,pk,lk", LEN_BAD, ids=[b[0] for b in LEN_BAD])
def test_length_checks(lib, name, pk, lk):
    assert _status(_prob(**pk), B.make_lengths(**lk)) == B.ERR_INVALID_ARGUMENT


def test_compressed_original_length_limit(lib):
    # the visibility rule works on original token positions, which must fit int32
    p = _prob(cmp_ratio=128, s2=(1 << 24) - 1)
    assert _status(p, B.make_lengths(cmp_residual_k=[127, 127])) == B.OK
    p = _prob(cmp_ratio=128, s2=1 << 24)
    assert _status(p, B.make_lengths(cmp_residual_k=[0, 0])) == B.ERR_UNSUPPORTED


def test_buffer_too_small_reports_size(lib):
    p = _prob()
    L = B.make_lengths()
    need = ctypes.c_size_t(0)
    buf = np.zeros(64, np.uint8)
    st = lib.li_metadata(ctypes.byref(p), ctypes.byref(L), 256, buf.ctypes.data, 64,
                         ctypes.byref(need))
    assert st == B.ERR_BUFFER_TOO_SMALL and need.value > 64


# ---------------------------------------------------------------------------
# task table
# ---------------------------------------------------------------------------
def _coverage(wl, meta):
    """Every visible (row, key) pair is covered by exactly one work item."""
    h, recs, items = B.parse_metadata(meta)
    tq = int(h["tile_q"])
    cover = {}
    for b in range(wl.B):
        sq, sk = int(recs[b]["s_q"]), int(recs[b]["s_k"])
        cover[b] = np.zeros((sq, max(sk, 1)), np.int32)
    for it in items:
        b, q0, k0, k1 = (int(it[f]) for f in ("b", "q0", "k0", "k1"))
        r = recs[b]
        assert k0 < k1
        for i in range(q0, min(q0 + tq, int(r["s_q"]))):
            nv = visible(wl, b, i)
            hi = min(nv, k1)
            if hi > k0:
                cover[b][i, k0:hi] += 1
    pairs = 0
    for b in range(wl.B):
        for i in range(int(recs[b]["s_q"])):
            nv = visible(wl, b, i)
            assert (cover[b][i, :nv] == 1).all(), f"row ({b},{i}) not covered exactly once"
            assert (cover[b][i, nv:] == 0).all()
            pairs += nv
    assert pairs == int(h["visible_pairs"]) == visible_pairs(wl)
    return h, recs, items


WORKLOADS = {
    "causal": lambda: synth.build("c", layout_q="BSND", layout_k="BSND", qk_dtype="bf16",
                                  w_dtype="bf16", N1=64, D=128, seqlens_q=[300], seqlens_k=[300],
                                  sparse_count=64, sparse_mode=3, seed=1),
    "nomask": lambda: synth.build("n", layout_q="BSND", layout_k="BSND", qk_dtype="f16",
                                  w_dtype="f32", N1=32, D=64, seqlens_q=[37, 37],
                                  seqlens_k=[500, 500], sparse_count=64, sparse_mode=0, seed=2),
    "seqused": lambda: synth.build("u", layout_q="BSND", layout_k="BSND", qk_dtype="bf16",
                                   w_dtype="bf16", N1=16, D=128, seqlens_q=[10, 33, 0],
                                   seqlens_k=[100, 20, 50], S1=40, S2=120, sparse_count=8,
                                   sparse_mode=3, seed=3),
    "varlen": lambda: synth.build("v", layout_q="TND", layout_k="TND", qk_dtype="e4m3fn",
                                  w_dtype="f32", N1=64, D=128, seqlens_q=[5, 0, 70, 19],
                                  seqlens_k=[5, 0, 70, 40], sparse_count=16, sparse_mode=3,
                                  seed=4),
    "paged": lambda: synth.paged_decode(B=6, lo=100, hi=900, block_size=64),
    # one or two rows per sequence, key lengths spanning every top-k size class
    "classes": lambda: synth.build("k", layout_q="TND", layout_k="TND", qk_dtype="bf16",
                                   w_dtype="bf16", N1=8, D=64, seqlens_q=[1, 2, 1, 1, 2, 1, 0],
                                   seqlens_k=[100, 3000, 5000, 9000, 20000, 40000, 7],
                                   sparse_count=64, sparse_mode=0, seed=6),
    # compressed keys: ratio 4 with per-batch residuals, and per-batch index offsets
    "compressed": lambda: synth.build("z", layout_q="BSND", layout_k="BSND", qk_dtype="bf16",
                                      w_dtype="bf16", N1=16, D=128, seqlens_q=[300, 7, 64],
                                      seqlens_k=[80, 3, 20], S1=300, S2=80, sparse_count=32,
                                      sparse_mode=3, cmp_ratio=4, cmp_residual_k=[3, 0, 1],
                                      output_idx_offset=[0, 1000, 77], seed=7),
    # key blocks of 16 over compressed keys, with sink and local blocks
    "blocks": lambda: synth.build("bl", layout_q="TND", layout_k="TND", qk_dtype="bf16",
                                  w_dtype="f32", N1=8, D=64, seqlens_q=[40, 3, 0, 9],
                                  seqlens_k=[500, 70, 5, 33], sparse_count=16, sparse_mode=3,
                                  cmp_ratio=2, cmp_residual_k=[1, 0, 1, 1], block_len=16,
                                  init_num=2, local_num=3, seed=10),
    "compressed_tnd": lambda: synth.build("zt", layout_q="TND", layout_k="TND",
                                          qk_dtype="e4m3fn", w_dtype="f32", N1=32, D=128,
                                          seqlens_q=[128, 1, 50], seqlens_k=[1000, 9, 13],
                                          sparse_count=16, sparse_mode=3, cmp_ratio=128,
                                          cmp_residual_k=[127, 5, 0], seed=8),
    # TND padding: seqused_q / seqused_k below the cu_seqlens lengths, one
    # sequence with no used query rows
    "tnd_padding": lambda: synth.build("tp", layout_q="TND", layout_k="TND", qk_dtype="bf16",
                                       w_dtype="bf16", N1=16, D=64, seqlens_q=[30, 0, 9, 4],
                                       seqlens_k=[90, 12, 9, 0], padded_q=[41, 5, 9, 6],
                                       padded_k=[100, 12, 20, 3], sparse_count=16,
                                       sparse_mode=3, seed=11),
    "tnd_padding_paged": lambda: synth.build("tpp", layout_q="TND", layout_k="PA_BSND",
                                             qk_dtype="e4m3fn", w_dtype="f32", N1=8, D=128,
                                             seqlens_q=[3, 0, 7], seqlens_k=[300, 40, 129],
                                             padded_q=[5, 2, 7], block_size=64,
                                             sparse_count=32, sparse_mode=3, seed=12),
    "compressed_nomask": lambda: synth.build("zn", layout_q="BSND", layout_k="BSND",
                                             qk_dtype="bf16", w_dtype="bf16", N1=8, D=64,
                                             seqlens_q=[9, 9], seqlens_k=[40, 40],
                                             sparse_count=8, sparse_mode=0, cmp_ratio=2,
                                             output_idx_offset=[5, 6], seed=9),
}


def _lengths(wl):
    return B.make_lengths(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.seqused_q, wl.seqused_k,
                          wl.cmp_residual_k, wl.output_idx_offset)


def _row_table(wl, meta, num_cus=256):
    """Every output row is one record -- of the first pass, or, when split, of
    the second pass with its chunks in the first -- carrying its visible-key
    count, the workspace offset of its scores and its index offset; first-pass
    records sit in the size class of their count, second-pass records all in
    the class of the longest, longest first inside a class; chunks tile
    the row with 16-byte aligned starts and lengths in (k, 8192], and their
    candidate lists lie side by side where the second-pass record reads them."""
    h, recs, _ = B.parse_metadata(meta)
    rows, bounds = B.parse_row_table(meta)
    C, k = B.TOPK_CLASSES, wl.sparse_count
    assert bounds[0] == 0 and bounds[-1] == len(rows) == int(h["num_recs"])
    assert (np.diff(bounds) >= 0).all()
    where = {}
    for b in range(wl.B):
        nrows_b = (int(wl.cu_seqlens_q[b + 1]) - int(wl.cu_seqlens_q[b])
                   if wl.layout_q == "TND" else wl.S1)
        for i in range(nrows_b):
            where[wl.row_of(b, i)] = (b, i)
    assert len(where) == wl.num_rows
    limits = (0,) + B.TOPK_CLASS_KEYS
    split_ok = (k <= 2048 and wl.init_num == 0 and wl.local_num == 0
                and wl.num_rows < 2 * num_cus)
    seen, chunks = [], {}
    cand_end = 0
    for q in range(2):
        for c in range(C):
            ns = []
            for rec in rows[bounds[q * C + c]:bounds[q * C + c + 1]]:
                n, kind = int(rec["n"]), int(rec["kind"])
                if q == 0:
                    assert (n == 0 and c == 0) or limits[c] < n <= limits[c + 1]
                else:   # one launch: every record in the class of the longest
                    assert n <= limits[c + 1] and (ns or limits[c] < n)
                    assert all(bounds[C + d] == bounds[C + d + 1] for d in range(C) if d != c)
                ns.append(n)
                if kind == B.ROW_CHUNK:
                    assert q == 0
                    chunks.setdefault(int(rec["row"]), []).append(rec)
                    continue
                assert kind == (B.ROW_WHOLE if q == 0 else B.ROW_MERGE)
                row = int(rec["row"])
                seen.append(row)
                assert int(rec["out_off"]) == row * k
                b, i = where[row]
                L = max(1, wl.block_len)
                nv = -(-visible(wl, b, i) // L) if i < int(wl.seqlens_q[b]) else 0
                off = 0 if wl.output_idx_offset is None else int(wl.output_idx_offset[b])
                assert int(rec["idx_offset"]) == off
                row_ws = int(recs[b]["ws_off"]) + i * int(recs[b]["ld"])
                if kind == B.ROW_WHOLE:
                    assert n == nv and not (split_ok and n > 8192)
                    if n > 0:
                        assert int(rec["ws_off"]) == row_ws
                    continue
                assert split_ok and nv > 8192
                ch = sorted(chunks.pop(row), key=lambda r: int(r["idx_offset"]))
                nc = -(-nv // 8188)
                assert len(ch) == nc and n == nc * k
                starts = [int(r["idx_offset"]) for r in ch] + [nv]
                assert starts[0] == 0 and all(x % 4 == 0 for x in starts[:-1])
                lens = np.diff(starts)
                assert (lens > k).all() and (lens <= 8192).all()
                assert [int(r["n"]) for r in ch] == list(lens)
                assert [int(r["ws_off"]) for r in ch] == [row_ws + x for x in starts[:-1]]
                base = int(rec["ws_off"]) - int(h["cand_val_off"])
                assert base % 4 == 0 and base >= 0
                assert [int(r["out_off"]) for r in ch] == [base + j * k for j in range(nc)]
                cand_end = max(cand_end, base + nc * k)
            ns_sorted = sorted(ns, reverse=True)
            assert ns == ns_sorted
    assert not chunks, "chunks without a second-pass record"
    assert sorted(seen) == list(range(wl.num_rows))
    nsplit = int(h["split_rows"])
    assert nsplit == sum(1 for r in rows if int(r["kind"]) == B.ROW_MERGE)
    if nsplit:
        vo, io = int(h["cand_val_off"]), int(h["cand_idx_off"])
        scores_end = max(int(r["ws_off"]) + int(r["s_q"]) * int(r["ld"]) for r in recs)
        assert vo >= scores_end and vo % 4 == 0
        assert io - vo >= cand_end and int(h["ws_floats"]) >= io + cand_end
    return nsplit


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_metadata_covers_every_pair_once(lib, name):
    wl = WORKLOADS[name]()
    dp = I.problem_of(wl)
    meta = B.li_metadata(dp, _lengths(wl))
    h, recs, items = _coverage(wl, meta)
    _row_table(wl, meta)
    assert int(h["num_rows"]) == wl.num_rows
    # workspace rows are 16-byte aligned and long enough
    L = max(1, wl.block_len)
    for b in range(wl.B):
        assert int(recs[b]["ld"]) % 4 == 0 and int(recs[b]["ld"]) >= -(-int(recs[b]["s_k"]) // L)
        assert int(recs[b]["ws_off"]) % 4 == 0
    assert B.li_workspace_size(dp, meta) >= 4 * int(sum(int(r["s_q"]) * int(r["ld"])
                                                        for r in recs))


def _split_wl(k=2048, rows=2, sk=30000, **kw):
    return synth.build("sp", layout_q="TND", layout_k="TND", qk_dtype="bf16", w_dtype="bf16",
                       N1=8, D=64, seqlens_q=[rows], seqlens_k=[sk], sparse_count=k,
                       sparse_mode=0, seed=1, **kw)


@pytest.mark.parametrize("case,cus,splits", [
    (dict(), 256, 2),                                  # few long rows: split
    (dict(sk=8192), 256, 0),                           # fits the first class: never split
    (dict(sk=8193), 256, 2),
    (dict(k=2049), 256, 0),                            # k above 2048: never split
    (dict(block_len=4, init_num=1, local_num=1), 256, 0),   # kept blocks: never split
    (dict(block_len=4, sk=40000), 256, 2),             # 10000 blocks per row: split
    (dict(rows=600), 256, 0),                          # rows enough to fill the CUs
    (dict(rows=600), 301, 600),                        # ... but not 301 of them
    (dict(rows=2), 1, 0),
])
def test_split_decision(lib, case, cus, splits):
    """Long rows are split only where rows are fewer than two per CU, k <= 2048
    and no blocks are always kept; the table stays consistent either way."""
    wl = _split_wl(**case)
    meta = B.li_metadata(I.problem_of(wl), _lengths(wl), cus)
    assert _row_table(wl, meta, cus) == splits
    h = B.parse_metadata(meta)[0]
    if splits:
        assert B.li_workspace_size(I.problem_of(wl), meta) == 4 * int(h["ws_floats"])
        assert int(h["cand_idx_off"]) > int(h["cand_val_off"]) > 0


@pytest.mark.parametrize("dtype,s1,variant,tile_q", [
    ("bf16", 2, 2, 2), ("bf16", 4, 1, 4), ("bf16", 64, 0, 8),
    ("e4m3fn", 2, 2, 2), ("e4m3fn", 4, 1, 4), ("e4m3fn", 64, 3, 4), ("i8", 5, 3, 4)])
def test_metadata_score_variant(lib, dtype, s1, variant, tile_q):
    """Decode (<= 2 query rows) and 3-4-row problems keep their variants whatever
    the dtype; longer fp8 / int8 sequences take the three-waves-per-SIMD variant
    of 4-row tiles, 16-bit ones the 8-row prefill tiles."""
    p = B.make_problem(layout_q="BSND", layout_k="BSND", dtype_qk=dtype, dtype_w="f32",
                       batch=2, s1=s1, s2=1024, n1=64, d=128, sparse_count=64, sparse_mode=0)
    h, _, items = B.parse_metadata(B.li_metadata(p, B.make_lengths()))
    assert int(h["variant"]) == variant and int(h["tile_q"]) == tile_q
    assert all(int(it["q0"]) % tile_q == 0 for it in items)


def test_metadata_heaviest_first_and_balanced(lib):
    p = B.make_problem(layout_q="BSND", layout_k="BSND", dtype_qk="bf16", dtype_w="bf16",
                       batch=1, s1=8192, s2=8192, n1=64, d=128, sparse_count=2048, sparse_mode=3)
    meta = B.li_metadata(p, B.make_lengths())
    h, recs, items = B.parse_metadata(meta)
    tq = int(h["tile_q"])
    cost = []
    for it in items:
        c = 0
        for i in range(int(it["q0"]), min(int(it["q0"]) + tq, 8192)):
            c += max(0, min(i + 1, int(it["k1"])) - int(it["k0"]))
        cost.append(c)
    cost = np.array(cost)
    assert (np.diff(cost) <= 0).all(), "items must be heaviest first"
    assert cost.sum() == int(h["visible_pairs"]) == 8192 * 8193 // 2
    # no item carries more than 1/200 of the work, so 256 CUs stay busy
    assert cost.max() * 200 < cost.sum()
    assert int(h["num_items"]) >= 4 * 256


MISMATCH = [
    ("s2", dict(s2=65)),
    ("k 8", dict(sparse_count=8)),        # row records would write row*2048 into rows*8
    ("k 4096", dict(sparse_count=4096)),  # ... or overrun the candidate lists
    ("k 2047", dict(sparse_count=2047)),
    ("init_num", dict(init_num=2)),       # kept blocks change the split decision
    ("local_num", dict(local_num=3)),
    ("block_len", dict(block_len=4)),
    ("cmp_ratio", dict(cmp_ratio=4, sparse_mode=0)),
    ("sparse_mode", dict(sparse_mode=0)),
    ("dtype", dict(dtype_qk="f16")),
]


@pytest.mark.parametrize("name,kw", MISMATCH, ids=[m[0] for m in MISMATCH])
def test_metadata_mismatch_rejected(lib, name, kw):
    """A table built for one problem (k = 2048, a few long rows that split) is
    rejected for another by every call that takes it, before any launch."""
    base = dict(layout_q="TND", layout_k="TND", t1=2, t2=30000, batch=1, n1=8, d=64,
                sparse_count=2048, sparse_mode=3)
    p = _prob(**base)
    L = B.make_lengths(cu_seqlens_q=[0, 2], cu_seqlens_k=[0, 30000])
    meta = B.li_metadata(p, L)
    assert int(B.parse_metadata(meta)[0]["split_rows"]) == 2
    ws = B.li_workspace_size(p, meta)
    q = _prob(**{**base, **kw})
    fake = 1 << 20   # never dereferenced: validation fails first
    inp = B.make_inputs(fake, fake, fake)
    calls = {
        "li_workspace_size": lambda: B.li_workspace_size(q, meta),
        "li_score": lambda: B.li_score(q, inp, meta, fake, fake, ws),
        "li_topk": lambda: B.li_topk(q, meta, fake, fake, ws, fake, 0),
        "li_indexer": lambda: B.li_indexer(q, inp, meta, fake, fake, ws, fake, 0),
    }
    for call, f in calls.items():
        with pytest.raises(B.LIError) as e:
            f()
        assert e.value.status == B.ERR_METADATA_MISMATCH, call


def test_metadata_junk_rejected(lib):
    p = _prob()
    meta = B.li_metadata(p, B.make_lengths())
    junk = np.zeros_like(meta)
    with pytest.raises(B.LIError) as e:
        B.li_workspace_size(p, junk)
    assert e.value.status == B.ERR_METADATA_MISMATCH
    h = B.parse_metadata(meta)[0]
    assert int(h["sparse_count"]) == 32 and int(h["init_num"]) == 0 and int(h["local_num"]) == 0


def test_metadata_header_fields_checked_apart_from_hash(lib):
    """The k the row records are laid out for is compared on its own too: a
    table whose stored k was altered (hash intact) is rejected."""
    p = _prob()
    meta = B.li_metadata(p, B.make_lengths()).copy()
    hdr = meta[:B.META_HEADER_DTYPE.itemsize].view(B.META_HEADER_DTYPE)
    hdr["sparse_count"] = 31
    with pytest.raises(B.LIError) as e:
        B.li_workspace_size(p, meta)
    assert e.value.status == B.ERR_METADATA_MISMATCH


def test_compute_calls_validate_before_launch(lib):
    """Error paths of li_score / li_topk / li_indexer return before any launch."""
    p = _prob()
    meta = B.li_metadata(p, B.make_lengths())
    ws = B.li_workspace_size(p, meta)
    fake = 1 << 20   # never dereferenced: every call below fails validation first
    inp = B.make_inputs(fake, fake, 0)
    with pytest.raises(B.LIError) as e:           # w missing
        B.li_score(p, inp, meta, fake, fake, ws)
    assert e.value.status == B.ERR_INVALID_ARGUMENT
    inp = B.make_inputs(fake, fake, fake)
    with pytest.raises(B.LIError) as e:           # workspace short
        B.li_score(p, inp, meta, fake, fake, ws - 4)
    assert e.value.status == B.ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(B.LIError) as e:           # no metadata on device
        B.li_score(p, inp, meta, 0, fake, ws)
    assert e.value.status == B.ERR_INVALID_ARGUMENT
    pv = _prob(return_value=True)
    metav = B.li_metadata(pv, B.make_lengths())
    with pytest.raises(B.LIError) as e:           # values requested, no buffer
        B.li_topk(pv, metav, fake, fake, ws, fake, 0)
    assert e.value.status == B.ERR_INVALID_ARGUMENT
    with pytest.raises(B.LIError) as e:
        B.li_indexer(pv, inp, metav, fake, fake, ws, fake, 0)
    assert e.value.status == B.ERR_INVALID_ARGUMENT
    q8 = _prob(dtype_qk="e4m3fn")
    meta8 = B.li_metadata(q8, B.make_lengths())
    with pytest.raises(B.LIError) as e:           # quantised inputs need scales
        B.li_score(q8, inp, meta8, fake, fake, B.li_workspace_size(q8, meta8))
    assert e.value.status == B.ERR_INVALID_ARGUMENT
    pa = _prob(layout_k="PA_BSND", block_size=16, num_blocks=16, max_blocks_per_seq=4)
    metapa = B.li_metadata(pa, B.make_lengths(seqused_k=[64, 10]))
    with pytest.raises(B.LIError) as e:           # paged keys need a block table
        B.li_score(pa, inp, metapa, fake, fake, B.li_workspace_size(pa, metapa))
    assert e.value.status == B.ERR_INVALID_ARGUMENT
