"""Plain fp64 CPU oracle of the LightningIndexer forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code with the HIP path (no decoders,
no tables, no helpers); its inputs are the raw host arrays of a seeded
workload, read by attribute.

What it computes (all pages agree on the formula; the MindSpore
``mindspore.ops.lightning_indexer`` page states it most cleanly, in its
formula block; the CANN LightningIndexerV2 guide gives the same three-step
description in "三步计算流程"; the VllmQuantLightningIndexer README gives the
quantised form in its "功能说明" formula):

    for every query token, every visible key j:
        s_j = sum_g  W[g] * ReLU( Q_index[g] . K_index[j] )            (plain)
        s_j = sum_g  W[g] * ReLU( Sq[g] * Sk[j] * (Qc[g] . Kc[j]) )    (quantised)
    Indices = Top-k over the visible keys of s.

Steps, in the order of the TileLang guide's ``index_golden`` (dot products
per head, ReLU, multiply by the per-head weight, sum over the heads, top-k
with largest first and sorted output):

1. actual lengths per batch: S_q, S_k (BSND: seqused or the padded dim;
   TND: seqused where given, else the cu_seqlens differences; PA_BSND:
   seqused_k). Under TND a seqused_q below the cu_seqlens_q length is the
   LightningIndexerV2 guide's "TND Padding" (constraint list, Ascend 950
   items): the query rows between the two lengths are allotted in the output
   but invalid, so they come out all -1 / -inf like any row past S_q;
2. visible keys of query row i: all S_k for sparse_mode 0; for sparse_mode 3
   (right-down causal) key j is visible iff j <= i + S_k - S_q, i.e. the
   first clamp(i + 1 + S_k - S_q, 0, S_k) keys;
3. decode the stored codes to float64 exactly (own IEEE-field decoders);
4. s_j in float64 as above (a float64 matrix product is the dot step);
5. order the visible keys by (s desc, j asc), keep the first m = min(k, n);
6. sparse_indices = those j (plus the batch's output_idx_offset, when one is
   given) then -1; sparse_values = float32(s_j) then -inf (fill values from the
   LightningIndexerV2 guide's constraint list).

Compressed keys (the LightningIndexerV2 guide's cmp_ratio r and
cmp_residual_k): k then holds S_k compressed keys of a sequence of
S_k * r + residual original tokens; the scores are computed on the compressed
keys as above, only the causal visibility changes (step 2).

Routing options of the forward operator the ops-transformer open-sourcing
issue lists (part 2, "LightningIndexer 族": block_len for key-block
granularity 1/2/4/8/16, init_num for sink tokens that are always kept,
local_num for the diagonal local window), which the issue names but does not
define; the oracle takes these readings:

7. with block_len L > 1 the selection runs over key blocks: block c holds
   keys [c*L, (c+1)*L) of the sequence, its score is the largest score of its
   visible keys, and a row has ceil(n / L) visible blocks; the output indices
   are block indices;
8. the first init_num visible blocks and the last local_num visible blocks
   (the latter end at the row's diagonal under the causal rule) are always
   kept: they fill the first output slots in ascending block order, and the
   remaining k - (number kept) slots take the other blocks ordered as in
   step 5.

Readings where the pages are silent (all listed in the design notes):
lowest index wins ties; output sorted by score; indices are 0-based positions
within the sequence; query rows past the actual query length are all padding;
sparse_values are float32; compressed key j summarises original tokens
[j*r, j*r + r - 1] and becomes visible under the right-down rule once its last
token does; output_idx_offset is one non-negative value per batch, added to
the valid indices only.

Every function here is pinned by ``tests/test_oracle.py`` against closed
forms, hand-worked examples, brute force or library routines.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Step 3: decoders, written from the IEEE / OCP field definitions
# ---------------------------------------------------------------------------


def decode_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int32))
    sub = np.ldexp(f / 1024.0, -14)
    special = np.where(f == 0, np.inf, np.nan)
    mag = np.where(e == 0, sub, np.where(e == 31, special, normal))
    return sign * mag


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(np.float64)
    normal = np.ldexp(1.0 + f / 128.0, (e - 127).astype(np.int32))
    sub = np.ldexp(f / 128.0, -126)
    special = np.where(f == 0, np.inf, np.nan)
    mag = np.where(e == 0, sub, np.where(e == 255, special, normal))
    return sign * mag


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits.

    No infinities; S.1111.111 is NaN; the largest finite value is 448.
    """
    b = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    f = (b & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + f / 8.0, (e - 7).astype(np.int32))
    sub = np.ldexp(f / 8.0, -6)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (f == 7), np.nan, mag)
    return sign * mag


def decode_i8(codes: np.ndarray) -> np.ndarray:
    return np.asarray(codes).astype(np.int8).astype(np.float64)


def decode_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


_DECODERS = {
    "f16": decode_f16,
    "bf16": decode_bf16,
    "e4m3fn": decode_e4m3fn,
    "i8": decode_i8,
    "f32": decode_f32,
}


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    return _DECODERS[dtype](arr)


# ---------------------------------------------------------------------------
# Steps 1-2: lengths and the visibility rule
# ---------------------------------------------------------------------------


def batch_lengths(wl) -> List[Tuple[int, int]]:
    """Actual (S_q, S_k) per batch, from the length inputs the pages define.

    seqused_* wins over the allotted length in every layout: the padded dim for
    BSND, the cu_seqlens difference for TND (the V2 guide's TND padding rule
    for queries; seqused_k is optional for BSND and TND keys, required for
    PA_BSND, in the same guide's constraint list)."""
    out = []
    for b in range(wl.B):
        if wl.seqused_q is not None:
            sq = int(wl.seqused_q[b])
        elif wl.layout_q == "TND":
            sq = int(wl.cu_seqlens_q[b + 1]) - int(wl.cu_seqlens_q[b])
        else:
            sq = int(wl.q.shape[1])
        if wl.seqused_k is not None:
            sk = int(wl.seqused_k[b])
        elif wl.layout_k == "TND":
            sk = int(wl.cu_seqlens_k[b + 1]) - int(wl.cu_seqlens_k[b])
        else:
            sk = int(wl.k.shape[1])
        out.append((sq, sk))
    return out


def visible_count(i: int, sq: int, sk: int, mode: int, cmp_ratio: int = 1,
                  residual: int = 0) -> int:
    """Keys visible to query row i: all of them for mode 0; the right-down
    causal rule j <= i + (S_k - S_q) for mode 3.

    With compressed keys (ratio r, residual res < r) the sequence has
    L = S_k * r + res original tokens and compressed key j covers original
    tokens j*r .. j*r + r - 1; it is visible to row i when its last token is,
    i.e. j*r + r - 1 <= i + L - S_q, so the first
    clamp(floor((i + 1 + L - S_q) / r), 0, S_k) compressed keys are visible
    (r = 1, res = 0 gives the plain rule)."""
    if i >= sq:
        return 0
    if mode == 0:
        return sk
    if mode == 3:
        orig = sk * cmp_ratio + residual
        return max(0, min(sk, (i + 1 + orig - sq) // cmp_ratio))
    raise ValueError(f"sparse_mode {mode} is not defined")


def compression(wl, b: int) -> Tuple[int, int]:
    """(cmp_ratio, residual of batch b) of a workload; (1, 0) when uncompressed."""
    r = int(getattr(wl, "cmp_ratio", 1) or 1)
    res = getattr(wl, "cmp_residual_k", None)
    return r, (int(res[b]) if res is not None else 0)


def index_offset(wl, b: int) -> int:
    """output_idx_offset of batch b (0 when none is given)."""
    off = getattr(wl, "output_idx_offset", None)
    return int(off[b]) if off is not None else 0


def routing(wl) -> Tuple[int, int, int]:
    """(block_len, init_num, local_num) of a workload; (1, 0, 0) when not given."""
    L = int(getattr(wl, "block_len", 1) or 1)
    return L, int(getattr(wl, "init_num", 0) or 0), int(getattr(wl, "local_num", 0) or 0)


# ---------------------------------------------------------------------------
# Step 3: per-batch operand gathering
# ---------------------------------------------------------------------------


def _query_block(wl, b: int, rows: np.ndarray):
    """Decoded query rows (len(rows), N1, D), weights (len(rows), N1) and
    query dequant scales (len(rows), N1) or None, for positions `rows` of batch b."""
    if wl.layout_q == "TND":
        r = int(wl.cu_seqlens_q[b]) + rows
        qc, wc = wl.q[r], wl.w[r]
        qs = wl.q_scale[r] if wl.q_scale is not None else None
    else:
        qc, wc = wl.q[b, rows], wl.w[b, rows]
        qs = wl.q_scale[b, rows] if wl.q_scale is not None else None
    q = decode(qc, wl.qk_dtype)
    w = decode(wc, wl.w_dtype)
    s = decode_f32(qs) if qs is not None else None
    return q, w, s


def _key_block(wl, b: int, sk: int):
    """Decoded keys (S_k, N2, D) of batch b in logical order, plus key dequant
    scales (S_k, N2) or None. PA_BSND: key j lives in physical block
    block_table[b, j // block_size], row j % block_size."""
    j = np.arange(sk)
    if wl.layout_k == "TND":
        r = int(wl.cu_seqlens_k[b]) + j
        kc = wl.k[r]
        ks = wl.k_scale[r] if wl.k_scale is not None else None
    elif wl.layout_k == "BSND":
        kc = wl.k[b, :sk]
        ks = wl.k_scale[b, :sk] if wl.k_scale is not None else None
    elif wl.layout_k == "PA_BSND":
        bs = int(wl.k.shape[1])
        blk = wl.block_table[b, j // bs]
        kc = wl.k[blk, j % bs]
        ks = wl.k_scale[blk, j % bs] if wl.k_scale is not None else None
    else:
        raise ValueError(wl.layout_k)
    k = decode(kc, wl.qk_dtype)
    s = decode_f32(ks) if ks is not None else None
    return k, s


# ---------------------------------------------------------------------------
# Step 4: scores, Step 5: ordering
# ---------------------------------------------------------------------------


def row_scores(q: np.ndarray, w: np.ndarray, k: np.ndarray,
               q_scale: Optional[np.ndarray] = None,
               k_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """s_j = sum_g w[g] * ReLU(x[g, j]) for one query row and one KV head.

    q: (G, D) decoded query heads, w: (G,), k: (n, D) decoded keys.
    Quantised inputs: x[g, j] = q_scale[g] * k_scale[j] * (q[g] . k[j]),
    i.e. ReLU is applied after dequantisation, as in the quantised formula.
    """
    x = q @ k.T                                    # (G, n) float64
    if q_scale is not None:
        x = (q_scale[:, None] * k_scale[None, :]) * x
    return w @ np.maximum(x, 0.0)


def row_magnitudes(q: np.ndarray, w: np.ndarray, k: np.ndarray,
                   q_scale: Optional[np.ndarray] = None,
                   k_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """P_j = sum_g |w[g]| * |q_scale[g] * k_scale[j]| * sum_d |q[g, d] * k[j, d]|.

    Not part of the method: the sum of the magnitudes of every product that
    enters s_j (same arguments as row_scores). Any floating-point evaluation
    of s_j (dot products over D, the head sum over G, the scale products) has
    a forward error of at most a small multiple of (D + G) * unit roundoff *
    P_j, whatever the summation order (the standard error bound for inner
    products and sums), which is how the tests judge how far a float32 result
    may lie from the exact score when the terms cancel."""
    x = np.abs(q) @ np.abs(k).T
    if q_scale is not None:
        x = (np.abs(q_scale)[:, None] * np.abs(k_scale)[None, :]) * x
    return np.abs(w) @ x


def topk_order(s: np.ndarray, k: int) -> np.ndarray:
    """Positions of the k largest entries of s, by (score desc, index asc)."""
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))
    return order[: min(k, n)]


def block_scores(s: np.ndarray, block_len: int) -> np.ndarray:
    """Step 7: score of key block c = max of s over its visible keys
    [c*L, min((c+1)*L, n)); ceil(n / L) blocks."""
    n = s.shape[0]
    nb = -(-n // block_len)
    return np.array([s[c * block_len:min((c + 1) * block_len, n)].max() for c in range(nb)])


def kept_blocks(nb: int, init_num: int, local_num: int) -> np.ndarray:
    """Step 8: the blocks always kept, ascending: the first init_num and the last
    local_num of the nb visible blocks (each block once)."""
    first = set(range(min(init_num, nb)))
    last = set(range(max(nb - local_num, 0), nb))
    return np.array(sorted(first | last), dtype=np.int64)


def select_blocks(sb: np.ndarray, k: int, init_num: int, local_num: int) -> Tuple[np.ndarray, int]:
    """Step 8 then step 5: (output order of block indices, number kept first)."""
    kept = kept_blocks(sb.shape[0], init_num, local_num)
    rest = np.setdiff1d(np.arange(sb.shape[0]), kept)
    chosen = rest[topk_order(sb[rest], k - kept.shape[0])]
    return np.concatenate([kept, chosen]), int(kept.shape[0])


# ---------------------------------------------------------------------------
# Driver
# ---------------------------------------------------------------------------


def all_rows(wl) -> List[Tuple[int, int]]:
    """Every output row as (batch, position): the rows allotted to each
    sequence (S1 for BSND, the cu_seqlens_q difference for TND), padding rows
    included."""
    rows = []
    for b in range(wl.B):
        n = (int(wl.cu_seqlens_q[b + 1]) - int(wl.cu_seqlens_q[b])
             if wl.layout_q == "TND" else int(wl.q.shape[1]))
        rows.extend((b, i) for i in range(n))
    return rows


def run(wl, rows: Optional[Iterable[Tuple[int, int]]] = None, want_scores: bool = False,
        row_block: int = 16) -> Dict[str, object]:
    """Oracle outputs for `rows` ((b, i) pairs; all rows when None).

    Returns a dict with
      'rows'    : list of (b, i)
      'indices' : int32 (R, N2, k)
      'values'  : float32 (R, N2, k)
      'scores'  : (if want_scores) list over rows of lists over N2 of float64
                  arrays holding s_j for every visible key j (block scores
                  for block_len > 1);
      'mags'    : (if want_scores) the same layout as 'scores', holding
                  row_magnitudes of each key (for blocks: the largest over
                  the block's visible keys);
      'kept'    : (if want_scores) int (R, N2): output slots taken by the
                  blocks that are always kept (0 without init_num / local_num).
    """
    rows = list(all_rows(wl) if rows is None else rows)
    kk = wl.sparse_count
    N2, G = wl.N2, wl.N1 // wl.N2
    R = len(rows)
    idx = np.full((R, N2, kk), -1, np.int32)
    val = np.full((R, N2, kk), -np.inf, np.float32)
    scores: List[List[np.ndarray]] = [[np.zeros(0)] * N2 for _ in range(R)]
    mags: List[List[np.ndarray]] = [[np.zeros(0)] * N2 for _ in range(R)]
    kept = np.zeros((R, N2), np.int64)
    lengths = batch_lengths(wl)
    L, init_num, local_num = routing(wl)

    by_batch: Dict[int, List[int]] = {}
    for r, (b, i) in enumerate(rows):
        by_batch.setdefault(b, []).append(r)
    for b, rlist in by_batch.items():
        sq, sk = lengths[b]
        cr, res = compression(wl, b)
        off = index_offset(wl, b)
        live = [r for r in rlist if rows[r][1] < sq and
                visible_count(rows[r][1], sq, sk, wl.sparse_mode, cr, res) > 0]
        if not live:
            continue
        keys, kscale = _key_block(wl, b, sk)
        for c in range(0, len(live), row_block):
            chunk = live[c:c + row_block]
            pos = np.array([rows[r][1] for r in chunk])
            q, w, qs = _query_block(wl, b, pos)
            for t, r in enumerate(chunk):
                n = visible_count(int(pos[t]), sq, sk, wl.sparse_mode, cr, res)
                for h in range(N2):
                    g = slice(h * G, (h + 1) * G)
                    s = row_scores(q[t, g], w[t, g], keys[:n, h],
                                   None if qs is None else qs[t, g],
                                   None if kscale is None else kscale[:n, h])
                    if L > 1 or init_num or local_num:
                        s = block_scores(s, L)
                        order, kept[r, h] = select_blocks(s, kk, init_num, local_num)
                    else:
                        order = topk_order(s, kk)
                    m = order.shape[0]
                    idx[r, h, :m] = order + off
                    val[r, h, :m] = s[order].astype(np.float32)
                    if want_scores:
                        scores[r][h] = s
                        p = row_magnitudes(q[t, g], w[t, g], keys[:n, h],
                                           None if qs is None else qs[t, g],
                                           None if kscale is None else kscale[:n, h])
                        mags[r][h] = block_scores(p, L) if L > 1 else p
    out: Dict[str, object] = {"rows": rows, "indices": idx, "values": val}
    if want_scores:
        out["scores"] = scores
        out["mags"] = mags
        out["kept"] = kept
    return out


def run_full(wl) -> Tuple[np.ndarray, np.ndarray]:
    """Whole-problem outputs shaped like the operator's: (B,S1,N2,k) for BSND
    queries, (T1,N2,k) for TND."""
    o = run(wl)
    idx, val = o["indices"], o["values"]
    if wl.layout_q == "BSND":
        shape = (wl.B, int(wl.q.shape[1]), wl.N2, wl.sparse_count)
        return idx.reshape(shape), val.reshape(shape)
    return idx, val
