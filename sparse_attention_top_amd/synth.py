"""Seeded synthetic inputs for the LightningIndexer forward pass.

This module only *draws* inputs: random normals, their rounding to the storage
dtype (fp16 / bf16 / OCP fp8-e4m3fn / int8 with per-token-head dequant scales),
sequence lengths, paged-cache block tables. It holds none of the indexer's
arithmetic (no dot products, ReLU, weighting or selection), so the CPU oracle
and the HIP path can both consume its output without sharing method code.

Shapes follow the MindSpore ``lightning_indexer`` reference page (parameter
list: query (B,S1,N1,D) or (T1,N1,D); key (B,S2,N2,D), (T2,N2,D) or paged
(block_count, block_size, N2, D); weights (B,S1,N1) or (T1,N1)) and the
VllmQuantLightningIndexer README (parameter table: per-token-head dequant
scales, fp8-e4m3fn or int8 codes).

Storage conventions of the host arrays (what is copied byte-for-byte to the
device):

==========  ===================  =============================
dtype name  numpy storage dtype  meaning
==========  ===================  =============================
f16         uint16               IEEE binary16 bit patterns
bf16        uint16               bfloat16 bit patterns
f32         float32              IEEE binary32
e4m3fn      uint8                OCP FP8 E4M3FN codes
i8          int8                 signed 8-bit integer codes
==========  ===================  =============================

Padding that must never be read (BSND and TND keys past ``seqused_k``, the
tail rows of a partly used paged block, unused physical blocks) is filled with
a poison value of +30 so any out-of-length read shows up as a dominant score.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

DTYPE_STORAGE = {
    "f16": np.uint16,
    "bf16": np.uint16,
    "f32": np.float32,
    "e4m3fn": np.uint8,
    "i8": np.int8,
}
QUANT_DTYPES = ("e4m3fn", "i8")
E4M3FN_MAX = 448.0
I8_MAX = 127.0
POISON = 30.0
SEED_BASE = 0x4C49_0000_0000_0000


# --------------------------------------------------------------------------
# float32 -> storage encoders (input rounding only)
# --------------------------------------------------------------------------
def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def encode_f16(x: np.ndarray) -> np.ndarray:
    """float32 -> binary16 bit patterns (numpy's cast rounds to nearest even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn codes, round-to-nearest-even, saturating at +-448."""
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32),
                                 -E4M3FN_MAX, E4M3FN_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def encode_i8(x: np.ndarray) -> np.ndarray:
    """float32 -> int8 codes, round-half-even, saturating at +-127."""
    return np.clip(np.rint(x), -I8_MAX, I8_MAX).astype(np.int8)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return encode_f16(x)
    if dtype == "bf16":
        return encode_bf16(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"no plain encoder for {dtype}")


def quantize_per_row(x: np.ndarray, dtype: str):
    """Per-row symmetric quantisation over the last axis.

    scale = absmax / QMAX (1 where the row is all zero); code = enc(x / scale).
    Returns (codes, scales) with scales of shape x.shape[:-1], float32.
    """
    qmax = E4M3FN_MAX if dtype == "e4m3fn" else I8_MAX
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(qmax), np.float32(1.0)).astype(np.float32)
    y = x / scale[..., None]
    codes = encode_e4m3fn(y) if dtype == "e4m3fn" else encode_i8(y)
    return codes, scale


# --------------------------------------------------------------------------
# Workload container
# --------------------------------------------------------------------------
@dataclass
class Workload:
    """One seeded indexer problem: attributes + host arrays (storage dtypes)."""

    name: str
    layout_q: str            # "BSND" | "TND"
    layout_k: str            # "BSND" | "TND" | "PA_BSND"
    qk_dtype: str            # "f16" | "bf16" | "e4m3fn" | "i8"
    w_dtype: str             # "f16" | "bf16" | "f32"
    B: int
    S1: int                  # BSND query seq dim (max over batch for TND)
    S2: int                  # BSND key seq dim (max over batch for TND / PA)
    N1: int
    N2: int
    D: int
    sparse_count: int
    sparse_mode: int
    return_value: bool
    seqlens_q: np.ndarray    # (B,) actual query lengths
    seqlens_k: np.ndarray    # (B,) actual key lengths
    q: np.ndarray
    k: np.ndarray
    w: np.ndarray
    q_scale: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    cu_seqlens_q: Optional[np.ndarray] = None
    cu_seqlens_k: Optional[np.ndarray] = None
    seqused_q: Optional[np.ndarray] = None
    seqused_k: Optional[np.ndarray] = None
    block_table: Optional[np.ndarray] = None
    block_size: int = 0
    cmp_ratio: int = 1                          # key compression ratio (1: none)
    cmp_residual_k: Optional[np.ndarray] = None  # (B,) leftover original tokens
    output_idx_offset: Optional[np.ndarray] = None  # (B,) added to returned indices
    block_len: int = 1                          # keys per selected block (1: tokens)
    init_num: int = 0                           # leading blocks always kept
    local_num: int = 0                          # trailing visible blocks always kept
    seed: int = 0
    notes: Dict[str, object] = field(default_factory=dict)

    @property
    def quant(self) -> bool:
        return self.qk_dtype in QUANT_DTYPES

    @property
    def T1(self) -> int:
        return int(self.q.shape[0]) if self.layout_q == "TND" else self.B * self.S1

    @property
    def num_rows(self) -> int:
        """Output rows: B*S1 for BSND queries, T1 for TND."""
        return self.T1

    def row_of(self, b: int, i: int) -> int:
        if self.layout_q == "TND":
            return int(self.cu_seqlens_q[b]) + i
        return b * self.S1 + i


# --------------------------------------------------------------------------
# Generic seeded builder
# --------------------------------------------------------------------------
class _Draw:
    """Seeded normal draws in a fixed order (one torch CPU generator)."""

    def __init__(self, seed: int):
        self.g = torch.Generator().manual_seed(int(seed) & ((1 << 63) - 1))

    def normal(self, shape: Sequence[int], std: float = 1.0) -> np.ndarray:
        x = torch.randn(tuple(int(s) for s in shape), generator=self.g, dtype=torch.float32)
        if std != 1.0:
            x.mul_(float(std))
        return x.numpy()

    def integers(self, lo: int, hi: int, n: int) -> np.ndarray:
        """n integers uniform in [lo, hi] inclusive."""
        return torch.randint(lo, hi + 1, (n,), generator=self.g, dtype=torch.int64).numpy()

    def permutation(self, n: int) -> np.ndarray:
        return torch.randperm(n, generator=self.g).numpy()


def _encode_qk(x: np.ndarray, dtype: str):
    if dtype in QUANT_DTYPES:
        return quantize_per_row(x, dtype)
    return encode(x, dtype), None


def _poison_code(dtype: str):
    if dtype in QUANT_DTYPES:
        c, _ = quantize_per_row(np.full((1, 1), POISON, np.float32), dtype)
        return c.reshape(())  # scale of a poison row is set to 1 below
    return encode(np.array(POISON, np.float32), dtype)


def build(name: str, *, layout_q: str, layout_k: str, qk_dtype: str, w_dtype: str,
          N1: int, D: int, seqlens_q: Sequence[int], seqlens_k: Sequence[int],
          sparse_count: int, sparse_mode: int, return_value: bool = False,
          N2: int = 1, S1: Optional[int] = None, S2: Optional[int] = None,
          block_size: int = 128, max_blocks: Optional[int] = None,
          w_std: float = 1.0, seed: int = 0,
          pass_seqused_q: Optional[bool] = None,
          pass_seqused_k: Optional[bool] = None,
          cmp_ratio: int = 1, cmp_residual_k: Optional[Sequence[int]] = None,
          output_idx_offset: Optional[Sequence[int]] = None, block_len: int = 1,
          init_num: int = 0, local_num: int = 0,
          padded_q: Optional[Sequence[int]] = None,
          padded_k: Optional[Sequence[int]] = None) -> Workload:
    """Draw one problem. Draw order: q, k, w, then the paged block permutation.

    seqlens_q / seqlens_k are the actual lengths. padded_q / padded_k (TND
    only) are the rows each sequence is allotted in the packed tensor (the
    cu_seqlens differences, each >= the actual length); the actual lengths are
    then passed as seqused_q / seqused_k (the V2 guide's TND padding), query
    rows in between are padding rows and keys in between are poisoned."""
    if layout_k != "PA_BSND" and layout_k != layout_q:
        raise ValueError("non-paged key layout must equal the query layout")
    sl_q = np.asarray(seqlens_q, dtype=np.int32)
    sl_k = np.asarray(seqlens_k, dtype=np.int32)
    B = int(sl_q.shape[0])
    assert sl_k.shape == (B,)
    if padded_q is not None:
        assert layout_q == "TND"
        pad_q = np.asarray(padded_q, dtype=np.int32)
        assert pad_q.shape == (B,) and (pad_q >= sl_q).all()
    if padded_k is not None:
        assert layout_k == "TND"
        pad_k = np.asarray(padded_k, dtype=np.int32)
        assert pad_k.shape == (B,) and (pad_k >= sl_k).all()
    dr = _Draw(seed)
    wl_kw = {}

    # ---------------- query ----------------
    if layout_q == "TND":
        cu_q = np.zeros(B + 1, np.int32)
        cu_q[1:] = np.cumsum(sl_q if padded_q is None else pad_q)
        T1 = int(cu_q[-1])
        qf = dr.normal((T1, N1, D))
        S1v = int(sl_q.max()) if B else 0
        wl_kw["cu_seqlens_q"] = cu_q
        if padded_q is not None:
            wl_kw["seqused_q"] = sl_q.copy()
    else:
        S1v = int(S1) if S1 is not None else int(sl_q.max())
        assert (sl_q <= S1v).all()
        qf = dr.normal((B, S1v, N1, D))
        use = pass_seqused_q if pass_seqused_q is not None else bool((sl_q < S1v).any())
        if use:
            wl_kw["seqused_q"] = sl_q.copy()
        else:
            assert (sl_q == S1v).all()
    q, q_scale = _encode_qk(qf, qk_dtype)
    del qf

    # ---------------- key ----------------
    if layout_k == "TND":
        cu_k = np.zeros(B + 1, np.int32)
        cu_k[1:] = np.cumsum(sl_k if padded_k is None else pad_k)
        kf = dr.normal((int(cu_k[-1]), N2, D))
        S2v = int(sl_k.max()) if B else 0
        wl_kw["cu_seqlens_k"] = cu_k
        if padded_k is not None:
            for b in range(B):                   # never-read padding
                kf[int(cu_k[b]) + int(sl_k[b]):int(cu_k[b + 1])] = POISON
            wl_kw["seqused_k"] = sl_k.copy()
        k, k_scale = _encode_qk(kf, qk_dtype)
    elif layout_k == "BSND":
        S2v = int(S2) if S2 is not None else int(sl_k.max())
        assert (sl_k <= S2v).all()
        kf = dr.normal((B, S2v, N2, D))
        for b in range(B):                       # never-read padding
            kf[b, int(sl_k[b]):] = POISON
        k, k_scale = _encode_qk(kf, qk_dtype)
        use = pass_seqused_k if pass_seqused_k is not None else bool((sl_k < S2v).any())
        if use:
            wl_kw["seqused_k"] = sl_k.copy()
        else:
            assert (sl_k == S2v).all()
    else:  # PA_BSND
        assert block_size % 16 == 0 and 16 <= block_size <= 1024
        nblk = [(int(s) + block_size - 1) // block_size for s in sl_k]
        pool = int(sum(nblk))
        S2v = int(sl_k.max()) if B else 0
        mb = int(max_blocks) if max_blocks is not None else max(1, max(nblk) if nblk else 1)
        assert mb >= max(nblk or [0])
        kf = dr.normal((pool, block_size, N2, D))
        k, k_scale = _encode_qk(kf, qk_dtype)
        del kf
        perm = dr.permutation(pool).astype(np.int32)
        bt = np.full((B, mb), -1, np.int32)
        pos = 0
        pc = _poison_code(qk_dtype)
        for b in range(B):
            ids = perm[pos:pos + nblk[b]]
            pos += nblk[b]
            bt[b, :nblk[b]] = ids
            tail = int(sl_k[b]) - (nblk[b] - 1) * block_size
            if nblk[b] and tail < block_size:     # partly used last block
                last = int(ids[-1])
                k[last, tail:] = pc
                if k_scale is not None:
                    k_scale[last, tail:] = 1.0
        wl_kw["block_table"] = bt
        wl_kw["seqused_k"] = sl_k.copy()
        kf = None
    del kf

    # ---------------- weights ----------------
    wshape = (q.shape[0], N1) if layout_q == "TND" else (B, S1v, N1)
    w = encode(dr.normal(wshape, w_std), w_dtype)

    return Workload(name=name, layout_q=layout_q, layout_k=layout_k, qk_dtype=qk_dtype,
                    w_dtype=w_dtype, B=B, S1=S1v, S2=S2v, N1=N1, N2=N2, D=D,
                    sparse_count=int(sparse_count), sparse_mode=int(sparse_mode),
                    return_value=bool(return_value), seqlens_q=sl_q, seqlens_k=sl_k,
                    q=q, k=k, w=w, q_scale=q_scale, k_scale=k_scale,
                    block_size=block_size if layout_k == "PA_BSND" else 0,
                    cmp_ratio=int(cmp_ratio),
                    cmp_residual_k=(None if cmp_residual_k is None
                                    else np.asarray(cmp_residual_k, np.int32)),
                    output_idx_offset=(None if output_idx_offset is None
                                       else np.asarray(output_idx_offset, np.int32)),
                    block_len=int(block_len), init_num=int(init_num), local_num=int(local_num),
                    seed=seed, **wl_kw)


# --------------------------------------------------------------------------
# The five workloads the indexer is measured on (and scaled-down variants)
# --------------------------------------------------------------------------
def _uniform_lengths(seed: int, lo: int, hi: int, n: int) -> np.ndarray:
    return _Draw(seed ^ 0x5EED).integers(lo, hi, n).astype(np.int32)


def tiny_bsnd(seed: int = SEED_BASE + 1) -> Workload:
    """B=1, S1=64, S2=256, N1=8, D=128, fp16 q/k/w ~ N(0,1), k=32, causal, values on."""
    return build("tiny_bsnd", layout_q="BSND", layout_k="BSND", qk_dtype="f16", w_dtype="f16",
                 N1=8, D=128, seqlens_q=[64], seqlens_k=[256], sparse_count=32,
                 sparse_mode=3, return_value=True, seed=seed)


def test_shape(seed: int = SEED_BASE + 2, S1: int = 512, S2: int = 4096,
               sparse_count: int = 1024) -> Workload:
    """B=2, S1=512, S2=4096, N1=G=32, D=64, fp16 q/k, fp32 w, k=1024, no mask."""
    return build("test_shape", layout_q="BSND", layout_k="BSND", qk_dtype="f16", w_dtype="f32",
                 N1=32, D=64, seqlens_q=[S1, S1], seqlens_k=[S2, S2],
                 sparse_count=sparse_count, sparse_mode=0, seed=seed)


def dsa_prefill(seed: int = SEED_BASE + 3, S: int = 8192, sparse_count: int = 2048,
                return_value: bool = False) -> Workload:
    """B=1, S1=S2=8192, N1=64, D=128, bf16 q/k ~N(0,1), bf16 w ~N(0,1)/8, k=2048, causal."""
    return build("dsa_prefill", layout_q="BSND", layout_k="BSND", qk_dtype="bf16",
                 w_dtype="bf16", N1=64, D=128, seqlens_q=[S], seqlens_k=[S],
                 sparse_count=sparse_count, sparse_mode=3, return_value=return_value,
                 w_std=1.0 / 8.0, seed=seed)


def paged_decode(seed: int = SEED_BASE + 4, B: int = 64, lo: int = 4096, hi: int = 65536,
                 block_size: int = 128, max_blocks: Optional[int] = None,
                 sparse_count: int = 2048, return_value: bool = False) -> Workload:
    """B=64 requests x 2 query tokens, N1=64, D=128, bf16, PA_BSND bs=128, S_k~U{4096..65536}."""
    sk = _uniform_lengths(seed, lo, hi, B)
    if max_blocks is None:
        max_blocks = (hi + block_size - 1) // block_size
    return build("paged_decode", layout_q="BSND", layout_k="PA_BSND", qk_dtype="bf16",
                 w_dtype="bf16", N1=64, D=128, seqlens_q=[2] * B, seqlens_k=sk,
                 sparse_count=sparse_count, sparse_mode=3, return_value=return_value,
                 block_size=block_size, max_blocks=max_blocks, w_std=1.0 / 8.0, seed=seed)


def quant_varlen_tnd(seed: int = SEED_BASE + 5, nseq: int = 16, lo: int = 1024,
                     hi: int = 16384, qk_dtype: str = "e4m3fn",
                     sparse_count: int = 2048, return_value: bool = False) -> Workload:
    """16 sequences, L~U{1024..16384}, TND, N1=64, D=128, fp8-e4m3fn per-token-head, fp32 w."""
    L = _uniform_lengths(seed, lo, hi, nseq)
    return build("quant_varlen_tnd", layout_q="TND", layout_k="TND", qk_dtype=qk_dtype,
                 w_dtype="f32", N1=64, D=128, seqlens_q=L, seqlens_k=L,
                 sparse_count=sparse_count, sparse_mode=3, return_value=return_value,
                 seed=seed)


CONFIGS = {
    "tiny_bsnd": tiny_bsnd,
    "test_shape": test_shape,
    "dsa_prefill": dsa_prefill,
    "paged_decode": paged_decode,
    "quant_varlen_tnd": quant_varlen_tnd,
}
