"""ctypes mirror of the C ABI in include/li.h (argument marshalling only).

Every function here has the name of the C entry point it calls. Device
pointers are plain integers (e.g. ``tensor.data_ptr()``); streams are raw
``hipStream_t`` handles as integers (``torch.cuda.current_stream().cuda_stream``).
A non-OK status raises :class:`LIError` carrying the library's message.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libli_mi355x.so")

API_VERSION = 4
INT64_MAX = (1 << 63) - 1

# li_status
OK = 0
ERR_INVALID_ARGUMENT = -1
ERR_UNSUPPORTED = -2
ERR_EMPTY_TENSOR = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_METADATA_MISMATCH = -5
ERR_HIP = -6
ERR_BUFFER_TOO_SMALL = -7
STATUS_NAMES = {
    OK: "LI_OK", ERR_INVALID_ARGUMENT: "LI_ERR_INVALID_ARGUMENT",
    ERR_UNSUPPORTED: "LI_ERR_UNSUPPORTED", ERR_EMPTY_TENSOR: "LI_ERR_EMPTY_TENSOR",
    ERR_WORKSPACE_TOO_SMALL: "LI_ERR_WORKSPACE_TOO_SMALL",
    ERR_METADATA_MISMATCH: "LI_ERR_METADATA_MISMATCH", ERR_HIP: "LI_ERR_HIP",
    ERR_BUFFER_TOO_SMALL: "LI_ERR_BUFFER_TOO_SMALL",
}

# li_layout / li_dtype
LAYOUTS = {"BSND": 0, "TND": 1, "PA_BSND": 2}
DTYPES = {"f16": 0, "bf16": 1, "f32": 2, "e4m3fn": 3, "i8": 4}


class LIError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class li_problem(ctypes.Structure):
    _fields_ = [
        ("api_version", ctypes.c_uint32),
        ("layout_q", ctypes.c_int32),
        ("layout_k", ctypes.c_int32),
        ("dtype_qk", ctypes.c_int32),
        ("dtype_w", ctypes.c_int32),
        ("dtype_scale", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("s1", ctypes.c_int32),
        ("s2", ctypes.c_int32),
        ("n1", ctypes.c_int32),
        ("n2", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("t1", ctypes.c_int64),
        ("t2", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("k_block_stride", ctypes.c_int64),
        ("sparse_count", ctypes.c_int32),
        ("sparse_mode", ctypes.c_int32),
        ("pre_tokens", ctypes.c_int64),
        ("next_tokens", ctypes.c_int64),
        ("return_value", ctypes.c_int32),
        ("cmp_ratio", ctypes.c_int32),
        ("block_len", ctypes.c_int32),
        ("init_num", ctypes.c_int32),
        ("local_num", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 3),
    ]


class li_lengths(ctypes.Structure):
    _fields_ = [
        ("cu_seqlens_q", ctypes.POINTER(ctypes.c_int32)),
        ("cu_seqlens_k", ctypes.POINTER(ctypes.c_int32)),
        ("seqused_q", ctypes.POINTER(ctypes.c_int32)),
        ("seqused_k", ctypes.POINTER(ctypes.c_int32)),
        ("cmp_residual_k", ctypes.POINTER(ctypes.c_int32)),
        ("output_idx_offset", ctypes.POINTER(ctypes.c_int32)),
    ]


class li_inputs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("w", ctypes.c_void_p),
        ("q_scale", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
    ]


def make_problem(*, layout_q="BSND", layout_k="BSND", dtype_qk="bf16", dtype_w="f32",
                 dtype_scale="f32", batch=1, s1=0, s2=0, n1=64, n2=1, d=128, t1=0, t2=0,
                 block_size=0, max_blocks_per_seq=0, num_blocks=0, k_block_stride=0,
                 sparse_count=2048, sparse_mode=3, pre_tokens=INT64_MAX,
                 next_tokens=INT64_MAX, return_value=False, cmp_ratio=1, block_len=1,
                 init_num=0, local_num=0) -> li_problem:
    p = li_problem()
    p.api_version = API_VERSION
    p.layout_q = LAYOUTS[layout_q] if isinstance(layout_q, str) else int(layout_q)
    p.layout_k = LAYOUTS[layout_k] if isinstance(layout_k, str) else int(layout_k)
    p.dtype_qk = DTYPES[dtype_qk] if isinstance(dtype_qk, str) else int(dtype_qk)
    p.dtype_w = DTYPES[dtype_w] if isinstance(dtype_w, str) else int(dtype_w)
    p.dtype_scale = DTYPES[dtype_scale] if isinstance(dtype_scale, str) else int(dtype_scale)
    p.batch, p.s1, p.s2 = int(batch), int(s1), int(s2)
    p.n1, p.n2, p.d = int(n1), int(n2), int(d)
    p.t1, p.t2 = int(t1), int(t2)
    p.block_size, p.max_blocks_per_seq = int(block_size), int(max_blocks_per_seq)
    p.num_blocks, p.k_block_stride = int(num_blocks), int(k_block_stride)
    p.sparse_count, p.sparse_mode = int(sparse_count), int(sparse_mode)
    p.pre_tokens, p.next_tokens = int(pre_tokens), int(next_tokens)
    p.return_value = int(bool(return_value))
    p.cmp_ratio = int(cmp_ratio)
    p.block_len = int(block_len)
    p.init_num, p.local_num = int(init_num), int(local_num)
    return p


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_attention_top_amd.build` "
                "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.li_metadata.argtypes = [P(li_problem), P(li_lengths), ctypes.c_int32, vp, sz, P(sz)]
        L.li_workspace_size.argtypes = [P(li_problem), vp, P(sz)]
        L.li_score.argtypes = [P(li_problem), P(li_inputs), vp, vp, vp, sz, vp]
        L.li_topk.argtypes = [P(li_problem), vp, vp, vp, sz, vp, vp, vp]
        L.li_indexer.argtypes = [P(li_problem), P(li_inputs), vp, vp, vp, sz, vp, vp, vp]
        L.li_indexer_noalloc.argtypes = [P(li_problem), P(li_inputs), vp, vp, vp, vp, vp]
        L.li_noalloc_capacity.argtypes = []
        L.li_noalloc_capacity.restype = sz
        for f in ("li_metadata", "li_workspace_size", "li_score", "li_topk", "li_indexer",
                  "li_indexer_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        L.li_last_error.argtypes = []
        L.li_last_error.restype = ctypes.c_char_p
        L.li_api_version.argtypes = []
        L.li_api_version.restype = ctypes.c_int32
        if L.li_api_version() != API_VERSION:
            raise RuntimeError("library API version mismatch; rebuild it")
        _lib = L
    return _lib


def li_last_error() -> str:
    return lib().li_last_error().decode()


def li_api_version() -> int:
    return int(lib().li_api_version())


def _check(status: int) -> None:
    if status != OK:
        raise LIError(status, li_last_error())


def _i32p(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def make_lengths(cu_seqlens_q=None, cu_seqlens_k=None, seqused_q=None, seqused_k=None,
                 cmp_residual_k=None, output_idx_offset=None):
    """Host lengths: arrays are converted to contiguous int32 and kept alive on the result."""
    keep = [None if a is None else np.ascontiguousarray(np.asarray(a), dtype=np.int32)
            for a in (cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, cmp_residual_k,
                      output_idx_offset)]
    L = li_lengths(*[_i32p(a) for a in keep])
    L._keep = keep  # type: ignore[attr-defined]
    return L


def li_metadata(p: li_problem, lengths: li_lengths, num_cus: int = 256) -> np.ndarray:
    """Build the task table; returns it as a host uint8 array."""
    need = ctypes.c_size_t(0)
    _check(lib().li_metadata(ctypes.byref(p), ctypes.byref(lengths), int(num_cus), None, 0,
                             ctypes.byref(need)))
    buf = np.zeros(max(int(need.value), 16), dtype=np.uint8)
    got = ctypes.c_size_t(0)
    _check(lib().li_metadata(ctypes.byref(p), ctypes.byref(lengths), int(num_cus),
                             buf.ctypes.data, buf.nbytes, ctypes.byref(got)))
    return buf[: int(got.value)]


def li_workspace_size(p: li_problem, meta_host: np.ndarray) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().li_workspace_size(ctypes.byref(p), meta_host.ctypes.data, ctypes.byref(out)))
    return int(out.value)


def make_inputs(q: int, k: int, w: int, q_scale: int = 0, k_scale: int = 0,
                block_table: int = 0) -> li_inputs:
    return li_inputs(q or None, k or None, w or None, q_scale or None, k_scale or None,
                     block_table or None)


def li_score(p: li_problem, inputs: li_inputs, meta_host: np.ndarray, meta_dev: int, ws: int,
             ws_bytes: int, stream: int = 0) -> None:
    _check(lib().li_score(ctypes.byref(p), ctypes.byref(inputs), meta_host.ctypes.data,
                          meta_dev or None, ws or None, int(ws_bytes), stream or None))


def li_topk(p: li_problem, meta_host: np.ndarray, meta_dev: int, ws: int, ws_bytes: int,
            sparse_indices: int, sparse_values: int = 0, stream: int = 0) -> None:
    _check(lib().li_topk(ctypes.byref(p), meta_host.ctypes.data, meta_dev or None, ws or None,
                         int(ws_bytes), sparse_indices or None, sparse_values or None,
                         stream or None))


def li_indexer(p: li_problem, inputs: li_inputs, meta_host: np.ndarray, meta_dev: int, ws: int,
               ws_bytes: int, sparse_indices: int, sparse_values: int = 0,
               stream: int = 0) -> None:
    _check(lib().li_indexer(ctypes.byref(p), ctypes.byref(inputs), meta_host.ctypes.data,
                            meta_dev or None, ws or None, int(ws_bytes), sparse_indices or None,
                            sparse_values or None, stream or None))


def li_indexer_noalloc(p: li_problem, inputs: li_inputs, meta_host: np.ndarray, meta_dev: int,
                       sparse_indices: int, sparse_values: int = 0, stream: int = 0) -> None:
    _check(lib().li_indexer_noalloc(ctypes.byref(p), ctypes.byref(inputs), meta_host.ctypes.data,
                                    meta_dev or None, sparse_indices or None,
                                    sparse_values or None, stream or None))


def li_noalloc_capacity() -> int:
    return int(lib().li_noalloc_capacity())


# Layout of the task table header (mirrors MetaHeader in csrc/li_internal.h),
# for tests and reports only.
TOPK_CLASSES = 4
TOPK_CLASS_KEYS = (8192, 16384, 32768, 0x7FFFFFFF)
META_HEADER_DTYPE = np.dtype([
    ("magic", "<u4"), ("version", "<u4"), ("problem_hash", "<u8"), ("batch", "<i4"),
    ("num_items", "<i4"), ("num_rows", "<i8"), ("variant", "<i4"), ("tile_q", "<i4"),
    ("key_chunk", "<i4"), ("num_cus", "<i4"), ("ws_floats", "<i8"), ("visible_pairs", "<i8"),
    ("off_batches", "<u8"), ("off_items", "<u8"), ("max_sk", "<i4"), ("max_sq", "<i4"),
    ("off_rows", "<u8"), ("row_class", "<i4", (2 * TOPK_CLASSES + 1,)), ("split_rows", "<i4"),
    ("cand_val_off", "<i8"), ("cand_idx_off", "<i8"), ("num_recs", "<i8"),
    ("sparse_count", "<i4"), ("init_num", "<i4"), ("local_num", "<i4"), ("reserved", "<i4"),
])
assert META_HEADER_DTYPE.itemsize == 176
BATCH_REC_DTYPE = np.dtype([("ws_off", "<i8"), ("row_base", "<i4"), ("k_base", "<i4"),
                            ("s_q", "<i4"), ("s_k", "<i4"), ("ld", "<i4"), ("rows", "<i4"),
                            ("cmp_res", "<i4"), ("reserved", "<i4")])
WORK_ITEM_DTYPE = np.dtype([("b", "<i4"), ("q0", "<i4"), ("k0", "<i4"), ("k1", "<i4")])
ROW_REC_DTYPE = np.dtype([("ws_off", "<i8"), ("out_off", "<i8"), ("n", "<i4"),
                          ("idx_offset", "<i4"), ("row", "<i4"), ("kind", "<i4")])
ROW_WHOLE, ROW_CHUNK, ROW_MERGE = 0, 1, 2   # top-k record kinds


def parse_metadata(meta: np.ndarray):
    """(header, batch records, work items) as numpy structured arrays."""
    h = meta[:META_HEADER_DTYPE.itemsize].view(META_HEADER_DTYPE)[0]
    ob, oi = int(h["off_batches"]), int(h["off_items"])
    recs = meta[ob:ob + BATCH_REC_DTYPE.itemsize * int(h["batch"])].view(BATCH_REC_DTYPE)
    items = meta[oi:oi + WORK_ITEM_DTYPE.itemsize * int(h["num_items"])].view(WORK_ITEM_DTYPE)
    return h, recs, items


def parse_row_table(meta: np.ndarray):
    """The top-k records of both passes and their boundaries: pass q, class c is
    records [bounds[q*TOPK_CLASSES + c], bounds[q*TOPK_CLASSES + c + 1])."""
    h = parse_metadata(meta)[0]
    orow = int(h["off_rows"])
    rows = meta[orow:orow + ROW_REC_DTYPE.itemsize * int(h["num_recs"])].view(ROW_REC_DTYPE)
    return rows, np.array(h["row_class"])
