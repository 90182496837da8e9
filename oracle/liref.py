"""ctypes wrapper of the plain C++17 fp64 oracle (li_oracle.cpp).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the CPU baseline of the benchmark use it. It takes a seeded workload
(the host arrays of sparse_attention_top_amd.synth, read by attribute) and
returns the operator's outputs; the arithmetic is all in li_oracle.cpp.

    python -m oracle.liref        # builds oracle/libliref.so with g++
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys
from typing import Iterable, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "li_oracle.cpp")
LIB = os.path.join(_HERE, "libliref.so")

_LAYOUT = {"BSND": 0, "TND": 1, "PA_BSND": 2}
_DTYPE = {"f16": 0, "bf16": 1, "f32": 2, "e4m3fn": 3, "i8": 4}


class liref_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("layout_q", "layout_k", "dtype_qk", "dtype_w",
                                              "batch", "s1", "s2", "n1", "n2", "d")] + \
               [("t1", ctypes.c_int64), ("t2", ctypes.c_int64)] + \
               [(n, ctypes.c_int32) for n in ("block_size", "max_blocks", "sparse_count",
                                              "sparse_mode", "cmp_ratio", "block_len",
                                              "init_num", "local_num")]


class liref_inputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q", "k", "w", "q_scale", "k_scale", "cu_seqlens_q", "cu_seqlens_k", "seqused_q",
        "seqused_k", "block_table", "cmp_residual_k", "output_idx_offset")]


def build(verbose: bool = False) -> str:
    """Compile the oracle with g++ (plain C++17, no GPU code)."""
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        L.liref_run.argtypes = [ctypes.POINTER(liref_problem), ctypes.POINTER(liref_inputs),
                                ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_int]
        L.liref_run.restype = ctypes.c_int
        L.liref_num_rows.argtypes = [ctypes.POINTER(liref_problem)]
        L.liref_num_rows.restype = ctypes.c_int64
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray], keep: list) -> Optional[int]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    keep.append(a)
    return a.ctypes.data


def run(wl, rows: Optional[Iterable[Tuple[int, int]]] = None,
        nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray, int]:
    """(indices (R, N2, k) int32, values (R, N2, k) float32, threads used) for
    `rows` ((b, i) pairs; every row of the problem, in order, when None)."""
    p = liref_problem()
    p.layout_q, p.layout_k = _LAYOUT[wl.layout_q], _LAYOUT[wl.layout_k]
    p.dtype_qk, p.dtype_w = _DTYPE[wl.qk_dtype], _DTYPE[wl.w_dtype]
    p.batch, p.n1, p.n2, p.d = int(wl.B), int(wl.N1), int(wl.N2), int(wl.D)
    if wl.layout_q == "TND":
        p.t1 = int(wl.q.shape[0])
    else:
        p.s1 = int(wl.q.shape[1])
    if wl.layout_k == "TND":
        p.t2 = int(wl.k.shape[0])
    elif wl.layout_k == "BSND":
        p.s2 = int(wl.k.shape[1])
    else:
        p.block_size = int(wl.k.shape[1])
        p.max_blocks = int(wl.block_table.shape[1])
    p.sparse_count, p.sparse_mode = int(wl.sparse_count), int(wl.sparse_mode)
    p.cmp_ratio = int(getattr(wl, "cmp_ratio", 1) or 1)
    p.block_len = int(getattr(wl, "block_len", 1) or 1)
    p.init_num = int(getattr(wl, "init_num", 0) or 0)
    p.local_num = int(getattr(wl, "local_num", 0) or 0)
    keep: list = []
    i32 = lambda a: None if a is None else np.asarray(a, np.int32)
    f32 = lambda a: None if a is None else np.asarray(a, np.float32)
    inp = liref_inputs(_ptr(wl.q, keep), _ptr(wl.k, keep), _ptr(wl.w, keep),
                       _ptr(f32(wl.q_scale), keep), _ptr(f32(wl.k_scale), keep),
                       _ptr(i32(wl.cu_seqlens_q), keep), _ptr(i32(wl.cu_seqlens_k), keep),
                       _ptr(i32(wl.seqused_q), keep), _ptr(i32(wl.seqused_k), keep),
                       _ptr(i32(wl.block_table), keep),
                       _ptr(i32(getattr(wl, "cmp_residual_k", None)), keep),
                       _ptr(i32(getattr(wl, "output_idx_offset", None)), keep))
    if rows is None:
        rp, nrows = None, int(lib().liref_num_rows(ctypes.byref(p)))
    else:
        ra = np.ascontiguousarray(np.asarray(list(rows), np.int32).reshape(-1, 2))
        rp, nrows = _ptr(ra, keep), ra.shape[0]
    idx = np.empty((nrows, p.n2, p.sparse_count), np.int32)
    val = np.empty((nrows, p.n2, p.sparse_count), np.float32)
    used = lib().liref_run(ctypes.byref(p), ctypes.byref(inp), rp, nrows, idx.ctypes.data,
                           val.ctypes.data, int(nthreads))
    if used < 0:
        raise RuntimeError("liref_run rejected the problem")
    return idx, val, used


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
