"""torch-facing wrapper of the C ABI.

torch supplies device memory and the current HIP stream; every step of the
indexer runs in the library's kernels. The keyword interface mirrors the
MindSpore ``lightning_indexer`` page (its signature and parameter list):
``actual_seq_lengths_query`` / ``actual_seq_lengths_key`` are per-batch
lengths for BSND and PA_BSND, and prefix sums without the leading zero for
TND; ``sparse_values`` comes back with shape (0,) when ``return_value`` is
False (CANN V2 guide, return value section). The V2 guide's compressed keys
(``cmp_ratio``, ``cmp_residual_k``) and per-batch ``output_idx_offset`` are
accepted as keywords too, and so are the key-block routing options the
ops-transformer issue lists for the forward operator (``block_len``,
``init_num``, ``local_num``).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import binding as B

_QK_DTYPES = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "e4m3fn",
              torch.int8: "i8"}
_W_DTYPES = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}
_STORAGE_TO_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32,
                     "e4m3fn": torch.float8_e4m3fn, "i8": torch.int8}


@dataclass
class Plan:
    """Task table (host + device copies) and workspace for one problem."""

    problem: B.li_problem
    meta_host: np.ndarray
    meta_dev: torch.Tensor
    ws: torch.Tensor
    ws_bytes: int

    @property
    def header(self):
        return B.parse_metadata(self.meta_host)[0]


def make_plan(problem: B.li_problem, lengths: B.li_lengths, device, num_cus: int = 256) -> Plan:
    meta = B.li_metadata(problem, lengths, num_cus)
    meta_dev = torch.from_numpy(meta.copy()).to(device)
    ws_bytes = B.li_workspace_size(problem, meta)
    ws = torch.empty((ws_bytes + 3) // 4, dtype=torch.float32, device=device)
    return Plan(problem, meta, meta_dev, ws, ws_bytes)


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_handle(device) -> int:
    return int(torch.cuda.current_stream(device).cuda_stream)


def _host_i32(t) -> Optional[np.ndarray]:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(t), dtype=np.int32)


def lightning_indexer(query: torch.Tensor, key: torch.Tensor, weights: torch.Tensor, *,
                      sparse_count: int = 2048,
                      actual_seq_lengths_query=None, actual_seq_lengths_key=None,
                      block_table: Optional[torch.Tensor] = None,
                      layout_query: str = "BSND", layout_key: str = "BSND",
                      sparse_mode: int = 3, pre_tokens: int = B.INT64_MAX,
                      next_tokens: int = B.INT64_MAX, return_value: bool = False,
                      query_dequant_scale: Optional[torch.Tensor] = None,
                      key_dequant_scale: Optional[torch.Tensor] = None,
                      cmp_ratio: int = 1, cmp_residual_k=None, output_idx_offset=None,
                      block_len: int = 1, init_num: int = 0, local_num: int = 0,
                      plan: Optional[Plan] = None, num_cus: int = 256):
    """Top-k key indices (int32) and optionally values (float32) per query token."""
    dev = query.device
    if query.dtype not in _QK_DTYPES or key.dtype != query.dtype:
        raise TypeError("query and key must share one of float16, bfloat16, float8_e4m3fn, int8")
    if weights.dtype not in _W_DTYPES:
        raise TypeError("weights must be float16, bfloat16 or float32")
    dt = _QK_DTYPES[query.dtype]
    query = query.contiguous()
    weights = weights.contiguous()
    if layout_key == "PA_BSND":
        if key.dim() != 4 or key.stride(3) != 1 or key.stride(2) != key.shape[3] or \
                key.stride(1) != key.shape[2] * key.shape[3]:
            raise ValueError("paged key must be contiguous within each block")
        k_block_stride = int(key.stride(0))
    else:
        key = key.contiguous()
        k_block_stride = 0
    if layout_query == "TND":
        t1, n1, d = query.shape
        b_sz, s1 = 0, 0
    else:
        b_sz, s1, n1, d = query.shape
        t1 = 0
    kw = dict(layout_q=layout_query, layout_k=layout_key, dtype_qk=dt,
              dtype_w=_W_DTYPES[weights.dtype], n1=n1, d=d, sparse_count=sparse_count,
              sparse_mode=sparse_mode, pre_tokens=pre_tokens, next_tokens=next_tokens,
              return_value=return_value, cmp_ratio=cmp_ratio, block_len=block_len,
              init_num=init_num, local_num=local_num)
    aq = _host_i32(actual_seq_lengths_query)
    ak = _host_i32(actual_seq_lengths_key)
    cu_q = cu_k = used_q = used_k = None
    if layout_query == "TND":
        if aq is None:
            raise ValueError("TND queries need actual_seq_lengths_query (prefix sums)")
        cu_q = np.concatenate([[0], aq]).astype(np.int32)
        b_sz = aq.shape[0]
    else:
        used_q = aq
    if layout_key == "TND":
        if ak is None:
            raise ValueError("TND keys need actual_seq_lengths_key (prefix sums)")
        cu_k = np.concatenate([[0], ak]).astype(np.int32)
        kw.update(t2=key.shape[0], n2=key.shape[1])
    elif layout_key == "BSND":
        used_k = ak
        kw.update(s2=key.shape[1], n2=key.shape[2])
    else:
        used_k = ak
        if block_table is None:
            raise ValueError("PA_BSND keys need block_table")
        kw.update(block_size=key.shape[1], n2=key.shape[2], num_blocks=key.shape[0],
                  max_blocks_per_seq=block_table.shape[1], k_block_stride=k_block_stride)
    kw.update(batch=b_sz, s1=s1, t1=t1)
    p = B.make_problem(**kw)
    if plan is None:
        plan = make_plan(p, B.make_lengths(cu_q, cu_k, used_q, used_k, _host_i32(cmp_residual_k),
                                           _host_i32(output_idx_offset)), dev, num_cus)
    n2 = p.n2
    rows = (b_sz, s1, n2, sparse_count) if layout_query == "BSND" else (t1, n2, sparse_count)
    idx = torch.empty(rows, dtype=torch.int32, device=dev)
    val = torch.empty(rows if return_value else (0,), dtype=torch.float32, device=dev)
    qs = query_dequant_scale.contiguous() if query_dequant_scale is not None else None
    ks = key_dequant_scale.contiguous() if key_dequant_scale is not None else None
    bt = block_table.contiguous() if block_table is not None else None
    inp = B.make_inputs(_ptr(query), _ptr(key), _ptr(weights), _ptr(qs), _ptr(ks), _ptr(bt))
    B.li_indexer(p, inp, plan.meta_host, _ptr(plan.meta_dev), _ptr(plan.ws), plan.ws_bytes,
                 _ptr(idx), _ptr(val) if return_value else 0, _stream_handle(dev))
    return idx, val


# ---------------------------------------------------------------------------
# Seeded workloads (sparse_attention_top_amd.synth) on the device
# ---------------------------------------------------------------------------
def to_device(arr: Optional[np.ndarray], dtype: str, device) -> Optional[torch.Tensor]:
    """Host storage array (see synth) -> device tensor of the matching torch dtype."""
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if dtype in ("f16", "bf16"):
        t = torch.from_numpy(a.view(np.int16)).view(_STORAGE_TO_TORCH[dtype])
    elif dtype == "e4m3fn":
        t = torch.from_numpy(a.view(np.uint8)).view(torch.float8_e4m3fn)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


@dataclass
class DeviceWorkload:
    problem: B.li_problem
    lengths: B.li_lengths
    q: torch.Tensor
    k: torch.Tensor
    w: torch.Tensor
    q_scale: Optional[torch.Tensor]
    k_scale: Optional[torch.Tensor]
    block_table: Optional[torch.Tensor]

    def inputs(self) -> B.li_inputs:
        return B.make_inputs(_ptr(self.q), _ptr(self.k), _ptr(self.w), _ptr(self.q_scale),
                             _ptr(self.k_scale), _ptr(self.block_table))


def problem_of(wl, return_value: Optional[bool] = None) -> B.li_problem:
    rv = wl.return_value if return_value is None else return_value
    kw = dict(layout_q=wl.layout_q, layout_k=wl.layout_k, dtype_qk=wl.qk_dtype,
              dtype_w=wl.w_dtype, batch=wl.B, n1=wl.N1, n2=wl.N2, d=wl.D,
              sparse_count=wl.sparse_count, sparse_mode=wl.sparse_mode, return_value=rv,
              cmp_ratio=getattr(wl, "cmp_ratio", 1), block_len=getattr(wl, "block_len", 1),
              init_num=getattr(wl, "init_num", 0), local_num=getattr(wl, "local_num", 0))
    if wl.layout_q == "TND":
        kw["t1"] = int(wl.q.shape[0])
    else:
        kw["s1"] = int(wl.q.shape[1])
    if wl.layout_k == "TND":
        kw["t2"] = int(wl.k.shape[0])
    elif wl.layout_k == "BSND":
        kw["s2"] = int(wl.k.shape[1])
    else:
        kw.update(block_size=int(wl.k.shape[1]), num_blocks=int(wl.k.shape[0]),
                  max_blocks_per_seq=int(wl.block_table.shape[1]))
    return B.make_problem(**kw)


def upload(wl, device="cuda", return_value: Optional[bool] = None) -> DeviceWorkload:
    p = problem_of(wl, return_value)
    L = B.make_lengths(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.seqused_q, wl.seqused_k,
                       getattr(wl, "cmp_residual_k", None), getattr(wl, "output_idx_offset", None))
    bt = None if wl.block_table is None else torch.from_numpy(wl.block_table).to(device)
    return DeviceWorkload(p, L, to_device(wl.q, wl.qk_dtype, device),
                          to_device(wl.k, wl.qk_dtype, device),
                          to_device(wl.w, wl.w_dtype, device),
                          to_device(wl.q_scale, "f32", device),
                          to_device(wl.k_scale, "f32", device), bt)


def output_shape(p: B.li_problem):
    if p.layout_q == B.LAYOUTS["BSND"]:
        return (p.batch, p.s1, p.n2, p.sparse_count)
    return (p.t1, p.n2, p.sparse_count)


def run_workload(wl, device="cuda", return_value: Optional[bool] = None, num_cus: int = 256):
    """Upload a seeded workload, run the indexer once, return (idx, val, plan, dev_workload)."""
    dw = upload(wl, device, return_value)
    plan = make_plan(dw.problem, dw.lengths, device, num_cus)
    shape = output_shape(dw.problem)
    idx = torch.empty(shape, dtype=torch.int32, device=device)
    val = torch.empty(shape if dw.problem.return_value else (0,), dtype=torch.float32,
                      device=device)
    B.li_indexer(dw.problem, dw.inputs(), plan.meta_host, _ptr(plan.meta_dev), _ptr(plan.ws),
                 plan.ws_bytes, _ptr(idx), _ptr(val) if dw.problem.return_value else 0,
                 _stream_handle(device))
    return idx, val, plan, dw
