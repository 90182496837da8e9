"""li_indexer_noalloc: li_indexer on the library's own device scratch.

It must give exactly what li_indexer gives with a caller workspace (same
kernels, same task table), call after call on the shared array -- the second
call here is smaller than the first -- and reject a problem whose workspace
exceeds the array before anything is enqueued.
"""
import numpy as np
import pytest
import torch

from sparse_attention_top_amd import binding as B
from sparse_attention_top_amd import indexer as I
from sparse_attention_top_amd import synth


def _noalloc(wl, device="cuda"):
    dw = I.upload(wl, device)
    meta = B.li_metadata(dw.problem, dw.lengths)
    meta_dev = torch.from_numpy(meta.copy()).to(device)
    shape = I.output_shape(dw.problem)
    idx = torch.empty(shape, dtype=torch.int32, device=device)
    val = torch.empty(shape if dw.problem.return_value else (0,), dtype=torch.float32,
                      device=device)
    need = B.li_workspace_size(dw.problem, meta)
    print(f"[gpu] noalloc {wl.name}: workspace {need} of {B.li_noalloc_capacity()} bytes",
          flush=True)
    B.li_indexer_noalloc(dw.problem, dw.inputs(), meta, int(meta_dev.data_ptr()),
                         int(idx.data_ptr()), int(val.data_ptr()) if dw.problem.return_value else 0,
                         int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return idx, val, need


@pytest.mark.gpu
def test_noalloc_equals_caller_workspace_twice():
    """Three calls in a row on the one array, each smaller than the one before:
    the full 8K causal prefill (the whole 256 MiB), a 3000-token prefill with
    values, and a paged decode whose long rows are split (candidate lists in
    the workspace). Each equals li_indexer bit for bit."""
    cases = [synth.dsa_prefill(),
             synth.dsa_prefill(S=3000, sparse_count=512, return_value=True),
             synth.paged_decode(B=6, lo=3000, hi=20000, sparse_count=512, return_value=True)]
    last = None
    for wl in cases:
        i_ref, v_ref, plan, _ = I.run_workload(wl, "cuda")
        torch.cuda.synchronize()
        i_na, v_na, need = _noalloc(wl)
        assert need == plan.ws_bytes
        assert last is None or need < last
        last = need
        assert torch.equal(i_na, i_ref), f"{wl.name}: indices differ"
        assert torch.equal(v_na, v_ref), f"{wl.name}: values differ"
    assert int(plan.header["split_rows"]) > 0


def test_noalloc_rejects_oversized_problem():
    """A prefill one row past 8192 needs more than the array: rejected with
    LI_ERR_WORKSPACE_TOO_SMALL before any HIP call (so this runs without a GPU)."""
    p = B.make_problem(layout_q="BSND", layout_k="BSND", dtype_qk="bf16", dtype_w="bf16",
                       batch=1, s1=8193, s2=8193, n1=64, d=128, sparse_count=2048,
                       sparse_mode=3)
    meta = B.li_metadata(p, B.make_lengths())
    assert B.li_workspace_size(p, meta) > B.li_noalloc_capacity()
    fake = 1 << 20   # never dereferenced
    inp = B.make_inputs(fake, fake, fake)
    with pytest.raises(B.LIError) as e:
        B.li_indexer_noalloc(p, inp, meta, fake, fake, 0)
    assert e.value.status == B.ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in B.li_last_error()
    # the headline prefill fits exactly
    q = B.make_problem(layout_q="BSND", layout_k="BSND", dtype_qk="bf16", dtype_w="bf16",
                       batch=1, s1=8192, s2=8192, n1=64, d=128, sparse_count=2048,
                       sparse_mode=3)
    assert B.li_workspace_size(q, B.li_metadata(q, B.make_lengths())) <= \
        B.li_noalloc_capacity() == 256 << 20
    # a table of another problem is rejected the same way as by li_indexer
    with pytest.raises(B.LIError) as e:
        B.li_indexer_noalloc(q, inp, meta, fake, fake, 0)
    assert e.value.status == B.ERR_METADATA_MISMATCH
