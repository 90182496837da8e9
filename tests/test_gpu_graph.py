"""A captured HIP graph of li_score + li_topk replays to the eager result.

bench.py times graph replays of the step, so the launches must be capture-safe
(no allocation, no memset, no host synchronisation) and every replay must give
what an eager call gives, with the program's own eager work (output fills, an
eager run over the same workspace) between the replays.
"""
import pytest
import torch

from sparse_attention_top_amd import binding as B
from sparse_attention_top_amd import indexer as I
from sparse_attention_top_amd import synth

pytestmark = pytest.mark.gpu

CASES = {
    "prefill": lambda: synth.dsa_prefill(S=1200, sparse_count=256),
    # six rows over 9K-30K keys: split rows, two top-k passes
    "paged_split_rows": lambda: synth.paged_decode(B=3, lo=9000, hi=30000, sparse_count=512),
    "quant_tnd": lambda: synth.quant_varlen_tnd(nseq=3, lo=100, hi=900, sparse_count=128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    wl = CASES[name]()
    print(f"[gpu] graph replay: {name} rows={wl.num_rows}", flush=True)
    dw = I.upload(wl, "cuda", return_value=True)
    plan = I.make_plan(dw.problem, dw.lengths, "cuda")
    p, inp = dw.problem, dw.inputs()
    shape = I.output_shape(p)

    def outputs():
        return (torch.empty(shape, dtype=torch.int32, device="cuda"),
                torch.empty(shape, dtype=torch.float32, device="cuda"))

    def run(idx, val):
        s = int(torch.cuda.current_stream().cuda_stream)
        md, ws = int(plan.meta_dev.data_ptr()), int(plan.ws.data_ptr())
        B.li_score(p, inp, plan.meta_host, md, ws, plan.ws_bytes, s)
        B.li_topk(p, plan.meta_host, md, ws, plan.ws_bytes, int(idx.data_ptr()),
                  int(val.data_ptr()), s)

    ei, ev = outputs()
    run(ei, ev)
    torch.cuda.synchronize()
    gi, gv = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(gi, gv)
    xi, xv = outputs()
    for rep in range(3):
        gi.fill_(-7)
        gv.fill_(1.5)
        run(xi, xv)   # eager work over the same workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gi, ei) and torch.equal(gv, ev), f"replay {rep} differs"
        assert torch.equal(xi, ei) and torch.equal(xv, ev)
