"""fp64 CPU oracle of the LightningIndexer forward pass (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package. The product path never does.
"""
from .li_oracle import (  # noqa: F401
    all_rows, batch_lengths, decode, decode_bf16, decode_e4m3fn, decode_f16,
    decode_f32, decode_i8, row_scores, run, run_full, topk_order, visible_count,
)
