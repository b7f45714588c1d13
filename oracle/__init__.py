"""FP64 CPU oracle -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The HIP path never does.
"""

from .gvattn_oracle import (  # noqa: F401
    SCORE_BUDGET_BYTES,
    attention_flops,
    attention_bwd,
    attention_bwd_magnitudes,
    attention_fwd,
    attention_fwd_ranges,
    bits_equal,
    host_cores,
    lse_merge,
    segment_head_rows,
    segment_key_rows,
    visible_limit,
)
