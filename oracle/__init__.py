"""CPU oracle for sparse-MLA prefill (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never calls it and shares no code with it.
"""
from .spmla_oracle import (  # noqa: F401
    INVISIBLE,
    attend_one,
    compress_rows,
    indexer_scores,
    key_rows,
    n_compressed,
    n_visible,
    prefill,
    select_one,
    sparse_attention,
    topk_select,
    window_range,
)
