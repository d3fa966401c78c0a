"""Float64 CPU oracle for tiled exact attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle.py`` and ``tests/test_oracle_backward.py``; the causal alignment for T != S is a reading that
the pages do not fix (parity unpinned beyond T == S and the decode case T=1).
"""
from .backward import attention_backward, attention_head_backward, row_dot
from .dense import (attention, attention_head, attention_rows, decode_paged,
                    gather_pages, kv_head_of, masked_scores, scaled_scores,
                    softmax_rows, softmax_rows_unstabilised, visible_mask)

__all__ = [
    "attention_backward", "attention_head_backward", "row_dot",
    "attention", "attention_head", "attention_rows", "decode_paged", "gather_pages",
    "kv_head_of", "masked_scores", "scaled_scores", "softmax_rows",
    "softmax_rows_unstabilised", "visible_mask",
]
