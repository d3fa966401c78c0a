"""Float64 CPU oracle for tiled exact attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle.py``, ``tests/test_oracle_backward.py`` and
``tests/test_oracle_next.py``; the causal alignment for T != S is a reading
that the pages do not fix (parity unpinned beyond T == S and the decode case
T=1), and so are the sliding-window rule and the fp8 and int8 page formats,
which the pages only name.
"""
from .backward import attention_backward, attention_head_backward, row_dot
from .dense import (attention, attention_head, attention_rows, decode_paged,
                    gather_pages, kv_head_of, masked_scores, prefill_paged, scaled_scores,
                    softmax_rows, softmax_rows_unstabilised, visible_mask)
from .quant import (decode_paged_fp8, decode_paged_int8, dequantise, dequantise_int8,
                    e4m3_to_float, int8_to_float)

__all__ = [
    "attention_backward", "attention_head_backward", "row_dot",
    "attention", "attention_head", "attention_rows", "decode_paged", "gather_pages",
    "kv_head_of", "masked_scores", "prefill_paged", "scaled_scores", "softmax_rows",
    "softmax_rows_unstabilised", "visible_mask",
    "decode_paged_fp8", "dequantise", "e4m3_to_float",
    "decode_paged_int8", "dequantise_int8", "int8_to_float",
]
