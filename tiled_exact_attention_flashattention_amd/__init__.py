"""Tiled exact attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libattn.so`` (hand-written HIP kernels behind the C ABI
of ``include/attn.h``); this package is its thin Python binding.  Importing it
does not load the library; the first call does, and raises if the library has
not been built (``python -m tiled_exact_attention_flashattention_amd.build``).
"""
from ._binding import (ATTN_BF16, ATTN_EHIP, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_F32,
                       ATTN_OK, PAGE, AttnError, attn_bwd, attn_bwd_workspace_size,
                       attn_decode_paged, attn_decode_paged_fp8, attn_decode_paged_int8,
                       attn_decode_paged_noalloc,
                       attn_decode_workspace_size,
                       attn_fwd, attn_fwd_window, attn_last_error, attn_prefill_paged,
                       attn_status_string, attn_time_next_call, bwd, check_paged_inputs,
                       decode_paged,
                       decode_workspace, fwd, lib, library_path)

__all__ = [
    "ATTN_BF16", "ATTN_EHIP", "ATTN_EINVAL", "ATTN_EUNSUPPORTED", "ATTN_F32", "ATTN_OK", "PAGE",
    "AttnError", "attn_bwd", "attn_bwd_workspace_size", "attn_decode_paged", "attn_decode_paged_fp8",
    "attn_decode_paged_int8", "attn_decode_paged_noalloc",
    "attn_decode_workspace_size", "attn_fwd", "attn_fwd_window", "attn_last_error",
    "attn_prefill_paged", "attn_status_string", "attn_time_next_call", "bwd", "check_paged_inputs",
    "decode_paged", "decode_workspace", "fwd", "lib", "library_path",
]
