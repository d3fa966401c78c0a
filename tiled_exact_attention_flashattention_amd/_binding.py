"""ctypes binding of libattn.so: argument marshalling only.

Each function mirrors one entry point of ``include/attn.h`` under the same
name.  Tensors are PyTorch tensors on a ROCm device; this module only reads
their shapes, dtypes, devices and data pointers, picks the caller's current
stream, and turns a non-OK status into :class:`AttnError`.  All computation
happens in the HIP kernels.  If the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP = 0, 1, 2, 3
ATTN_F32, ATTN_BF16 = 0, 1
PAGE = 16

_LIB = None


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{attn_status_string(status)} ({detail})")


def library_path() -> str:
    return LIB_PATH


def hip_runtimes_loaded() -> list:
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                    paths.add(os.path.realpath(parts[-1]))
    except OSError:
        pass
    return sorted(paths)


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it was never built).

    torch is imported first so that its HIP runtime is the one in the process:
    libattn.so asks for ``libamdhip64.so.7``, which the loader then satisfies
    with torch's copy (same SONAME).  Loaded the other way round, torch would
    map a second HIP runtime next to the system one, and device pointers and
    streams from one runtime are meaningless to the other.
    """
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m tiled_exact_attention_flashattention_amd.build` (there is no fallback)")
    import torch  # noqa: F401  (must precede the CDLL below)
    L = ctypes.CDLL(LIB_PATH)
    runtimes = hip_runtimes_loaded()
    if len(runtimes) > 1:
        raise RuntimeError(f"more than one HIP runtime is mapped into this process: {runtimes}")
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    L.attn_fwd.restype = i32
    L.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    f32, i32, vp, sz, vp]
    L.attn_decode_paged.restype = i32
    L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                  vp]
    L.attn_fwd_window.restype = i32
    L.attn_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     i32, i32, f32, i32, i32, vp]
    L.attn_prefill_paged.restype = i32
    L.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            i32, i32, f32, i32, vp]
    L.attn_decode_paged_noalloc.restype = i32
    L.attn_decode_paged_fp8.argtypes = [vp, vp, vp, f32, f32, vp, vp, vp, vp, i32, i32, i32, i32,
                                        i32, i32, i32, f32, vp, sz, vp]
    L.attn_decode_paged_fp8.restype = i32
    L.attn_decode_paged_int8.argtypes = list(L.attn_decode_paged_fp8.argtypes)
    L.attn_decode_paged_int8.restype = i32
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                           i32, i32, vp, sz, vp]
    L.attn_bwd.restype = i32
    L.attn_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.attn_bwd_workspace_size.restype = sz
    L.attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.attn_decode_workspace_size.restype = sz
    L.attn_status_string.argtypes = [i32]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_time_next_call.argtypes = [vp, vp]
    L.attn_time_next_call.restype = i32
    _LIB = L
    return L


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def attn_last_error() -> str:
    return lib().attn_last_error().decode()


def attn_time_next_call(start, stop) -> None:
    """The calling thread's next computing call records ``start`` when its
    first kernel begins and ``stop`` when its last kernel ends.

    start/stop: ``torch.cuda.Event(enable_timing=True)`` objects that have been
    recorded once (torch creates the underlying event on its first record), or
    both None to cancel.
    """
    if start is None and stop is None:
        _check(lib().attn_time_next_call(None, None))
        return
    handles = [int(e.cuda_event) for e in (start, stop)]
    if not all(handles):
        raise ValueError("record each event once before passing it (torch creates it then)")
    _check(lib().attn_time_next_call(handles[0], handles[1]))


def attn_decode_workspace_size(N: int, Hq: int, d: int, max_blocks: int, page: int = PAGE) -> int:
    return int(lib().attn_decode_workspace_size(N, Hq, d, max_blocks, page))


def attn_bwd_workspace_size(B: int, Hq: int, Hkv: int, T: int, S: int, d: int) -> int:
    return int(lib().attn_bwd_workspace_size(B, Hq, Hkv, T, S, d))


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_ptr(device, stream) -> int:
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return int(s.cuda_stream)


def _require_device_tensors(*ts) -> None:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")


def attn_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    """Enqueue attn_fwd on ``stream`` (default: the current stream of q's device).

    q/o [B,Hq,T,d], k/v [B,Hkv,S,d] in one dtype (bf16 or f32); lse [B,Hq,T]
    float32 or None.
    """
    import torch
    _require_device_tensors(q, k, v, o, lse)
    B, Hq, T, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, S, d) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o")
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise TypeError("q, k, v, o must share one dtype")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (B, Hq, T)):
        raise ValueError("lse must be float32 [B, Hq, T]")
    st = lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                        lse.data_ptr() if lse is not None else None,
                        B, Hq, Hkv, T, S, d, float(scale), int(bool(causal)), _dtype_code(q),
                        _stream_ptr(q.device, stream))
    _check(st)


def attn_fwd_window(q, k, v, o, lse, scale: float, window: int, stream=None) -> None:
    """Enqueue attn_fwd_window (causal, sliding window of ``window`` keys)."""
    import torch
    _require_device_tensors(q, k, v, o, lse)
    B, Hq, T, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, S, d) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o")
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise TypeError("q, k, v, o must share one dtype")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (B, Hq, T)):
        raise ValueError("lse must be float32 [B, Hq, T]")
    st = lib().attn_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr() if lse is not None else None,
                               B, Hq, Hkv, T, S, d, float(scale), int(window), _dtype_code(q),
                               _stream_ptr(q.device, stream))
    _check(st)


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale: float, causal: bool, workspace,
             stream=None) -> None:
    """Enqueue attn_bwd on ``stream`` (default: the current stream of q's device).

    q/o/dout/dq [B,Hq,T,d], k/v/dk/dv [B,Hkv,S,d], all bf16; lse [B,Hq,T]
    float32 from attn_fwd; workspace: a device tensor of at least
    attn_bwd_workspace_size bytes.
    """
    import torch
    _require_device_tensors(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    B, Hq, T, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, S, d) or v.shape != k.shape or dk.shape != k.shape or dv.shape != k.shape:
        raise ValueError("k, v, dk, dv must be [B, Hkv, S, d]")
    if o.shape != q.shape or dout.shape != q.shape or dq.shape != q.shape:
        raise ValueError("o, dout, dq must have q's shape")
    if len({t.dtype for t in (q, k, v, o, dout, dq, dk, dv)}) != 1:
        raise TypeError("q, k, v, o, dout, dq, dk, dv must share one dtype")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, T):
        raise ValueError("lse must be float32 [B, Hq, T]")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                        B, Hq, Hkv, T, S, d, float(scale), int(bool(causal)), _dtype_code(q),
                        workspace.data_ptr(), ws_bytes, _stream_ptr(q.device, stream))
    _check(st)


def attn_decode_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, scale: float,
                      workspace, page: int = PAGE, stream=None) -> None:
    """Enqueue attn_decode_paged on ``stream``.

    q/o [N,Hq,d] bf16; pools [num_pages,Hkv,page,d] bf16; block_table int32
    [N,max_blocks]; seq_lens int32 [N]; lse float32 [N,Hq] or None;
    workspace: a device tensor of at least attn_decode_workspace_size bytes.
    """
    import torch
    _require_device_tensors(q, k_pool, v_pool, block_table, seq_lens, o, lse, workspace)
    N, Hq, d = q.shape
    num_pages, Hkv = k_pool.shape[0], k_pool.shape[1]
    if k_pool.shape != (num_pages, Hkv, page, d) or v_pool.shape != k_pool.shape:
        raise ValueError("pools must be [num_pages, Hkv, page, d]")
    if o.shape != q.shape or block_table.dim() != 2 or block_table.shape[0] != N:
        raise ValueError("shape mismatch among q, o, block_table")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or seq_lens.shape != (N,):
        raise TypeError("block_table and seq_lens must be int32")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (N, Hq)):
        raise ValueError("lse must be float32 [N, Hq]")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().attn_decode_paged(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                 block_table.data_ptr(), seq_lens.data_ptr(), o.data_ptr(),
                                 lse.data_ptr() if lse is not None else None,
                                 N, Hq, Hkv, d, page, num_pages, block_table.shape[1],
                                 float(scale), _dtype_code(q), workspace.data_ptr(), ws_bytes,
                                 _stream_ptr(q.device, stream))
    _check(st)


def attn_decode_paged_noalloc(q, k_pool, v_pool, block_table, seq_lens, o, lse, scale: float,
                              page: int = PAGE, stream=None) -> None:
    """Enqueue attn_decode_paged_noalloc on ``stream``: attn_decode_paged with
    its scratch in the library's device-resident array (no workspace; calls
    that overlap in time on one device race).  Arguments as for
    attn_decode_paged without ``workspace``."""
    import torch
    _require_device_tensors(q, k_pool, v_pool, block_table, seq_lens, o, lse)
    N, Hq, d = q.shape
    num_pages, Hkv = k_pool.shape[0], k_pool.shape[1]
    if k_pool.shape != (num_pages, Hkv, page, d) or v_pool.shape != k_pool.shape:
        raise ValueError("pools must be [num_pages, Hkv, page, d]")
    if o.shape != q.shape or block_table.dim() != 2 or block_table.shape[0] != N:
        raise ValueError("shape mismatch among q, o, block_table")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or seq_lens.shape != (N,):
        raise TypeError("block_table and seq_lens must be int32")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (N, Hq)):
        raise ValueError("lse must be float32 [N, Hq]")
    st = lib().attn_decode_paged_noalloc(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                         block_table.data_ptr(), seq_lens.data_ptr(), o.data_ptr(),
                                         lse.data_ptr() if lse is not None else None,
                                         N, Hq, Hkv, d, page, num_pages, block_table.shape[1],
                                         float(scale), _dtype_code(q),
                                         _stream_ptr(q.device, stream))
    _check(st)


def check_paged_inputs(block_table, seq_lens, num_pages: int, page: int = PAGE,
                       q_lens=None, T: Optional[int] = None) -> None:
    """Host-side check of what the paged entry points take on trust.

    The kernels read the block table and the lengths on the device, so the C
    ABI cannot validate them: every page id a sequence uses (block b <
    ceil(seq_len / page)) must lie in [0, num_pages), every length in
    [0, max_blocks * page], and for chunked prefill 0 <= q_len <= min(T,
    seq_len).  (The kernels still never read outside the pools: a bad page id
    is masked in decode and clamped in prefill, so only that sequence's
    result is wrong.)  This copies the tensors to the host; it is a debugging
    aid for callers, not part of any launch.  Raises ValueError naming the
    first offending sequence.
    """
    import numpy as np

    def host(t):
        return np.asarray(t.detach().cpu().numpy() if hasattr(t, "detach") else t)

    bt, sl = host(block_table), host(seq_lens)
    if bt.ndim != 2 or sl.ndim != 1 or sl.shape[0] != bt.shape[0]:
        raise ValueError("block_table must be [N, max_blocks] and seq_lens [N]")
    max_blocks = bt.shape[1]
    for n, L in enumerate(sl.tolist()):
        if L < 0 or L > max_blocks * page:
            raise ValueError(f"sequence {n}: seq_len {L} outside [0, {max_blocks * page}]")
        used = bt[n, :(L + page - 1) // page]
        bad = np.flatnonzero((used < 0) | (used >= num_pages))
        if bad.size:
            raise ValueError(f"sequence {n}: block {int(bad[0])} holds page id {int(used[bad[0]])}"
                             f" outside [0, {num_pages})")
    if q_lens is not None:
        ql = host(q_lens)
        if ql.shape != sl.shape:
            raise ValueError("q_lens must be [N]")
        for n, (Tn, L) in enumerate(zip(ql.tolist(), sl.tolist())):
            hi = L if T is None else min(T, L)
            if Tn < 0 or Tn > hi:
                raise ValueError(f"sequence {n}: q_len {Tn} outside [0, {hi}]")


def attn_prefill_paged(q, k_pool, v_pool, block_table, seq_lens, q_lens, o, lse, scale: float,
                       window: int = 0, page: int = PAGE, stream=None) -> None:
    """Enqueue attn_prefill_paged on ``stream``.

    q/o [N,Hq,T,d] bf16; pools [num_pages,Hkv,page,d] bf16; block_table int32
    [N,max_blocks]; seq_lens, q_lens int32 [N]; lse float32 [N,Hq,T] or None.
    """
    import torch
    _require_device_tensors(q, k_pool, v_pool, block_table, seq_lens, q_lens, o, lse)
    N, Hq, T, d = q.shape
    num_pages, Hkv = k_pool.shape[0], k_pool.shape[1]
    if k_pool.shape != (num_pages, Hkv, page, d) or v_pool.shape != k_pool.shape:
        raise ValueError("pools must be [num_pages, Hkv, page, d]")
    if o.shape != q.shape or block_table.dim() != 2 or block_table.shape[0] != N:
        raise ValueError("shape mismatch among q, o, block_table")
    for t in (block_table, seq_lens, q_lens):
        if t.dtype != torch.int32:
            raise TypeError("block_table, seq_lens and q_lens must be int32")
    if seq_lens.shape != (N,) or q_lens.shape != (N,):
        raise ValueError("seq_lens and q_lens must be [N]")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (N, Hq, T)):
        raise ValueError("lse must be float32 [N, Hq, T]")
    st = lib().attn_prefill_paged(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                  block_table.data_ptr(), seq_lens.data_ptr(), q_lens.data_ptr(),
                                  o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                  N, Hq, Hkv, T, d, page, num_pages, block_table.shape[1],
                                  float(scale), int(window), _dtype_code(q),
                                  _stream_ptr(q.device, stream))
    _check(st)


def attn_decode_paged_fp8(q, k_codes, v_codes, k_scale: float, v_scale: float, block_table,
                          seq_lens, o, lse, scale: float, workspace, page: int = PAGE,
                          stream=None) -> None:
    """Enqueue attn_decode_paged_fp8: pools are uint8 E4M3 codes [num_pages,Hkv,page,d]."""
    import torch
    _require_device_tensors(q, k_codes, v_codes, block_table, seq_lens, o, lse, workspace)
    N, Hq, d = q.shape
    num_pages, Hkv = k_codes.shape[0], k_codes.shape[1]
    if k_codes.shape != (num_pages, Hkv, page, d) or v_codes.shape != k_codes.shape:
        raise ValueError("pools must be [num_pages, Hkv, page, d]")
    if k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise TypeError("fp8 pools must be uint8 E4M3 codes")
    if o.shape != q.shape or block_table.dim() != 2 or block_table.shape[0] != N:
        raise ValueError("shape mismatch among q, o, block_table")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or seq_lens.shape != (N,):
        raise TypeError("block_table and seq_lens must be int32")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (N, Hq)):
        raise ValueError("lse must be float32 [N, Hq]")
    if q.dtype != torch.bfloat16 or o.dtype != torch.bfloat16:
        raise TypeError("q and o must be bfloat16")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().attn_decode_paged_fp8(q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
                                     float(k_scale), float(v_scale), block_table.data_ptr(),
                                     seq_lens.data_ptr(), o.data_ptr(),
                                     lse.data_ptr() if lse is not None else None,
                                     N, Hq, Hkv, d, page, num_pages, block_table.shape[1],
                                     float(scale), workspace.data_ptr(), ws_bytes,
                                     _stream_ptr(q.device, stream))
    _check(st)


def attn_decode_paged_int8(q, k_codes, v_codes, k_scale: float, v_scale: float, block_table,
                           seq_lens, o, lse, scale: float, workspace, page: int = PAGE,
                           stream=None) -> None:
    """Enqueue attn_decode_paged_int8: pools are int8 codes (torch int8 or their
    uint8 bytes) [num_pages,Hkv,page,d] with per-tensor scales."""
    import torch
    _require_device_tensors(q, k_codes, v_codes, block_table, seq_lens, o, lse, workspace)
    N, Hq, d = q.shape
    num_pages, Hkv = k_codes.shape[0], k_codes.shape[1]
    if k_codes.shape != (num_pages, Hkv, page, d) or v_codes.shape != k_codes.shape:
        raise ValueError("pools must be [num_pages, Hkv, page, d]")
    if k_codes.dtype not in (torch.int8, torch.uint8) or v_codes.dtype != k_codes.dtype:
        raise TypeError("int8 pools must be int8 codes (or their uint8 bytes)")
    if o.shape != q.shape or block_table.dim() != 2 or block_table.shape[0] != N:
        raise ValueError("shape mismatch among q, o, block_table")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or seq_lens.shape != (N,):
        raise TypeError("block_table and seq_lens must be int32")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (N, Hq)):
        raise ValueError("lse must be float32 [N, Hq]")
    if q.dtype != torch.bfloat16 or o.dtype != torch.bfloat16:
        raise TypeError("q and o must be bfloat16")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().attn_decode_paged_int8(q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
                                      float(k_scale), float(v_scale), block_table.data_ptr(),
                                      seq_lens.data_ptr(), o.data_ptr(),
                                      lse.data_ptr() if lse is not None else None,
                                      N, Hq, Hkv, d, page, num_pages, block_table.shape[1],
                                      float(scale), workspace.data_ptr(), ws_bytes,
                                      _stream_ptr(q.device, stream))
    _check(st)


# ---- conveniences that allocate outputs with torch ---------------------------

def fwd(q, k, v, scale: Optional[float] = None, causal: bool = False, with_lse: bool = True,
        window: int = 0):
    """Allocate O (and LSE) and run attn_fwd (attn_fwd_window if window > 0,
    which implies causal).  Returns (o, lse)."""
    import torch
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if with_lse else None
    if window:
        attn_fwd_window(q, k, v, o, lse, scale, window)
    else:
        attn_fwd(q, k, v, o, lse, scale, causal)
    return o, lse


def bwd(q, k, v, o, lse, dout, scale: Optional[float] = None, causal: bool = False,
        workspace=None):
    """Allocate dQ, dK, dV (and the workspace if not given) and run attn_bwd."""
    import torch
    B, Hq, T, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(attn_bwd_workspace_size(B, Hq, k.shape[1], T, k.shape[2], d),
                                dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale, causal, workspace)
    return dq, dk, dv


def decode_workspace(N: int, Hq: int, d: int, max_blocks: int, device) -> "object":
    import torch
    nbytes = attn_decode_workspace_size(N, Hq, d, max_blocks, PAGE)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale: Optional[float] = None,
                 workspace=None, with_lse: bool = True):
    """Allocate O (and LSE, and the workspace if not given) and run attn_decode_paged."""
    import torch
    N, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = decode_workspace(N, Hq, d, block_table.shape[1], q.device)
    o = torch.empty_like(q)
    lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device) if with_lse else None
    attn_decode_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, scale, workspace)
    return o, lse
