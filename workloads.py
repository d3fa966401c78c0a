"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the float64 oracle and the HIP path receive the
arrays produced here, so the two sides see bit-identical inputs.

Recipe (shared by tests and the benchmark):

* generator: ``numpy.random.default_rng(seed)``; draws are float32
  ``standard_normal`` in the order q, k, v;
* bf16 workloads are rounded to nearest-even by ``torch.Tensor.to(bfloat16)``;
  the oracle receives exactly those bf16 values widened to float64;
* paged decode draws, in order: sequence lengths (discrete uniform, inclusive
  bounds), one permutation of the shared page pool, then q, k_pool, v_pool.
  Logical block ``b`` of sequence ``n`` lives in physical page
  ``perm[off_n + b]`` with ``off_n`` the number of pages of the sequences before
  ``n``; block-table entries past a sequence's last page are -1.

The five named workloads:

========  =====================================================================
prefill_1  B=1, H=1, T=S=256, d=64, fp32, non-causal, seed 1001
prefill_2  B=8, Hq=Hkv=12, T=S=1024, d=64, bf16, causal, seed 1002
prefill_3  B=4, Hq=12, Hkv=2, T=S=4096, d=128, bf16, causal, seed 1003
prefill_4  B=1, Hq=Hkv=32, T=S=16384, d=128, bf16, causal, x0.5, seed 1004
decode_5   64 sequences, Hq=12, Hkv=2, d=128, bf16, lengths U[512, 8192],
           16-token pages, seed 1005
========  =====================================================================

Backward inputs (``make_backward``) draw q, k, v exactly as ``make_prefill``
and then the output gradient dO, float32 ``standard_normal`` of q's shape,
rounded to bf16.  ``backward_3`` is the gradient pass of prefill_3: its q, k,
v are prefill_3's (same seed), with dO drawn after them.

``make_prefill_paged`` lays chunked-prefill inputs out like ``make_decode``;
``chunked_prefill_6`` is its benchmark case: 16 sequences with 1024..8192
cached tokens whose last 512 are the chunk, on the decode model shape.
``make_decode_fp8`` draws as ``make_decode`` and quantises K and V to E4M3
codes (value / scale, torch's float8_e4m3fn cast; quantising is input
preparation, the attention only ever sees the codes and the scales);
``decode_fp8_7`` is decode_5's shape with such pages.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE = 16


@dataclass
class PrefillInputs:
    B: int
    Hq: int
    Hkv: int
    T: int
    S: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    scale: float
    q: object           # torch CPU tensor [B,Hq,T,d] in dtype
    k: object           # torch CPU tensor [B,Hkv,S,d]
    v: object
    name: str = ""

    def f64(self):
        """The exact input values widened to float64 numpy arrays."""
        return (self.q.double().numpy(), self.k.double().numpy(), self.v.double().numpy())


@dataclass
class BackwardInputs(PrefillInputs):
    do: object = None   # torch CPU tensor [B,Hq,T,d]: gradient of the loss w.r.t. O

    def f64(self):
        return super().f64() + (self.do.double().numpy(),)


@dataclass
class PagedPrefillInputs:
    N: int
    Hq: int
    Hkv: int
    T: int                      # row stride of q / o (largest chunk)
    d: int
    page: int
    num_pages: int
    max_blocks: int
    scale: float
    window: int
    seq_lens: np.ndarray        # int32 [N], cached tokens incl. the chunk
    q_lens: np.ndarray          # int32 [N], chunk tokens (the last of seq_lens)
    block_table: np.ndarray     # int32 [N, max_blocks], -1 past the end
    q: object                   # torch CPU bf16 [N, Hq, T, d]
    k_pool: object              # torch CPU bf16 [num_pages, Hkv, page, d]
    v_pool: object
    name: str = ""

    def f64(self):
        return (self.q.double().numpy(), self.k_pool.double().numpy(), self.v_pool.double().numpy())


@dataclass
class DecodeInputs:
    N: int
    Hq: int
    Hkv: int
    d: int
    page: int
    num_pages: int
    max_blocks: int
    scale: float
    seq_lens: np.ndarray        # int32 [N]
    block_table: np.ndarray     # int32 [N, max_blocks], -1 past the end
    q: object                   # torch CPU bf16 [N, Hq, d]
    k_pool: object              # torch CPU bf16 [num_pages, Hkv, page, d]
    v_pool: object
    name: str = ""
    meta: dict = field(default_factory=dict)

    def f64(self):
        return (self.q.double().numpy(), self.k_pool.double().numpy(), self.v_pool.double().numpy())


def _torch():
    import torch
    return torch


def _cast(arr32: np.ndarray, dtype: str):
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(arr32, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).contiguous()
    if dtype == "f32":
        return t.contiguous()
    raise ValueError(f"unknown dtype {dtype!r}")


def make_prefill(B, Hq, Hkv, T, S, d, dtype="bf16", causal=True, seed=0,
                 amplitude=1.0, scale=None, name="") -> PrefillInputs:
    """q, k, v iid N(0,1) (times ``amplitude``), drawn in the order q, k, v."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, d), dtype=np.float32)
    if amplitude != 1.0:
        a = np.float32(amplitude)
        q, k, v = q * a, k * a, v * a
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return PrefillInputs(B, Hq, Hkv, T, S, d, dtype, bool(causal), float(scale),
                         _cast(q, dtype), _cast(k, dtype), _cast(v, dtype), name=name)


def make_backward(B, Hq, Hkv, T, S, d, causal=True, seed=0, amplitude=1.0, scale=None,
                  name="") -> BackwardInputs:
    """q, k, v exactly as ``make_prefill`` (bf16), then dO iid N(0,1) [B,Hq,T,d]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, d), dtype=np.float32)
    if amplitude != 1.0:
        a = np.float32(amplitude)
        q, k, v = q * a, k * a, v * a
    do = rng.standard_normal((B, Hq, T, d), dtype=np.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return BackwardInputs(B, Hq, Hkv, T, S, d, "bf16", bool(causal), float(scale),
                          _cast(q, "bf16"), _cast(k, "bf16"), _cast(v, "bf16"), name=name,
                          do=_cast(do, "bf16"))


def make_decode(N, Hq, Hkv, d, min_len, max_len, page=PAGE, max_blocks=None, seed=0,
                poison_tail=False, lens=None, scale=None, name="") -> DecodeInputs:
    """Paged decode inputs.

    ``lens`` overrides the drawn lengths (the draw still happens so that the
    rest of the stream is unchanged).  With ``poison_tail`` the unused slots
    of every sequence's last page are set to NaN after the draw.
    """
    rng = np.random.default_rng(seed)
    drawn = rng.integers(min_len, max_len + 1, N)
    seq_lens = np.asarray(drawn if lens is None else lens, dtype=np.int64)
    assert seq_lens.shape == (N,) and (seq_lens >= 1).all()
    pages_per = (seq_lens + page - 1) // page
    if max_blocks is None:
        max_blocks = int((max_len + page - 1) // page)
    assert (pages_per <= max_blocks).all()
    P = int(pages_per.sum())
    perm = rng.permutation(P)
    block_table = np.full((N, max_blocks), -1, dtype=np.int32)
    off = 0
    for n in range(N):
        cnt = int(pages_per[n])
        block_table[n, :cnt] = perm[off:off + cnt]
        off += cnt
    q = rng.standard_normal((N, Hq, d), dtype=np.float32)
    k_pool = rng.standard_normal((P, Hkv, page, d), dtype=np.float32)
    v_pool = rng.standard_normal((P, Hkv, page, d), dtype=np.float32)
    if poison_tail:
        for n in range(N):
            L = int(seq_lens[n])
            used = L - (int(pages_per[n]) - 1) * page
            if used < page:
                last = block_table[n, int(pages_per[n]) - 1]
                k_pool[last, :, used:, :] = np.nan
                v_pool[last, :, used:, :] = np.nan
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return DecodeInputs(N, Hq, Hkv, d, page, P, max_blocks, float(scale),
                        seq_lens.astype(np.int32), block_table,
                        _cast(q, "bf16"), _cast(k_pool, "bf16"), _cast(v_pool, "bf16"),
                        name=name, meta={"numpy": np.__version__, "sum_len": int(seq_lens.sum())})


def make_prefill_paged(N, Hq, Hkv, T, d, min_len, max_len, q_lens=None, lens=None, page=PAGE,
                       window=0, seed=0, poison_tail=False, extra_pages=0, name=""):
    """Chunked-prefill inputs on a paged cache.

    Draws, in order: cached lengths (discrete uniform [min_len, max_len],
    overridden by ``lens``), chunk lengths (uniform [1, min(T, len)], unless
    ``q_lens`` is given: an int for all or a list), one permutation of the
    pool (the sequences' pages plus ``extra_pages`` unused ones), then q,
    k_pool, v_pool iid N(0,1).  Page layout and the -1 padding of the block
    table are those of ``make_decode``; ``poison_tail`` sets the unused slots
    of every last page to NaN.
    """
    rng = np.random.default_rng(seed)
    drawn = rng.integers(min_len, max_len + 1, N)
    seq_lens = np.asarray(drawn if lens is None else lens, dtype=np.int64)
    drawn_q = rng.integers(1, np.minimum(T, seq_lens) + 1)
    if q_lens is None:
        ql = drawn_q
    elif np.isscalar(q_lens):
        ql = np.full(N, int(q_lens))
    else:
        ql = np.asarray(q_lens)
    ql = np.asarray(ql, dtype=np.int64)
    assert (ql >= 1).all() and (ql <= np.minimum(T, seq_lens)).all()
    pages_per = (seq_lens + page - 1) // page
    max_blocks = int(pages_per.max())
    P = int(pages_per.sum()) + extra_pages
    perm = rng.permutation(P)
    block_table = np.full((N, max_blocks), -1, dtype=np.int32)
    off = 0
    for n in range(N):
        cnt = int(pages_per[n])
        block_table[n, :cnt] = perm[off:off + cnt]
        off += cnt
    q = rng.standard_normal((N, Hq, T, d), dtype=np.float32)
    k_pool = rng.standard_normal((P, Hkv, page, d), dtype=np.float32)
    v_pool = rng.standard_normal((P, Hkv, page, d), dtype=np.float32)
    if poison_tail:
        for n in range(N):
            used = int(seq_lens[n]) - (int(pages_per[n]) - 1) * page
            if used < page:
                last = block_table[n, int(pages_per[n]) - 1]
                k_pool[last, :, used:, :] = np.nan
                v_pool[last, :, used:, :] = np.nan
    return PagedPrefillInputs(N, Hq, Hkv, T, d, page, P, max_blocks, 1.0 / math.sqrt(d), window,
                              seq_lens.astype(np.int32), ql.astype(np.int32), block_table,
                              _cast(q, "bf16"), _cast(k_pool, "bf16"), _cast(v_pool, "bf16"),
                              name=name)


@dataclass
class DecodeFp8Inputs:
    """Paged decode with 8-bit key/value pages (E4M3 or int8 codes as uint8
    bytes) and per-tensor scales."""
    N: int
    Hq: int
    Hkv: int
    d: int
    page: int
    num_pages: int
    max_blocks: int
    scale: float
    k_scale: float
    v_scale: float
    seq_lens: np.ndarray
    block_table: np.ndarray
    q: object                   # torch CPU bf16 [N, Hq, d]
    k_codes: object             # torch CPU uint8 [num_pages, Hkv, page, d]
    v_codes: object
    name: str = ""


def make_decode_fp8(N, Hq, Hkv, d, min_len, max_len, page=PAGE, max_blocks=None, seed=0,
                    k_scale=2.0 ** -5, v_scale=2.0 ** -5, poison_tail=False, lens=None, name=""):
    """The draws of ``make_decode`` (same order and seed use), then K and V
    quantised to E4M3 codes of value / scale by torch's float8_e4m3fn cast
    (round to nearest even; |value| / scale stays far below 448 for N(0,1)
    draws at the default scale 2^-5).  ``poison_tail`` writes the NaN code
    0x7F into the unused slots of every last page."""
    import torch
    rng = np.random.default_rng(seed)
    drawn = rng.integers(min_len, max_len + 1, N)
    seq_lens = np.asarray(drawn if lens is None else lens, dtype=np.int64)
    pages_per = (seq_lens + page - 1) // page
    if max_blocks is None:
        max_blocks = int((max_len + page - 1) // page)
    P = int(pages_per.sum())
    perm = rng.permutation(P)
    block_table = np.full((N, max_blocks), -1, dtype=np.int32)
    off = 0
    for n in range(N):
        cnt = int(pages_per[n])
        block_table[n, :cnt] = perm[off:off + cnt]
        off += cnt
    q = rng.standard_normal((N, Hq, d), dtype=np.float32)
    k = rng.standard_normal((P, Hkv, page, d), dtype=np.float32)
    v = rng.standard_normal((P, Hkv, page, d), dtype=np.float32)

    def codes(x, sc):
        return (torch.from_numpy(x / np.float32(sc)).to(torch.float8_e4m3fn)
                .view(torch.uint8).contiguous())
    kc, vc = codes(k, k_scale), codes(v, v_scale)
    if poison_tail:
        for n in range(N):
            used = int(seq_lens[n]) - (int(pages_per[n]) - 1) * page
            if used < page:
                last = block_table[n, int(pages_per[n]) - 1]
                kc[last, :, used:, :] = 0x7F
                vc[last, :, used:, :] = 0x7F
    return DecodeFp8Inputs(N, Hq, Hkv, d, page, P, max_blocks, 1.0 / math.sqrt(d), float(k_scale),
                           float(v_scale), seq_lens.astype(np.int32), block_table, _cast(q, "bf16"),
                           kc, vc, name=name)


def make_decode_int8(N, Hq, Hkv, d, min_len, max_len, page=PAGE, max_blocks=None, seed=0,
                     k_scale=2.0 ** -5, v_scale=2.0 ** -5, poison_tail=False, lens=None, name=""):
    """The draws of ``make_decode`` (same order and seed use), then K and V
    quantised symmetrically to int8 codes: value / scale rounded to nearest
    even and clipped to [-127, 127] (N(0,1) draws at the default scale 2^-5
    clip beyond 3.97).  Codes are stored as their two's-complement bytes
    (torch uint8).  ``poison_tail`` writes the code -128 into the unused slots
    of every last page (never used by a correct kernel)."""
    import torch
    rng = np.random.default_rng(seed)
    drawn = rng.integers(min_len, max_len + 1, N)
    seq_lens = np.asarray(drawn if lens is None else lens, dtype=np.int64)
    pages_per = (seq_lens + page - 1) // page
    if max_blocks is None:
        max_blocks = int((max_len + page - 1) // page)
    P = int(pages_per.sum())
    perm = rng.permutation(P)
    block_table = np.full((N, max_blocks), -1, dtype=np.int32)
    off = 0
    for n in range(N):
        cnt = int(pages_per[n])
        block_table[n, :cnt] = perm[off:off + cnt]
        off += cnt
    q = rng.standard_normal((N, Hq, d), dtype=np.float32)
    k = rng.standard_normal((P, Hkv, page, d), dtype=np.float32)
    v = rng.standard_normal((P, Hkv, page, d), dtype=np.float32)

    def codes(x, sc):
        c = np.clip(np.rint(x / np.float32(sc)), -127, 127).astype(np.int8)
        return torch.from_numpy(c.view(np.uint8).copy())
    kc, vc = codes(k, k_scale), codes(v, v_scale)
    if poison_tail:
        for n in range(N):
            used = int(seq_lens[n]) - (int(pages_per[n]) - 1) * page
            if used < page:
                last = block_table[n, int(pages_per[n]) - 1]
                kc[last, :, used:, :] = 0x80
                vc[last, :, used:, :] = 0x80
    return DecodeFp8Inputs(N, Hq, Hkv, d, page, P, max_blocks, 1.0 / math.sqrt(d), float(k_scale),
                           float(v_scale), seq_lens.astype(np.int32), block_table, _cast(q, "bf16"),
                           kc, vc, name=name)


# --- the five named workloads -------------------------------------------------

def prefill_1():
    return make_prefill(1, 1, 1, 256, 256, 64, "f32", causal=False, seed=1001, name="prefill_1")


def prefill_2():
    return make_prefill(8, 12, 12, 1024, 1024, 64, "bf16", causal=True, seed=1002, name="prefill_2")


def prefill_3():
    return make_prefill(4, 12, 2, 4096, 4096, 128, "bf16", causal=True, seed=1003, name="prefill_3")


def prefill_4():
    return make_prefill(1, 32, 32, 16384, 16384, 128, "bf16", causal=True, seed=1004,
                        amplitude=0.5, name="prefill_4")


def decode_5(poison_tail=False):
    return make_decode(64, 12, 2, 128, 512, 8192, page=PAGE, max_blocks=512, seed=1005,
                       poison_tail=poison_tail, name="decode_5")


def chunked_prefill_6():
    """Chunked prefill on the decode model shape: 16 sequences, chunks of 512
    new tokens at the end of 1024..8192 cached ones, Hq=12, Hkv=2, d=128."""
    return make_prefill_paged(16, 12, 2, 512, 128, 1024, 8192, q_lens=512, seed=1006,
                              name="chunked_prefill_6")


def decode_fp8_7(poison_tail=False):
    """decode_5's shape (64 sequences, lengths U[512, 8192], Hq=12, Hkv=2,
    d=128, 16-token pages) with E4M3 key/value pages."""
    return make_decode_fp8(64, 12, 2, 128, 512, 8192, page=PAGE, max_blocks=512, seed=1007,
                           poison_tail=poison_tail, name="decode_fp8_7")


def decode_int8_8(poison_tail=False):
    """decode_5's shape (64 sequences, lengths U[512, 8192], Hq=12, Hkv=2,
    d=128, 16-token pages) with int8 key/value pages."""
    return make_decode_int8(64, 12, 2, 128, 512, 8192, page=PAGE, max_blocks=512, seed=1008,
                            poison_tail=poison_tail, name="decode_int8_8")


def backward_3():
    """The gradient pass of prefill_3 (same q, k, v), dO drawn after v."""
    return make_backward(4, 12, 2, 4096, 4096, 128, causal=True, seed=1003, name="backward_3")


WORKLOADS = {
    "prefill_1": prefill_1,
    "prefill_2": prefill_2,
    "prefill_3": prefill_3,
    "prefill_4": prefill_4,
    "decode_5": decode_5,
    "backward_3": backward_3,
    "chunked_prefill_6": chunked_prefill_6,
    "decode_fp8_7": decode_fp8_7,
    "decode_int8_8": decode_int8_8,
}

# Human-readable shapes, used for labels in the benchmark output.
SHAPES = {
    "prefill_1": dict(B=1, Hq=1, Hkv=1, T=256, S=256, d=64, dtype="f32", causal=False),
    "prefill_2": dict(B=8, Hq=12, Hkv=12, T=1024, S=1024, d=64, dtype="bf16", causal=True),
    "prefill_3": dict(B=4, Hq=12, Hkv=2, T=4096, S=4096, d=128, dtype="bf16", causal=True),
    "prefill_4": dict(B=1, Hq=32, Hkv=32, T=16384, S=16384, d=128, dtype="bf16", causal=True),
    "decode_5": dict(N=64, Hq=12, Hkv=2, d=128, page=16, min_len=512, max_len=8192, dtype="bf16"),
    "backward_3": dict(B=4, Hq=12, Hkv=2, T=4096, S=4096, d=128, dtype="bf16", causal=True),
    "chunked_prefill_6": dict(N=16, Hq=12, Hkv=2, T=512, d=128, page=16, min_len=1024,
                              max_len=8192, dtype="bf16"),
    "decode_fp8_7": dict(N=64, Hq=12, Hkv=2, d=128, page=16, min_len=512, max_len=8192,
                         dtype="bf16 q, e4m3 kv"),
    "decode_int8_8": dict(N=64, Hq=12, Hkv=2, d=128, page=16, min_len=512, max_len=8192,
                          dtype="bf16 q, int8 kv"),
}
