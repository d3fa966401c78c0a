"""Float64 CPU oracle for attention over 8-bit quantised KV pages (fp8, int8).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
It shares no code with the HIP library and the HIP library never calls it.

Source: "Fast attention kernels and operator fusion accelerate AI models",
section on kernel fusion: dequantisation is fused with the matrix product
that consumes it.  The pages fix no format; the reading here (listed in the
design notes) is:

* K and V pages hold 8-bit codes in the OCP E4M3 format ("fn": no
  infinities): bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0
  mantissa; exponent 0 is subnormal (m/8 * 2^-6); code S.1111.111 is NaN;
  the largest finite magnitude is 448;
* one float scale per tensor: K = k_scale * e4m3(k_code), V likewise;
* attention is then the plain definition on the dequantised values.

The integer reading (also listed in the design notes): int8 pages hold
signed two's-complement bytes, -128 .. 127, with one float scale per tensor,
K = k_scale * code and V = v_scale * code (symmetric quantisation).
"""
from __future__ import annotations

import numpy as np

from .dense import decode_paged


def e4m3_to_float(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array) as float64; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 0xF) & (c & 0x7 == 0x7), np.nan, out)


def dequantise(codes, scale) -> np.ndarray:
    """scale * e4m3(code), float64."""
    return float(scale) * e4m3_to_float(codes)


def decode_paged_fp8(q, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, scale,
                     page=16, seqs=None):
    """decode_paged on the dequantised pools (codes [num_pages,Hkv,page,d] uint8)."""
    return decode_paged(q, dequantise(k_codes, k_scale), dequantise(v_codes, v_scale),
                        block_table, seq_lens, scale, page=page, seqs=seqs)


def int8_to_float(codes) -> np.ndarray:
    """Value of each byte read as a signed two's-complement integer, float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def dequantise_int8(codes, scale) -> np.ndarray:
    """scale * int8(code), float64."""
    return float(scale) * int8_to_float(codes)


def decode_paged_int8(q, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, scale,
                      page=16, seqs=None):
    """decode_paged on the dequantised pools (codes [num_pages,Hkv,page,d] bytes)."""
    return decode_paged(q, dequantise_int8(k_codes, k_scale), dequantise_int8(v_codes, v_scale),
                        block_table, seq_lens, scale, page=page, seqs=seqs)
