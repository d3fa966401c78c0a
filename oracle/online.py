"""Float64 blocked online-softmax recurrence and split combine.

TEST INFRASTRUCTURE ONLY (same import rule as ``oracle/dense.py``).  These
functions are never compared against the GPU; they exist so the tests can show
that the tile-by-tile method the pages describe reaches the plain definition
in ``oracle/dense.py``, which is what pins the reading of the missing
formulas.

"Advanced Attention Mechanisms - II", section "Incremental / online softmax":
the softmax of each block is computed without the full denominator; the value
is incomplete at every step but the last, where it becomes the required one.
The formula images of that section are lost, so the recurrence below is the
reading: keep a running maximum m and sum l per query row, and when a block
raises the maximum from m to m', rescale the old sum and accumulator by
exp(m - m').  Nothing is normalised until the last block.

"Fast attention kernels and operator fusion accelerate AI models", section on
FlashAttention-style attention: per block the kernel computes part of the
scores, updates the softmax statistics and accumulates the outputs.

The split combine merges results computed over disjoint key ranges by their
log-sum-exp; it follows from the same rescaling algebra and is what the paged
decode uses to merge its splits.
"""
from __future__ import annotations

import numpy as np

from .dense import scaled_scores, visible_mask


def online_attention_head(q_bh, k_bh, v_bh, scale, causal, block):
    """Process keys in blocks of ``block`` with the running (m, l, acc) state.

    Returns (O [T,d], LSE [T]).
    """
    T, S = q_bh.shape[0], k_bh.shape[0]
    rows = np.arange(T)
    m = np.full(T, -np.inf)
    l = np.zeros(T)
    acc = np.zeros((T, v_bh.shape[1]))
    for j0 in range(0, S, block):
        kb = k_bh[j0:j0 + block]
        vb = v_bh[j0:j0 + block]
        s = scaled_scores(q_bh, kb, scale)
        vis = visible_mask(rows, S, T, causal)[:, j0:j0 + block]
        s = np.where(vis, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        # rows that have seen no visible key yet keep m = -inf; shift by 0 there
        shift = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - shift)
        p = np.exp(s - shift[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ vb
        m = m_new
    return acc / l[:, None], m + np.log(l)


def combine_partials(parts):
    """Merge [(O_s [..,d], lse_s [..])] from disjoint key ranges.

    LSE = M + ln sum_s exp(lse_s - M) with M = max_s lse_s, and
    O = sum_s exp(lse_s - LSE) * O_s.  Partials with lse_s = -inf (no key)
    carry zero weight.
    """
    lses = np.stack([p[1] for p in parts])          # [n_s, ...]
    outs = np.stack([p[0] for p in parts])          # [n_s, ..., d]
    M = lses.max(axis=0)
    lse = M + np.log(np.exp(lses - M).sum(axis=0))
    w = np.exp(lses - lse)
    return (w[..., None] * outs).sum(axis=0), lse
