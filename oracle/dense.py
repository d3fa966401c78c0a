"""Float64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
It shares no code with the HIP library and the HIP library never calls it.

This is the plain definition, written out the slow way: the whole score matrix
of a (batch, head) pair is materialised, masked, pushed through the
max-subtracted softmax and multiplied by V.  There is no tiling and no online
softmax here; the tiled kernels must land on this result up to rounding.

Sources (page titles and sections):

* "Advanced Attention Mechanisms - II" (A. Das), section Tiling, step 2:
  per query/key pair the scaled dot product gives the score matrix, softmax
  normalises it and the weights multiply V.
* same page, section "Softmax stabiliser": p_i = exp(l_i) / sum_j exp(l_j),
  and the stabilised form that subtracts the maximum logit m first.
* same page, section "Flash Attention": the row statistics are kept instead of
  the attention matrix; the log-sum-exp output is our reading of that.
* "Accelerating Mamba-2 with high-performance forward-pass kernels in NVIDIA
  CUDA Tile", paragraph on exp(G - G^T): terms with i < j are removed by the
  causal mask.
* "Fast attention kernels and operator fusion accelerate AI models", section
  on FlashAttention-style and paged attention: the paged cache keeps keys and
  values in fixed-size blocks, and a block table maps logical positions to
  physical blocks that the kernel must translate.

Readings where the pages are silent (each listed in the design notes):

* scale multiplies the logits before masking;
* causal alignment is bottom-right: query i sees key j iff j <= i + (S - T);
  for T == S this is the pages' "i < j is masked" rule (T != S: parity unpinned);
* masked logits are -inf, i.e. exactly zero weight;
* LSE is the natural log of sum_j exp(scale * q.k_j) over visible keys;
* GQA groups consecutive query heads: query head h reads KV head h // (Hq/Hkv);
* layouts: q/o [B,Hq,T,d], k/v [B,Hkv,S,d]; pools [num_pages,Hkv,page,d];
* sliding window (the pages only name sliding-window attention as a
  predecessor, in "Advanced Attention Mechanisms - II", section "Flash
  Attention"): a causal window of W keys, query i sees key j iff
  i + (S - T) - W < j <= i + (S - T), i.e. its own position and the W - 1
  before it;
* chunked prefill on a paged cache: the T new queries of a sequence are the
  last T of its S cached positions, which is the bottom-right causal rule.
"""
from __future__ import annotations

import numpy as np

# Rows of the score matrix materialised at once (memory bound for big S).
ROW_CHUNK = 1024


def scaled_scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """scale * Q K^T for one (batch, head): q_rows [R,d], k [S,d] -> [R,S]."""
    return scale * (q_rows @ k.T)


def visible_mask(rows: np.ndarray, S: int, T: int, causal: bool, window: int = 0) -> np.ndarray:
    """Boolean [R,S]: True where key j may be attended by query row i.

    Causal rule (bottom-right aligned): key j is visible to query i iff
    j <= i + (S - T).  Non-causal: every key is visible.  window W > 0 (causal
    only) also hides keys j <= i + (S - T) - W.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if not causal:
        if window:
            raise ValueError("a sliding window needs the causal mask")
        return np.ones((rows.shape[0], S), dtype=bool)
    j = np.arange(S, dtype=np.int64)[None, :]
    diag = rows[:, None] + (S - T)
    vis = j <= diag
    if window:
        vis &= j > diag - window
    return vis


def masked_scores(scores: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """Masked logits are replaced by -inf (exactly zero weight after exp)."""
    return np.where(visible, scores, -np.inf)


def softmax_rows(logits: np.ndarray):
    """Max-subtracted softmax along the last axis.

    Returns (P, m, l): probabilities, the row maximum m and the row sum
    l = sum_j exp(logit_j - m).  Masked (-inf) logits give exactly 0.
    """
    m = np.max(logits, axis=-1, keepdims=True)
    e = np.exp(logits - m)
    l = np.sum(e, axis=-1, keepdims=True)
    return e / l, m[..., 0], l[..., 0]


def softmax_rows_unstabilised(logits: np.ndarray) -> np.ndarray:
    """The textbook form p_i = exp(l_i) / sum_j exp(l_j), without the max shift.

    Kept only so the tests can show it equals the stabilised form where it
    does not overflow.
    """
    e = np.exp(logits)
    return e / np.sum(e, axis=-1, keepdims=True)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Consecutive GQA grouping: Hq/Hkv query heads share one KV head."""
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def attention_head(q_bh, k_bh, v_bh, scale, causal, rows=None, window=0):
    """Attention for one (batch, query head).

    q_bh [T,d], k_bh/v_bh [S,d] float64.  ``rows`` selects query rows (all by
    default); ``window`` > 0 adds the causal sliding window.  Returns
    (O [R,d], LSE [R]).  A row that sees no key gets O = 0 and LSE = -inf.
    """
    T, S = q_bh.shape[0], k_bh.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.shape[0], v_bh.shape[1]), dtype=np.float64)
    lse = np.empty(rows.shape[0], dtype=np.float64)
    for r0 in range(0, rows.shape[0], ROW_CHUNK):
        rr = rows[r0:r0 + ROW_CHUNK]
        sc = scaled_scores(q_bh[rr], k_bh, scale)
        vis = visible_mask(rr, S, T, causal, window)
        sc = masked_scores(sc, vis)
        empty = ~vis.any(axis=1)
        sc[empty] = 0.0                      # placeholder, overwritten below
        p, m, l = softmax_rows(sc)
        o[r0:r0 + rr.shape[0]] = p @ v_bh
        lse[r0:r0 + rr.shape[0]] = m + np.log(l)
        o[r0:r0 + rr.shape[0]][empty] = 0.0
        lse[r0:r0 + rr.shape[0]][empty] = -np.inf
    return o, lse


def attention(q, k, v, scale, causal, window=0):
    """Full attention: q [B,Hq,T,d], k/v [B,Hkv,S,d] float64 -> (O, LSE).

    O is [B,Hq,T,d]; LSE is [B,Hq,T].  ``window`` > 0: causal sliding window.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    o = np.empty((B, Hq, T, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, Hq, T), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, hk], v[b, hk], scale, causal,
                                                window=window)
    return o, lse


def attention_rows(q, k, v, scale, causal, b, h, rows, window=0):
    """Sampled rows of one (b, h): the same definition on a subset of queries."""
    Hq, Hkv = q.shape[1], k.shape[1]
    hk = kv_head_of(h, Hq, Hkv)
    return attention_head(np.asarray(q[b, h], dtype=np.float64),
                          np.asarray(k[b, hk], dtype=np.float64),
                          np.asarray(v[b, hk], dtype=np.float64), scale, causal, rows, window)


def gather_pages(pool, block_table_row, length, hk, page):
    """Contiguous [length, d] keys (or values) of one sequence and KV head.

    Logical position t lives in physical page block_table_row[t // page], slot
    t % page.  Slots at or past ``length`` are never touched.
    """
    t = np.arange(length, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // page]
    if (pages < 0).any():
        raise ValueError("block table entry < 0 inside the sequence")
    return np.asarray(pool, dtype=np.float64)[pages, hk, t % page, :]


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale, page=16, seqs=None):
    """One query token per sequence against its paged KV cache.

    q [N,Hq,d]; pools [num_pages,Hkv,page,d]; block_table int [N,max_blocks];
    seq_lens int [N].  Returns (O [N,Hq,d], LSE [N,Hq]) over the sequences in
    ``seqs`` (all by default), in that order.  A single query attends every
    cached position, so there is no mask beyond the sequence length.
    """
    q = np.asarray(q, dtype=np.float64)
    N, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    seqs = range(N) if seqs is None else list(seqs)
    o = np.empty((len(seqs), Hq, v_pool.shape[3]), dtype=np.float64)
    lse = np.empty((len(seqs), Hq), dtype=np.float64)
    for i, n in enumerate(seqs):
        L = int(seq_lens[n])
        if L < 1:
            raise ValueError("sequence length must be >= 1")
        for hk in range(Hkv):
            kn = gather_pages(k_pool, block_table[n], L, hk, page)
            vn = gather_pages(v_pool, block_table[n], L, hk, page)
            for h in range(Hq):
                if kv_head_of(h, Hq, Hkv) != hk:
                    continue
                oo, ll = attention_head(q[n, h][None, :], kn, vn, scale, causal=False)
                o[i, h], lse[i, h] = oo[0], ll[0]
    return o, lse


def prefill_paged(q, k_pool, v_pool, block_table, seq_lens, q_lens, scale, page=16, window=0):
    """Chunked prefill against a paged cache.

    q [N,Hq,T,d]: row i < q_lens[n] of sequence n is the query at position
    seq_lens[n] - q_lens[n] + i, i.e. the new tokens are the last q_lens[n] of
    the seq_lens[n] cached ones; it attends causally (and within ``window`` if
    > 0) to the cached keys.  Returns (O [N,Hq,T,d], LSE [N,Hq,T]); rows at or
    past q_lens[n] are NaN (they are not part of the result).
    """
    q = np.asarray(q, dtype=np.float64)
    N, Hq, T, d = q.shape
    Hkv = k_pool.shape[1]
    o = np.full((N, Hq, T, v_pool.shape[3]), np.nan)
    lse = np.full((N, Hq, T), np.nan)
    for n in range(N):
        L, Tn = int(seq_lens[n]), int(q_lens[n])
        if not (1 <= Tn <= min(T, L)):
            raise ValueError("need 1 <= q_lens[n] <= min(T, seq_lens[n])")
        for hk in range(Hkv):
            kn = gather_pages(k_pool, block_table[n], L, hk, page)
            vn = gather_pages(v_pool, block_table[n], L, hk, page)
            for h in range(Hq):
                if kv_head_of(h, Hq, Hkv) != hk:
                    continue
                o[n, h, :Tn], lse[n, h, :Tn] = attention_head(q[n, h, :Tn], kn, vn, scale,
                                                              causal=True, window=window)
    return o, lse
