"""Float64 CPU oracle for the backward pass of exact attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
It shares no code with the HIP library and the HIP library never calls it.

Source: "Advanced Attention Mechanisms - II" (A. Das), section "Flash
Attention": the method keeps the row statistics instead of storing the
attention matrix for the backward pass, so the backward pass must rebuild the
probabilities from the inputs and those statistics.  The pages give no
gradient formulas; the gradient of the forward definition (the one in
``dense.py``) is plain calculus, written out here with the whole matrices
materialised:

    S  = scale * Q K^T, masked entries -inf          (forward definition)
    P  = softmax over each row of S
    O  = P V
    dV = P^T dO
    dP = dO V^T
    D  = rowsum(dO * O)          (equals rowsum(P * dP))
    dS = P * (dP - D)            (Jacobian of the row softmax)
    dQ = scale * dS K
    dK = scale * dS^T Q

With grouped-query heads a KV head receives the sum of the gradients of every
query head that reads it.  Pinned in ``tests/test_oracle_backward.py`` by
central finite differences of the forward oracle and by closed forms.
"""
from __future__ import annotations

import numpy as np

from .dense import kv_head_of, masked_scores, scaled_scores, softmax_rows, visible_mask


def attention_head_backward(q, k, v, do, scale, causal):
    """Gradients of one (batch, head): q [T,d], k/v [S,d], do [T,d].

    Returns (dq [T,d], dk [S,d], dv [S,d], o [T,d], lse [T]) in float64; o and
    lse are the forward results the gradients are taken at.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    T, S = q.shape[0], k.shape[0]
    s = masked_scores(scaled_scores(q, k, scale), visible_mask(np.arange(T), S, T, causal))
    p, m, l = softmax_rows(s)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(do * o, axis=1, keepdims=True)
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    lse = m + np.log(l)
    return dq, dk, dv, o, lse


def attention_backward(q, k, v, do, scale, causal):
    """Batched gradients: q/do [B,Hq,T,d], k/v [B,Hkv,S,d] -> dq, dk, dv (float64)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            gq, gk, gv, _, _ = attention_head_backward(q[b, h], k[b, hk], v[b, hk], do[b, h],
                                                       scale, causal)
            dq[b, h] = gq
            dk[b, hk] += gk
            dv[b, hk] += gv
    return dq, dk, dv


def row_dot(do, o):
    """D = rowsum(dO * O) over the last axis (float64)."""
    return np.sum(np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64), axis=-1)
