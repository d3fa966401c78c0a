"""Pins of the float64 backward-pass oracle (CPU only).

The oracle writes the chain rule of the forward definition out in closed
form.  These tests fix it against things it does not compute itself:
central finite differences of the forward oracle (a different computation:
forward evaluations only), closed forms of special inputs, conservation
laws of the softmax, and the grouped-query sum.  A planted mistake (the
softmax Jacobian's D term dropped) must fail the finite-difference pin.
"""
import zlib

import numpy as np
import pytest

import oracle
import oracle.backward as ob


def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention_head(q, k, v, scale, causal)
    return float(np.sum(o * do))


def _numeric_grads(q, k, v, do, scale, causal, h=1e-6):
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, causal)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


CASES = [
    # name, T, S, d, dv, causal
    ("square_causal", 5, 5, 4, 3, True),
    ("square_noncausal", 4, 4, 3, 5, False),
    ("t_lt_s_causal_bottom_right", 3, 7, 4, 2, True),
    ("t_gt_s_noncausal", 6, 3, 2, 4, False),
    ("single_key", 3, 1, 4, 4, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gradients_match_finite_differences(case):
    name, T, S, d, dv, causal = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q, k = rng.standard_normal((T, d)), rng.standard_normal((S, d))
    v, do = rng.standard_normal((S, dv)), rng.standard_normal((T, dv))
    scale = 0.8
    dq, dk, dvv, _, _ = oracle.attention_head_backward(q, k, v, do, scale, causal)
    nq, nk, nv = _numeric_grads(q.copy(), k.copy(), v.copy(), do, scale, causal)
    for got, ref, what in ((dq, nq, "dq"), (dk, nk, "dk"), (dvv, nv, "dv")):
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-8, err_msg=f"{name} {what}")


def test_planted_mistake_fails_the_finite_difference_pin():
    """Dropping D (dS = P * dP) is caught by the finite differences."""
    rng = np.random.default_rng(7)
    T, S, d = 4, 5, 3
    q, k, v, do = (rng.standard_normal(sh) for sh in ((T, d), (S, d), (S, d), (T, d)))
    scale = 0.9
    s = oracle.masked_scores(oracle.scaled_scores(q, k, scale),
                             oracle.visible_mask(np.arange(T), S, T, False))
    p, _, _ = oracle.softmax_rows(s)
    wrong_dq = scale * ((p * (do @ v.T)) @ k)
    nq, _, _ = _numeric_grads(q.copy(), k.copy(), v.copy(), do, scale, False)
    assert np.abs(wrong_dq - nq).max() > 1e-3
    right_dq = oracle.attention_head_backward(q, k, v, do, scale, False)[0]
    np.testing.assert_allclose(right_dq, nq, rtol=1e-6, atol=1e-8)


def test_value_gradient_conserves_the_output_gradient():
    """Rows of P sum to 1, so sum_j dV_j = sum_i dO_i (columnwise)."""
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.standard_normal(sh) for sh in ((9, 8), (12, 8), (12, 6), (9, 6)))
    for causal in (False, True):
        _, _, dv, _, _ = oracle.attention_head_backward(q, k, v, do, 0.35, causal)
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_key_gradient_sums_to_zero():
    """Each row of dS sums to zero (softmax is shift-invariant), so sum_j dK_j = 0."""
    rng = np.random.default_rng(12)
    q, k, v, do = (rng.standard_normal(sh) for sh in ((7, 5), (10, 5), (10, 4), (7, 4)))
    for causal in (False, True):
        _, dk, _, _, _ = oracle.attention_head_backward(q, k, v, do, 0.6, causal)
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)


def test_identical_keys_give_zero_query_gradient():
    """With every key equal the scores do not depend on q: dQ = 0."""
    rng = np.random.default_rng(13)
    q, v, do = rng.standard_normal((6, 4)), rng.standard_normal((8, 3)), rng.standard_normal((6, 3))
    k = np.tile(rng.standard_normal((1, 4)), (8, 1))
    dq, _, _, _, _ = oracle.attention_head_backward(q, k, v, do, 0.5, False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)


def test_single_visible_key_passes_the_gradient_straight_through():
    """Causal row 0 sees only key 0: P[0,0] = 1, so dV_0 gets dO_0 and row 0 has no dQ."""
    rng = np.random.default_rng(14)
    q, k, v, do = (rng.standard_normal(sh) for sh in ((1, 4), (1, 4), (1, 3), (1, 3)))
    dq, dk, dv, o, lse = oracle.attention_head_backward(q, k, v, do, 0.5, True)
    np.testing.assert_allclose(dv, do, rtol=0, atol=0)
    np.testing.assert_allclose(dq, 0.0, atol=0)
    np.testing.assert_allclose(dk, 0.0, atol=0)
    np.testing.assert_allclose(o, v, rtol=0, atol=0)


def test_grouped_heads_sum_into_their_kv_head():
    """Hq=4 over Hkv=2 equals MHA with repeated KV heads, dK/dV summed over repeats."""
    rng = np.random.default_rng(15)
    B, Hq, Hkv, T, S, d = 2, 4, 2, 5, 6, 3
    q, do = rng.standard_normal((B, Hq, T, d)), rng.standard_normal((B, Hq, T, d))
    k, v = rng.standard_normal((B, Hkv, S, d)), rng.standard_normal((B, Hkv, S, d))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.7, True)
    krep, vrep = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    dq2, dk2, dv2 = oracle.attention_backward(q, krep, vrep, do, 0.7, True)
    np.testing.assert_allclose(dq, dq2, rtol=0, atol=0)
    np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, Hq // Hkv, S, d).sum(axis=2), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, Hq // Hkv, S, d).sum(axis=2), rtol=1e-14, atol=1e-14)


def test_row_dot_equals_rowsum_of_p_times_dp():
    """D = rowsum(dO * O) = rowsum(P * dP), the two readings of the same term."""
    rng = np.random.default_rng(16)
    q, k, v, do = (rng.standard_normal(sh) for sh in ((6, 4), (9, 4), (9, 5), (6, 5)))
    s = oracle.masked_scores(oracle.scaled_scores(q, k, 0.4), oracle.visible_mask(np.arange(6), 9, 6, True))
    p, _, _ = oracle.softmax_rows(s)
    o = p @ v
    np.testing.assert_allclose(ob.row_dot(do, o), np.sum(p * (do @ v.T), axis=1), rtol=1e-12, atol=1e-12)
