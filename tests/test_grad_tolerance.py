"""The gradient tolerances of the GPU parity tests, derived from a model of the
roundings rather than from the kernels' own errors (CPU only).

The backward pass computes in fp32 from bf16 inputs and rounds exactly where
an MFMA takes an operand or a result is stored: the forward output O (bf16,
which D = rowsum(dO * O) is formed from), P before dV = P^T dO, dS before
dQ = scale dS K and dK = scale dS^T Q, and the three gradients themselves.
This test applies those roundings (round to nearest even to bf16) to a float64
evaluation of the same formulas ("Advanced Attention Mechanisms - II", section
"Flash Attention": the backward pass recomputes P from the saved statistics)
and measures the result against the float64 oracle with the GPU tests' own
metrics: max|dG| / max|G| and mean|dG| / mean|G|.  The tolerances must sit
above what the roundings alone produce, with room for the fp32 accumulation
order, and not so far above that a real mistake (an error of the size of a
dropped term) would pass.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import GRAD_MAX_REL, GRAD_MEAN_REL


def _bf16(x):
    """Round to the nearest bf16 (ties to even), returned as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _rounded_backward(q, k, v, do, scale, causal):
    B, Hq, T, _ = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    g = Hq // Hkv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            s = q[b, h] @ k[b, hk].T * scale
            if causal:
                i, j = np.arange(T)[:, None], np.arange(S)[None, :]
                s = np.where(j > i + (S - T), -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
            p = np.exp(s - lse)
            o = _bf16(p @ v[b, hk])
            dd = (do[b, h] * o).sum(axis=1, keepdims=True)
            ds = _bf16(p * (do[b, h] @ v[b, hk].T - dd))
            dv[b, hk] += _bf16(p).T @ do[b, h]
            dq[b, h] = scale * ds @ k[b, hk]
            dk[b, hk] += scale * ds.T @ q[b, h]
    return _bf16(dq), _bf16(dk), _bf16(dv)


def test_bf16_rounding_helper():
    assert _bf16(1.0) == 1.0
    assert _bf16(1.0 + 2.0 ** -8) == 1.0            # tie: to even (mantissa 0)
    assert _bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6   # tie: to even (mantissa 2)
    assert _bf16(1.0 + 2.0 ** -7) == 1.0 + 2.0 ** -7
    assert _bf16(-3.3) == -_bf16(3.3)


# name, B, Hq, Hkv, T, S, d, causal
CASES = [
    ("causal_d128", 1, 2, 2, 257, 257, 128, True),
    ("noncausal_gqa_t_ne_s", 2, 4, 2, 130, 200, 128, False),
    ("causal_gqa6_d64", 1, 12, 2, 300, 300, 64, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tolerances_sit_just_above_the_rounding_model(case):
    name, B, Hq, Hkv, T, S, d, causal = case
    x = workloads.make_backward(B, Hq, Hkv, T, S, d, causal, seed=7, name=name)
    q, k, v, do = x.f64()
    ref = oracle.attention_backward(q, k, v, do, x.scale, causal)
    got = _rounded_backward(q, k, v, do, x.scale, causal)
    for g, r, what in zip(got, ref, ("dq", "dk", "dv")):
        err = np.abs(g - r)
        rmax = err.max() / np.abs(r).max()
        rmean = err.mean() / np.abs(r).mean()
        # the bounds leave a margin over the model ...
        assert rmax <= GRAD_MAX_REL / 1.5, (what, rmax)
        assert rmean <= GRAD_MEAN_REL / 1.3, (what, rmean)
        # ... and are of its size, not orders of magnitude looser
        assert rmean >= GRAD_MEAN_REL / 2.5, (what, rmean)
        assert rmax >= GRAD_MAX_REL / 6, (what, rmax)
