"""CPU pins of the float64 oracle (no GPU).

The oracle is the plain definition of attention.  Before any kernel is
compared with it, these tests tie it to things other than itself: hand-derived
closed forms (tests/golden), invariants the pages state (rows of P sum to 1,
stabilised == unstabilised softmax, tile-by-tile accumulation reaches the full
result, paging changes storage only), brute-force loops on tiny inputs, and a
library routine the pages name (PyTorch's scaled_dot_product_attention, run on
the CPU in float64).  The last block plants mistakes in the oracle and checks
that the pins catch each of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.dense as oa
from oracle.online import combine_partials, online_attention_head
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")
TOL = 1e-12


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def _value(s: str) -> float:
    """Evaluate a fixture entry: integer, a/b, ln(x), x/y of those, or nan."""
    s = s.strip()
    if s == "nan":
        return float("nan")
    if "/" in s and not s.startswith("ln("):
        a, b = s.split("/", 1)
        return _value(a) / _value(b)
    if s.startswith("ln(") and ")/" in s:
        a, b = s.split(")/", 1)
        return _value(a + ")") / _value(b)
    if s.startswith("ln(") and s.endswith(")"):
        return math.log(float(Fraction(s[3:-1])))
    return float(Fraction(s))


def _arr(nested):
    return np.vectorize(_value, otypes=[np.float64])(np.array(nested, dtype=object))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def brute_force(q, k, v, scale, causal):
    """Pure-Python loops over one (batch, head): lists in, lists out."""
    T, S, d, dv = len(q), len(k), len(q[0]), len(v[0])
    out, lses = [], []
    for i in range(T):
        logits = []
        for j in range(S):
            if causal and j > i + (S - T):
                continue
            dot = 0.0
            for c in range(d):
                dot += q[i][c] * k[j][c]
            logits.append((j, scale * dot))
        m = max(x for _, x in logits)
        z = sum(math.exp(x - m) for _, x in logits)
        row = [0.0] * dv
        for j, x in logits:
            w = math.exp(x - m) / z
            for c in range(dv):
                row[c] += w * v[j][c]
        out.append(row)
        lses.append(m + math.log(z))
    return np.array(out), np.array(lses)


def sdpa_reference(q, k, v, scale, causal):
    """CPU float64 torch SDPA (KV heads repeated for GQA) + logsumexp."""
    import torch
    import torch.nn.functional as F
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1)
    vt = vt.repeat_interleave(g, dim=1)
    T, S = qt.shape[2], kt.shape[2]
    mask = None
    if causal:
        i = torch.arange(T)[:, None]
        j = torch.arange(S)[None, :]
        mask = j <= i + (S - T)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    logits = scale * (qt @ kt.transpose(-1, -2))
    if mask is not None:
        logits = logits.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(logits, dim=-1).numpy()


# ----------------------------------------------------------------------------
# golden closed forms
# ----------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["prefill"], ids=lambda c: c["name"])
def test_golden_prefill(case):
    q, k, v = (_arr(case[n])[None] for n in ("q", "k", "v"))
    o, lse = oracle.attention(q, k, v, _value(case["scale"]), case["causal"])
    np.testing.assert_allclose(o[0], _arr(case["o"]), rtol=0, atol=TOL)
    np.testing.assert_allclose(lse[0], _arr(case["lse"]), rtol=0, atol=TOL)


@pytest.mark.parametrize("case", _golden()["decode"], ids=lambda c: c["name"])
def test_golden_decode(case):
    o, lse = oracle.decode_paged(_arr(case["q"]), _arr(case["k_pool"]), _arr(case["v_pool"]),
                                 np.array(case["block_table"]), np.array(case["seq_lens"]),
                                 _value(case["scale"]), page=case["page"])
    np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=TOL)
    np.testing.assert_allclose(lse, _arr(case["lse"]), rtol=0, atol=TOL)


# ----------------------------------------------------------------------------
# pins against the pages' statements
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one_and_masked_weights_are_zero(causal):
    rng = np.random.default_rng(1)
    T = S = 33
    sc = oa.scaled_scores(_rand(rng, T, 16), _rand(rng, S, 16), 0.25)
    vis = oa.visible_mask(np.arange(T), S, T, causal)
    p, _, _ = oa.softmax_rows(oa.masked_scores(sc, vis))
    assert np.all(np.abs(p.sum(axis=1) - 1.0) <= TOL)
    assert np.all(p[~vis] == 0.0)
    assert np.all(p[vis] > 0.0)


def test_stabilised_equals_unstabilised_on_small_logits():
    rng = np.random.default_rng(2)
    logits = rng.uniform(-20, 20, size=(50, 40))
    p_stab, _, _ = oa.softmax_rows(logits)
    p_raw = oa.softmax_rows_unstabilised(logits)
    np.testing.assert_allclose(p_stab, p_raw, rtol=1e-12, atol=0)


def test_stabiliser_keeps_large_logits_finite():
    logits = np.array([[1000.0, 999.0, 998.0], [-1000.0, -1001.0, -1002.0]])
    p_stab, m, l = oa.softmax_rows(logits)
    assert np.all(np.isfinite(p_stab))
    np.testing.assert_allclose(p_stab[0], p_stab[1], rtol=1e-12)
    # the exponentiated numerators stay in [0, 1]
    assert np.all(np.exp(logits - m[:, None]) <= 1.0)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        p_raw = oa.softmax_rows_unstabilised(logits)
    assert not np.all(np.isfinite(p_raw))


@pytest.mark.parametrize("T,S", [(1, 1), (2, 2), (3, 3), (5, 5), (17, 17), (64, 64), (3, 17), (5, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_blocked_online_recurrence_equals_direct(T, S, causal):
    rng = np.random.default_rng(3 + T * 100 + S)
    q, k, v = _rand(rng, T, 8), _rand(rng, S, 8), _rand(rng, S, 6)
    o_ref, lse_ref = oracle.attention_head(q, k, v, 0.4, causal)
    for block in sorted({1, 2, 4, 16, S}):
        o, lse = online_attention_head(q, k, v, 0.4, causal, block)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=TOL)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=TOL)


@pytest.mark.parametrize("cuts", [[], [1], [7], [3, 10], [1, 2, 3, 4, 5], [16, 32, 48]])
def test_split_combine_equals_direct(cuts):
    rng = np.random.default_rng(4)
    S = 64
    q, k, v = _rand(rng, 3, 16), _rand(rng, S, 16) * 3, _rand(rng, S, 16)
    o_ref, lse_ref = oracle.attention_head(q, k, v, 0.3, False)
    edges = [0] + cuts + [S]
    parts = [oracle.attention_head(q, k[a:b], v[a:b], 0.3, False) for a, b in zip(edges[:-1], edges[1:])]
    o, lse = combine_partials(parts)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=TOL)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=TOL)


def test_split_combine_ignores_empty_partials():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 2, 8), _rand(rng, 10, 8), _rand(rng, 10, 8)
    ref = oracle.attention_head(q, k, v, 0.5, False)
    empty = (np.zeros((2, 8)), np.full(2, -np.inf))
    o, lse = combine_partials([ref, empty])
    np.testing.assert_allclose(o, ref[0], atol=TOL)
    np.testing.assert_allclose(lse, ref[1], atol=TOL)


def _contiguous_reference(inp):
    """Decode through an explicit dense KV: unpage with plain Python indexing."""
    q, kp, vp = inp.f64()
    N, Hq, d = q.shape
    Hkv, page = kp.shape[1], kp.shape[2]
    o = np.zeros((N, Hq, d))
    lse = np.zeros((N, Hq))
    for n in range(N):
        L = int(inp.seq_lens[n])
        k_dense = np.zeros((1, Hkv, L, d))
        v_dense = np.zeros((1, Hkv, L, d))
        for t in range(L):
            pg = inp.block_table[n, t // page]
            k_dense[0, :, t] = kp[pg, :, t % page]
            v_dense[0, :, t] = vp[pg, :, t % page]
        oo, ll = oracle.attention(q[n][None, :, None, :], k_dense, v_dense, inp.scale, False)
        o[n], lse[n] = oo[0, :, 0], ll[0, :, 0]
    return o, lse


@pytest.mark.parametrize("poison", [False, True])
def test_paged_equals_contiguous_bitwise(poison):
    inp = workloads.make_decode(5, 6, 2, 16, 1, 70, page=16, max_blocks=6, seed=6,
                                poison_tail=poison, lens=[1, 15, 16, 17, 70])
    q, kp, vp = inp.f64()
    o, lse = oracle.decode_paged(q, kp, vp, inp.block_table, inp.seq_lens, inp.scale, page=16)
    o_ref, lse_ref = _contiguous_reference(inp)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)


def test_causal_first_row_is_first_value_and_t1_is_noncausal():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 9, 8), _rand(rng, 9, 8), _rand(rng, 9, 8)
    o, lse = oracle.attention_head(q, k, v, 0.7, True)
    np.testing.assert_allclose(o[0], v[0], atol=TOL)
    np.testing.assert_allclose(lse[0], 0.7 * q[0] @ k[0], atol=TOL)
    # bottom-right alignment: a single query row sees every key
    o1, l1 = oracle.attention_head(q[:1], k, v, 0.7, True)
    o2, l2 = oracle.attention_head(q[:1], k, v, 0.7, False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    rng = np.random.default_rng(8)
    T = S = 12
    q, k, v = np.zeros((T, 8)), _rand(rng, S, 8), _rand(rng, S, 5)
    o, lse = oracle.attention_head(q, k, v, 1.3, causal)
    for i in range(T):
        n = (i + 1) if causal else S
        np.testing.assert_allclose(o[i], v[:n].mean(axis=0), atol=TOL)
        np.testing.assert_allclose(lse[i], math.log(n), atol=TOL)


def test_identical_keys_and_constant_values():
    rng = np.random.default_rng(9)
    q = _rand(rng, 6, 8)
    k = np.repeat(_rand(rng, 1, 8), 10, axis=0)
    v = _rand(rng, 10, 4)
    o, lse = oracle.attention_head(q, k, v, 0.9, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=TOL)
    np.testing.assert_allclose(lse, 0.9 * q @ k[0] + math.log(10), atol=TOL)
    o_c, _ = oracle.attention_head(q, _rand(rng, 10, 8), np.full((10, 4), -2.5), 0.9, False)
    np.testing.assert_allclose(o_c, -2.5, atol=TOL)


def test_joint_key_value_permutation_invariance_and_single_key():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 7, 8), _rand(rng, 11, 8), _rand(rng, 11, 8)
    perm = rng.permutation(11)
    o, lse = oracle.attention_head(q, k, v, 0.5, False)
    o_p, lse_p = oracle.attention_head(q, k[perm], v[perm], 0.5, False)
    np.testing.assert_allclose(o_p, o, atol=TOL)
    np.testing.assert_allclose(lse_p, lse, atol=TOL)
    o1, _ = oracle.attention_head(q, k[:1], v[:1], 0.5, False)
    np.testing.assert_allclose(o1, np.broadcast_to(v[0], o1.shape), atol=TOL)


def test_gqa_equals_mha_on_repeated_kv_heads():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, T, d = 2, 6, 2, 9, 8
    q, k, v = _rand(rng, B, Hq, T, d), _rand(rng, B, Hkv, T, d), _rand(rng, B, Hkv, T, d)
    g = Hq // Hkv
    k_rep = np.stack([k[:, h // g] for h in range(Hq)], axis=1)
    v_rep = np.stack([v[:, h // g] for h in range(Hq)], axis=1)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.3, causal)
        o2, lse2 = oracle.attention(q, k_rep, v_rep, 0.3, causal)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("B,Hq,Hkv,T,S,d,causal", [
    (1, 1, 1, 16, 16, 8, False), (2, 4, 4, 33, 33, 16, True), (1, 6, 2, 20, 20, 8, True),
    (2, 3, 1, 5, 40, 8, False), (1, 2, 2, 7, 19, 8, True)])
def test_matches_torch_sdpa_float64(B, Hq, Hkv, T, S, d, causal):
    rng = np.random.default_rng(12 + T + S)
    q, k, v = _rand(rng, B, Hq, T, d), _rand(rng, B, Hkv, S, d), _rand(rng, B, Hkv, S, d)
    o, lse = oracle.attention(q, k, v, 0.35, causal)
    o_t, lse_t = sdpa_reference(q, k, v, 0.35, causal)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse, lse_t, rtol=0, atol=1e-10)


@pytest.mark.parametrize("T,S,d,causal", [(1, 1, 1, False), (3, 5, 4, False), (8, 8, 8, True),
                                           (4, 7, 3, True), (6, 6, 5, False)])
def test_matches_brute_force_loops(T, S, d, causal):
    rng = np.random.default_rng(13 + T * S)
    q, k, v = _rand(rng, T, d), _rand(rng, S, d), _rand(rng, S, d)
    o, lse = oracle.attention_head(q, k, v, 0.6, causal)
    o_b, lse_b = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.6, causal)
    np.testing.assert_allclose(o, o_b, rtol=0, atol=TOL)
    np.testing.assert_allclose(lse, lse_b, rtol=0, atol=TOL)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_reconstructs_the_output(causal):
    rng = np.random.default_rng(14)
    T = S = 20
    q, k, v = _rand(rng, T, 8), _rand(rng, S, 8), _rand(rng, S, 8)
    o, lse = oracle.attention_head(q, k, v, 0.8, causal)
    sc = 0.8 * q @ k.T
    vis = oa.visible_mask(np.arange(T), S, T, causal)
    w = np.where(vis, np.exp(sc - lse[:, None]), 0.0)
    np.testing.assert_allclose(w @ v, o, atol=TOL)


def test_sampled_rows_equal_full_rows():
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 1, 4, 50, 8), _rand(rng, 1, 2, 50, 8), _rand(rng, 1, 2, 50, 8)
    o, lse = oracle.attention(q, k, v, 0.4, True)
    rows = [0, 7, 49, 23]
    o_r, lse_r = oracle.attention_rows(q, k, v, 0.4, True, 0, 3, rows)
    assert np.array_equal(o_r, o[0, 3, rows]) and np.array_equal(lse_r, lse[0, 3, rows])


def test_row_chunking_does_not_change_results(monkeypatch):
    rng = np.random.default_rng(16)
    q, k, v = _rand(rng, 37, 8), _rand(rng, 37, 8), _rand(rng, 37, 8)
    o, lse = oracle.attention_head(q, k, v, 0.4, True)
    monkeypatch.setattr(oa, "ROW_CHUNK", 5)
    o5, lse5 = oracle.attention_head(q, k, v, 0.4, True)
    assert np.array_equal(o, o5) and np.array_equal(lse, lse5)


def test_decode_workload_generator_is_pinned():
    """default_rng(1005) lengths: sum 308,010 and 19,277 pages (numpy 2.x PCG64)."""
    rng = np.random.default_rng(1005)
    lens = rng.integers(512, 8193, 64)
    assert int(lens.sum()) == 308010
    assert list(lens[:3]) == [3820, 1143, 7870]
    assert int(((lens + 15) // 16).sum()) == 19277


def test_decode_workload_block_table_is_a_permutation():
    inp = workloads.make_decode(7, 4, 2, 16, 1, 100, page=16, max_blocks=8, seed=17)
    used = []
    for n in range(inp.N):
        cnt = (int(inp.seq_lens[n]) + 15) // 16
        assert (inp.block_table[n, :cnt] >= 0).all()
        assert (inp.block_table[n, cnt:] == -1).all()
        used.extend(inp.block_table[n, :cnt].tolist())
    assert sorted(used) == list(range(inp.num_pages))


# ----------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must fail at least one pin
# ----------------------------------------------------------------------------

def _pins_pass():
    """Run a compact set of the pins above; False if any fails."""
    checks = [
        lambda: [test_golden_prefill(c) for c in _golden()["prefill"]],
        lambda: [test_golden_decode(c) for c in _golden()["decode"]],
        lambda: test_matches_torch_sdpa_float64(1, 6, 2, 20, 20, 8, True),
        lambda: test_matches_brute_force_loops(4, 7, 3, True),
        lambda: test_causal_first_row_is_first_value_and_t1_is_noncausal(),
        lambda: test_gqa_equals_mha_on_repeated_kv_heads(),
        lambda: test_paged_equals_contiguous_bitwise(True),
        lambda: test_lse_reconstructs_the_output(True),
    ]
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return False
    return True


def test_unmodified_oracle_passes_the_pin_set():
    assert _pins_pass()


def _mask_off_by_one(rows, S, T, causal, window=0):
    rows = np.asarray(rows)
    if not causal:
        return np.ones((rows.shape[0], S), dtype=bool)
    return np.arange(S)[None, :] < (rows[:, None] + (S - T))


def _mask_top_left(rows, S, T, causal, window=0):
    rows = np.asarray(rows)
    if not causal:
        return np.ones((rows.shape[0], S), dtype=bool)
    return np.arange(S)[None, :] <= rows[:, None]


def _scores_scale_twice(q_rows, k, scale):
    return scale * scale * (q_rows @ k.T)


def _scores_transposed_k(q_rows, k, scale):
    return scale * (q_rows @ k[::-1].T)


_TRUE_SOFTMAX = oa.softmax_rows


def _softmax_no_max_in_lse(logits):
    p, m, l = _TRUE_SOFTMAX(logits)
    return p, np.zeros_like(m), l


def _softmax_dropped_denominator(logits):
    m = np.max(logits, axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e, m[..., 0], np.sum(e, axis=-1)


def _gqa_modulo(h, Hq, Hkv):
    return h % Hkv


def _gather_swapped(pool, row, length, hk, page):
    t = np.arange(length)
    pages = np.asarray(row, dtype=np.int64)[np.minimum(t % page, len(row) - 1)]
    return np.asarray(pool, dtype=np.float64)[np.maximum(pages, 0), hk, np.minimum(t // page, page - 1), :]


@pytest.mark.parametrize("name,target,mutant", [
    ("causal mask off by one", "visible_mask", _mask_off_by_one),
    ("causal mask top-left aligned", "visible_mask", _mask_top_left),
    ("scale applied twice", "scaled_scores", _scores_scale_twice),
    ("keys in the wrong order", "scaled_scores", _scores_transposed_k),
    ("LSE without the row max", "softmax_rows", _softmax_no_max_in_lse),
    ("softmax denominator dropped", "softmax_rows", _softmax_dropped_denominator),
    ("GQA heads interleaved", "kv_head_of", _gqa_modulo),
    ("page index and slot swapped", "gather_pages", _gather_swapped),
])
def test_planted_mistake_is_caught(monkeypatch, name, target, mutant):
    monkeypatch.setattr(oa, target, mutant)
    assert not _pins_pass(), f"pins did not catch: {name}"
