"""Pins of the oracle for the sliding-window mask, chunked prefill on a paged
cache, and fp8 (E4M3) KV pages (CPU only).

Each is checked against something it does not compute itself: pure-Python
brute force, closed forms, attention over explicit key slices, contiguous
key/value layouts built here rather than gathered, the decode oracle for the
last token, and torch's own float8_e4m3fn conversion for every code.
"""
import math
import zlib

import numpy as np
import pytest

import oracle


def _rng(name):
    return np.random.default_rng(zlib.crc32(name.encode()))


# --- sliding window -------------------------------------------------------------

def _brute_window_row(q, k, v, scale, i, S, T, W):
    """Pure-Python loops: keys i+(S-T)-W < j <= i+(S-T)."""
    diag = i + (S - T)
    keys = [j for j in range(S) if diag - W < j <= diag]
    logits = [scale * sum(q[i][c] * k[j][c] for c in range(len(q[i]))) for j in keys]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    tot = sum(w)
    o = [sum(w[a] * v[j][c] for a, j in enumerate(keys)) / tot for c in range(len(v[0]))]
    return o, m + math.log(tot)


@pytest.mark.parametrize("T,S,W", [(5, 5, 1), (5, 5, 2), (6, 9, 3), (4, 7, 7), (3, 3, 10), (7, 7, 4)])
def test_window_matches_brute_force(T, S, W):
    rng = _rng(f"win{T}_{S}_{W}")
    q, k, v = rng.standard_normal((T, 3)), rng.standard_normal((S, 3)), rng.standard_normal((S, 2))
    o, lse = oracle.attention_head(q, k, v, 0.7, True, window=W)
    for i in range(T):
        ob, lb = _brute_window_row(q.tolist(), k.tolist(), v.tolist(), 0.7, i, S, T, W)
        np.testing.assert_allclose(o[i], ob, rtol=1e-12, atol=1e-12)
        assert abs(lse[i] - lb) < 1e-12


def test_window_equals_attention_over_the_key_slice():
    """Row i with window W is non-causal attention over keys [i+S-T-W+1, i+S-T]."""
    rng = _rng("slice")
    T, S, W = 40, 70, 13
    q, k, v = rng.standard_normal((T, 8)), rng.standard_normal((S, 8)), rng.standard_normal((S, 5))
    o, lse = oracle.attention_head(q, k, v, 0.4, True, window=W)
    for i in range(T):
        lo, hi = max(0, i + S - T - W + 1), i + S - T
        os_, ls = oracle.attention_head(q[i:i + 1], k[lo:hi + 1], v[lo:hi + 1], 0.4, False)
        np.testing.assert_allclose(o[i], os_[0], rtol=1e-12, atol=1e-13)
        assert abs(lse[i] - ls[0]) < 1e-12


def test_window_one_is_the_diagonal_value():
    rng = _rng("w1")
    T, S = 6, 10
    q, k, v = rng.standard_normal((T, 4)), rng.standard_normal((S, 4)), rng.standard_normal((S, 3))
    o, lse = oracle.attention_head(q, k, v, 0.5, True, window=1)
    for i in range(T):
        j = i + S - T
        np.testing.assert_allclose(o[i], v[j], rtol=0, atol=1e-15)
        assert abs(lse[i] - 0.5 * q[i] @ k[j]) < 1e-13


def test_window_covering_all_keys_is_plain_causal():
    rng = _rng("wall")
    q, k, v = rng.standard_normal((9, 4)), rng.standard_normal((12, 4)), rng.standard_normal((12, 4))
    a = oracle.attention_head(q, k, v, 0.3, True, window=12)
    b = oracle.attention_head(q, k, v, 0.3, True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_window_off_by_one_is_caught():
    """A window that keeps one key too many (j >= diag - W) differs from the pin."""
    rng = _rng("offbyone")
    T, S, W = 5, 8, 3
    q, k, v = rng.standard_normal((T, 3)), rng.standard_normal((S, 3)), rng.standard_normal((S, 2))
    good, _ = oracle.attention_head(q, k, v, 0.9, True, window=W)
    wrong, _ = oracle.attention_head(q, k, v, 0.9, True, window=W + 1)
    ob, _ = _brute_window_row(q.tolist(), k.tolist(), v.tolist(), 0.9, T - 1, S, T, W)
    np.testing.assert_allclose(good[T - 1], ob, atol=1e-12)
    assert np.abs(wrong[T - 1] - ob).max() > 1e-3


def test_window_needs_causal():
    with pytest.raises(ValueError):
        oracle.visible_mask(np.arange(3), 3, 3, False, window=2)


# --- chunked prefill on a paged cache -------------------------------------------

def _paged_case(name, N=3, Hq=4, Hkv=2, T=20, d=8, page=16, lens=(40, 17, 33), qlens=(20, 5, 1)):
    rng = _rng(name)
    lens, qlens = np.array(lens), np.array(qlens)
    pages_per = (lens + page - 1) // page
    P = int(pages_per.sum()) + 3                        # a few pages nobody uses
    perm = rng.permutation(P)
    max_blocks = int(pages_per.max()) + 1
    bt = np.full((N, max_blocks), -1, dtype=np.int64)
    kc = [rng.standard_normal((Hkv, int(L), d)) for L in lens]   # contiguous, built here
    vc = [rng.standard_normal((Hkv, int(L), d)) for L in lens]
    k_pool = rng.standard_normal((P, Hkv, page, d))
    v_pool = rng.standard_normal((P, Hkv, page, d))
    off = 0
    for n in range(N):
        for b in range(int(pages_per[n])):
            pg = perm[off + b]
            bt[n, b] = pg
            lo, hi = b * page, min((b + 1) * page, int(lens[n]))
            k_pool[pg, :, :hi - lo] = kc[n][:, lo:hi]
            v_pool[pg, :, :hi - lo] = vc[n][:, lo:hi]
        off += int(pages_per[n])
    q = rng.standard_normal((N, Hq, T, d))
    return q, k_pool, v_pool, bt, lens, qlens, kc, vc


def test_prefill_paged_equals_contiguous_causal():
    q, kp, vp, bt, lens, qlens, kc, vc = _paged_case("pp_contig")
    o, lse = oracle.prefill_paged(q, kp, vp, bt, lens, qlens, 0.35)
    Hq, Hkv = q.shape[1], kp.shape[1]
    for n in range(len(lens)):
        Tn = int(qlens[n])
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            oc, lc = oracle.attention_head(q[n, h, :Tn], kc[n][hk], vc[n][hk], 0.35, True)
            np.testing.assert_allclose(o[n, h, :Tn], oc, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse[n, h, :Tn], lc, rtol=1e-13, atol=1e-13)
        assert np.isnan(o[n, :, Tn:]).all() and np.isnan(lse[n, :, Tn:]).all()


def test_prefill_paged_last_token_equals_decode():
    """A chunk of one query is the decode step of that sequence."""
    q, kp, vp, bt, lens, _, _, _ = _paged_case("pp_dec", qlens=(1, 1, 1))
    o, lse = oracle.prefill_paged(q, kp, vp, bt, lens, np.ones(3, dtype=np.int64), 0.6)
    od, ld = oracle.decode_paged(q[:, :, 0, :], kp, vp, bt, lens, 0.6)
    np.testing.assert_allclose(o[:, :, 0], od, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[:, :, 0], ld, rtol=1e-13, atol=1e-13)


def test_prefill_paged_whole_sequence_with_window():
    """q_len = seq_len is plain windowed causal prefill on the contiguous keys."""
    q, kp, vp, bt, lens, _, kc, vc = _paged_case("pp_full", T=40, qlens=(40, 17, 33))
    o, lse = oracle.prefill_paged(q, kp, vp, bt, lens, lens, 0.5, window=9)
    for n in range(3):
        L = int(lens[n])
        for h in range(4):
            oc, lc = oracle.attention_head(q[n, h, :L], kc[n][h // 2], vc[n][h // 2], 0.5, True,
                                           window=9)
            np.testing.assert_allclose(o[n, h, :L], oc, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse[n, h, :L], lc, rtol=1e-13, atol=1e-13)


def test_prefill_paged_rejects_bad_lengths():
    q, kp, vp, bt, lens, _, _, _ = _paged_case("pp_bad")
    with pytest.raises(ValueError):
        oracle.prefill_paged(q, kp, vp, bt, lens, np.array([21, 1, 1]), 0.5)   # > T
    with pytest.raises(ValueError):
        oracle.prefill_paged(q, kp, vp, bt, lens, np.array([1, 18, 1]), 0.5)   # > seq_len


# --- fp8 E4M3 pages --------------------------------------------------------------

def test_e4m3_closed_forms():
    f = oracle.e4m3_to_float
    assert f([0x00])[0] == 0.0 and math.copysign(1.0, f([0x80])[0]) == -1.0
    assert f([0x38])[0] == 1.0 and f([0xB8])[0] == -1.0          # exponent field 7 = bias
    assert f([0x7E])[0] == 448.0 and f([0xFE])[0] == -448.0      # largest finite
    assert f([0x01])[0] == 2.0 ** -9                             # smallest subnormal
    assert f([0x07])[0] == 7 * 2.0 ** -9
    assert f([0x08])[0] == 2.0 ** -6                             # smallest normal
    assert f([0x3C])[0] == 1.5 and f([0x40])[0] == 2.0
    assert np.isnan(f([0x7F])[0]) and np.isnan(f([0xFF])[0])
    assert not np.isnan(f([0x78, 0x7D])).any()                   # no infinities in "fn"


def test_e4m3_all_codes_match_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_float(codes)
    assert (np.isnan(ref) == np.isnan(got)).all()
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_e4m3_positive_codes_increase():
    vals = oracle.e4m3_to_float(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(vals) > 0).all()


def _fp8_case(name):
    rng = _rng(name)
    N, Hq, Hkv, d, page = 3, 4, 2, 8, 16
    lens = np.array([20, 33, 7])
    P = int(((lens + page - 1) // page).sum())
    perm = rng.permutation(P)
    bt = np.full((N, 3), -1, dtype=np.int64)
    off = 0
    for n in range(N):
        c = int((lens[n] + page - 1) // page)
        bt[n, :c] = perm[off:off + c]
        off += c
    kc = rng.integers(0, 256, (P, Hkv, page, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (P, Hkv, page, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x11                               # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x22
    q = rng.standard_normal((N, Hq, d))
    return q, kc, vc, bt, lens


def test_fp8_value_scale_scales_the_output():
    """O is linear in V and the LSE does not depend on V."""
    q, kc, vc, bt, lens = _fp8_case("fp8v")
    o1, l1 = oracle.decode_paged_fp8(q, kc, vc, 0.01, 1.0, bt, lens, 0.3)
    o2, l2 = oracle.decode_paged_fp8(q, kc, vc, 0.01, 0.125, bt, lens, 0.3)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(l1, l2)


def test_fp8_key_scale_is_a_softmax_temperature():
    """k_scale multiplies every logit, the same as multiplying the attention scale."""
    q, kc, vc, bt, lens = _fp8_case("fp8k")
    o1, l1 = oracle.decode_paged_fp8(q, kc, vc, 0.02, 0.5, bt, lens, 0.3)
    o2, l2 = oracle.decode_paged_fp8(q, kc, vc, 1.0, 0.5, bt, lens, 0.3 * 0.02)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-13)


def test_fp8_single_code_value_cache():
    """All V codes equal (0x38 = 1.0): O is v_scale in every component."""
    q, kc, vc, bt, lens = _fp8_case("fp8c")
    vc[:] = 0x38
    o, _ = oracle.decode_paged_fp8(q, kc, vc, 0.05, 0.75, bt, lens, 0.3)
    np.testing.assert_allclose(o, 0.75, rtol=1e-14, atol=1e-14)


# --- int8 pages ------------------------------------------------------------------

def test_int8_closed_forms():
    f = oracle.int8_to_float
    assert list(f([0x00, 0x01, 0x7F, 0x80, 0x81, 0xFE, 0xFF])) == [0, 1, 127, -128, -127, -2, -1]


def test_int8_all_codes_match_numpy_view():
    codes = np.arange(256, dtype=np.uint8)
    np.testing.assert_array_equal(oracle.int8_to_float(codes),
                                  codes.view(np.int8).astype(np.float64))


def _int8_case(name):
    q, kc, vc, bt, lens = _fp8_case(name)       # any bytes are valid int8 codes
    return q, kc, vc, bt, lens


def test_int8_value_scale_scales_the_output():
    q, kc, vc, bt, lens = _int8_case("i8v")
    o1, l1 = oracle.decode_paged_int8(q, kc, vc, 0.01, 1.0, bt, lens, 0.3)
    o2, l2 = oracle.decode_paged_int8(q, kc, vc, 0.01, 0.125, bt, lens, 0.3)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(l1, l2)


def test_int8_key_scale_is_a_softmax_temperature():
    q, kc, vc, bt, lens = _int8_case("i8k")
    o1, l1 = oracle.decode_paged_int8(q, kc, vc, 0.02, 0.5, bt, lens, 0.3)
    o2, l2 = oracle.decode_paged_int8(q, kc, vc, 1.0, 0.5, bt, lens, 0.3 * 0.02)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-13)


def test_int8_constant_value_cache_and_zero_keys():
    """V codes all -3: O = -3 v_scale.  K codes all 0: every logit is 0, so the
    LSE is ln(length) and O is the mean of the visible values."""
    q, kc, vc, bt, lens = _int8_case("i8c")
    vc2 = np.full_like(vc, 0xFD)                                  # -3
    o, _ = oracle.decode_paged_int8(q, kc, vc2, 0.05, 0.75, bt, lens, 0.3)
    np.testing.assert_allclose(o, -2.25, rtol=1e-14, atol=1e-14)
    kz = np.zeros_like(kc)
    o, lse = oracle.decode_paged_int8(q, kz, vc, 0.05, 0.5, bt, lens, 0.3)
    np.testing.assert_allclose(lse, np.log(lens.astype(np.float64))[:, None] * np.ones(q.shape[1]),
                               rtol=1e-14, atol=1e-14)
    vals = oracle.int8_to_float(vc) * 0.5
    for n in range(len(lens)):
        L = int(lens[n])
        for h in range(q.shape[1]):
            hk = h // (q.shape[1] // kc.shape[1])
            rows = [vals[bt[n, t // 16], hk, t % 16] for t in range(L)]
            np.testing.assert_allclose(o[n, h], np.mean(rows, axis=0), rtol=1e-12, atol=1e-14)


def test_int8_sign_mistake_is_caught():
    """A reading of the bytes as unsigned changes the result (the pins above see it)."""
    q, kc, vc, bt, lens = _int8_case("i8s")
    kc = kc | 0x80                                                # every key code negative
    o_s, _ = oracle.decode_paged_int8(q, kc, vc, 0.05, 0.5, bt, lens, 0.3)
    o_u, _ = oracle.decode_paged(q, 0.05 * kc.astype(np.float64), 0.5 * vc.astype(np.float64), bt,
                                 lens, 0.3)
    assert np.abs(o_s - o_u).max() > 1e-3
