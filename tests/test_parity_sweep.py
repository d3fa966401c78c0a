"""Seeded random-shape sweep of attn_fwd, attn_fwd_window and attn_bwd against
the float64 oracle (needs an MI355X).

The hand-picked cases elsewhere pin the edges one at a time; this sweep draws
shapes that combine them: batch, query and KV head counts (GQA group sizes 1,
2, 3, 6 and 16), ragged and exact-tile lengths, T below, equal to and (non-
causal) above S, both head dimensions, with and without the causal mask and
the sliding window, and grids on both sides of the one-block/two-block kernel
switch (fewer or more than 256 workgroups of 128 rows).  Every element of O
and the LSE (and of dQ, dK, dV) is compared at the tolerances of the other
parity tests.  The draw is fixed by its seed, so a failure names a shape that
can be rerun alone.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, check_grad, check_lse, check_o, seed_of, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")

SWEEP_SEED = 20261203


def _draw(n, seed):
    """n shapes (B, Hq, Hkv, T, S, d, causal, window); oracle work per case is
    kept below ~2e10 multiply-adds so the sweep runs in seconds."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 4]))
        grp = int(rng.choice([1, 2, 3, 6, 16]))
        hq = hkv * grp
        b = int(rng.integers(1, 5))
        causal = bool(rng.random() < 0.7)
        t = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 1300)),
                            128 * int(rng.integers(1, 9))]))
        if causal:
            s = t + int(rng.choice([0, 0, int(rng.integers(1, 400))]))
        else:
            s = int(rng.choice([t, int(rng.integers(1, 1500))]))
        window = int(rng.integers(1, s + 64)) if causal and rng.random() < 0.35 else 0
        if b * hq * t * s * d > 2e10:
            continue
        out.append((b, hq, hkv, t, s, d, causal, window))
    return out


FWD = _draw(28, SWEEP_SEED)


def _name(c):
    b, hq, hkv, t, s, d, causal, window = c
    return (f"B{b}_Hq{hq}_Hkv{hkv}_T{t}_S{s}_d{d}" + ("_causal" if causal else "") +
            (f"_w{window}" if window else ""))


def test_sweep_reaches_both_kernels_and_every_feature():
    """The draw covers what it claims (checked on the host, no GPU work)."""
    big = [c for c in FWD if ((c[3] + 127) // 128) * c[0] * c[1] >= 256]
    assert big and len(big) < len(FWD)
    assert {c[5] for c in FWD} == {64, 128}
    assert any(c[6] and c[7] for c in FWD) and any(c[6] and not c[7] for c in FWD)
    assert any(not c[6] for c in FWD) and any(c[3] < c[4] for c in FWD)
    assert any(c[3] % 128 == 0 for c in FWD) and any(c[3] % 128 for c in FWD)


@pytest.mark.parametrize("case", FWD, ids=[_name(c) for c in FWD])
def test_forward_sweep(case):
    b, hq, hkv, t, s, d, causal, window = case
    name = _name(case)
    inp = workloads.make_prefill(b, hq, hkv, t, s, d, "bf16", causal,
                                 seed=seed_of(name), name=name)
    announce(f"sweep attn_fwd{'_window' if window else ''} {name}")
    q, k, v = (x.cuda() for x in (inp.q, inp.k, inp.v))
    if window:
        o, lse = tea.fwd(q, k, v, scale=inp.scale, window=window)
    else:
        o, lse = tea.fwd(q, k, v, scale=inp.scale, causal=causal)
    torch.cuda.synchronize()
    qd, kd, vd = inp.f64()
    o_ref, lse_ref = oracle.attention(qd, kd, vd, inp.scale, causal, window=window)
    check_o(to_np(o), o_ref, "bf16", name)
    check_lse(to_np(lse), lse_ref, name)


# The backward on a smaller draw (its oracle forms P, dP and dS in float64).
BWD = [c for c in _draw(40, SWEEP_SEED + 1) if c[7] == 0 and c[0] * c[1] * c[3] * c[4] * c[5] <= 4e9][:10]


@pytest.mark.parametrize("case", BWD, ids=[_name(c) for c in BWD])
def test_backward_sweep(case):
    b, hq, hkv, t, s, d, causal, _ = case
    name = _name(case)
    inp = workloads.make_backward(b, hq, hkv, t, s, d, causal,
                                  seed=seed_of("bwd " + name), name=name)
    announce(f"sweep attn_bwd {name}")
    q, k, v, do = (x.cuda() for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = tea.fwd(q, k, v, scale=inp.scale, causal=causal)
    dq, dk, dv = tea.bwd(q, k, v, o, lse, do, scale=inp.scale, causal=causal)
    torch.cuda.synchronize()
    qd, kd, vd, dod = inp.f64()
    rq, rk, rv = oracle.attention_backward(qd, kd, vd, dod, inp.scale, causal)
    for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        check_grad(to_np(got), ref, f"{name} {what}")


def _draw_decode(n, seed):
    """n decode shapes (N, Hq, Hkv, d, min_len, max_len)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        grp = int(rng.choice([1, 2, 4, 6, 8, 16]))
        d = int(rng.choice([64, 128]))
        nseq = int(rng.choice([int(rng.integers(1, 8)), int(rng.integers(8, 200))]))
        lo = int(rng.integers(1, 600))
        hi = lo + int(rng.integers(0, 4000))
        out.append((nseq, hkv * grp, hkv, d, lo, hi))
    return out


DEC = _draw_decode(12, SWEEP_SEED + 2)


@pytest.mark.parametrize("case", DEC, ids=[f"N{c[0]}_Hq{c[1]}_Hkv{c[2]}_d{c[3]}_len{c[4]}-{c[5]}"
                                           for c in DEC])
def test_decode_sweep(case):
    nseq, hq, hkv, d, lo, hi = case
    name = f"decode N{nseq} Hq{hq} Hkv{hkv} d{d} len {lo}-{hi}"
    inp = workloads.make_decode(nseq, hq, hkv, d, lo, hi, seed=seed_of(name), poison_tail=True,
                                name=name)
    announce(f"sweep attn_decode_paged {name}")
    q, kp, vp = inp.q.cuda(), inp.k_pool.cuda(), inp.v_pool.cuda()
    bt, sl = torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.seq_lens).cuda()
    o, lse = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale)
    torch.cuda.synchronize()
    qd, kd, vd = inp.f64()
    o_ref, lse_ref = oracle.decode_paged(qd, kd, vd, inp.block_table, inp.seq_lens, inp.scale,
                                         page=inp.page)
    check_o(to_np(o), o_ref, "bf16", name)
    check_lse(to_np(lse), lse_ref, name)


def _draw_chunked(n, seed):
    """n chunked-prefill shapes (N, Hq, Hkv, T, d, min_len, max_len, window)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        grp = int(rng.choice([1, 2, 3, 6]))
        d = int(rng.choice([64, 128]))
        nseq = int(rng.integers(1, 10))
        t = int(rng.integers(1, 400))
        lo = int(rng.integers(1, 500))
        hi = lo + int(rng.integers(0, 1500))
        window = int(rng.integers(1, 600)) if rng.random() < 0.3 else 0
        out.append((nseq, hkv * grp, hkv, t, d, lo, hi, window))
    return out


CHUNKED = _draw_chunked(10, SWEEP_SEED + 3)


@pytest.mark.parametrize("case", CHUNKED, ids=[
    f"N{c[0]}_Hq{c[1]}_Hkv{c[2]}_T{c[3]}_d{c[4]}_len{c[5]}-{c[6]}" + (f"_w{c[7]}" if c[7] else "")
    for c in CHUNKED])
def test_chunked_prefill_sweep(case):
    from tests.test_parity_prefill_paged import _check, _run
    nseq, hq, hkv, t, d, lo, hi, window = case
    name = f"chunked N{nseq} Hq{hq} Hkv{hkv} T{t} d{d} len {lo}-{hi} w{window}"
    inp = workloads.make_prefill_paged(nseq, hq, hkv, t, d, lo, hi, window=window,
                                       seed=seed_of(name), poison_tail=True, extra_pages=3,
                                       name=name)
    announce(f"sweep attn_prefill_paged {name}: seq_lens={inp.seq_lens.tolist()} "
             f"q_lens={inp.q_lens.tolist()}")
    o, lse = _run(inp)
    _check(inp, name, o, lse)


# The quantised page formats over the same kind of draw (fewer shapes).
QDEC = _draw_decode(6, SWEEP_SEED + 4)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("case", QDEC, ids=[f"N{c[0]}_Hq{c[1]}_Hkv{c[2]}_d{c[3]}_len{c[4]}-{c[5]}"
                                            for c in QDEC])
def test_quantised_decode_sweep(case, fmt):
    nseq, hq, hkv, d, lo, hi = case
    name = f"decode {fmt} N{nseq} Hq{hq} Hkv{hkv} d{d} len {lo}-{hi}"
    make = workloads.make_decode_fp8 if fmt == "fp8" else workloads.make_decode_int8
    inp = make(nseq, hq, hkv, d, lo, hi, seed=seed_of(name), poison_tail=True, name=name)
    if fmt == "fp8":
        from tests.test_parity_decode_fp8 import _check
    else:
        from tests.test_parity_decode_int8 import _check
    _check(inp, name)
