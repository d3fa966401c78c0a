"""GPU parity of attn_fwd against the float64 oracle (needs an MI355X).

Small and ragged shapes are compared element by element over the whole
output; the named workloads at full size are compared in full where the
oracle finishes in seconds (prefill_1, prefill_2) and otherwise (prefill_3,
prefill_4) on sampled query rows of every head, with NaN-filled outputs so
that an unwritten row fails, in the same launch configuration the benchmark
times.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, check_lse, check_o, seed_of, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


def _run(inp):
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    o, lse = tea.fwd(q, k, v, scale=inp.scale, causal=inp.causal)
    torch.cuda.synchronize()
    return o, lse


def _full_check(inp, name):
    announce(f"attn_fwd {name}: B={inp.B} Hq={inp.Hq} Hkv={inp.Hkv} T={inp.T} S={inp.S} d={inp.d} "
             f"{inp.dtype} causal={inp.causal}")
    o, lse = _run(inp)
    q, k, v = inp.f64()
    o_ref, lse_ref = oracle.attention(q, k, v, inp.scale, inp.causal)
    check_o(to_np(o), o_ref, inp.dtype, name)
    check_lse(to_np(lse), lse_ref, name)


# name, B, Hq, Hkv, T, S, d, dtype, causal
SMALL = [
    ("t1_s1", 1, 1, 1, 1, 1, 64, "bf16", False),
    ("t1_s1_causal_d128", 1, 2, 1, 1, 1, 128, "bf16", True),
    ("t17_causal", 1, 2, 2, 17, 17, 64, "bf16", True),
    ("t63_causal_d128", 2, 2, 2, 63, 63, 128, "bf16", True),
    ("t65_causal", 1, 3, 3, 65, 65, 64, "bf16", True),
    ("t128_exact_tiles", 1, 2, 2, 128, 128, 128, "bf16", True),
    ("t256_exact_tiles_d64", 1, 2, 2, 256, 256, 64, "bf16", True),
    ("t129_s127", 1, 2, 2, 129, 127, 64, "bf16", False),
    ("t1000_gqa6", 1, 12, 2, 1000, 1000, 128, "bf16", True),
    ("t1000_mqa_noncausal", 1, 4, 1, 1000, 1000, 64, "bf16", False),
    ("gqa2_ragged", 2, 4, 2, 300, 300, 128, "bf16", True),
    ("gqa12_mqa", 1, 12, 1, 257, 257, 64, "bf16", True),
    ("noncausal_t_lt_s", 1, 2, 2, 100, 333, 128, "bf16", False),
    ("noncausal_t_gt_s", 1, 2, 1, 333, 100, 64, "bf16", False),
    ("causal_t_lt_s_bottom_right", 1, 2, 2, 100, 333, 128, "bf16", True),
    ("group_count_multiple_of_8", 4, 4, 2, 200, 200, 64, "bf16", True),
    ("f32_t1", 1, 1, 1, 1, 1, 64, "f32", False),
    ("f32_causal_d128", 2, 2, 1, 200, 200, 128, "f32", True),
    ("f32_ragged_d64", 1, 3, 3, 77, 130, 64, "f32", False),
    ("f32_causal_t_lt_s", 1, 1, 1, 50, 120, 64, "f32", True),
    ("f32_gqa_causal_d64", 1, 6, 2, 129, 129, 64, "f32", True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(case):
    name, B, Hq, Hkv, T, S, d, dtype, causal = case
    inp = workloads.make_prefill(B, Hq, Hkv, T, S, d, dtype, causal, seed=seed_of(name), name=name)
    _full_check(inp, name)


# Grids of at least 256 workgroups at 128 query rows take the two-blocks-per-
# wave kernel (the small shapes above take the one-block kernel): non-causal,
# ragged tails, bottom-right causal with T < S, GQA.
MEDIUM = [
    ("medium_noncausal_d128", 2, 8, 8, 2048, 2048, 128, "bf16", False),
    ("medium_ragged_causal_d64", 3, 12, 4, 1000, 1000, 64, "bf16", True),
    ("medium_causal_t_lt_s_gqa", 2, 16, 2, 1000, 1500, 128, "bf16", True),
    ("medium_noncausal_t_gt_s_d64", 1, 32, 8, 1100, 700, 64, "bf16", False),
]


@pytest.mark.parametrize("case", MEDIUM, ids=[c[0] for c in MEDIUM])
def test_medium_shapes(case):
    name, B, Hq, Hkv, T, S, d, dtype, causal = case
    inp = workloads.make_prefill(B, Hq, Hkv, T, S, d, dtype, causal, seed=seed_of(name), name=name)
    assert ((T + 127) // 128) * B * Hq >= 256
    _full_check(inp, name)


def test_prefill_1_fp32_full():
    _full_check(workloads.prefill_1(), "prefill_1")


def test_prefill_2_full():
    _full_check(workloads.prefill_2(), "prefill_2")


def _sampled_check(inp, name, rows_per_head):
    """Every (batch, head) on sampled rows against the oracle, with O and LSE
    allocated NaN-filled so that a row the kernel never wrote cannot pass; on
    every head, causal row 0 (a single visible key) must be v_0 exactly."""
    announce(f"attn_fwd {name} full size, sampled rows of every head")
    q, k, v = inp.q, inp.k, inp.v
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((inp.B, inp.Hq, inp.T), float("nan"), dtype=torch.float32, device="cuda")
    tea.attn_fwd(qd, kd, vd, o, lse, inp.scale, inp.causal)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "unwritten rows"
    rng = np.random.default_rng(seed_of(name))
    T = inp.T
    g = inp.Hq // inp.Hkv
    edge = np.array([0, 1, 2, 127, 128, 129, T // 2, T - 129, T - 128, T - 2, T - 1])
    worst = [0.0, 0.0, 0.0]
    for b in range(inp.B):
        for h in range(inp.Hq):
            rows = np.unique(np.concatenate([edge, rng.integers(0, T, rows_per_head)]))
            qf = q[b, h].double().numpy()
            kf = k[b, h // g].double().numpy()
            vf = v[b, h // g].double().numpy()
            o_ref, lse_ref = oracle.attention_head(qf, kf, vf, inp.scale, inp.causal, rows)
            og = to_np(o[b, h][torch.from_numpy(rows).cuda()])
            lg = to_np(lse[b, h][torch.from_numpy(rows).cuda()])
            mx, mean = check_o(og, o_ref, inp.dtype, f"{name} b={b} h={h}")
            lmx = check_lse(lg, lse_ref, f"{name} b={b} h={h}")
            worst = [max(worst[0], mx), max(worst[1], mean), max(worst[2], lmx)]
            if inp.causal:
                assert torch.equal(o[b, h, 0].cpu(), v[b, h // g, 0]), f"{name} b={b} h={h} row 0"
    print(f"[{name}] worst max|dO| {worst[0]:.3g} mean|dO| {worst[1]:.3g} max|dLSE| {worst[2]:.3g}")


def test_prefill_3_sampled():
    _sampled_check(workloads.prefill_3(), "prefill_3", 40)


def test_prefill_4_sampled():
    _sampled_check(workloads.prefill_4(), "prefill_4", 24)


def test_repeat_runs_are_bitwise_identical():
    inp = workloads.make_prefill(2, 6, 2, 700, 700, 128, "bf16", True, seed=5, name="repeat")
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    announce("attn_fwd repeat x10")
    o0, l0 = tea.fwd(q, k, v, scale=inp.scale, causal=True)
    for _ in range(9):
        o1, l1 = tea.fwd(q, k, v, scale=inp.scale, causal=True)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_lse_optional_and_output_unchanged():
    inp = workloads.make_prefill(1, 2, 2, 130, 130, 64, "bf16", True, seed=6, name="nolse")
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    announce("attn_fwd without lse")
    o_a, _ = tea.fwd(q, k, v, scale=inp.scale, causal=True)
    o_b, none = tea.fwd(q, k, v, scale=inp.scale, causal=True, with_lse=False)
    assert none is None and torch.equal(o_a, o_b)


def test_gpu_rejects_unsupported_without_fallback():
    q = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tea.AttnError) as e:
        tea.fwd(q, q, q, scale=0.1)
    assert e.value.status == tea.ATTN_EUNSUPPORTED
