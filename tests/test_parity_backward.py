"""GPU parity of attn_bwd against the float64 backward oracle (needs an MI355X).

The HIP path runs attn_fwd and then attn_bwd on the same bf16 inputs, so the
saved log-sum-exp and output it differentiates through are the library's own;
the oracle differentiates its own float64 forward.  Small and ragged shapes
are compared over every element of dQ, dK and dV; the full-size gradient pass
of the GQA causal workload (B=4, Hq=12, Hkv=2, T=S=4096, d=128) is compared on
whole sampled head groups in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, check_grad, seed_of, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


def _run(inp, workspace=None):
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    o, lse = tea.fwd(q, k, v, scale=inp.scale, causal=inp.causal)
    dq, dk, dv = tea.bwd(q, k, v, o, lse, do, scale=inp.scale, causal=inp.causal,
                         workspace=workspace)
    torch.cuda.synchronize()
    return dq, dk, dv


def _describe(inp, name):
    return (f"{name}: B={inp.B} Hq={inp.Hq} Hkv={inp.Hkv} T={inp.T} S={inp.S} d={inp.d} "
            f"causal={inp.causal}")


def _full_check(inp, name):
    announce(f"attn_bwd {_describe(inp, name)}")
    dq, dk, dv = _run(inp)
    q, k, v, do = inp.f64()
    rq, rk, rv = oracle.attention_backward(q, k, v, do, inp.scale, inp.causal)
    worst = {}
    for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        worst[what] = check_grad(to_np(got), ref, f"{name} {what}")
    print(f"[{name}] " + " ".join(f"{w}: max {a:.3g} mean {b:.3g}" for w, (a, b) in worst.items()))


# name, B, Hq, Hkv, T, S, d, causal
SMALL = [
    ("b_t1_s1", 1, 1, 1, 1, 1, 64, False),
    ("b_t1_s1_causal_d128", 1, 2, 1, 1, 1, 128, True),
    ("b_t17_causal", 1, 2, 2, 17, 17, 64, True),
    ("b_t63_causal_d128", 2, 2, 2, 63, 63, 128, True),
    ("b_exact_tiles_d128", 1, 2, 2, 256, 256, 128, True),
    ("b_t130_s200_noncausal_gqa", 2, 4, 2, 130, 200, 128, False),
    ("b_t257_causal", 1, 4, 4, 257, 257, 128, True),
    ("b_t300_s100_noncausal_mqa_d64", 1, 4, 1, 300, 100, 64, False),
    ("b_causal_t_lt_s_bottom_right", 1, 2, 2, 100, 333, 128, True),
    ("b_causal_t1_s333", 1, 2, 2, 1, 333, 128, True),
    ("b_gqa6_causal_d64", 1, 12, 2, 500, 500, 64, True),
    ("b_group_count_multiple_of_8", 4, 4, 2, 200, 200, 64, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(case):
    name, B, Hq, Hkv, T, S, d, causal = case
    inp = workloads.make_backward(B, Hq, Hkv, T, S, d, causal, seed=seed_of(name), name=name)
    _full_check(inp, name)


MEDIUM = [
    ("b_medium_causal_gqa_d128", 2, 16, 4, 1024, 1024, 128, True),
    ("b_medium_noncausal_ragged_d64", 1, 24, 8, 1100, 900, 64, False),
]


@pytest.mark.parametrize("case", MEDIUM, ids=[c[0] for c in MEDIUM])
def test_medium_shapes(case):
    name, B, Hq, Hkv, T, S, d, causal = case
    inp = workloads.make_backward(B, Hq, Hkv, T, S, d, causal, seed=seed_of(name), name=name)
    _full_check(inp, name)


def test_backward_3_sampled_groups():
    """Full size: every gradient of two sampled (batch, KV head) groups."""
    inp = workloads.backward_3()
    announce(f"attn_bwd {_describe(inp, 'backward_3')} sampled groups")
    dq, dk, dv = _run(inp)
    hpg = inp.Hq // inp.Hkv
    for b, hk in ((0, 0), (3, 1)):
        heads = range(hk * hpg, (hk + 1) * hpg)
        kf, vf = inp.k[b, hk].double().numpy(), inp.v[b, hk].double().numpy()
        rk, rv = np.zeros_like(kf), np.zeros_like(vf)
        for h in heads:
            qf, dof = inp.q[b, h].double().numpy(), inp.do[b, h].double().numpy()
            gq, gk, gv, _, _ = oracle.attention_head_backward(qf, kf, vf, dof, inp.scale, True)
            rk += gk
            rv += gv
            a, m = check_grad(to_np(dq[b, h]), gq, f"backward_3 dq b={b} h={h}")
            print(f"[backward_3] dq b={b} h={h}: max {a:.3g} mean {m:.3g}")
        for got, ref, what in ((dk[b, hk], rk, "dk"), (dv[b, hk], rv, "dv")):
            a, m = check_grad(to_np(got), ref, f"backward_3 {what} b={b} hk={hk}")
            print(f"[backward_3] {what} b={b} hk={hk}: max {a:.3g} mean {m:.3g}")
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())


def test_repeat_runs_are_bitwise_identical():
    inp = workloads.make_backward(2, 6, 2, 700, 700, 128, True, seed=5, name="bwd_repeat")
    announce("attn_bwd repeat x5")
    first = _run(inp)
    for _ in range(4):
        again = _run(inp)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_workspace_contents_are_ignored():
    inp = workloads.make_backward(1, 4, 2, 300, 300, 64, True, seed=8, name="bwd_ws")
    announce("attn_bwd workspace zero vs 0xff")
    nbytes = tea.attn_bwd_workspace_size(inp.B, inp.Hq, inp.Hkv, inp.T, inp.S, inp.d)
    ws0 = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ws1 = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")
    for a, b in zip(_run(inp, ws0), _run(inp, ws1)):
        assert torch.equal(a, b)


def test_gpu_rejects_f32_without_fallback():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float32, device="cuda")
    lse = torch.zeros(1, 1, 8, dtype=torch.float32, device="cuda")
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(tea.AttnError) as e:
        tea.attn_bwd(q, q.clone(), q.clone(), q.clone(), lse, q.clone(), torch.empty_like(q),
                     torch.empty_like(q), torch.empty_like(q), 0.125, False, ws)
    assert e.value.status == tea.ATTN_EUNSUPPORTED
