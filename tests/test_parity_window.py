"""GPU parity of attn_fwd_window (causal sliding window) against the float64
oracle (needs an MI355X).

Whole outputs are compared for small, ragged and medium shapes in both
dtypes; a window at least as long as the keys must reproduce attn_fwd's
causal result bit for bit (same kernel path, nothing extra masked); the
full-size GQA shape (B=4, Hq=12, Hkv=2, T=S=4096, d=128, window 1024) is
compared on sampled rows in the configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, check_lse, check_o, seed_of, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


def _run(inp, window):
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    o, lse = tea.fwd(q, k, v, scale=inp.scale, window=window)
    torch.cuda.synchronize()
    return o, lse


# name, B, Hq, Hkv, T, S, d, dtype, window
CASES = [
    ("w_t1", 1, 2, 1, 1, 1, 64, "bf16", 1),
    ("w_one_key", 1, 2, 2, 130, 130, 64, "bf16", 1),
    ("w37_ragged", 1, 2, 1, 300, 300, 64, "bf16", 37),
    ("w64_t_lt_s_gqa", 1, 4, 2, 100, 333, 128, "bf16", 64),
    ("w128_exact_tiles", 1, 2, 2, 512, 512, 128, "bf16", 128),
    ("w129_d64", 2, 3, 3, 700, 700, 64, "bf16", 129),
    ("w_longer_than_rows", 1, 2, 2, 200, 450, 128, "bf16", 300),
    ("w512_medium_gqa", 2, 16, 2, 2048, 2048, 128, "bf16", 512),
    ("w200_medium_d64", 3, 12, 4, 1000, 1000, 64, "bf16", 200),
    ("w50_f32", 1, 2, 1, 200, 200, 64, "f32", 50),
    ("w33_f32_t_lt_s", 1, 1, 1, 77, 130, 128, "f32", 33),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_shapes(case):
    name, B, Hq, Hkv, T, S, d, dtype, W = case
    inp = workloads.make_prefill(B, Hq, Hkv, T, S, d, dtype, True, seed=seed_of(name), name=name)
    announce(f"attn_fwd_window {name}: B={B} Hq={Hq} Hkv={Hkv} T={T} S={S} d={d} {dtype} W={W}")
    o, lse = _run(inp, W)
    q, k, v = inp.f64()
    o_ref, lse_ref = oracle.attention(q, k, v, inp.scale, True, window=W)
    check_o(to_np(o), o_ref, dtype, name)
    check_lse(to_np(lse), lse_ref, name)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_window_covering_every_key_is_bitwise_causal(dtype, d):
    inp = workloads.make_prefill(2, 4, 2, 333, 333, d, dtype, True, seed=31, name="wall")
    announce(f"attn_fwd_window window >= S vs attn_fwd causal, {dtype} d={d}")
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    o_w, l_w = tea.fwd(q, k, v, scale=inp.scale, window=333)
    o_c, l_c = tea.fwd(q, k, v, scale=inp.scale, causal=True)
    assert torch.equal(o_w, o_c) and torch.equal(l_w, l_c)


def test_window_full_size_sampled():
    inp = workloads.prefill_3()
    W = 1024
    announce(f"attn_fwd_window prefill_3 full size W={W}, sampled rows")
    o, lse = _run(inp, W)
    rng = np.random.default_rng(seed_of("window_full"))
    T = inp.T
    edge = np.array([0, 1, W - 2, W - 1, W, W + 1, 2047, 2048, T - 2, T - 1])
    for (b, h) in [(0, 0), (1, 7), (3, 11)]:
        rows = np.unique(np.concatenate([edge, rng.integers(0, T, 64)]))
        hk = h // (inp.Hq // inp.Hkv)
        o_ref, lse_ref = oracle.attention_head(inp.q[b, h].double().numpy(),
                                               inp.k[b, hk].double().numpy(),
                                               inp.v[b, hk].double().numpy(), inp.scale, True,
                                               rows, window=W)
        idx = torch.from_numpy(rows).cuda()
        check_o(to_np(o[b, h][idx]), o_ref, "bf16", f"window b={b} h={h}")
        check_lse(to_np(lse[b, h][idx]), lse_ref, f"window b={b} h={h}")
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
