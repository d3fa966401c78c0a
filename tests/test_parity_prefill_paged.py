"""GPU parity of attn_prefill_paged (chunked prefill on a paged cache) against
the float64 oracle (needs an MI355X).

Small cases cover ragged chunk and context lengths, chunks that fill the
whole context, one-token chunks, the sliding window, poisoned (NaN) slots
past each sequence's end, GQA ratios and both head sizes; a chunk equal to
the whole sequence must reproduce attn_fwd on the contiguous keys bit for
bit.  Sequences are dispatched longest first by a selection the kernel makes
from the lengths (ties by index): equal lengths and many sequences must
still give every sequence its own workgroups.  The full-size chunked workload (16 sequences,
512-token chunks, up to 8192 cached tokens) is compared on sampled rows in
the configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, check_lse, check_o, seed_of, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


def _run(inp, fill=7.0):
    dev = "cuda"
    q, kp, vp = (t.to(dev) for t in (inp.q, inp.k_pool, inp.v_pool))
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    ql = torch.from_numpy(inp.q_lens).to(dev)
    o = torch.full_like(q, fill)                    # rows past q_lens must keep the fill
    lse = torch.full((inp.N, inp.Hq, inp.T), fill, dtype=torch.float32, device=dev)
    tea.attn_prefill_paged(q, kp, vp, bt, sl, ql, o, lse, inp.scale, window=inp.window)
    torch.cuda.synchronize()
    return o, lse


def _check(inp, name, o, lse, seqs=None, rows_of=None):
    """Every computed row against the oracle: the maximum errors element by
    element, the mean error of O over all the rows checked (the bf16 bound is
    a mean over the output, which a single short row, its values rounded once
    to bf16, can exceed on its own)."""
    q, kp, vp = inp.f64()
    seqs = range(inp.N) if seqs is None else seqs
    got_o, ref_o = [], []
    for n in seqs:
        L, Tn = int(inp.seq_lens[n]), int(inp.q_lens[n])
        rows = np.arange(Tn) if rows_of is None else rows_of(n, Tn)
        for hk in range(inp.Hkv):
            kn = oracle.gather_pages(kp, inp.block_table[n], L, hk, inp.page)
            vn = oracle.gather_pages(vp, inp.block_table[n], L, hk, inp.page)
            for h in range(hk * (inp.Hq // inp.Hkv), (hk + 1) * (inp.Hq // inp.Hkv)):
                o_ref, l_ref = oracle.attention_head(q[n, h, :Tn], kn, vn, inp.scale, True, rows,
                                                     window=inp.window)
                got_o.append(to_np(o[n, h, rows]).reshape(-1))
                ref_o.append(np.asarray(o_ref).reshape(-1))
                check_lse(to_np(lse[n, h, rows]), l_ref, f"{name} n={n} h={h}")
        if rows_of is None:
            assert bool((o[n, :, Tn:] == 7.0).all()) and bool((lse[n, :, Tn:] == 7.0).all())
    check_o(np.concatenate(got_o), np.concatenate(ref_o), "bf16", name)


# name, N, Hq, Hkv, T, d, min_len, max_len, q_lens, window, poison
CASES = [
    ("pp_tiny", 2, 2, 1, 8, 64, 1, 20, None, 0, False),
    ("pp_ragged_d128", 4, 4, 2, 100, 128, 40, 400, None, 0, True),
    ("pp_ragged_d64_mqa", 3, 6, 1, 130, 64, 130, 700, None, 0, True),
    ("pp_one_token_chunks", 5, 12, 2, 16, 128, 1, 300, 1, 0, True),
    ("pp_full_context", 3, 4, 4, 257, 128, 100, 257, "full", 0, False),
    ("pp_window", 4, 8, 2, 200, 128, 200, 900, None, 77, True),
    ("pp_window_d64", 3, 4, 2, 300, 64, 300, 600, 300, 128, False),
    ("pp_medium_gqa", 8, 12, 2, 512, 128, 512, 3000, 512, 0, True),
    # 256 workgroups: the two-row-block kernel (64-key tiles at d = 64)
    ("pp_d64_full_grid", 8, 16, 2, 256, 64, 256, 700, None, 0, True),
    ("pp_d64_full_grid_window", 8, 16, 2, 256, 64, 256, 700, 256, 90, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_paged_shapes(case):
    name, N, Hq, Hkv, T, d, lo, hi, qlens, window, poison = case
    seed = seed_of(name)
    if qlens == "full":
        lens = np.random.default_rng(seed).integers(lo, hi + 1, N)
        inp = workloads.make_prefill_paged(N, Hq, Hkv, T, d, lo, hi, q_lens=list(lens), lens=lens,
                                           window=window, seed=seed, poison_tail=poison,
                                           extra_pages=3, name=name)
    else:
        inp = workloads.make_prefill_paged(N, Hq, Hkv, T, d, lo, hi, q_lens=qlens, window=window,
                                           seed=seed, poison_tail=poison, extra_pages=3, name=name)
    announce(f"attn_prefill_paged {name}: N={N} Hq={Hq} Hkv={Hkv} T={T} d={d} window={window} "
             f"seq_lens={inp.seq_lens.tolist()} q_lens={inp.q_lens.tolist()}")
    o, lse = _run(inp)
    _check(inp, name, o, lse)


@pytest.mark.parametrize("d", [64, 128])
def test_whole_sequence_chunk_is_bitwise_attn_fwd(d):
    """q_len = seq_len = T on every sequence: the dense causal kernel on the
    gathered keys must give the very same bits."""
    T = 300
    inp = workloads.make_prefill_paged(3, 4, 2, T, d, T, T, q_lens=T, seed=41 + d,
                                       name="pp_vs_fwd")
    announce(f"attn_prefill_paged vs attn_fwd, d={d}")
    o, lse = _run(inp)
    k = torch.stack([torch.stack([inp.k_pool[torch.from_numpy(inp.block_table[n]).long(), hk]
                                  .reshape(-1, d)[:T] for hk in range(inp.Hkv)])
                     for n in range(inp.N)]).cuda().contiguous()
    v = torch.stack([torch.stack([inp.v_pool[torch.from_numpy(inp.block_table[n]).long(), hk]
                                  .reshape(-1, d)[:T] for hk in range(inp.Hkv)])
                     for n in range(inp.N)]).cuda().contiguous()
    o_f, l_f = tea.fwd(inp.q.cuda(), k, v, scale=inp.scale, causal=True)
    assert torch.equal(o, o_f) and torch.equal(lse, l_f)


def test_equal_lengths_each_sequence_computed_once():
    name = "pp_ties"
    lens = [300, 300, 120, 300, 120, 57, 300]
    qls = [40, 40, 40, 1, 120, 57, 33]
    inp = workloads.make_prefill_paged(7, 4, 2, 120, 128, 0, 0, q_lens=qls, lens=lens,
                                       seed=seed_of(name), poison_tail=True, extra_pages=2,
                                       name=name)
    announce(f"attn_prefill_paged {name}: seq_lens={lens} q_lens={qls}")
    o, lse = _run(inp)
    _check(inp, name, o, lse)


@pytest.mark.parametrize("N", [256, 300, 1000, 1100])
def test_many_sequences_each_get_their_workgroups(N):
    """The longest-first dispatch selects every sequence exactly once at any N
    (the selection reads the lengths in passes over all N)."""
    name = f"pp_many_{N}"
    inp = workloads.make_prefill_paged(N, 2, 1, 8, 64, 1, 64, seed=seed_of(name),
                                       poison_tail=True, extra_pages=3, name=name)
    announce(f"attn_prefill_paged {name}: N={N} Hq=2 Hkv=1 T=8 d=64")
    o, lse = _run(inp)
    _check(inp, name, o, lse)


def test_chunked_prefill_6_sampled():
    """Sampled rows of every sequence and head, outputs NaN-filled: a row the
    kernel never wrote cannot pass (every row is below q_lens here)."""
    inp = workloads.chunked_prefill_6()
    assert (inp.q_lens == inp.T).all()
    announce("attn_prefill_paged chunked_prefill_6 full size, sampled rows of every sequence")
    o, lse = _run(inp, fill=float("nan"))
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "unwritten rows"
    rng = np.random.default_rng(seed_of("cp6"))

    def rows_of(n, Tn):
        return np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, Tn - 2, Tn - 1],
                                         rng.integers(0, Tn, 16)]))
    _check(inp, "chunked_prefill_6", o, lse, seqs=range(inp.N), rows_of=rows_of)
