"""GPU parity of attn_decode_paged against the float64 oracle (needs an MI355X)."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, check_lse, check_o, seed_of, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


def _dev(inp):
    return (inp.q.cuda(), inp.k_pool.cuda(), inp.v_pool.cuda(),
            torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.seq_lens).cuda())


def _run(inp):
    q, kp, vp, bt, sl = _dev(inp)
    o, lse = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale)
    torch.cuda.synchronize()
    return o, lse


def _oracle(inp):
    q, kp, vp = inp.f64()
    return oracle.decode_paged(q, kp, vp, inp.block_table, inp.seq_lens, inp.scale, page=inp.page)


def _check(inp, name):
    announce(f"attn_decode_paged {name}: N={inp.N} Hq={inp.Hq} Hkv={inp.Hkv} d={inp.d} "
             f"lens {int(inp.seq_lens.min())}..{int(inp.seq_lens.max())}")
    o, lse = _run(inp)
    o_ref, lse_ref = _oracle(inp)
    mx, mean = check_o(to_np(o), o_ref, "bf16", name)
    lmx = check_lse(to_np(lse), lse_ref, name)
    print(f"[{name}] max|dO| {mx:.3g} mean|dO| {mean:.3g} max|dLSE| {lmx:.3g}")
    return o, lse


def test_decode_5_full():
    _check(workloads.decode_5(), "decode_5")


def test_decode_5_poisoned_tails_are_ignored():
    clean = workloads.decode_5()
    poisoned = workloads.decode_5(poison_tail=True)
    assert torch.isnan(poisoned.k_pool.float()).any()
    o_c, l_c = _run(clean)
    o_p, l_p = _check(poisoned, "decode_5_poisoned")
    assert torch.equal(o_c, o_p) and torch.equal(l_c, l_p)


# name, N, Hq, Hkv, d, lens
EDGE = [
    ("lens_edge", 6, 12, 2, 128, [1, 15, 16, 17, 8192, 513]),
    ("lens_edge_d64", 5, 8, 2, 64, [1, 16, 31, 33, 1000]),
    ("mha_g1", 3, 4, 4, 128, [100, 700, 2049]),
    ("mqa_g16", 2, 16, 1, 128, [300, 5000]),
    ("gqa_g3_d64", 4, 6, 2, 64, [47, 48, 49, 4096]),
    ("one_page", 2, 12, 2, 128, [16, 7]),
    ("split_boundaries", 4, 12, 2, 128, [511, 512, 513, 1025]),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_decode_edge_lengths(case):
    name, N, Hq, Hkv, d, lens = case
    max_len = max(lens)
    inp = workloads.make_decode(N, Hq, Hkv, d, 1, max_len, seed=seed_of(name), lens=lens,
                                poison_tail=True, name=name)
    _check(inp, name)


def test_paged_equals_contiguous_on_gpu():
    """Same logical cache stored in permuted pages vs in order: identical bits."""
    inp = workloads.make_decode(8, 12, 2, 128, 200, 3000, seed=21, name="perm")
    q, kp, vp, bt, sl = _dev(inp)
    # rebuild the pool with every sequence's pages in logical order
    order = []
    for n in range(inp.N):
        cnt = (int(inp.seq_lens[n]) + 15) // 16
        order.extend(inp.block_table[n, :cnt].tolist())
    order_t = torch.tensor(order, dtype=torch.long, device="cuda")
    kp2, vp2 = kp[order_t].contiguous(), vp[order_t].contiguous()
    bt2 = torch.full_like(bt, -1)
    off = 0
    for n in range(inp.N):
        cnt = (int(inp.seq_lens[n]) + 15) // 16
        bt2[n, :cnt] = torch.arange(off, off + cnt, dtype=torch.int32, device="cuda")
        off += cnt
    announce("attn_decode_paged permuted vs ordered pages")
    o1, l1 = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale)
    o2, l2 = tea.decode_paged(q, kp2, vp2, bt2, sl, scale=inp.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_zero_length_sequence_gives_zero_and_minus_inf():
    inp = workloads.make_decode(3, 12, 2, 128, 1, 500, seed=22, lens=[300, 1, 500], name="zero")
    q, kp, vp, bt, sl = _dev(inp)
    sl[1] = 0
    announce("attn_decode_paged with a zero-length sequence")
    o, lse = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale)
    torch.cuda.synchronize()
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(lse[1]))
    o_ref, lse_ref = _oracle(inp)
    check_o(to_np(o[[0, 2]]), o_ref[[0, 2]], "bf16", "zero-len neighbours")
    check_lse(to_np(lse[[0, 2]]), lse_ref[[0, 2]], "zero-len neighbours")


def test_out_of_range_page_is_skipped_and_neighbours_exact():
    inp = workloads.make_decode(3, 12, 2, 128, 100, 600, seed=23, lens=[600, 400, 200], name="badpage")
    q, kp, vp, bt, sl = _dev(inp)
    bt[1, 3] = -5                       # inside sequence 1: never dereferenced
    bt[1, 7] = inp.num_pages + 9
    announce("attn_decode_paged with out-of-range page ids in one sequence")
    o, lse = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(inp)
    check_o(to_np(o[[0, 2]]), o_ref[[0, 2]], "bf16", "bad-page neighbours")
    check_lse(to_np(lse[[0, 2]]), lse_ref[[0, 2]], "bad-page neighbours")


def test_decode_repeat_runs_are_bitwise_identical():
    inp = workloads.make_decode(16, 12, 2, 128, 512, 8192, seed=24, name="repeat")
    q, kp, vp, bt, sl = _dev(inp)
    ws = tea.decode_workspace(inp.N, inp.Hq, inp.d, inp.max_blocks, "cuda")
    announce("attn_decode_paged repeat x10")
    o0, l0 = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale, workspace=ws)
    for _ in range(9):
        o1, l1 = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale, workspace=ws)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_decode_rejects_small_workspace():
    inp = workloads.make_decode(2, 12, 2, 128, 10, 40, seed=25, name="ws")
    q, kp, vp, bt, sl = _dev(inp)
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(tea.AttnError) as e:
        tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale, workspace=ws)
    assert e.value.status == tea.ATTN_EINVAL


# Work-distribution cases: the page pairs of all sequences are divided evenly
# over up to 768 waves, so these exercise several 64-sequence planning
# chunks (up to 4000 sequences), runs of empty sequences, totals too small
# for every wave (down to a single wave), and one sequence cut into many
# pieces (more than 16, the combine's load batch, and more than 64, its lane
# count).
# name, N, Hq, Hkv, d, lens (0: the sequence is emptied on the device)
def _dist_cases():
    rng = np.random.default_rng(31)
    many = rng.integers(0, 301, 150)
    many[::7] = 0
    mid = rng.integers(1, 4000, 60)
    lots = rng.integers(0, 49, 4000)
    lots[::9] = 0
    return [
        ("many_seqs_chunks", 150, 8, 2, 128, many.tolist()),
        ("tiny_total_one_wave", 3, 12, 2, 128, [1, 0, 2]),
        ("zeros_at_ends", 70, 4, 1, 64, [0] * 5 + mid.tolist() + [0] * 5),
        ("one_long_sequence", 1, 12, 2, 128, [8192]),
        ("one_very_long_sequence", 1, 8, 1, 128, [65536]),
        # every wave plans over 63 chunks of 64 lengths; most sequences are
        # cut between waves or lie inside one, a ninth are empty
        ("four_thousand_short_sequences", 4000, 4, 1, 64, lots.tolist()),
    ]


DIST = _dist_cases()


@pytest.mark.parametrize("case", DIST, ids=[c[0] for c in DIST])
def test_decode_work_distribution(case):
    name, N, Hq, Hkv, d, lens = case
    gen_lens = [max(1, int(x)) for x in lens]
    inp = workloads.make_decode(N, Hq, Hkv, d, 1, max(gen_lens), seed=seed_of(name),
                                lens=gen_lens, poison_tail=True, name=name)
    q, kp, vp, bt, _ = _dev(inp)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    announce(f"attn_decode_paged distribution {name}: N={N} Hq={Hq} Hkv={Hkv} d={d} "
             f"total tokens {int(sum(lens))}")
    o, lse = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale)
    torch.cuda.synchronize()
    live = [n for n in range(N) if lens[n] > 0]
    dead = [n for n in range(N) if lens[n] == 0]
    if dead:
        assert torch.all(o[dead] == 0) and torch.all(torch.isneginf(lse[dead]))
    qd, kd, vd = inp.f64()
    o_ref, lse_ref = oracle.decode_paged(qd, kd, vd, inp.block_table, np.asarray(lens), inp.scale,
                                         page=inp.page, seqs=live)
    mx, mean = check_o(to_np(o[live]), o_ref, "bf16", name)
    lmx = check_lse(to_np(lse[live]), lse_ref, name)
    print(f"[{name}] max|dO| {mx:.3g} mean|dO| {mean:.3g} max|dLSE| {lmx:.3g}")


def test_decode_workspace_contents_are_ignored():
    """A workspace full of all-ones bytes (NaN floats, -1 ints) gives the same bits."""
    inp = workloads.make_decode(16, 12, 2, 128, 512, 8192, seed=26, name="ws_poison")
    q, kp, vp, bt, sl = _dev(inp)
    ws = tea.decode_workspace(inp.N, inp.Hq, inp.d, inp.max_blocks, "cuda")
    announce("attn_decode_paged with a poisoned workspace")
    ws.zero_()
    o0, l0 = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale, workspace=ws)
    ws.fill_(255)
    o1, l1 = tea.decode_paged(q, kp, vp, bt, sl, scale=inp.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
