"""GPU test of attn_decode_paged_noalloc (needs an MI355X).

The entry point runs attn_decode_paged's kernels with their scratch in the
library's device-resident array instead of a caller workspace.  It must give
attn_decode_paged's result bit for bit (same kernels, same work division) and
meet the float64 oracle's bounds, on consecutive calls that reuse the array:
the second call is smaller and has empty sequences, so anything the first
call left behind that the second one read would show.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, check_lse, check_o, seed_of, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


def _case(name, N, Hq, Hkv, d, lens):
    gen = [max(1, int(x)) for x in lens]
    inp = workloads.make_decode(N, Hq, Hkv, d, 1, max(gen), seed=seed_of(name), lens=gen,
                                poison_tail=True, name=name)
    return inp, np.asarray(lens, dtype=np.int32)


def _compare(inp, lens, with_lse=True):
    q, kp, vp = inp.q.cuda(), inp.k_pool.cuda(), inp.v_pool.cuda()
    bt = torch.from_numpy(inp.block_table).cuda()
    sl = torch.from_numpy(lens).cuda()
    announce(f"attn_decode_paged_noalloc {inp.name}: N={inp.N} Hq={inp.Hq} Hkv={inp.Hkv} "
             f"d={inp.d} tokens {int(lens.sum())}")
    o_ws = torch.empty_like(q)
    l_ws = torch.empty((inp.N, inp.Hq), dtype=torch.float32, device="cuda")
    ws = tea.decode_workspace(inp.N, inp.Hq, inp.d, inp.max_blocks, "cuda")
    tea.attn_decode_paged(q, kp, vp, bt, sl, o_ws, l_ws, inp.scale, ws)
    o_na = torch.full_like(q, float("nan"))
    l_na = torch.full((inp.N, inp.Hq), float("nan"), dtype=torch.float32, device="cuda")
    tea.attn_decode_paged_noalloc(q, kp, vp, bt, sl, o_na, l_na if with_lse else None, inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws), f"{inp.name}: O differs from attn_decode_paged"
    if with_lse:
        assert torch.equal(l_na, l_ws), f"{inp.name}: LSE differs from attn_decode_paged"
    else:
        assert torch.isnan(l_na).all()
    live = [n for n in range(inp.N) if lens[n] > 0]
    dead = [n for n in range(inp.N) if lens[n] == 0]
    if dead:
        assert torch.all(o_na[dead] == 0)
        if with_lse:
            assert torch.all(torch.isneginf(l_na[dead]))
    qd, kd, vd = inp.f64()
    o_ref, lse_ref = oracle.decode_paged(qd, kd, vd, inp.block_table, lens, inp.scale,
                                         page=inp.page, seqs=live)
    mx, mean = check_o(to_np(o_na[live]), o_ref, "bf16", inp.name)
    msg = f"[{inp.name}] max|dO| {mx:.3g} mean|dO| {mean:.3g}"
    if with_lse:
        msg += f" max|dLSE| {check_lse(to_np(l_na[live]), lse_ref, inp.name):.3g}"
    print(msg)


def test_noalloc_equals_workspace_entry_on_consecutive_calls():
    rng = np.random.default_rng(41)
    big = rng.integers(1, 6000, 48)
    big[3] = 8192
    small = rng.integers(1, 700, 9)
    small[[1, 5]] = 0
    _compare(*_case("noalloc_first", 48, 12, 2, 128, big.tolist()))
    _compare(*_case("noalloc_second_smaller", 9, 12, 2, 128, small.tolist()))


def test_noalloc_other_shapes_and_no_lse():
    _compare(*_case("noalloc_d64_g3", 5, 6, 2, 64, [47, 0, 4096, 1, 300]), with_lse=False)
    _compare(*_case("noalloc_one_long", 1, 16, 1, 128, [20000]))


def test_noalloc_rejects_more_rows_than_the_scratch_holds():
    inp = workloads.make_decode(2, 12, 2, 128, 10, 40, seed=27, name="noalloc_big")
    q = torch.empty((5462, 12, 128), dtype=torch.bfloat16, device="cuda")   # N*Hq > 65536
    kp, vp = inp.k_pool.cuda(), inp.v_pool.cuda()
    bt = torch.zeros((5462, inp.max_blocks), dtype=torch.int32, device="cuda")
    sl = torch.ones(5462, dtype=torch.int32, device="cuda")
    with pytest.raises(tea.AttnError) as e:
        tea.attn_decode_paged_noalloc(q, kp, vp, bt, sl, torch.empty_like(q), None, inp.scale)
    assert e.value.status == tea.ATTN_EINVAL and "scratch" in str(e.value)
