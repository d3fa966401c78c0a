"""GPU parity of attn_decode_paged_int8 (int8 key/value pages) against the
float64 oracle on the dequantised cache (needs an MI355X).

The codes are widened exactly, so the bounds are those of the bf16 decode.
Covered: the full-size workload (64 sequences, lengths U[512, 8192]) over
every output, junk codes in the unused slots of last pages (must not change a
single bit), edge lengths, head sizes 64 and 128, one to sixteen query heads
per KV head, zero-length sequences, the value scale (a power of two scales
the output exactly) and every one of the 256 codes through the kernel.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, check_lse, check_o, seed_of, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


def _run(inp, k_scale=None, v_scale=None):
    q, kc, vc = inp.q.cuda(), inp.k_codes.cuda(), inp.v_codes.cuda()
    bt, sl = torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.seq_lens).cuda()
    o = torch.full_like(q, float("nan"))
    lse = torch.full((inp.N, inp.Hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = tea.decode_workspace(inp.N, inp.Hq, inp.d, inp.max_blocks, q.device)
    tea.attn_decode_paged_int8(q, kc, vc, inp.k_scale if k_scale is None else k_scale,
                               inp.v_scale if v_scale is None else v_scale, bt, sl, o, lse,
                               inp.scale, ws)
    torch.cuda.synchronize()
    return o, lse


def _oracle(inp, seqs=None):
    return oracle.decode_paged_int8(inp.q.double().numpy(), inp.k_codes.numpy(),
                                    inp.v_codes.numpy(), inp.k_scale, inp.v_scale,
                                    inp.block_table, inp.seq_lens, inp.scale, page=inp.page,
                                    seqs=seqs)


def _check(inp, name):
    announce(f"attn_decode_paged_int8 {name}: N={inp.N} Hq={inp.Hq} Hkv={inp.Hkv} d={inp.d} "
             f"lens {int(inp.seq_lens.min())}..{int(inp.seq_lens.max())}")
    o, lse = _run(inp)
    o_ref, lse_ref = _oracle(inp)
    mx, mean = check_o(to_np(o), o_ref, "bf16", name)
    lmx = check_lse(to_np(lse), lse_ref, name)
    print(f"[{name}] max|dO| {mx:.3g} mean|dO| {mean:.3g} max|dLSE| {lmx:.3g}")
    return o, lse


def test_decode_int8_8_full():
    _check(workloads.decode_int8_8(), "decode_int8_8")


def test_decode_int8_junk_codes_past_the_end_are_ignored():
    clean = workloads.decode_int8_8()
    poisoned = workloads.decode_int8_8(poison_tail=True)
    assert bool((poisoned.k_codes == 0x80).any())
    o_c, l_c = _run(clean)
    o_p, l_p = _run(poisoned)
    assert torch.equal(o_c, o_p) and torch.equal(l_c, l_p)


# name, N, Hq, Hkv, d, lens
EDGE = [
    ("i8_lens_edge", 6, 12, 2, 128, [1, 15, 16, 17, 8192, 513]),
    ("i8_lens_edge_d64", 5, 8, 2, 64, [1, 16, 31, 33, 1000]),
    ("i8_mha", 3, 4, 4, 128, [100, 700, 2049]),
    ("i8_g16", 2, 16, 1, 128, [300, 4000]),
    ("i8_many_short", 200, 12, 2, 64, None),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_decode_int8_edge(case):
    name, N, Hq, Hkv, d, lens = case
    if lens is None:
        inp = workloads.make_decode_int8(N, Hq, Hkv, d, 1, 100, seed=seed_of(name), name=name)
    else:
        inp = workloads.make_decode_int8(N, Hq, Hkv, d, 1, 8192, lens=lens, seed=seed_of(name),
                                         name=name)
    _check(inp, name)


def test_decode_int8_zero_length_sequence():
    inp = workloads.make_decode_int8(4, 12, 2, 128, 1, 500, lens=[300, 1, 40, 200], seed=9,
                                     name="i8_zero")
    inp.seq_lens[2] = 0
    o, lse = _run(inp)
    keep = [0, 1, 3]
    o_ref, lse_ref = _oracle(inp, seqs=keep)
    check_o(to_np(o[keep]), o_ref, "bf16", "i8_zero")
    check_lse(to_np(lse[keep]), lse_ref, "i8_zero")
    assert bool((o[2] == 0).all()) and bool(torch.isinf(lse[2]).all()) and bool((lse[2] < 0).all())


def test_decode_int8_value_scale_is_exact():
    """Doubling v_scale doubles every output bit-exactly (a power of two)."""
    inp = workloads.make_decode_int8(8, 12, 2, 128, 1, 3000, seed=17, name="i8_vscale")
    o1, l1 = _run(inp, v_scale=inp.v_scale)
    o2, l2 = _run(inp, v_scale=2 * inp.v_scale)
    assert torch.equal(o1.float() * 2, o2.float()) and torch.equal(l1, l2)


def test_every_int8_code_decodes_exactly():
    """One cached token: O is that token's V row, so all 256 codes (two KV
    heads x 128 columns) come out through the kernel as exact values."""
    inp = workloads.make_decode_int8(1, 2, 2, 128, 1, 1, lens=[1], seed=3, name="i8_codes")
    inp.v_codes[:] = 0
    page = int(inp.block_table[0, 0])
    inp.v_codes[page, :, 0, :] = torch.arange(256, dtype=torch.uint8).reshape(2, 128)
    announce("attn_decode_paged_int8 all 256 codes")
    o, _ = _run(inp, v_scale=1.0)
    got = to_np(o[0]).reshape(-1)
    ref = oracle.int8_to_float(np.arange(256, dtype=np.uint8))
    np.testing.assert_array_equal(got, ref)
