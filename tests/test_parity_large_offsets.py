"""GPU parity where element offsets pass 2^31 (needs an MI355X; up to ~50 GB of HBM).

The kernels address one head (or one page) with 32-bit offsets from a 64-bit
base; these cases make the bases themselves exceed 2^31 elements, so a base
computed in 32 bits would wrap to the wrong head or page.  The inputs are
drawn on the device from a seeded torch generator (host generation of ~7.5e9
values would take minutes); only the checked heads and sequences come back to
the host, where the float64 oracle recomputes them.  Checked: the first head,
heads whose offsets lie past 2^31, and the very last head (prefill and the
backward pass); for decode and chunked prefill, sequences whose pages sit at
the top of a pool of more than 2^31 elements.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import announce, check_lse, check_o, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")

TWO31 = 1 << 31


def _randn(shape, gen):
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("B,Hq,Hkv,T,S,causal", [
    (2048, 32, 32, 300, 300, True),       # q, k, v, o each 2.5e9 elements
    (2048, 32, 8, 300, 1200, False),      # GQA, keys longer than queries: q and k past 2^31
])
def test_prefill_heads_past_2_31_elements(B, Hq, Hkv, T, S, causal):
    d = 128
    assert B * Hq * T * d > TWO31 and B * Hkv * S * d > TWO31
    announce(f"attn_fwd large offsets: B={B} Hq={Hq} Hkv={Hkv} T={T} S={S} d={d} causal={causal}")
    gen = torch.Generator(device="cuda").manual_seed(B + Hq + T + S)
    q = _randn((B, Hq, T, d), gen)
    k = _randn((B, Hkv, S, d), gen)
    v = _randn((B, Hkv, S, d), gen)
    scale = 1.0 / np.sqrt(d)
    o, lse = tea.fwd(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    g = Hq // Hkv
    first_past = TWO31 // (T * d) + 1                    # first (b*Hq + h) whose base is past 2^31
    picks = [0, first_past, (first_past + B * Hq) // 2, B * Hq - 1]
    for bh in picks:
        b, h = divmod(bh, Hq)
        qh = q[b, h].double().cpu().numpy()
        kh = k[b, h // g].double().cpu().numpy()
        vh = v[b, h // g].double().cpu().numpy()
        o_ref, lse_ref = oracle.attention_head(qh, kh, vh, scale, causal)
        name = f"head b={b} h={h} base={(bh * T * d) / TWO31:.2f}*2^31"
        check_o(to_np(o[b, h]), o_ref, "bf16", name)
        check_lse(to_np(lse[b, h]), lse_ref, name)
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def _decode_tables(num_pages, lens, rng, page=16):
    """Block tables whose pages are half from the top 8192 pages of the pool
    (including the last one) and half anywhere, all distinct."""
    nblk = [(int(L) + page - 1) // page for L in lens]
    total = sum(nblk)
    top = np.arange(num_pages - 8192, num_pages)
    low = rng.choice(num_pages - 8192, size=total, replace=False)
    ids = np.concatenate([top[-(total // 2):], low[: total - total // 2]])
    ids = rng.permutation(ids)
    table = -np.ones((len(lens), max(nblk)), dtype=np.int32)
    off = 0
    for n, nb in enumerate(nblk):
        table[n, :nb] = ids[off:off + nb]
        off += nb
    return table


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_pages_past_2_31_elements(fp8):
    N, Hq, Hkv, d, page = 8, 12, 2, 128, 16
    per_page = Hkv * page * d
    num_pages = TWO31 // per_page + 80_000                # pool of ~2.5e9 elements
    assert num_pages * per_page > TWO31
    rng = np.random.default_rng(77 + fp8)
    lens = rng.integers(2000, 8001, N).astype(np.int32)
    table = _decode_tables(num_pages, lens, rng, page)
    assert int(table.max()) * per_page > TWO31
    announce(f"attn_decode_paged{'_fp8' if fp8 else ''} large offsets: {num_pages} pages "
             f"({num_pages * per_page / TWO31:.2f}*2^31 elements per pool), lens {lens.tolist()}")
    gen = torch.Generator(device="cuda").manual_seed(5 + fp8)
    q = _randn((N, Hq, d), gen)
    scale = 1.0 / np.sqrt(d)
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(lens).cuda()
    if fp8:
        # E4M3 codes, NaN codes (0x7f, 0xff) replaced by 0; small scales keep
        # |V| < 1 so the bf16 output's own rounding stays far below the bound
        def codes():
            c = torch.randint(0, 255, (num_pages, Hkv, page, d), generator=gen, device="cuda",
                              dtype=torch.uint8)
            c[c == 0x7F] = 0
            return c
        kp, vp = codes(), codes()
        k_scale, v_scale = 2.0 ** -7, 2.0 ** -9
        o = torch.empty_like(q)
        lse = torch.empty((N, Hq), dtype=torch.float32, device="cuda")
        ws = tea.decode_workspace(N, Hq, d, table.shape[1], q.device)
        tea.attn_decode_paged_fp8(q, kp, vp, k_scale, v_scale, bt, sl, o, lse, scale, ws)
    else:
        kp = _randn((num_pages, Hkv, page, d), gen)
        vp = _randn((num_pages, Hkv, page, d), gen)
        o, lse = tea.decode_paged(q, kp, vp, bt, sl, scale=scale)
    torch.cuda.synchronize()
    qd = q.double().cpu().numpy()
    for n in range(N):
        nb = (int(lens[n]) + page - 1) // page
        pages = torch.from_numpy(table[n, :nb].astype(np.int64)).cuda()
        sub_k = kp.index_select(0, pages).cpu()
        sub_v = vp.index_select(0, pages).cpu()
        local = np.arange(nb, dtype=np.int32)[None, :]
        if fp8:
            o_ref, lse_ref = oracle.decode_paged_fp8(qd[n:n + 1], sub_k.numpy(), sub_v.numpy(),
                                                     k_scale, v_scale, local, lens[n:n + 1],
                                                     scale, page=page)
        else:
            o_ref, lse_ref = oracle.decode_paged(qd[n:n + 1], sub_k.double().numpy(),
                                                 sub_v.double().numpy(), local, lens[n:n + 1],
                                                 scale, page=page)
        name = f"sequence {n} (top page {int(table[n, :nb].max())})"
        check_o(to_np(o[n:n + 1]), o_ref, "bf16", name)
        check_lse(to_np(lse[n:n + 1]), lse_ref, name)
    del q, kp, vp, o, lse
    torch.cuda.empty_cache()


def test_backward_heads_past_2_31_elements():
    """q, k, v, o, dO and the three gradients of 2.5e9 elements each (~50 GB)."""
    from tests.gpu_helpers import check_grad
    B, H, T, d = 2048, 32, 300, 128
    assert B * H * T * d > TWO31
    announce(f"attn_bwd large offsets: B={B} Hq=Hkv={H} T=S={T} d={d} causal")
    gen = torch.Generator(device="cuda").manual_seed(11)
    q, k, v, do = (_randn((B, H, T, d), gen) for _ in range(4))
    scale = 1.0 / np.sqrt(d)
    o, lse = tea.fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = tea.bwd(q, k, v, o, lse, do, scale=scale, causal=True)
    torch.cuda.synchronize()
    first_past = TWO31 // (T * d) + 1
    for bh in (0, first_past, B * H - 1):
        b, h = divmod(bh, H)
        host = [x[b, h].double().cpu().numpy() for x in (q, k, v, do)]
        rq, rk, rv, _, _ = oracle.attention_head_backward(*host, scale, True)
        for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
            check_grad(to_np(got[b, h]), ref, f"head b={b} h={h} {what}")
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_chunked_prefill_pages_past_2_31_elements():
    """Chunks of 4 sequences against a pool of 1.15 * 2^31 elements, half of
    each block table in its top pages."""
    N, Hq, Hkv, d, page, T = 4, 12, 2, 128, 16, 256
    per_page = Hkv * page * d
    num_pages = TWO31 // per_page + 80_000
    rng = np.random.default_rng(91)
    lens = rng.integers(2000, 6001, N).astype(np.int32)
    q_lens = np.array([T, T - 1, 100, 1], dtype=np.int32)
    table = _decode_tables(num_pages, lens, rng, page)
    assert int(table.max()) * per_page > TWO31
    announce(f"attn_prefill_paged large offsets: {num_pages} pages, lens {lens.tolist()}, "
             f"chunks {q_lens.tolist()}")
    gen = torch.Generator(device="cuda").manual_seed(13)
    q = _randn((N, Hq, T, d), gen)
    kp = _randn((num_pages, Hkv, page, d), gen)
    vp = _randn((num_pages, Hkv, page, d), gen)
    o = torch.zeros_like(q)
    lse = torch.zeros((N, Hq, T), dtype=torch.float32, device="cuda")
    scale = 1.0 / np.sqrt(d)
    tea.attn_prefill_paged(q, kp, vp, torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(),
                           torch.from_numpy(q_lens).cuda(), o, lse, scale)
    torch.cuda.synchronize()
    qd = q.double().cpu().numpy()
    for n in range(N):
        nb = (int(lens[n]) + page - 1) // page
        pages = torch.from_numpy(table[n, :nb].astype(np.int64)).cuda()
        sub_k = kp.index_select(0, pages).cpu().double().numpy()
        sub_v = vp.index_select(0, pages).cpu().double().numpy()
        o_ref, lse_ref = oracle.prefill_paged(qd[n:n + 1], sub_k, sub_v,
                                              np.arange(nb, dtype=np.int32)[None, :],
                                              lens[n:n + 1], q_lens[n:n + 1], scale, page=page)
        t = int(q_lens[n])
        name = f"sequence {n} ({t} new of {int(lens[n])}, top page {int(table[n, :nb].max())})"
        check_o(to_np(o[n, :, :t]), o_ref[0, :, :t], "bf16", name)
        check_lse(to_np(lse[n, :, :t]), lse_ref[0, :, :t], name)
    del q, kp, vp, o, lse
    torch.cuda.empty_cache()
