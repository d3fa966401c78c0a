"""The entry points under HIP graph capture (needs an MI355X).

A serving loop captures its per-step launches once and replays them.  The
library allocates nothing and issues no memset or copy, so its calls can be
captured: prefill (causal GQA) and the backward pass through its output,
sliding-window prefill, chunked prefill on a paged cache, and paged decode
over bf16 and fp8 pages are captured together into one graph on a side
stream, then replayed several times.  Between replays the program writes new
inputs into the captured buffers and runs its own eager work; after every
replay each output must equal, bit for bit, an eager call on the same inputs
(the kernels are deterministic).
"""
import pytest

import workloads
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


CHUNK_LENS = [2900, 700, 1500, 2222]
DECODE_LENS = [100, 3000, 17, 1024, 2500, 640, 33, 1999, 2048, 777, 1500, 1, 2900, 260, 1234, 3000]


def _inputs(seed):
    """Same shapes for every seed (fixed lengths); values, page permutations
    and chunk lengths change."""
    p = workloads.make_prefill(2, 12, 2, 700, 700, 128, "bf16", True, seed=seed, name="graph")
    c = workloads.make_prefill_paged(4, 12, 2, 128, 128, 600, 3000, lens=CHUNK_LENS,
                                     seed=seed + 1, name="graph")
    d = workloads.make_decode(16, 12, 2, 128, 1, 3000, lens=DECODE_LENS, seed=seed + 2,
                              name="graph")
    f = workloads.make_decode_fp8(16, 12, 2, 128, 1, 3000, lens=DECODE_LENS, seed=seed + 3,
                                  name="graph")
    g = torch.randn(p.q.shape, generator=torch.Generator().manual_seed(seed + 4)).to(torch.bfloat16)
    return p, c, d, f, g


def test_graph_replays_equal_eager_calls():
    p, c, d, f, g = _inputs(100)
    dev = torch.device("cuda")
    # captured buffers
    q, k, v = (t.to(dev) for t in (p.q, p.k, p.v))
    o, lse = torch.empty_like(q), torch.empty((p.B, p.Hq, p.T), dtype=torch.float32, device=dev)
    ow, lsew = torch.empty_like(q), torch.empty_like(lse)
    cq, ckp, cvp = (t.to(dev) for t in (c.q, c.k_pool, c.v_pool))
    cbt, csl, cql = (torch.from_numpy(a).to(dev) for a in (c.block_table, c.seq_lens, c.q_lens))
    co = torch.zeros_like(cq)
    clse = torch.zeros((c.N, c.Hq, c.T), dtype=torch.float32, device=dev)
    dq, dkp, dvp = (t.to(dev) for t in (d.q, d.k_pool, d.v_pool))
    dbt, dsl = torch.from_numpy(d.block_table).to(dev), torch.from_numpy(d.seq_lens).to(dev)
    do = torch.empty_like(dq)
    dlse = torch.empty((d.N, d.Hq), dtype=torch.float32, device=dev)
    ws = tea.decode_workspace(d.N, d.Hq, d.d, d.max_blocks, dev)
    fq, fkc, fvc = (t.to(dev) for t in (f.q, f.k_codes, f.v_codes))
    fbt, fsl = torch.from_numpy(f.block_table).to(dev), torch.from_numpy(f.seq_lens).to(dev)
    fo = torch.empty_like(fq)
    flse = torch.empty((f.N, f.Hq), dtype=torch.float32, device=dev)
    fws = tea.decode_workspace(f.N, f.Hq, f.d, f.max_blocks, dev)
    gout = g.to(dev)                                # dO of the backward pass
    bws = torch.empty(tea.attn_bwd_workspace_size(p.B, p.Hq, p.Hkv, p.T, p.S, p.d),
                      dtype=torch.uint8, device=dev)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step(outs):
        o_, lse_, ow_, lsew_, co_, clse_, do_, dlse_, fo_, flse_, gq_, gk_, gv_ = outs
        tea.attn_fwd(q, k, v, o_, lse_, p.scale, True)
        tea.attn_bwd(q, k, v, o_, lse_, gout, gq_, gk_, gv_, p.scale, True, bws)
        tea.attn_fwd_window(q, k, v, ow_, lsew_, p.scale, 256)
        tea.attn_prefill_paged(cq, ckp, cvp, cbt, csl, cql, co_, clse_, c.scale)
        tea.attn_decode_paged(dq, dkp, dvp, dbt, dsl, do_, dlse_, d.scale, ws)
        tea.attn_decode_paged_fp8(fq, fkc, fvc, f.k_scale, f.v_scale, fbt, fsl, fo_, flse_,
                                  f.scale, fws)

    captured = (o, lse, ow, lsew, co, clse, do, dlse, fo, flse, gq, gk, gv)
    eager = tuple(torch.zeros_like(t) for t in captured)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        step(captured)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    announce("graph capture: attn_fwd + attn_bwd + attn_fwd_window + attn_prefill_paged + "
             "attn_decode_paged + attn_decode_paged_fp8")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(captured)
    torch.cuda.synchronize()

    for rep in range(4):
        # new inputs into the captured buffers, and some eager work of the program's own
        p2, c2, d2, f2, g2 = _inputs(200 + rep)
        q.copy_(p2.q); k.copy_(p2.k); v.copy_(p2.v)
        cq.copy_(c2.q); ckp.copy_(c2.k_pool); cvp.copy_(c2.v_pool)
        cbt.copy_(torch.from_numpy(c2.block_table)); csl.copy_(torch.from_numpy(c2.seq_lens))
        cql.copy_(torch.from_numpy(c2.q_lens))
        dq.copy_(d2.q); dkp.copy_(d2.k_pool); dvp.copy_(d2.v_pool)
        dbt.copy_(torch.from_numpy(d2.block_table)); dsl.copy_(torch.from_numpy(d2.seq_lens))
        fq.copy_(f2.q); fkc.copy_(f2.k_codes); fvc.copy_(f2.v_codes)
        fbt.copy_(torch.from_numpy(f2.block_table)); fsl.copy_(torch.from_numpy(f2.seq_lens))
        gout.copy_(g2)
        scratch = (q.float() * 2).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(eager)
        torch.cuda.synchronize()
        names = ("o", "lse", "o_window", "lse_window", "o_chunked", "lse_chunked", "o_decode",
                 "lse_decode", "o_decode_fp8", "lse_decode_fp8", "dq", "dk", "dv")
        for got, ref, what in zip(captured, eager, names):
            if what.endswith("chunked"):
                # rows past each sequence's chunk are not part of the result
                for n, t in enumerate(c2.q_lens.tolist()):
                    assert torch.equal(got[n, :, :t], ref[n, :, :t]), f"replay {rep}: {what} seq {n}"
            else:
                assert torch.equal(got, ref), f"replay {rep}: {what} differs from the eager call"
        scratch.item()
        print(f"replay {rep}: all outputs bit-identical to eager calls")
