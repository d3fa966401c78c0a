"""GPU checks of attn_time_next_call (needs an MI355X).

A timed call must compute exactly what an untimed call computes, its events
must bracket its kernels (a positive time, no longer than stream markers
recorded around the same call), and the events must apply to one call only.
"""
import pytest

import workloads
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()                           # torch creates the event on its first record
    torch.cuda.synchronize()
    return evs


def _timed(call):
    """(kernel ms from the call's own events, ms between stream markers)."""
    k0, k1, s0, s1 = _events(4)
    s0.record()
    tea.attn_time_next_call(k0, k1)
    call()
    s1.record()
    torch.cuda.synchronize()
    return k0.elapsed_time(k1), s0.elapsed_time(s1)


def test_timed_prefill_is_bit_identical_and_bracketed():
    inp = workloads.make_prefill(2, 4, 2, 640, 640, 128, causal=True, seed=41)
    announce("attn_fwd timed: B=2 Hq=4 Hkv=2 T=S=640 d=128 causal")
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1 = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    tea.attn_fwd(q, k, v, o1, l1, inp.scale, True)
    kms, sms = _timed(lambda: tea.attn_fwd(q, k, v, o2, l2, inp.scale, True))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    print(f"kernel {kms * 1e3:.1f} us, stream markers {sms * 1e3:.1f} us")
    assert 0.0 < kms <= sms


def test_timed_decode_spans_both_kernels():
    inp = workloads.make_decode(16, 12, 2, 128, 100, 3000, seed=43)
    announce("attn_decode_paged timed: N=16 Hq=12 Hkv=2 d=128")
    q, kp, vp = inp.q.cuda(), inp.k_pool.cuda(), inp.v_pool.cuda()
    bt, sl = torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.seq_lens).cuda()
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1 = torch.empty((inp.N, inp.Hq), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    ws = tea.decode_workspace(inp.N, inp.Hq, inp.d, inp.max_blocks, q.device)
    tea.attn_decode_paged(q, kp, vp, bt, sl, o1, l1, inp.scale, ws)
    kms, sms = _timed(lambda: tea.attn_decode_paged(q, kp, vp, bt, sl, o2, l2, inp.scale, ws))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    print(f"kernels {kms * 1e3:.1f} us, stream markers {sms * 1e3:.1f} us")
    assert 0.0 < kms <= sms


def test_timed_backward_spans_its_three_kernels():
    # one KV head of four query heads at S = 256: the dK/dV pass splits the
    # query heads, so the call runs the dQ, dK/dV and reduction kernels
    inp = workloads.make_prefill(1, 4, 1, 256, 256, 128, causal=True, seed=45)
    announce("attn_bwd timed: B=1 Hq=4 Hkv=1 T=S=256 d=128 causal (three kernels)")
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    o, lse = tea.fwd(q, k, v, scale=inp.scale, causal=True)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(46)).to(q.dtype).cuda()
    ws = torch.empty(tea.attn_bwd_workspace_size(1, 4, 1, 256, 256, 128), dtype=torch.uint8,
                     device="cuda")
    g1 = tea.bwd(q, k, v, o, lse, do, scale=inp.scale, causal=True, workspace=ws)
    torch.cuda.synchronize()
    out = {}
    kms, sms = _timed(lambda: out.update(g=tea.bwd(q, k, v, o, lse, do, scale=inp.scale,
                                                   causal=True, workspace=ws)))
    for a, b in zip(g1, out["g"]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    print(f"kernels {kms * 1e3:.1f} us, stream markers {sms * 1e3:.1f} us")
    assert 0.0 < kms <= sms


def test_events_apply_to_one_call_only():
    inp = workloads.make_prefill(1, 2, 2, 256, 256, 64, causal=False, seed=47)
    announce("attn_fwd events then an untimed call: B=1 H=2 T=S=256 d=64")
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    o = torch.empty_like(q)
    k0, k1 = _events(2)
    tea.attn_time_next_call(k0, k1)
    tea.attn_fwd(q, k, v, o, None, inp.scale, False)
    torch.cuda.synchronize()
    first = k0.elapsed_time(k1)
    # a later untimed call must not move the events
    tea.attn_fwd(q, k, v, o, None, inp.scale, False)
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == first
