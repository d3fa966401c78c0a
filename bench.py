#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path on resident synthetic inputs, each
launch preceded by a 512 MiB read that evicts L2 and the Infinity Cache:
  1. causal prefill attn_fwd on the three prefill workloads:
     prefill_2 (GPT-2-small-shaped: B=8, H=12, T=S=1024, d=64, bf16),
     prefill_3 (GQA: B=4, Hq=12, Hkv=2, T=S=4096, d=128, bf16),
     prefill_4 (long: B=1, H=32, T=S=16384, d=128, bf16, inputs x0.5);
  2. paged decode attn_decode_paged on decode_5: 64 sequences, 12 query / 2 KV
     heads, d=128, 16-token pages, lengths U[512, 8192] (stream kernel +
     combine).
`--only <workload>` makes the step that one launch (profiling runs).

Reported (one JSON line on stdout):
  value               prefill_2 TFLOP/s = algorithmic FLOPs / mean kernel time,
                      FLOPs = 4*d per visible (query, key) pair; kernel time
                      is taken by HIP events that the call's kernels record
                      themselves as they begin and end (attn_time_next_call),
                      the interval a kernel trace reports; `ms_stream` beside
                      each `ms` is the time between events recorded on the
                      launch stream around the call, which adds the stream's
                      launch gaps;
  roofline_per_kernel every workload of the step against its published peak
                      (bf16 dense MFMA 2516.6 TFLOP/s; HBM 8 TB/s for decode,
                      bytes = K+V of every cached token once plus q, o, lse,
                      seq_lens and the used block-table entries), with its
                      measured HBM traffic per launch (`traffic`, from
                      profiles/counters.json while the kernel sources still
                      match the recorded hash, else null) and the float64
                      oracle timed on a bounded sample of the same workload on
                      the host cores (`cpu_baseline`);
  roofline            the entry of the workload that takes the most time;
  hbm_probe           a read-only kernel (libattn_probe.so) on the decode
                      workload's key/value chunks in the decode's order, split
                      like the decode's grid (768 waves, and 1024: the faster
                      kept), and on as many bytes in sequence: the read rate
                      the chip reaches on those bytes with no compute;
  window              attn_fwd_window on prefill_3's inputs with a 1024-key
                      sliding window (FLOPs over the visible pairs only);
  chunked             attn_prefill_paged on 16 sequences of 1024..8192 cached
                      tokens whose last 512 are the new chunk, Hq=12, Hkv=2,
                      d=128, keys through the block table;
  decode_fp8          attn_decode_paged_fp8 on decode_5's shape with E4M3 pages
                      (decode_fp8_7): GB/s over the bytes it must read;
  decode_int8         attn_decode_paged_int8 on the same shape with int8 pages
                      (decode_int8_8), likewise;
  backward            the gradient pass attn_bwd on prefill_3's shape,
                      TFLOP/s with FLOPs = 10*d per visible (query, key) pair
                      (recomputed scores, dP, dV, dQ, dK);
  (window, chunked, decode_fp8, decode_int8 and backward each carry their own
  cpu_baseline)
  cpu_baseline        the oracle's figure for the headline workload.
The flush reads sit outside both kinds of events but inside ms_per_step.

Measurement helpers (each runs and exits):
  --copy-probe        a 256 MiB device copy, to calibrate the HBM counters;
  --hbm-probe         the read-only probe alone;
  --write-counters D  profiles/counters.json from rocprofv3 FETCH_SIZE /
                      WRITE_SIZE collections under D (D/copy_{fetch,write}
                      from --copy-probe runs, D/<workload>_{fetch,write} from
                      --only <workload> runs): HBM bytes per launch, each
                      counter scaled by what it reads for a copy of known size;
  --summarize D       a markdown table of a rocprofv3 kernel trace or counter
                      collection under D, per kernel and grid size.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 FLOP/clk x 2.4 GHz (dense)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = {
    "prefill": ["tiled_exact_attention_flashattention_amd/csrc/prefill_bf16.hip",
                "tiled_exact_attention_flashattention_amd/csrc/cdna4.hpp",
                "tiled_exact_attention_flashattention_amd/csrc/lds_stage.hpp",
                "tiled_exact_attention_flashattention_amd/csrc/kernels.hpp"],
    "decode": ["tiled_exact_attention_flashattention_amd/csrc/decode_paged.hip",
               "tiled_exact_attention_flashattention_amd/csrc/cdna4.hpp",
               "tiled_exact_attention_flashattention_amd/csrc/kernels.hpp"],
}


def sources_sha(kind):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_work(B, Hq, Hkv, T, S, d, causal, elem, window=0):
    if causal:
        pairs = sum(min(S, i + (S - T) + 1, window if window else S) for i in range(T))
    else:
        pairs = T * S
    flops = 4 * d * pairs * B * Hq
    nbytes = (2 * B * Hq * T * d + 2 * B * Hkv * S * d) * elem + B * Hq * T * 4
    return flops, nbytes


def chunked_pairs(seq_lens, q_lens):
    """Visible (query, key) pairs of a chunked prefill: the chunk's row i of a
    sequence with L cached tokens (its T new ones last) sees L - T + i + 1 keys."""
    return sum(int(L) * int(T) - int(T) * (int(T) - 1) // 2 for L, T in zip(seq_lens, q_lens))


def decode_work(inp):
    tokens = int(inp.seq_lens.astype("int64").sum())
    pages = int(((inp.seq_lens.astype("int64") + inp.page - 1) // inp.page).sum())
    kv = tokens * inp.Hkv * inp.d * 2 * 2
    qo = 2 * inp.N * inp.Hq * inp.d * 2
    nbytes = kv + qo + inp.N * inp.Hq * 4 + inp.N * 4 + pages * 4
    flops = 4 * inp.d * tokens * inp.Hq
    return flops, nbytes, tokens


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def oracle_sample(budget_s, units, run_unit, work_of):
    """Run the oracle on units[0], units[1], ... (cycling) until budget_s seconds
    are spent; returns (units done, algorithmic work done, seconds)."""
    done, work, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        u = units[done % len(units)]
        run_unit(u)
        work += work_of(u)
        done += 1
    return done, work, time.perf_counter() - t0


def kernel_events(n):
    """n pairs of timing events, each recorded once (torch creates an event on
    its first record), for attn_time_next_call."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b_ in evs:
        a.record()
        b_.record()
    torch.cuda.synchronize()
    return evs


def timed_launches(stream, flush, launch, n=7, skip=2):
    """Cold launches of launch(events) (the first `skip` untimed): the mean time
    from the start of the call's first kernel to the end of its last (events the
    call's kernels record, passed to launch), and the mean time between stream
    markers recorded around the call (which adds the stream's launch gaps).
    Returns (kernel ms, stream ms, launches timed)."""
    import torch
    kev = kernel_events(n)
    times = []
    for i in range(n):
        if flush is not None:
            flush.sum()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch(kev[i])
        b_.record(stream)
        if i >= skip:
            times.append((kev[i], (a, b_)))
    torch.cuda.synchronize()
    km = sum(k0.elapsed_time(k1) for (k0, k1), _ in times) / len(times)
    sm = sum(a.elapsed_time(b_) for _, (a, b_) in times) / len(times)
    return km, sm, len(times)


def bench_window(tea, workloads, dev, stream, flush, cpu_budget_s=None, window=1024):
    """attn_fwd_window on the GQA causal workload (and the oracle on sampled heads)."""
    import torch
    x = workloads.prefill_3()
    xq, xk, xv = (t.to(dev) for t in (x.q, x.k, x.v))
    xo = torch.empty_like(xq)
    xl = torch.empty((x.B, x.Hq, x.T), dtype=torch.float32, device=dev)
    ms, ms_stream, n = timed_launches(stream, flush, lambda ev: (
        tea.attn_time_next_call(*ev),
        tea.attn_fwd_window(xq, xk, xv, xo, xl, x.scale, window, stream=stream)))
    fl, _ = prefill_work(x.B, x.Hq, x.Hkv, x.T, x.S, x.d, True, 2, window=window)
    tf = fl / (ms * 1e-3) / 1e12
    rec = {"config": f"B={x.B}, Hq={x.Hq}, Hkv={x.Hkv}, T=S={x.T}, d={x.d}, bf16, causal, "
                     f"window {window}", "kernel": "prefill_bf16_kernel", "ms": ms,
           "ms_stream": ms_stream, "value": tf,
           "unit": "TFLOP/s", "algorithmic_flops": fl, "bound": "mfma",
           "peak": PEAK_BF16_TFLOPS, "frac_of_mfma_peak": tf / PEAK_BF16_TFLOPS, "launches": n,
           "cpu_baseline": None}
    del xq, xk, xv, xo, xl
    if cpu_budget_s:
        import oracle
        g = x.Hq // x.Hkv
        heads = [(b, h) for b in range(x.B) for h in range(x.Hq)]
        done, work, tc = oracle_sample(
            cpu_budget_s, heads,
            lambda bh: oracle.attention_head(x.q[bh[0], bh[1]].double().numpy(),
                                             x.k[bh[0], bh[1] // g].double().numpy(),
                                             x.v[bh[0], bh[1] // g].double().numpy(),
                                             x.scale, True, window=window),
            lambda bh: fl // len(heads))
        rec["cpu_baseline"] = {"value": work / tc / 1e12, "unit": "TFLOP/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{done} (batch, head) windowed attention problems of "
                                         f"this workload ({tc:.1f} s)"}
    return rec


def bench_chunked(tea, workloads, dev, stream, flush, cpu_budget_s=None):
    """attn_prefill_paged on chunked_prefill_6 (and the oracle on sampled sequences)."""
    import torch
    x = workloads.chunked_prefill_6()
    xq, kp, vp = (t.to(dev) for t in (x.q, x.k_pool, x.v_pool))
    bt, sl, ql = (torch.from_numpy(a).to(dev) for a in (x.block_table, x.seq_lens, x.q_lens))
    xo = torch.empty_like(xq)
    xl = torch.empty((x.N, x.Hq, x.T), dtype=torch.float32, device=dev)
    ms, ms_stream, n = timed_launches(stream, flush, lambda ev: (
        tea.attn_time_next_call(*ev),
        tea.attn_prefill_paged(xq, kp, vp, bt, sl, ql, xo, xl, x.scale, stream=stream)))
    fl = 4 * x.d * x.Hq * chunked_pairs(x.seq_lens, x.q_lens)
    tf = fl / (ms * 1e-3) / 1e12
    rec = {"config": f"N={x.N}, Hq={x.Hq}, Hkv={x.Hkv}, chunk {x.T}, cached "
                     f"{int(x.seq_lens.min())}..{int(x.seq_lens.max())} tokens, d={x.d}, bf16, "
                     f"16-token pages", "kernel": "prefill_bf16_kernel (paged)", "ms": ms,
           "ms_stream": ms_stream,
           "value": tf, "unit": "TFLOP/s", "algorithmic_flops": fl, "bound": "mfma",
           "peak": PEAK_BF16_TFLOPS, "frac_of_mfma_peak": tf / PEAK_BF16_TFLOPS, "launches": n,
           "cpu_baseline": None}
    del xq, kp, vp, bt, sl, ql, xo, xl
    if cpu_budget_s:
        import oracle
        qd, kd, vd = x.f64()
        done, work, tc = oracle_sample(
            cpu_budget_s, list(range(x.N)),
            lambda n: oracle.prefill_paged(qd[n:n + 1], kd, vd, x.block_table[n:n + 1],
                                           x.seq_lens[n:n + 1], x.q_lens[n:n + 1], x.scale),
            lambda n: 4 * x.d * x.Hq * (int(x.seq_lens[n]) * int(x.q_lens[n])
                                        - int(x.q_lens[n]) * (int(x.q_lens[n]) - 1) // 2))
        rec["cpu_baseline"] = {"value": work / tc / 1e12, "unit": "TFLOP/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{done} sequences of this workload, one oracle call "
                                         f"each ({tc:.1f} s)"}
    return rec


def bench_decode_q8(tea, workloads, dev, stream, flush, cpu_budget_s=None, fmt="fp8"):
    """attn_decode_paged_fp8 on decode_fp8_7 (E4M3 pages) or attn_decode_paged_int8 on
    decode_int8_8 (int8 pages): stream + combine kernels, and the oracle on
    sampled sequences."""
    import torch
    x = workloads.decode_fp8_7() if fmt == "fp8" else workloads.decode_int8_8()
    entry = tea.attn_decode_paged_fp8 if fmt == "fp8" else tea.attn_decode_paged_int8
    xq, kc, vc = x.q.to(dev), x.k_codes.to(dev), x.v_codes.to(dev)
    bt, sl = torch.from_numpy(x.block_table).to(dev), torch.from_numpy(x.seq_lens).to(dev)
    xo = torch.empty_like(xq)
    xl = torch.empty((x.N, x.Hq), dtype=torch.float32, device=dev)
    ws = tea.decode_workspace(x.N, x.Hq, x.d, x.max_blocks, dev)
    ms, ms_stream, n = timed_launches(stream, flush, lambda ev: (
        tea.attn_time_next_call(*ev),
        entry(xq, kc, vc, x.k_scale, x.v_scale, bt, sl, xo, xl, x.scale, ws, stream=stream)), n=12)
    tokens = int(x.seq_lens.astype("int64").sum())
    pages = int(((x.seq_lens.astype("int64") + x.page - 1) // x.page).sum())
    nbytes = tokens * x.Hkv * x.d * 2 + 2 * x.N * x.Hq * x.d * 2 + x.N * x.Hq * 4 + x.N * 4 + pages * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    rec = {"config": f"N={x.N}, Hq={x.Hq}, Hkv={x.Hkv}, d={x.d}, "
                     f"{'E4M3' if fmt == 'fp8' else 'int8'} K/V pages, lengths "
                     f"U[512,8192] (sum {tokens})",
           "kernel": f"decode_stream_kernel<{fmt}>+decode_combine_kernel",
           "ms": ms, "ms_stream": ms_stream, "value": gbs,
           "unit": "GB/s",
           "algorithmic_bytes": nbytes, "bound": "hbm", "peak": PEAK_HBM_GBS,
           "frac_of_hbm_peak": gbs / PEAK_HBM_GBS, "launches": n,
           "tokens_per_s": tokens / (ms * 1e-3), "cpu_baseline": None}
    del xq, kc, vc, bt, sl, xo, xl, ws
    if cpu_budget_s:
        import numpy as np

        import oracle
        qd = x.q.double().numpy()
        kcodes, vcodes = x.k_codes.numpy(), x.v_codes.numpy()
        ref = oracle.decode_paged_fp8 if fmt == "fp8" else oracle.decode_paged_int8

        def one_sequence(n):
            # the pages sequence n uses, as a pool of their own with the table renumbered
            nb = (int(x.seq_lens[n]) + x.page - 1) // x.page
            pages = x.block_table[n, :nb]
            ref(qd[n:n + 1], kcodes[pages], vcodes[pages], x.k_scale, x.v_scale,
                np.arange(nb, dtype=np.int32)[None, :], x.seq_lens[n:n + 1], x.scale, page=x.page)

        done, work, tc = oracle_sample(
            cpu_budget_s, list(range(x.N)), one_sequence,
            lambda n: int(x.seq_lens[n]) * x.Hkv * x.d * 2 + 2 * x.Hq * x.d * 2)
        rec["cpu_baseline"] = {"value": work / tc / 1e9, "unit": "GB/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": f"{done} sequences of this workload, one oracle call "
                                         f"each on the {fmt} pages it uses ({tc:.1f} s)"}
    return rec


def bench_backward(tea, workloads, dev, stream, flush, cpu_budget_s):
    """Time attn_bwd on backward_3 (7 cold launches, the first 2 untimed)."""
    import torch
    x = workloads.backward_3()
    xq, xk, xv, xdo = (t.to(dev) for t in (x.q, x.k, x.v, x.do))
    xo, xl = tea.fwd(xq, xk, xv, scale=x.scale, causal=x.causal)
    gq, gk, gv = torch.empty_like(xq), torch.empty_like(xk), torch.empty_like(xv)
    ws = torch.empty(tea.attn_bwd_workspace_size(x.B, x.Hq, x.Hkv, x.T, x.S, x.d), dtype=torch.uint8,
                     device=dev)
    ms, ms_stream, n = timed_launches(stream, flush, lambda ev: (
        tea.attn_time_next_call(*ev),
        tea.attn_bwd(xq, xk, xv, xo, xl, xdo, gq, gk, gv, x.scale, x.causal, ws, stream=stream)))
    fwd_flops, _ = prefill_work(x.B, x.Hq, x.Hkv, x.T, x.S, x.d, x.causal, 2)
    flops = fwd_flops // 4 * 10
    tf = flops / (ms * 1e-3) / 1e12
    rec = {"config": f"{x.name}: B={x.B}, Hq={x.Hq}, Hkv={x.Hkv}, T=S={x.T}, d={x.d}, bf16, causal",
           "kernels": "bwd_dq_kernel+bwd_dkdv_kernel+bwd_kv_reduce_kernel", "ms": ms,
           "ms_stream": ms_stream, "value": tf,
           "unit": "TFLOP/s", "algorithmic_flops": flops, "bound": "mfma",
           "peak": PEAK_BF16_TFLOPS, "frac_of_mfma_peak": tf / PEAK_BF16_TFLOPS,
           "launches": n, "cpu_baseline": None}
    del xq, xk, xv, xdo, xo, xl, gq, gk, gv, ws
    if cpu_budget_s:
        import oracle
        g = x.Hq // x.Hkv
        head_flops = flops // (x.B * x.Hq)
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < cpu_budget_s:
            b, h = divmod(done % (x.B * x.Hq), x.Hq)
            oracle.attention_head_backward(x.q[b, h].double().numpy(), x.k[b, h // g].double().numpy(),
                                           x.v[b, h // g].double().numpy(), x.do[b, h].double().numpy(),
                                           x.scale, x.causal)
            done += 1
        tc = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": done * head_flops / tc / 1e12, "unit": "TFLOP/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{done} (batch, head) gradient problems of {x.name} "
                                         f"({tc:.1f} s)"}
    return rec


# --- the main step: causal prefill on the three prefill workloads, then decode ----

MAIN_STEP = ["prefill_2", "prefill_3", "prefill_4", "decode_5"]
HEADLINE = "prefill_2"
# Kernel names (substrings) per workload, for traces and counters.
KERNEL_OF = {"prefill_2": "prefill_bf16_kernel", "prefill_3": "prefill_bf16_kernel",
             "prefill_4": "prefill_bf16_kernel",
             "decode_5": "decode_stream_kernel+decode_combine_kernel"}
# Oracle seconds per workload out of --cpu-budget (fractions).
CPU_SHARE = {"prefill_2": 0.3, "prefill_3": 0.25, "prefill_4": 0.25, "decode_5": 0.2}


def prefill_grid_threads(x):
    """Threads of one prefill launch (the grid the kernel trace reports): 128 query
    rows per 256-thread workgroup, or 64 rows per workgroup on grids under 256
    workgroups."""
    wgs = -(-x.T // 128) * x.B * x.Hq
    if wgs < 256:
        wgs = -(-x.T // 64) * x.B * x.Hq
    return wgs * 256


def oracle_prefill_sample(x, budget_s, window=0):
    """Float64 oracle on (batch, head) problems of prefill workload x, in order
    and cycling, for about budget_s seconds."""
    import oracle
    g = x.Hq // x.Hkv
    heads = [(b, h) for b in range(x.B) for h in range(x.Hq)]
    fl, _ = prefill_work(x.B, x.Hq, x.Hkv, x.T, x.S, x.d, x.causal, 2, window=window)
    q, k, v = x.q, x.k, x.v
    done, work, tc = oracle_sample(
        budget_s, heads,
        lambda bh: oracle.attention_head(q[bh[0], bh[1]].double().numpy(),
                                         k[bh[0], bh[1] // g].double().numpy(),
                                         v[bh[0], bh[1] // g].double().numpy(),
                                         x.scale, x.causal, window=window),
        lambda bh: fl // len(heads))
    return {"value": work / tc / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{done} (batch, head) attention problems of {x.name} ({done / len(heads):.2f} "
                      f"passes over its {len(heads)}, {tc:.1f} s, {fl // len(heads) * done / 1e9:.1f} "
                      f"GFLOP)", "host_cpus": len(os.sched_getaffinity(0))}


def oracle_decode_sample(x, budget_s):
    """Float64 oracle on whole sequences of decode workload x for about budget_s
    seconds; GB/s over the same algorithmic bytes per sequence as the GPU figure."""
    import oracle
    qd, kd, vd = x.f64()

    def one(n):
        oracle.decode_paged(qd, kd, vd, x.block_table, x.seq_lens, x.scale, seqs=[n])

    def nbytes(n):
        L = int(x.seq_lens[n])
        return L * x.Hkv * x.d * 2 * 2 + 2 * x.Hq * x.d * 2 + x.Hq * 4 + 4 + -(-L // x.page) * 4

    done, work, tc = oracle_sample(budget_s, list(range(x.N)), one, nbytes)
    return {"value": work / tc / 1e9, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} sequences of {x.name} ({done / x.N:.2f} passes over its {x.N}, "
                      f"{tc:.1f} s), one oracle call each", "host_cpus": len(os.sched_getaffinity(0))}


def hbm_probe(dinp, dev, stream, flush, launches=12):
    """Read-only probe (libattn_probe.so): the decode workload's key and value
    slabs, one 4 KiB chunk each per (page, KV head), read in the decode's
    sequence-major order by one-wave workgroups splitting them into equal
    contiguous ranges, at the decode's 768 waves and at 1024 (the faster is
    reported: the ceiling); then the same byte count read in order from a
    contiguous buffer.  GB/s = bytes / mean event time."""
    import ctypes

    import numpy as np
    import torch
    from tiled_exact_attention_flashattention_amd import build as B
    if not os.path.exists(B.PROBE_LIB_PATH):
        raise RuntimeError(f"{B.PROBE_LIB_PATH} is missing: build with "
                           "`python -m tiled_exact_attention_flashattention_amd.build`")
    L = ctypes.CDLL(B.PROBE_LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    L.attn_probe_read_units.argtypes = [vp, vp, vp, i32, i32, vp, i32, vp, vp, vp]
    L.attn_probe_read_units.restype = i32
    unit_bytes = dinp.page * dinp.d * 2
    units = []
    for n in range(dinp.N):
        nb = -(-int(dinp.seq_lens[n]) // dinp.page)
        for hk in range(dinp.Hkv):
            units.append(dinp.block_table[n, :nb].astype(np.int64) * dinp.Hkv + hk)
    units = np.concatenate(units).astype(np.int32)
    pool_units = dinp.k_pool.numel() * 2 // unit_bytes
    assert units.min() >= 0 and units.max() < pool_units
    sink = torch.empty(1024 * 64, dtype=torch.int32, device=dev)
    kp, vpl = dinp.k_pool.to(dev), dinp.v_pool.to(dev)
    u_dev = torch.from_numpy(units).to(dev)
    n = len(units)
    seq = torch.empty(2 * n * unit_bytes, dtype=torch.uint8, device=dev)
    seq_units = torch.arange(n, dtype=torch.int32, device=dev)
    res = {}
    for name, (kb, vb, ub) in {"decode_pages": (kp, vpl, u_dev),
                               "sequential": (seq, seq[n * unit_bytes:], seq_units)}.items():
        for waves in (768, 1024):
            def launch(ev):
                st = L.attn_probe_read_units(kb.data_ptr(), vb.data_ptr(), ub.data_ptr(), n,
                                             unit_bytes, sink.data_ptr(), waves,
                                             ctypes.c_void_p(stream.cuda_stream),
                                             ctypes.c_void_p(ev[0].cuda_event),
                                             ctypes.c_void_p(ev[1].cuda_event))
                if st != 0:
                    raise RuntimeError(f"probe launch failed ({st})")
            ms, ms_stream, cnt = timed_launches(stream, flush, launch, n=launches, skip=2)
            nbytes = 2 * n * unit_bytes
            rec = {"bytes": nbytes, "ms": ms, "ms_stream": ms_stream,
                   "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s",
                   "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                   "launches": cnt, "waves": waves}
            if name not in res or rec["value"] > res[name]["value"]:
                res[name] = rec
    res["note"] = (f"{n} chunks of {unit_bytes} B of K and as many of V (768 or 1024 one-wave "
                   "workgroups, equal contiguous ranges, the faster kept); cold caches")
    del kp, vpl, u_dev, seq, seq_units, sink
    return res


def write_counters(pmc_dir):
    """profiles/counters.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE CSVs.

    Expects DIR/copy_{fetch,write}/ (this script with --copy-probe) and
    DIR/<workload>_{fetch,write}/ for each workload of the main step (this
    script with --only <workload>); every dispatch of the workload's kernels is
    averaged, the flush's reduction kernel excluded by name."""
    import csv
    import glob

    def rows(sub):
        files = glob.glob(os.path.join(pmc_dir, sub, "**", "*_counter_collection.csv"), recursive=True)
        if len(files) != 1:
            raise SystemExit(f"need exactly one counter_collection.csv under {pmc_dir}/{sub}")
        return list(csv.DictReader(open(files[0])))

    copy_bytes = 256 << 20
    factors = {}
    for counter, sub in (("FETCH_SIZE", "copy_fetch"), ("WRITE_SIZE", "copy_write")):
        # the copy dispatches (the runtime's buffer copy), KiB per dispatch
        vals = [float(r["Counter_Value"]) for r in rows(sub) if "copy" in r["Kernel_Name"].lower()]
        if not vals:
            raise SystemExit(f"no copy dispatch under {pmc_dir}/{sub}")
        factors[counter] = copy_bytes / (sum(vals) / len(vals) * 1024.0)

    out = {"factors": factors, "copy_probe_bytes": copy_bytes,
           "commands": {"copy": "rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv -d <dir> "
                                "-- python3 bench.py --copy-probe",
                        "workload": "rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv -d <dir> "
                                    "-- python3 bench.py --only <workload> --steps 3 --warmup 1 "
                                    "--no-cpu-baseline (flush on: cold caches as in the timed run)"}}
    for name in MAIN_STEP:
        kinds = KERNEL_OF[name].split("+")
        kind = "decode" if name.startswith("decode") else "prefill"
        tot = {}
        for counter, suffix in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            per = {}
            for r in rows(f"{name}_{suffix}"):
                if any(k in r["Kernel_Name"] for k in kinds):
                    per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            if not per:
                raise SystemExit(f"no {kinds} dispatch in {name}_{suffix}")
            kib = sum(sum(v) / len(v) for v in per.values())
            tot[counter] = kib * 1024.0 * factors[counter]
        out[name] = {"sources_sha": sources_sha(kind), "kernels": kinds,
                     "fetch_bytes_per_launch": tot["FETCH_SIZE"],
                     "write_bytes_per_launch": tot["WRITE_SIZE"],
                     "hbm_bytes_per_launch": tot["FETCH_SIZE"] + tot["WRITE_SIZE"]}
    path = os.path.join(ROOT, "profiles", "counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def counters_for(name):
    path = os.path.join(ROOT, "profiles", "counters.json")
    kind = "decode" if name.startswith("decode") else "prefill"
    try:
        with open(path) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha") != sources_sha(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def summarize(prof_dir):
    """Markdown summary of a rocprofv3 run under prof_dir: per (kernel, grid)
    dispatch count and mean / median / min / max duration from the kernel
    trace, or the mean of every counter per (kernel, grid) from a counter
    collection."""
    import csv
    import glob
    from collections import defaultdict
    traces = glob.glob(os.path.join(prof_dir, "**", "*_kernel_trace.csv"), recursive=True)
    counters = glob.glob(os.path.join(prof_dir, "**", "*_counter_collection.csv"), recursive=True)
    lines = []

    def short(name):
        import re
        n = name.replace("(anonymous namespace)::", "")
        m = re.match(r"_ZN\d+attn\d+_GLOBAL__N_1(\d+)", n)
        if m:                                  # mangled: identifier and integer template args
            ln = int(m.group(1))
            rest = n[m.end():]
            ident, rest = rest[:ln], rest[ln:]
            args = re.findall(r"L[a-z](\d+)E", rest.split("EE")[0] + "E") if rest.startswith("I") else []
            return f"{ident}<{','.join(args)}>" if args else ident
        m = re.match(r"(?:void\s+)?(?:[\w]+::)*(\w+(?:<.*?>)?)\(", n)
        return (m.group(1) if m else n)[:90]

    for f in traces:
        acc = defaultdict(list)
        for r in csv.DictReader(open(f)):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            acc[(r["Kernel_Name"], grid)].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += [f"kernel trace `{os.path.relpath(f, prof_dir)}`", "",
                  "| kernel | grid (threads) | dispatches | mean µs | median µs | min µs | max µs |",
                  "|---|---|---|---|---|---|---|"]
        for (k, g), d in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
            ds = sorted(d)
            med = ds[len(ds) // 2] if len(ds) % 2 else (ds[len(ds) // 2 - 1] + ds[len(ds) // 2]) / 2
            lines.append(f"| `{short(k)}` | {g} | {len(d)} | {sum(d) / len(d):.2f} | {med:.2f} | "
                         f"{min(d):.2f} | {max(d):.2f} |")
        lines.append("")
    for f in counters:
        acc = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(f)):
            acc[(r["Kernel_Name"], int(r["Grid_Size"]))][r["Counter_Name"]].append(
                float(r["Counter_Value"]))
        names = sorted({c for v in acc.values() for c in v})
        lines += [f"counters `{os.path.relpath(f, prof_dir)}` (mean per dispatch)", "",
                  "| kernel | grid | dispatches | " + " | ".join(names) + " |",
                  "|---|---|---|" + "---|" * len(names)]
        for (k, g), cs in sorted(acc.items(), key=lambda kv: kv[0][1]):
            n = max(len(v) for v in cs.values())
            vals = [f"{sum(cs[c]) / len(cs[c]):.4g}" if cs.get(c) else "" for c in names]
            lines.append(f"| `{short(k)}` | {g} | {n} | " + " | ".join(vals) + " |")
        lines.append("")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=MAIN_STEP,
                    help="the step runs only this workload (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=16.0,
                    help="seconds of oracle work for the main step's workloads")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration) and exit")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only run the read-only HBM probe on the decode workload's pages and exit")
    ap.add_argument("--write-counters", metavar="DIR",
                    help="write profiles/counters.json from rocprofv3 CSVs under DIR and exit")
    ap.add_argument("--summarize", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 output directory and exit")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the sliding-window, chunked-prefill and fp8-decode timings")
    ap.add_argument("--no-probe", action="store_true", help="skip the read-only HBM probe")
    args = ap.parse_args()
    if args.write_counters:
        write_counters(args.write_counters)
        return
    if args.summarize:
        summarize(args.summarize)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the kernels run on one device's share and nothing here is sharded.", flush=True)
        sys.exit(1)

    import torch

    import tiled_exact_attention_flashattention_amd as tea
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_probe:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 256 << 20, "launches": 5}))
        return
    # float32 so that sum() only reads it (an int32 sum would first write an
    # int64 copy, leaving dirty cache lines whose write-back slows the kernels)
    flush = None if args.no_flush else torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
    if args.hbm_probe:
        print(json.dumps(hbm_probe(workloads.decode_5(), dev, stream, flush)), flush=True)
        return

    names = [args.only] if args.only else MAIN_STEP
    inputs, launchers = {}, {}
    for name in names:
        x = getattr(workloads, name)()
        inputs[name] = x
        if name.startswith("prefill"):
            q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
            o = torch.empty_like(q)
            lse = torch.empty((x.B, x.Hq, x.T), dtype=torch.float32, device=dev)
            launchers[name] = (lambda q=q, k=k, v=v, o=o, lse=lse, x=x:
                               tea.attn_fwd(q, k, v, o, lse, x.scale, x.causal, stream=stream))
        else:
            dq, dk, dv = x.q.to(dev), x.k_pool.to(dev), x.v_pool.to(dev)
            bt = torch.from_numpy(x.block_table).to(dev)
            sl = torch.from_numpy(x.seq_lens).to(dev)
            do = torch.empty_like(dq)
            dlse = torch.empty((x.N, x.Hq), dtype=torch.float32, device=dev)
            ws = tea.decode_workspace(x.N, x.Hq, x.d, x.max_blocks, dev)
            launchers[name] = (lambda dq=dq, dk=dk, dv=dv, bt=bt, sl=sl, do=do, dlse=dlse, ws=ws, x=x:
                               tea.attn_decode_paged(dq, dk, dv, bt, sl, do, dlse, x.scale, ws,
                                                     stream=stream))

    events = {name: [] for name in names}
    kev = {name: kernel_events(args.steps) for name in names}
    smark = {name: kernel_events(args.steps) for name in names}

    def step(record):
        for name in names:
            if flush is not None:
                flush.sum()
            if record:
                i = len(events[name])
                a, b_ = smark[name][i]
                a.record(stream)
                tea.attn_time_next_call(*kev[name][i])
            launchers[name]()
            if record:
                b_.record(stream)
                events[name].append((kev[name][i], (a, b_)))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    kernels = {}
    for name in names:
        x = inputs[name]
        times = [k0.elapsed_time(k1) for (k0, k1), _ in events[name]]
        ms = sum(times) / len(times)
        ms_stream = sum(a.elapsed_time(b_) for _, (a, b_) in events[name]) / len(times)
        if name.startswith("prefill"):
            fl, nb = prefill_work(x.B, x.Hq, x.Hkv, x.T, x.S, x.d, x.causal, 2)
            rate = fl / (ms * 1e-3) / 1e12
            rec = {"kernel": KERNEL_OF[name], "bound": "mfma", "achieved": rate,
                   "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": rate / PEAK_BF16_TFLOPS,
                   "config": f"B={x.B}, Hq={x.Hq}, Hkv={x.Hkv}, T=S={x.T}, d={x.d}, bf16, causal"
                             f"{', inputs x0.5' if name == 'prefill_4' else ''}",
                   "grid_threads": prefill_grid_threads(x)}
        else:
            fl, nb, tokens = decode_work(x)
            rate = nb / (ms * 1e-3) / 1e9
            rec = {"kernel": KERNEL_OF[name], "bound": "hbm", "achieved": rate,
                   "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": rate / PEAK_HBM_GBS,
                   "config": f"N={x.N}, Hq={x.Hq}, Hkv={x.Hkv}, d={x.d}, page {x.page}, lengths "
                             f"U[512,8192] (sum {tokens}), bf16", "tokens": tokens,
                   "tokens_per_s": tokens / (ms * 1e-3)}
        rec.update({"traffic": counters_for(name), "algorithmic_flops": fl,
                    "algorithmic_bytes": nb, "ms": ms, "ms_min": min(times),
                    "ms_stream": ms_stream,
                    "launches": len(times)})
        kernels[name] = rec

    if not args.no_probe and "decode_5" in names:
        probe = hbm_probe(inputs["decode_5"], dev, stream, flush)
        kernels["decode_5"]["frac_of_probe_ceiling"] = (
            kernels["decode_5"]["achieved"] / probe["decode_pages"]["value"])
    else:
        probe = None

    dominant = max(names, key=lambda n: kernels[n]["ms"])
    head = HEADLINE if HEADLINE in names else names[0]
    hx = inputs[head]
    out = {
        "metric": "causal prefill attention TFLOP/s + paged decode GB/s, % of MFMA/HBM peak",
        "value": kernels[head]["achieved"],
        "unit": kernels[head]["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{head}: {kernels[head]['config']}; the step also runs "
                        + ", ".join(f"{n} ({kernels[n]['config']})" for n in names if n != head),
            "global_batch": getattr(hx, "B", getattr(hx, "N", None)),
            "seq_len": getattr(hx, "T", None),
            "parallelism": "single GPU",
            "cold_cache": flush is not None,
            "step": names,
        },
        "roofline": dict(kernels[dominant], workload=dominant),
        "roofline_per_kernel": kernels,
    }
    if probe is not None:
        out["hbm_probe"] = probe
    if not args.only:
        if not args.no_next:
            nb_ = None if args.no_cpu_baseline else args.cpu_budget / 5
            out["window"] = bench_window(tea, workloads, dev, stream, flush, nb_)
            out["chunked"] = bench_chunked(tea, workloads, dev, stream, flush, nb_)
            out["decode_fp8"] = bench_decode_q8(tea, workloads, dev, stream, flush, nb_, "fp8")
            out["decode_int8"] = bench_decode_q8(tea, workloads, dev, stream, flush, nb_, "int8")
        if not args.no_backward:
            out["backward"] = bench_backward(tea, workloads, dev, stream, flush,
                                             None if args.no_cpu_baseline else args.cpu_budget / 3)
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        for name in names:
            x = inputs[name]
            budget = args.cpu_budget * CPU_SHARE[name]
            cb = (oracle_prefill_sample(x, budget) if name.startswith("prefill")
                  else oracle_decode_sample(x, budget))
            kernels[name]["cpu_baseline"] = cb
        out["cpu_baseline"] = kernels[head]["cpu_baseline"]
        out["roofline"]["cpu_baseline"] = kernels[dominant]["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
