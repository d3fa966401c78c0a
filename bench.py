#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path on resident synthetic inputs:
  1. causal prefill attn_fwd on the GPT-2-small-shaped workload
     (B=8, H=12, T=S=1024, d=64, bf16; override with --prefill), then
  2. paged decode attn_decode_paged on 64 sequences, 12 query / 2 KV heads,
     d=128, 16-token pages, lengths U[512, 8192] (stream kernel + combine).

Reported (one JSON line on stdout):
  value          causal-prefill TFLOP/s = algorithmic FLOPs / mean kernel time
                 (HIP events on the launch stream), FLOPs = 4*d per visible
                 (query, key) pair;
  decode         paged-decode GB/s = algorithmic bytes / mean time of the stream
                 + combine kernels, bytes = K+V of every cached token once plus
                 q, o, lse, seq_lens and the used block-table entries;
  roofline       the kernel that takes the most time per step against its
                 published peak (bf16 dense MFMA 2516.6 TFLOP/s, HBM 8 TB/s);
                 `traffic` comes from profiles/counters.json when the measured
                 kernel sources still match the recorded hash, else null;
  prefill_other  the same causal prefill timing on the two larger prefill
                 workloads (GQA B=4 T=4096 d=128; long B=1 H=32 T=16384 d=128);
  window         attn_fwd_window on the GQA causal workload with a 1024-key
                 sliding window (FLOPs over the visible pairs only);
  chunked        attn_prefill_paged on 16 sequences of 1024..8192 cached
                 tokens whose last 512 are the new chunk, Hq=12, Hkv=2,
                 d=128, keys through the block table (FLOPs over the
                 visible pairs);
  decode_fp8     attn_decode_paged_fp8 on decode_5's shape with E4M3 pages
                 (decode_fp8_7): GB/s over the bytes it must read (one byte
                 per cached K/V element, plus q, o, lse, lengths, block table);
  (window, chunked and decode_fp8 each carry their own cpu_baseline: the
  oracle timed on sampled heads or sequences of the same workload)
  backward       the gradient pass attn_bwd (D = rowsum(dO*O), dQ, dK/dV
                 kernels) on the GQA causal workload (B=4, Hq=12, Hkv=2,
                 T=S=4096, d=128), TFLOP/s with FLOPs = 10*d per visible
                 (query, key) pair (recomputed scores, dP, dV, dQ, dK: five
                 products of 2*d each), next to the float64 backward oracle
                 timed on a bounded sample of its heads;
  cpu_baseline   the float64 oracle timed on the host on a bounded sample of
                 the same workloads.
`--write-counters DIR` turns rocprofv3 FETCH_SIZE / WRITE_SIZE collections
(DIR/{bench,copy}_{fetch,write}/*_counter_collection.csv, taken on this script
with the default workload and with --copy-probe) into profiles/counters.json:
HBM bytes per launch, each counter scaled by what it reads for a copy of
known size.
Between steps a 512 MiB buffer is read (summed) so both kernels start with
cold L2 / Infinity Cache without dirty lines whose write-back would compete
with them; that read is outside the kernel events but inside ms_per_step.
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


def cpu_baseline(pinp, dinp, budget_s):
    """Time the oracle on a bounded sample of both workloads (host cores).

    Whole passes over the (batch, head) pairs of the prefill workload, then
    over the sequences of the decode workload, are repeated until about 70 %
    (prefill) and 30 % (decode) of budget_s is spent; a pass that runs out of
    budget stops where it is, so the sample is a prefix of the workload
    repeated."""
    import numpy as np

    import oracle
    q, k, v = (t.double().numpy() for t in (pinp.q, pinp.k, pinp.v))
    g = pinp.Hq // pinp.Hkv
    heads = [(b, h) for b in range(pinp.B) for h in range(pinp.Hq)]
    head_flops = prefill_work(1, 1, 1, pinp.T, pinp.S, pinp.d, pinp.causal, 2)[0]
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s * 0.7:
        b, h = heads[done % len(heads)]
        oracle.attention_head(q[b, h], k[b, h // g], v[b, h // g], pinp.scale, pinp.causal)
        done += 1
    tp = time.perf_counter() - t0
    qd, kd, vd = dinp.f64()
    nseq, dbytes, t1 = 0, 0, time.perf_counter()
    while time.perf_counter() - t1 < budget_s * 0.3:
        n = nseq % dinp.N
        oracle.decode_paged(qd, kd, vd, dinp.block_table, dinp.seq_lens, dinp.scale, seqs=[n])
        L = int(dinp.seq_lens[n])
        dbytes += L * dinp.Hkv * dinp.d * 4 + 2 * dinp.Hq * dinp.d * 2
        nseq += 1
    td = time.perf_counter() - t1
    return {
        "value": done * head_flops / tp / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{done} (batch, head) attention problems of {pinp.name} ({done / len(heads):.2f} "
                  f"passes over its {len(heads)}, {tp:.1f} s); decode: {nseq} sequences of "
                  f"{dinp.name} ({nseq / dinp.N:.2f} passes over its {dinp.N}, {td:.1f} s)",
        "decode_value": dbytes / td / 1e9, "decode_unit": "GB/s",
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def timed_launches(stream, flush, launch, n=7, skip=2):
    """Mean HIP-event time (ms) of launch() over n cold launches, the first `skip` untimed."""
    import torch
    times = []
    for i in range(n):
        if flush is not None:
            flush.sum()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch()
        b_.record(stream)
        if i >= skip:
            times.append((a, b_))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b_) for a, b_ in times) / len(times), len(times)


def bench_window(tea, workloads, dev, stream, flush, cpu_budget_s=None, window=1024):
    """attn_fwd_window on the GQA causal workload (and the oracle on sampled heads)."""
    import torch
    x = workloads.prefill_3()
    xq, xk, xv = (t.to(dev) for t in (x.q, x.k, x.v))
    xo = torch.empty_like(xq)
    xl = torch.empty((x.B, x.Hq, x.T), dtype=torch.float32, device=dev)
    ms, n = timed_launches(stream, flush, lambda: tea.attn_fwd_window(
        xq, xk, xv, xo, xl, x.scale, window, stream=stream))
    fl, _ = prefill_work(x.B, x.Hq, x.Hkv, x.T, x.S, x.d, True, 2, window=window)
    tf = fl / (ms * 1e-3) / 1e12
    rec = {"config": f"B={x.B}, Hq={x.Hq}, Hkv={x.Hkv}, T=S={x.T}, d={x.d}, bf16, causal, "
                     f"window {window}", "kernel": "prefill_bf16_kernel", "ms": ms, "value": tf,
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
    ms, n = timed_launches(stream, flush, lambda: tea.attn_prefill_paged(
        xq, kp, vp, bt, sl, ql, xo, xl, x.scale, stream=stream))
    fl = 4 * x.d * x.Hq * chunked_pairs(x.seq_lens, x.q_lens)
    tf = fl / (ms * 1e-3) / 1e12
    rec = {"config": f"N={x.N}, Hq={x.Hq}, Hkv={x.Hkv}, chunk {x.T}, cached "
                     f"{int(x.seq_lens.min())}..{int(x.seq_lens.max())} tokens, d={x.d}, bf16, "
                     f"16-token pages", "kernel": "prefill_bf16_kernel (paged)", "ms": ms,
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


def bench_decode_fp8(tea, workloads, dev, stream, flush, cpu_budget_s=None):
    """attn_decode_paged_fp8 on decode_fp8_7 (stream + combine kernels), and the
    oracle on sampled sequences."""
    import torch
    x = workloads.decode_fp8_7()
    xq, kc, vc = x.q.to(dev), x.k_codes.to(dev), x.v_codes.to(dev)
    bt, sl = torch.from_numpy(x.block_table).to(dev), torch.from_numpy(x.seq_lens).to(dev)
    xo = torch.empty_like(xq)
    xl = torch.empty((x.N, x.Hq), dtype=torch.float32, device=dev)
    ws = tea.decode_workspace(x.N, x.Hq, x.d, x.max_blocks, dev)
    ms, n = timed_launches(stream, flush, lambda: tea.attn_decode_paged_fp8(
        xq, kc, vc, x.k_scale, x.v_scale, bt, sl, xo, xl, x.scale, ws, stream=stream), n=12)
    tokens = int(x.seq_lens.astype("int64").sum())
    pages = int(((x.seq_lens.astype("int64") + x.page - 1) // x.page).sum())
    nbytes = tokens * x.Hkv * x.d * 2 + 2 * x.N * x.Hq * x.d * 2 + x.N * x.Hq * 4 + x.N * 4 + pages * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    rec = {"config": f"N={x.N}, Hq={x.Hq}, Hkv={x.Hkv}, d={x.d}, E4M3 K/V pages, lengths "
                     f"U[512,8192] (sum {tokens})", "kernel": "decode_stream_kernel<fp8>+"
                     "decode_combine_kernel", "ms": ms, "value": gbs, "unit": "GB/s",
           "algorithmic_bytes": nbytes, "bound": "hbm", "peak": PEAK_HBM_GBS,
           "frac_of_hbm_peak": gbs / PEAK_HBM_GBS, "launches": n,
           "tokens_per_s": tokens / (ms * 1e-3), "cpu_baseline": None}
    del xq, kc, vc, bt, sl, xo, xl, ws
    if cpu_budget_s:
        import numpy as np

        import oracle
        qd = x.q.double().numpy()
        kcodes, vcodes = x.k_codes.numpy(), x.v_codes.numpy()

        def one_sequence(n):
            # the pages sequence n uses, as a pool of their own with the table renumbered
            nb = (int(x.seq_lens[n]) + x.page - 1) // x.page
            pages = x.block_table[n, :nb]
            oracle.decode_paged_fp8(qd[n:n + 1], kcodes[pages], vcodes[pages], x.k_scale,
                                    x.v_scale, np.arange(nb, dtype=np.int32)[None, :],
                                    x.seq_lens[n:n + 1], x.scale, page=x.page)

        done, work, tc = oracle_sample(
            cpu_budget_s, list(range(x.N)), one_sequence,
            lambda n: int(x.seq_lens[n]) * x.Hkv * x.d * 2 + 2 * x.Hq * x.d * 2)
        rec["cpu_baseline"] = {"value": work / tc / 1e9, "unit": "GB/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": f"{done} sequences of this workload, one oracle call "
                                         f"each on the E4M3 pages it uses ({tc:.1f} s)"}
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
    times = []
    for i in range(7):
        if flush is not None:
            flush.sum()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        tea.attn_bwd(xq, xk, xv, xo, xl, xdo, gq, gk, gv, x.scale, x.causal, ws, stream=stream)
        b_.record(stream)
        if i >= 2:
            times.append((a, b_))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b_) for a, b_ in times) / len(times)
    fwd_flops, _ = prefill_work(x.B, x.Hq, x.Hkv, x.T, x.S, x.d, x.causal, 2)
    flops = fwd_flops // 4 * 10
    tf = flops / (ms * 1e-3) / 1e12
    rec = {"config": f"{x.name}: B={x.B}, Hq={x.Hq}, Hkv={x.Hkv}, T=S={x.T}, d={x.d}, bf16, causal",
           "kernels": "bwd_prep_kernel+bwd_dq_kernel+bwd_dkdv_kernel", "ms": ms, "value": tf,
           "unit": "TFLOP/s", "algorithmic_flops": flops, "bound": "mfma",
           "peak": PEAK_BF16_TFLOPS, "frac_of_mfma_peak": tf / PEAK_BF16_TFLOPS,
           "launches": len(times), "cpu_baseline": None}
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


def write_counters(pmc_dir):
    """profiles/counters.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE CSVs."""
    import csv
    import glob

    def per_kernel(sub):
        files = glob.glob(os.path.join(pmc_dir, sub, "*_counter_collection.csv"))
        if len(files) != 1:
            raise SystemExit(f"need exactly one counter_collection.csv under {pmc_dir}/{sub}")
        vals = {}
        for r in csv.DictReader(open(files[0])):
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    copy_bytes = 256 << 20
    factors = {}
    for counter, sub in (("FETCH_SIZE", "copy_fetch"), ("WRITE_SIZE", "copy_write")):
        vals = per_kernel(sub)
        # the copy is the dispatch with the largest reading (KiB per dispatch)
        kib = max(max(v) for v in vals.values())
        factors[counter] = copy_bytes / (kib * 1024.0)
    fetch, write = per_kernel("bench_fetch"), per_kernel("bench_write")

    def bytes_of(pattern):
        tot = {}
        for counter, vals in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
            kib = sum(sum(v) / len(v) for k, v in vals.items() if any(p in k for p in pattern))
            tot[counter] = kib * 1024.0 * factors[counter]
        return tot

    out = {"factors": factors, "copy_probe_bytes": copy_bytes,
           "commands": {"copy": "rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv -d <dir> "
                                "-- python3 bench.py --copy-probe",
                        "bench": "rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv -d <dir> "
                                 "-- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-flush --no-other-prefill "
                                 "--no-backward --no-next"}}
    for kind, pattern in (("prefill", ["prefill_bf16_kernel"]),
                          ("decode", ["decode_stream_kernel", "decode_combine_kernel"])):
        t = bytes_of(pattern)
        out[kind] = {"sources_sha": sources_sha(kind), "kernels": pattern,
                     "fetch_bytes_per_launch": t["FETCH_SIZE"], "write_bytes_per_launch": t["WRITE_SIZE"],
                     "hbm_bytes_per_launch": t["FETCH_SIZE"] + t["WRITE_SIZE"]}
    path = os.path.join(ROOT, "profiles", "counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def counters_for(kind):
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha") != sources_sha(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill", default="prefill_2",
                    choices=["prefill_2", "prefill_3", "prefill_4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration) and exit")
    ap.add_argument("--write-counters", metavar="DIR",
                    help="write profiles/counters.json from rocprofv3 CSVs under DIR and exit")
    ap.add_argument("--no-other-prefill", action="store_true",
                    help="skip the timing of the two larger prefill workloads")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the sliding-window, chunked-prefill and fp8-decode timings")
    args = ap.parse_args()
    if args.write_counters:
        write_counters(args.write_counters)
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

    if args.copy_probe:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 256 << 20, "launches": 5}))
        return

    pinp = getattr(workloads, args.prefill)()
    dinp = workloads.decode_5()
    q, k, v = (t.to(dev) for t in (pinp.q, pinp.k, pinp.v))
    o = torch.empty_like(q)
    lse = torch.empty((pinp.B, pinp.Hq, pinp.T), dtype=torch.float32, device=dev)
    dq, dk, dv = dinp.q.to(dev), dinp.k_pool.to(dev), dinp.v_pool.to(dev)
    bt = torch.from_numpy(dinp.block_table).to(dev)
    sl = torch.from_numpy(dinp.seq_lens).to(dev)
    do = torch.empty_like(dq)
    dlse = torch.empty((dinp.N, dinp.Hq), dtype=torch.float32, device=dev)
    ws = tea.decode_workspace(dinp.N, dinp.Hq, dinp.d, dinp.max_blocks, dev)
    # float32 so that sum() only reads it (an int32 sum would first write an
    # int64 copy, leaving dirty cache lines whose write-back slows the kernels)
    flush = None if args.no_flush else torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)

    stream = torch.cuda.current_stream(dev)
    events = []

    def step(record):
        if flush is not None:
            flush.sum()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            e[0].record(stream)
        tea.attn_fwd(q, k, v, o, lse, pinp.scale, pinp.causal, stream=stream)
        if record:
            e[1].record(stream)
            e[2].record(stream)
        tea.attn_decode_paged(dq, dk, dv, bt, sl, do, dlse, dinp.scale, ws, stream=stream)
        if record:
            e[3].record(stream)
            events.append(e)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    prefill_ms = sum(e[0].elapsed_time(e[1]) for e in events) / len(events)
    decode_ms = sum(e[2].elapsed_time(e[3]) for e in events) / len(events)

    elem = 2 if pinp.dtype == "bf16" else 4
    pflops, pbytes = prefill_work(pinp.B, pinp.Hq, pinp.Hkv, pinp.T, pinp.S, pinp.d, pinp.causal, elem)
    dflops, dbytes, tokens = decode_work(dinp)
    p_tflops = pflops / (prefill_ms * 1e-3) / 1e12
    d_gbs = dbytes / (decode_ms * 1e-3) / 1e9
    peak_p = PEAK_BF16_TFLOPS if pinp.dtype == "bf16" else PEAK_F32_TFLOPS

    kernels = {
        "prefill": {"kernel": "prefill_bf16_kernel", "bound": "mfma", "achieved": p_tflops,
                    "peak": peak_p, "unit": "TFLOP/s", "frac": p_tflops / peak_p,
                    "traffic": counters_for("prefill"), "algorithmic_bytes": pbytes,
                    "algorithmic_flops": pflops, "ms": prefill_ms},
        "decode": {"kernel": "decode_stream_kernel+decode_combine_kernel", "bound": "hbm",
                   "achieved": d_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": d_gbs / PEAK_HBM_GBS, "traffic": counters_for("decode"),
                   "algorithmic_bytes": dbytes, "algorithmic_flops": dflops, "ms": decode_ms},
    }
    dominant = "prefill" if prefill_ms >= decode_ms else "decode"

    out = {
        "metric": "causal prefill attention TFLOP/s + paged decode GB/s, % of MFMA/HBM peak",
        "value": p_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": pinp.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{pinp.name} causal prefill (B={pinp.B}, Hq={pinp.Hq}, Hkv={pinp.Hkv}, "
                        f"T=S={pinp.T}, d={pinp.d}, {pinp.dtype}) + {dinp.name} paged decode "
                        f"(N={dinp.N}, Hq={dinp.Hq}, Hkv={dinp.Hkv}, d={dinp.d}, page {dinp.page}, "
                        f"lengths U[512,8192], sum {tokens})",
            "global_batch": pinp.B,
            "seq_len": pinp.T,
            "parallelism": "single GPU",
            "cold_cache": flush is not None,
        },
        "decode": {"value": d_gbs, "unit": "GB/s", "frac_of_hbm_peak": d_gbs / PEAK_HBM_GBS,
                   "ms": decode_ms, "tokens": tokens},
        "prefill_frac_of_mfma_peak": p_tflops / peak_p,
        "roofline": dict(kernels[dominant]),
        "roofline_per_kernel": kernels,
    }
    if not args.no_other_prefill:
        other = {}
        for name in ("prefill_3", "prefill_4"):
            if name == pinp.name:
                continue
            x = getattr(workloads, name)()
            xq, xk, xv = (t.to(dev) for t in (x.q, x.k, x.v))
            xo = torch.empty_like(xq)
            xl = torch.empty((x.B, x.Hq, x.T), dtype=torch.float32, device=dev)
            times = []
            for i in range(7):
                if flush is not None:
                    flush.sum()
                a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                tea.attn_fwd(xq, xk, xv, xo, xl, x.scale, x.causal, stream=stream)
                b_.record(stream)
                if i >= 2:
                    times.append((a, b_))
            torch.cuda.synchronize()
            ms = sum(a.elapsed_time(b_) for a, b_ in times) / len(times)
            fl, _ = prefill_work(x.B, x.Hq, x.Hkv, x.T, x.S, x.d, x.causal, 2)
            tf = fl / (ms * 1e-3) / 1e12
            other[name] = {"config": f"B={x.B}, Hq={x.Hq}, Hkv={x.Hkv}, T=S={x.T}, d={x.d}, bf16, causal",
                           "ms": ms, "value": tf, "unit": "TFLOP/s", "frac_of_mfma_peak": tf / peak_p,
                           "launches": len(times)}
            del xq, xk, xv, xo, xl
        out["prefill_other"] = other
    if not args.no_next:
        nb = None if args.no_cpu_baseline else args.cpu_budget / 5
        out["window"] = bench_window(tea, workloads, dev, stream, flush, nb)
        out["chunked"] = bench_chunked(tea, workloads, dev, stream, flush, nb)
        out["decode_fp8"] = bench_decode_fp8(tea, workloads, dev, stream, flush, nb)
    if not args.no_backward:
        out["backward"] = bench_backward(tea, workloads, dev, stream, flush,
                                         None if args.no_cpu_baseline else args.cpu_budget / 3)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pinp, dinp, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
