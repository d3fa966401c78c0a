"""The algorithmic work bench.py divides by, checked against explicit counts.

The benchmark reports throughput as algorithmic FLOPs (4 d per visible
(query, key) pair: the two products of each pair, 2 d each) or bytes per
second.  Its closed forms for the number of visible pairs (causal with the
bottom-right alignment, sliding window, chunked prefill on a paged cache) are
compared here with the pairs the float64 oracle's own visibility mask lets
through, and the decode byte count with a sum over the sequences' pages.
"""
import numpy as np
import pytest

import bench
import oracle
import workloads


@pytest.mark.parametrize("T,S,causal,window", [
    (1, 1, True, 0), (17, 17, True, 0), (100, 333, True, 0), (333, 100, False, 0),
    (256, 256, False, 0), (300, 300, True, 37), (512, 512, True, 128), (100, 333, True, 64),
    (200, 450, True, 300), (130, 130, True, 1), (64, 64, True, 1000),
])
def test_prefill_pairs_match_the_oracle_mask(T, S, causal, window):
    flops, nbytes = bench.prefill_work(2, 6, 3, T, S, 64, causal, 2, window=window)
    visible = int(oracle.visible_mask(np.arange(T), S, T, causal, window).sum())
    assert flops == 4 * 64 * visible * 2 * 6
    # Q and O of every query head, K and V of every KV head (bf16), LSE fp32
    assert nbytes == (2 * 2 * 6 * T * 64 + 2 * 2 * 3 * S * 64) * 2 + 2 * 6 * T * 4


def test_headline_workload_pair_counts():
    # causal T = S: T (T + 1) / 2 pairs per (batch, head)
    flops, _ = bench.prefill_work(8, 12, 12, 1024, 1024, 64, True, 2)
    assert flops == 12_897_484_800
    flops, _ = bench.prefill_work(1, 32, 32, 16384, 16384, 128, True, 2)
    assert flops == 2_199_157_473_280


def test_chunked_pairs_match_the_oracle_mask():
    rng = np.random.default_rng(3)
    q_lens = rng.integers(1, 40, 12)
    seq_lens = q_lens + rng.integers(0, 90, 12)
    explicit = sum(int(oracle.visible_mask(np.arange(t), int(L), int(t), True).sum())
                   for L, t in zip(seq_lens, q_lens))
    assert bench.chunked_pairs(seq_lens, q_lens) == explicit


def test_decode_bytes_and_flops_by_explicit_sum():
    inp = workloads.make_decode(9, 12, 2, 128, 1, 700, seed=4, name="work")
    flops, nbytes, tokens = bench.decode_work(inp)
    L = [int(x) for x in inp.seq_lens]
    kv = sum(2 * l * inp.Hkv * inp.d * 2 for l in L)          # K and V, bf16, every KV head
    table = sum(4 * -(-l // inp.page) for l in L)             # the used block-table entries
    qo = 2 * inp.N * inp.Hq * inp.d * 2                        # q in, o out (bf16)
    assert tokens == sum(L)
    assert nbytes == kv + table + qo + inp.N * inp.Hq * 4 + inp.N * 4
    assert flops == sum(4 * inp.d * l * inp.Hq for l in L)


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU's share; asked for more it says so and exits non-zero."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
