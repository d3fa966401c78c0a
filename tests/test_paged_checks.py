"""check_paged_inputs: the host-side check of what the paged entry points take
on trust (page ids of the used blocks, lengths, chunk lengths).  CPU only."""
import numpy as np
import pytest

import workloads

tea = pytest.importorskip("tiled_exact_attention_flashattention_amd")


def _decode_inputs():
    inp = workloads.make_decode(4, 4, 2, 64, 1, 70, seed=5, lens=[1, 16, 17, 70], name="chk")
    return inp.block_table.copy(), inp.seq_lens.copy(), inp.num_pages


def test_valid_tables_pass():
    bt, sl, P = _decode_inputs()
    tea.check_paged_inputs(bt, sl, P)
    # entries past each sequence's last block are never read: anything goes
    bt[0, 1:] = -7
    tea.check_paged_inputs(bt, sl, P)
    # a zero length uses no block at all
    sl[1] = 0
    bt[1, :] = 10 ** 6
    tea.check_paged_inputs(bt, sl, P)


@pytest.mark.parametrize("bad", [-1, "num_pages"])
def test_used_page_id_out_of_range_is_named(bad):
    bt, sl, P = _decode_inputs()
    bt[3, 4] = P if bad == "num_pages" else bad      # block 4 of a 70-token sequence is used
    with pytest.raises(ValueError, match="sequence 3: block 4"):
        tea.check_paged_inputs(bt, sl, P)


def test_length_beyond_the_table_is_named():
    bt, sl, P = _decode_inputs()
    sl[2] = bt.shape[1] * 16 + 1
    with pytest.raises(ValueError, match="sequence 2: seq_len"):
        tea.check_paged_inputs(bt, sl, P)
    sl[2] = -1
    with pytest.raises(ValueError, match="sequence 2: seq_len"):
        tea.check_paged_inputs(bt, sl, P)


def test_chunk_lengths():
    inp = workloads.make_prefill_paged(3, 2, 1, 40, 64, 10, 90, seed=9, name="chk_pp")
    tea.check_paged_inputs(inp.block_table, inp.seq_lens, inp.num_pages, q_lens=inp.q_lens,
                           T=inp.T)
    ql = inp.q_lens.copy()
    ql[1] = int(inp.seq_lens[1]) + 1                  # more new tokens than the sequence holds
    with pytest.raises(ValueError, match="sequence 1: q_len"):
        tea.check_paged_inputs(inp.block_table, inp.seq_lens, inp.num_pages, q_lens=ql)
    ql = inp.q_lens.copy()
    ql[0] = inp.T + 1                                  # more than the rows of q
    with pytest.raises(ValueError, match="sequence 0: q_len"):
        tea.check_paged_inputs(inp.block_table, inp.seq_lens, inp.num_pages, q_lens=ql, T=inp.T)


def test_shapes_are_checked():
    bt, sl, P = _decode_inputs()
    with pytest.raises(ValueError):
        tea.check_paged_inputs(bt[0], sl, P)
    with pytest.raises(ValueError):
        tea.check_paged_inputs(bt, sl[:2], P)
    torch = pytest.importorskip("torch")
    tea.check_paged_inputs(torch.from_numpy(bt), torch.from_numpy(sl), P)
