"""The device-side precondition check (pa_check_inputs): clean inputs report
nothing; each kind of violation is counted and located; table entries that
hold no visible position are never counted (they may hold anything).  Bad
inputs are only ever given to the check, never to pa_decode."""

import pytest
import torch

import decode_attention_pa_amd as pa
import workloads
from tests.test_gpu_parity import small

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def report(c, window, seq_lens=None, query_lens=None, tables=None):
    w = c.w
    dims = pa.dims_for(c.q, c.k_cache, c.block_tables, max(w.query_len, 1), w.max_seq_len)
    return pa.check_inputs(c.block_tables if tables is None else tables,
                           c.seq_lens if seq_lens is None else seq_lens,
                           c.query_lens if query_lens is None else query_lens,
                           window, w.num_kv_heads, w.block_size, dims)


CLEAN = {"bad_lengths": 0, "bad_entries": 0, "first_bad_sequence": None, "first_bad_entry": None}


@pytest.mark.parametrize("name,window", [("gqa_bf16", 0), ("swa_mtp_bf16", 128),
                                         ("large_block_mtp_bf16", 4096), ("tiny_f32", 5)])
def test_clean_workloads_report_nothing(name, window):
    c = workloads.make_case(name, device="cuda", window=window)
    assert report(c, window) == CLEAN


def test_length_violations_are_counted():
    w = small(21, batch=4, seq_lens=(90, 60, 40, 70), query_lens=(2, 1, 2, 1), query_len=2,
              block_size=16, max_seq_len=90, max_blocks_per_seq=7)
    c = workloads.make_case(w, device="cuda", window=0)
    assert report(c, 0) == CLEAN
    cases = [((90, 60, 40, 70), (2, 1, 41, 1), 2),    # q_b > L_b
             ((90, 91, 40, 70), (2, 1, 2, 1), 1),     # L_b > max_seq_len
             ((90, 60, 40, 70), (2, 1, 2, 3), 3),     # q_b > max_query_len
             ((-1, 60, 40, 70), (2, 1, 2, 1), 0),     # L_b < 0
             ((90, 60, 40, 70), (2, -1, 2, 1), 1)]    # q_b < 0
    for lens, qls, first in cases:
        r = report(c, 0, seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"),
                   query_lens=torch.tensor(qls, dtype=torch.int32, device="cuda"))
        assert (r["bad_lengths"], r["first_bad_sequence"], r["bad_entries"]) == (1, first, 0), (lens, qls)


def test_table_entries_of_visible_blocks_are_checked():
    w = small(22, batch=3, seq_lens=(200, 75, 33), query_lens=(1, 2, 1), query_len=2,
              block_size=16, max_seq_len=200, max_blocks_per_seq=14)
    c = workloads.make_case(w, device="cuda", window=40)
    M = w.max_blocks_per_seq
    nb = c.num_blocks
    assert report(c, 40) == CLEAN
    # sequence 0: L = 200, window 40 -> visible 161..199 -> logical blocks 10..12
    for bad in (-1, nb, nb + 1000):
        t = c.block_tables.clone()
        t[0, 11] = bad
        r = report(c, 40, tables=t)
        assert (r["bad_entries"], r["first_bad_entry"], r["bad_lengths"]) == (1, 11, 0), bad
    # entries that hold no visible position may hold anything
    t = c.block_tables.clone()
    t[0, 3] = -5          # before the window
    t[0, 13] = nb + 7     # past the last block of sequence 0
    t[2, 3:] = -1         # sequence 2 has 33 positions: blocks 0..2 only
    assert report(c, 40, tables=t) == CLEAN
    assert report(c, 0, tables=t)["bad_entries"] == 1          # without a window block 3 of seq 0 is seen
    # two bad entries in two sequences: both counted, the first located
    t = c.block_tables.clone()
    t[1, 4] = -2
    t[2, 1] = nb
    r = report(c, 40, tables=t)
    assert (r["bad_entries"], r["first_bad_entry"]) == (2, 1 * M + 4)
    # a sequence with bad lengths is not scanned
    lens = torch.tensor((200, 75, 9999), dtype=torch.int32, device="cuda")
    r = report(c, 40, seq_lens=lens, tables=t)
    assert (r["bad_lengths"], r["first_bad_sequence"], r["bad_entries"]) == (1, 2, 1)
