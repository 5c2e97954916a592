"""bench.py's accounting, on the CPU.

The roofline figure divides the partition kernel's algorithmic bytes by its
duration; here those bytes are checked against a count made position by
position from the oracle's visibility rule (K and V of every position some
row of a (sequence, KV head) sees, the table entries of the blocks holding
them, Q and the two length arrays).  Also: more than one GPU is refused
before anything touches a device.
"""

import os
import subprocess
import sys

import pytest

import bench
import workloads
from oracle import paged_attention as ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def counted_bytes(case):
    w = case.w
    s = 2 if w.dtype == "bf16" else 4
    skv = 1 if w.kv_dtype == "fp8" else s
    sq = 1 if w.q_dtype == "fp8" else s
    kv = tables = 0
    for L, q in zip(case.seq_lens_host, case.query_lens_host):
        seen = set()
        for i in range(q):
            lo, p = ref.visible_range(L, q, i, case.window)
            seen.update(range(lo, p + 1))
        kv += len(seen) * w.num_kv_heads * w.head_dim * 2 * skv
        tables += 4 * len({t // w.block_size for t in seen})
    T = sum(case.query_lens_host)
    return dict(kv=kv, tables=tables, q=T * w.num_q_heads * w.head_dim * sq,
                out=T * w.num_q_heads * w.head_dim * s, lens=8 * w.batch)


def _cases():
    yield workloads.make_case("tiny_f32", device="cpu", window=0)
    yield workloads.make_case("tiny_f32", device="cpu", window=5)
    mtp = workloads.custom(name="mtp", dtype="bf16", batch=5, num_q_heads=8, num_kv_heads=2,
                           head_dim=64, block_size=16, query_len=4,
                           seq_lens=(1, 17, 40, 300, 301), query_lens=(1, 4, 0, 3, 4),
                           max_seq_len=301, max_blocks_per_seq=20, pool=0, seed=7,
                           scale=0.125, windows=(0,))
    for win in (0, 1, 2, 16, 33, 1000):
        yield workloads.make_case(mtp, device="cpu", window=win)
    fp8 = workloads.custom(name="fp8", dtype="bf16", kv_dtype="fp8", q_dtype="fp8", batch=3,
                           num_q_heads=4, num_kv_heads=1, head_dim=128, block_size=32,
                           query_len=2, seq_lens=(70, 5, 129), max_seq_len=129,
                           max_blocks_per_seq=6, pool=0, seed=8, scale=0.08, windows=(0,))
    for win in (0, 7):
        yield workloads.make_case(fp8, device="cpu", window=win)


@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: f"{c.w.name}-w{c.window}")
def test_algorithmic_bytes_match_a_position_count(case):
    got = bench.algorithmic_bytes(case)
    exp = counted_bytes(case)
    for k, v in exp.items():
        assert got[k] == v, (k, got[k], v)
    assert got["partition_kernel"] == exp["kv"] + exp["q"] + exp["tables"] + exp["lens"]
    assert got["total"] == got["partition_kernel"] + exp["out"]
    # a one-shot plan's partition kernel writes the output itself
    whole = bench.algorithmic_bytes(case, one_shot=True)
    assert whole["partition_kernel"] == whole["total"] == got["total"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_scaling_uses_the_calibration_copies():
    """Traffic per launch: the counter scaled by what it reads for the 1 GiB
    calibration copies issued just before the first partition kernel (input
    staging copies of other sizes, earlier, are ignored), averaged over the
    partition dispatches after the cold first one."""
    gib = float(1 << 20)                                     # KiB
    rows = [(0, "copyBuffer", 3 * gib),                      # staging, earlier: ignored
            (1, "copyBuffer", 0.25 * gib),                   # staging: ignored
            (2, "fill", 7.0),
            (3, "copyBuffer", 0.5 * gib), (4, "copyBuffer", 0.5 * gib),
            (5, "copyBuffer", 0.5 * gib),                    # calibration: reads half
            (6, "pa::part_mfma_ps<...>", 999.0),             # cold first dispatch
            (7, "pa::lse_reduce<...>", 5.0),
            (8, "pa::part_mfma_ps<...>", 100.0),
            (9, "pa::part_mfma_ps<...>", 300.0),
            (10, "copyBuffer", 8 * gib)]                     # after: ignored
    rec = bench.counter_bytes(list(reversed(rows)), "FETCH_SIZE")
    assert rec["scale"] == 2.0
    assert rec["copy_kib"] == 0.5 * gib
    assert rec["partition_kib_raw"] == 200.0
    assert rec["partition_bytes"] == 200 * 2 * 1024
    assert rec["dispatches"] == 3
    with pytest.raises(SystemExit):
        bench.counter_bytes([(0, "pa::part_mfma<...>", 1.0)], "WRITE_SIZE")   # no copy


def test_parity_sample_keeps_extremes():
    """The sampled full-size parity cases always compare the longest and the
    shortest sequence besides the seeded draw, and never fewer than asked."""
    import numpy as np
    from tests._gpu_util import sample_sequences
    import workloads
    for name in ("large_block_mtp_bf16", "gqa_bf16", "swa_mtp_bf16"):
        w = workloads.WORKLOADS[name]
        g = __import__("torch").Generator().manual_seed(w.seed)
        lens, _ = workloads._lengths(w, g)
        for n, seed in ((2, 5), (10, 5), (10, 6), (24, 5)):
            s = sample_sequences(lens, n, seed)
            assert int(np.argmax(lens)) in s and int(np.argmin(lens)) in s
            assert len(s) >= min(n, len(lens)) and s == sorted(set(s))
    assert sample_sequences([5, 6, 7], None, 0) == [0, 1, 2]


def test_side_figures_that_fail_are_recorded_not_lost(capsys):
    # a failing figure beside the headline is reported in the line and on
    # stderr; a working one passes through unchanged
    got = bench.guarded("side line x", lambda: 1 // 0)
    assert got == {"error": "ZeroDivisionError: integer division or modulo by zero"}
    assert "side line x failed" in capsys.readouterr().err
    assert bench.guarded("y", lambda: {"value": 1}) == {"value": 1}
