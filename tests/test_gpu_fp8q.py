"""GPU parity of FP8 (OCP E4M3) queries over an FP8 KV cache against the
float64 oracle.

The oracle dequantizes the query codes with its own E4M3 decoder and the
query scale, exactly as it does the caches (aiter PR #2914, review of
pa_decode_gluon: an FP8 query comes with its query_scale, and a call
without it must be refused).  QK^T runs on the FP8 matrix cores (E4M3 x E4M3
products are exact in fp32), PV in bf16.  Bar: max-abs 2e-2.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import decode_attention_pa_amd as pa
import workloads
from tests._gpu_util import BF16_TOL, compare, oracle_out, run_gpu, say
from tests.test_gpu_general import many_rows
from tests.test_gpu_parity import small

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def fp8q(w):
    return replace(w, kv_dtype="fp8", q_dtype="fp8", name=w.name + "_fp8q")


@pytest.mark.parametrize("sched", [pa.SCHED_GRID, pa.SCHED_PERSISTENT], ids=["grid", "ps"])
@pytest.mark.parametrize("seed", range(6))
def test_fp8q_small(seed, sched):
    w = fp8q(small(100 + seed))
    for win in (0, 1, 5, 37, 100000):
        c = workloads.make_case(w, device="cuda", window=win)
        say(f"[case] fp8q small seed={100 + seed} schedule={sched} window={win} {w}")
        exp, rows = oracle_out(c)
        for P in (0, 32, 64):
            compare(run_gpu(c, part_size=P, schedule=sched), exp, rows, BF16_TOL,
                    f"fp8q small{100 + seed} sched={sched} w={win} P={P}")


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_fp8q_negative_and_zero_scale(scale):
    """A negative logit scale goes into the FP8 query codes' sign bits; a
    zero one weighs every visible position the same."""
    w = fp8q(small(105, scale=scale))
    for win in (0, 5):
        c = workloads.make_case(w, device="cuda", window=win)
        say(f"[case] fp8q scale={scale} window={win}")
        exp, rows = oracle_out(c)
        for P in (0, 32):
            compare(run_gpu(c, part_size=P), exp, rows, BF16_TOL, f"fp8q scale={scale} w={win} P={P}")


@pytest.mark.parametrize("seed", range(2))
def test_fp8q_head_dim_256(seed):
    w = fp8q(small(200 + seed, head_dim=256))
    for win in (0, 9):
        c = workloads.make_case(w, device="cuda", window=win)
        exp, rows = oracle_out(c)
        for P in (0, 32):
            say(f"[case] fp8q D=256 seed={200 + seed} window={win} P={P}")
            compare(run_gpu(c, part_size=P), exp, rows, BF16_TOL, f"fp8q d256 w={win} P={P}")


def test_fp8q_more_than_64_rows():
    w = fp8q(many_rows(1, 128, "bf16", "fp8"))
    for win in (0, 300):
        c = workloads.make_case(w, device="cuda", window=win)
        exp, rows = oracle_out(c)
        for P in (0, 64):
            say(f"[case] fp8q rows w={win} P={P}")
            compare(run_gpu(c, part_size=P), exp, rows, BF16_TOL, f"fp8q rows w={win} P={P}")


FP8Q_FULL = [("gqa_fp8qkv", 0, None), ("swa_mtp_bf16", 128, 16), ("long_splitk_bf16", 0, None)]


@pytest.mark.parametrize("name,window,nsample", FP8Q_FULL)
def test_fp8q_full_workload(name, window, nsample):
    w = workloads.WORKLOADS[name]
    if w.q_dtype != "fp8":
        w = fp8q(w)
    say(f"[case] fp8q full {w.name} window={window}")
    c = workloads.make_case(w, device="cuda", window=window)
    out = run_gpu(c)
    seqs = list(range(w.batch))
    if nsample is not None:
        seqs = sorted(np.random.default_rng(w.seed).choice(w.batch, size=nsample, replace=False).tolist())
    exp, rows = oracle_out(c, seqs)
    compare(out, exp, rows, BF16_TOL, f"fp8q {w.name} w={window}")
    assert torch.isfinite(out.float()).all()


def test_fp8q_scales_enter_as_a_product():
    """Moving a factor of 2 from q_scale to k_scale leaves every output bit
    unchanged (both only scale the logits, and powers of two multiply
    exactly); a different q_scale changes the output."""
    w = fp8q(small(7))
    c = workloads.make_case(w, device="cuda", window=0)
    base = run_gpu(c).clone()
    moved = run_gpu(c, q_scale=c.q_scale * 2, k_scale=c.k_scale / 2).clone()
    assert torch.equal(moved, base)
    other = run_gpu(c, q_scale=c.q_scale * 1.5)
    assert not torch.equal(other, base)


def test_fp8q_without_scale_is_refused():
    w = fp8q(small(8))
    c = workloads.make_case(w, device="cuda", window=0)
    out = c.new_out().fill_(7.0)
    with pytest.raises(pa.PaError) as e:
        pa.decode(out, c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.query_lens,
                  c.scale, 0, w.num_kv_heads, w.block_size, max_seq_len=w.max_seq_len,
                  max_query_len=w.query_len, k_scale=c.k_scale, v_scale=c.v_scale)
    assert e.value.status == pa.ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)          # nothing was launched


def test_fp8q_nan_codes_in_invisible_blocks_change_nothing():
    w = fp8q(small(9, seq_lens=(150, 77, 33), batch=3, query_len=2, block_size=16,
                   max_seq_len=150, max_blocks_per_seq=11))
    for win in (0, 5):
        for sched in (pa.SCHED_GRID, pa.SCHED_PERSISTENT):
            clean = run_gpu(workloads.make_case(w, device="cuda", window=win, poison=False),
                            schedule=sched).clone()
            dirty = run_gpu(workloads.make_case(w, device="cuda", window=win, poison=True),
                            schedule=sched)
            assert torch.equal(clean, dirty), (win, sched)
