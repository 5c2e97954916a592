"""GPU parity of the FP8 (OCP E4M3) KV cache path against the float64 oracle.

The oracle dequantizes the same codes with its own E4M3 decoder and the same
per-tensor scales (aiter PR #2914, review of pa_decode_gluon: FP8 key / value
caches come with key_scale / value_scale, and a call without them must be
refused).  Bar: max-abs 2e-2 (bf16 queries and output, fp32 accumulation).
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import decode_attention_pa_amd as pa
import workloads
from tests._gpu_util import BF16_TOL, compare, oracle_out, run_gpu, say
from tests.test_gpu_parity import small

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def fp8_small(seed, **over):
    w = small(seed, kv_dtype="fp8", **over)
    return w


@pytest.mark.parametrize("sched", [pa.SCHED_GRID, pa.SCHED_PERSISTENT], ids=["grid", "ps"])
@pytest.mark.parametrize("seed", range(8))
def test_fp8_small(seed, sched):
    w = fp8_small(seed)
    for win in (0, 1, 5, 37, 100000):
        c = workloads.make_case(w, device="cuda", window=win)
        say(f"[case] fp8 small seed={seed} schedule={sched} window={win} {w}")
        exp, rows = oracle_out(c)
        for P in (0, 32, 64):
            compare(run_gpu(c, part_size=P, schedule=sched), exp, rows, BF16_TOL,
                    f"fp8 small{seed} sched={sched} w={win} P={P}")


FP8_FULL = [("gqa_fp8kv", 0, None), ("swa_mtp_bf16", 128, 16), ("long_splitk_bf16", 0, None)]


@pytest.mark.parametrize("name,window,nsample", FP8_FULL)
def test_fp8_full_workload(name, window, nsample):
    w = workloads.WORKLOADS[name]
    if w.kv_dtype != "fp8":
        w = replace(w, kv_dtype="fp8", name=name + "_fp8")
    say(f"[case] fp8 full {w.name} window={window}")
    c = workloads.make_case(w, device="cuda", window=window)
    out = run_gpu(c)
    seqs = list(range(w.batch))
    if nsample is not None:
        seqs = sorted(np.random.default_rng(w.seed).choice(w.batch, size=nsample, replace=False).tolist())
    exp, rows = oracle_out(c, seqs)
    compare(out, exp, rows, BF16_TOL, f"fp8 {w.name} w={window}")
    assert torch.isfinite(out.float()).all()


def test_fp8_nan_codes_in_invisible_blocks_change_nothing():
    """Invisible blocks and tail slots hold the E4M3 NaN code: the output is
    bit-identical to a run over a clean cache."""
    w = fp8_small(3, seq_lens=(150, 77, 33), batch=3, query_len=2, block_size=16,
                  max_seq_len=150, max_blocks_per_seq=11)
    for win in (0, 5, 40):
        for sched in (pa.SCHED_GRID, pa.SCHED_PERSISTENT):
            for P in (0, 32):
                clean = run_gpu(workloads.make_case(w, device="cuda", window=win, poison=False),
                                part_size=P, schedule=sched).clone()
                dirty = run_gpu(workloads.make_case(w, device="cuda", window=win, poison=True),
                                part_size=P, schedule=sched)
                assert torch.equal(clean, dirty), (win, sched, P)


def test_fp8_value_scale_is_applied_once():
    """Doubling v_scale doubles every output bit-exactly (a power-of-two
    factor on the fp32 normalisation); changing k_scale changes the output."""
    w = fp8_small(5)
    c = workloads.make_case(w, device="cuda", window=0)
    base = run_gpu(c).clone()
    two = run_gpu(c, v_scale=c.v_scale * 2).clone()
    assert torch.equal(two, base * 2)
    other = run_gpu(c, k_scale=c.k_scale * 1.5)
    assert not torch.equal(other, base)


def test_fp8_without_scales_is_refused():
    w = fp8_small(2)
    c = workloads.make_case(w, device="cuda", window=0)
    out = c.new_out().fill_(7.0)
    for ks, vs in ((None, None), (c.k_scale, None), (None, c.v_scale)):
        with pytest.raises(pa.PaError) as e:
            pa.decode(out, c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.query_lens,
                      c.scale, 0, w.num_kv_heads, w.block_size, max_seq_len=w.max_seq_len,
                      max_query_len=w.query_len, k_scale=ks, v_scale=vs)
        assert e.value.status == pa.ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)          # nothing was launched


def test_fp8_load_forms_agree_bit_for_bit():
    w = workloads.WORKLOADS["gqa_fp8kv"]
    c = workloads.make_case(w, device="cuda")
    a = run_gpu(c, loads=pa.LOADS_CACHED).clone()
    assert torch.equal(run_gpu(c, loads=pa.LOADS_STREAMING), a)
    say("[fp8] cached and non-temporal outputs identical")
