"""pa_decode_noalloc: the allocation-free entry point (partial states in the
library's static per-GPU scratch) against pa_decode_ex with a caller-owned
workspace, through the C ABI, on two calls in a row (the second smaller),
and against the float64 oracle at the bf16 bars; plans needing more than the
scratch are refused before any launch."""

import ctypes
from dataclasses import replace

import pytest
import torch

import decode_attention_pa_amd as pa
import workloads
from tests._gpu_util import BF16_TOL, F32_TOL, compare, oracle_out, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def noalloc(case, **opts):
    out = case.new_out().fill_(float("nan"))
    if case.k_scale is not None:
        opts.setdefault("k_scale", case.k_scale)
        opts.setdefault("v_scale", case.v_scale)
    pa.decode_noalloc(out, case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                      case.query_lens, case.scale, case.window, case.w.num_kv_heads,
                      case.w.block_size, max_seq_len=case.w.max_seq_len,
                      max_query_len=case.w.query_len, **opts)
    torch.cuda.synchronize()
    return out


# (workload overrides, window, plan options): the persistent and the grid
# schedule with split partitions, FP8, and a one-shot plan (no scratch use)
CASES = [
    (dict(name="gqa_bf16", batch=12), 0, {}),
    (dict(name="gqa_bf16", batch=12), 0, dict(schedule=pa.SCHED_GRID, part_size=256)),
    (dict(name="long_splitk_bf16"), 0, {}),
    (dict(name="gqa_fp8kv", batch=9), 0, {}),
    (dict(name="swa_mtp_bf16", batch=16), 128, {}),
    (dict(name="gqa_f32", batch=12), 0, {}),          # the vector kernels' persistent plan
]


def _case(over, window, shrink=False):
    w = workloads.WORKLOADS[over["name"]]
    w = replace(w, **{k: v for k, v in over.items() if k != "name"})
    if shrink:   # a smaller call: fewer sequences, or a shorter context
        if w.batch > 1:
            w = replace(w, batch=max(1, w.batch // 3), seed=w.seed + 100)
        else:
            w = replace(w, seq_lens=(w.seq_lens[0] // 5,), seed=w.seed + 100)
    return workloads.make_case(w, device="cuda", window=window)


@pytest.mark.parametrize("over,window,opts", CASES)
def test_noalloc_matches_workspace_entry_point(over, window, opts):
    for step, shrink in enumerate((False, True)):
        c = _case(over, window, shrink)
        say(f"[case] noalloc {over} window={window} opts={opts} call {step} "
            f"batch={c.w.batch} lens={c.seq_lens_host[:4]}")
        got = noalloc(c, **opts)
        expect = run_gpu(c, **opts)
        assert torch.equal(got, expect), (over, opts, step)
        seqs = list(range(min(c.w.batch, 6)))
        exp, rows = oracle_out(c, seqs)
        compare(got, exp, rows, F32_TOL if c.w.dtype == "f32" else BF16_TOL,
                f"noalloc {over['name']} call {step}")


def test_noalloc_refuses_plans_beyond_the_scratch():
    """A grid plan with 32-position partitions over a long batch needs far
    more than the scratch: refused with PA_ERR_WORKSPACE, nothing launched."""
    lib = pa.load()
    size = pa.noalloc_scratch_bytes()
    assert size == 64 << 20
    d = pa.make_dims(128, 64, 128, 2, 65536, 64, 6000, pa.BF16)
    need = pa.workspace_size(d, 0, 8, 1024, schedule=pa.SCHED_GRID, part_size=32)
    assert need > size
    o = pa.make_options(schedule=pa.SCHED_GRID, part_size=32)
    P = ctypes.c_void_p
    st = lib.pa_decode_noalloc(*([P(4096)] * 7), ctypes.c_float(0.1), 0, 8, 1024,
                               ctypes.byref(d), None, ctypes.byref(o))
    assert st == pa.ERR_WORKSPACE, st
    assert b"static scratch" in lib.pa_last_error()
