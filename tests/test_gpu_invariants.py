"""GPU invariants that hold bit for bit, independent of tolerances.

* window 1: each query token returns its own value vector exactly;
* constant V returns the constant exactly;
* spike probe: a key aligned with one query row and a logit gap of ~400
  makes every other weight underflow to exactly 0, so the output equals that
  position's value vector iff the position is visible, and is bit-identical
  to the spike-free run iff it is not - checked at window edges, MTP
  neighbours, block and chunk edges, across forced partition sizes;
* NaN poison in every block no row can see (including blocks before the
  window) leaves the output bit-identical;
* a different physical placement of the same logical blocks, and a second
  run, give bit-identical outputs;
* query heads of one group with identical query vectors give identical
  outputs; one partition versus many agree within 2 bf16 ulps of each
  output row's largest magnitude;
* a window at least as long as the context equals window 0, and a GQA call
  equals an MHA call over repeated KV heads, bit for bit; an MTP row equals
  the one-token call whose context ends at that row.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import decode_attention_pa_amd as pa
import workloads
from oracle import paged_attention as ref
from tests._gpu_util import BF16_TOL, compare, oracle_out, run_gpu, say

pytestmark = pytest.mark.gpu

PATHS = [pa.PATH_MFMA, pa.PATH_VALU, pa.PATH_VALU_LDS]
KERNELS = [(pa.PATH_MFMA, pa.SCHED_GRID), (pa.PATH_MFMA, pa.SCHED_PERSISTENT),
           (pa.PATH_VALU, pa.SCHED_GRID), (pa.PATH_VALU, pa.SCHED_PERSISTENT),
           (pa.PATH_VALU_LDS, pa.SCHED_GRID)]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def mtp_workload(**over):
    kw = dict(name="inv", dtype="bf16", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=128,
              block_size=16, query_len=3, seq_lens=(150, 77), max_seq_len=150,
              max_blocks_per_seq=11, pool=0, seed=77, scale=1.0 / np.sqrt(128.0), windows=(0,))
    kw.update(over)
    return workloads.custom(**kw)


def v_at(case, blk, h, slot):
    return case.v_cache[blk, h, slot // 8, :, slot % 8]


@pytest.mark.parametrize("path", PATHS)
def test_window_one_returns_own_value(path):
    w = mtp_workload()
    c = workloads.make_case(w, device="cuda", window=1)
    for P in (0, 32, 64):
        out = run_gpu(c, path=path, part_size=P)
        row = 0
        for b, (L, q) in enumerate(zip(c.seq_lens_host, c.query_lens_host)):
            for i in range(q):
                p = L - q + i
                blk = c.used_blocks[b][p // w.block_size]
                for hq in range(w.num_q_heads):
                    h = hq // (w.num_q_heads // w.num_kv_heads)
                    assert torch.equal(out[row, hq], v_at(c, blk, h, p % w.block_size)), (path, P, b, i, hq)
                row += 1


@pytest.mark.parametrize("path", PATHS)
def test_constant_values_return_constant(path):
    w = mtp_workload()
    for win in (0, 5, 40):
        c = workloads.make_case(w, device="cuda", window=win)
        c.v_cache.fill_(-0.3125)
        for P in (0, 32, 96):
            out = run_gpu(c, path=path, part_size=P)
            assert torch.all(out == -0.3125), (path, win, P)


def _spike_positions(L, q, i, window, bs):
    p = L - q + i
    lo = 0 if window == 0 else max(0, p + 1 - window)
    cand = {p, p - 1, lo, lo - 1, lo + 1, p + 1, p + 2, 0,
            (p // bs) * bs, (p // bs) * bs - 1, (p // 32) * 32, (p // 32) * 32 - 1,
            (lo // bs) * bs, (lo // 32) * 32 + 31}
    return sorted(t for t in cand if 0 <= t < L)


@pytest.mark.parametrize("path,sched", KERNELS)
@pytest.mark.parametrize("window", [0, 5, 40])
def test_spike_probe_visibility(path, sched, window):
    w = mtp_workload(num_q_heads=2, num_kv_heads=2)   # G = 1: one query row per key head
    base = workloads.make_case(w, device="cuda", window=window, poison=False)
    bs = w.block_size
    for P in (0, 32, 64):
        clean = run_gpu(base, path=path, part_size=P, schedule=sched).clone()
        row0 = 0
        for b, (L, q) in enumerate(zip(base.seq_lens_host, base.query_lens_host)):
            for i in range(q):
                row = row0 + i
                lo_i, p_i = ref.visible_range(L, q, i, window)
                for t in _spike_positions(L, q, i, window, bs):
                    c = workloads.make_case(w, device="cuda", window=window, poison=False)
                    blk = c.used_blocks[b][t // bs]
                    h = 0
                    qv = c.q[row, h].float()
                    alpha = 400.0 / (w.scale * float(qv.dot(qv)))
                    workloads.write_k_row(c.k_cache, blk, h, t % bs,
                                          (alpha * qv).to(torch.bfloat16))
                    out = run_gpu(c, path=path, part_size=P, schedule=sched)
                    if lo_i <= t <= p_i:
                        expect = v_at(c, blk, h, t % bs)
                        assert torch.equal(out[row, h], expect), (path, window, P, b, i, t)
                    else:
                        assert torch.equal(out[row, h], clean[row, h]), (path, window, P, b, i, t)
            row0 += q
    say(f"[spike] path={path} window={window}: all probes bit-exact")


@pytest.mark.parametrize("path,sched", KERNELS)
def test_nan_poison_of_invisible_blocks(path, sched):
    for win in (0, 5, 40):
        w = mtp_workload(seq_lens=(150, 77, 33), batch=3, query_len=2)
        c = workloads.make_case(w, device="cuda", window=win, poison=True)
        for P in (0, 32):
            clean = run_gpu(c, path=path, part_size=P, schedule=sched).clone()
            sp = ref.spans(c.tables_host.numpy(), c.seq_lens_host, c.query_lens_host, win,
                           w.block_size)
            visible = set(int(x) for s in sp for x in s["blocks"] if x >= 0)
            dead = [x for x in range(c.num_blocks) if x not in visible]
            ids = torch.tensor(dead, dtype=torch.long, device="cuda")
            c.k_cache.index_fill_(0, ids, float("nan"))
            c.v_cache.index_fill_(0, ids, float("nan"))
            out = run_gpu(c, path=path, part_size=P, schedule=sched)
            assert torch.equal(out, clean), (path, sched, win, P)
            c = workloads.make_case(w, device="cuda", window=win, poison=True)


def test_block_placement_and_rerun_are_bit_identical():
    w = workloads.WORKLOADS["gqa_bf16"]
    c = workloads.make_case(w, device="cuda")
    a = run_gpu(c).clone()
    b = run_gpu(c)
    assert torch.equal(a, b)
    # move every used block to a new physical slot (reverse order)
    perm = torch.arange(c.num_blocks - 1, -1, -1, device="cuda")
    k2 = torch.empty_like(c.k_cache)
    v2 = torch.empty_like(c.v_cache)
    k2[perm] = c.k_cache
    v2[perm] = c.v_cache
    c.k_cache, c.v_cache = k2, v2
    c.block_tables = perm.to(torch.int32)[c.block_tables.long()]
    assert torch.equal(run_gpu(c), a)


@pytest.mark.parametrize("path", PATHS)
def test_identical_queries_in_a_group_agree(path):
    w = mtp_workload(num_q_heads=8, num_kv_heads=2)
    c = workloads.make_case(w, device="cuda", window=40)
    G = 4
    for g in range(1, G):
        c.q[:, g::G] = c.q[:, 0::G]
    out = run_gpu(c, path=path, part_size=32)
    for g in range(1, G):
        assert torch.equal(out[:, g::G], out[:, 0::G])


def _split_gap(one, many):
    """Largest |one - many| in bf16 ulps of each output row's largest
    magnitude (bf16 keeps 8 significant bits: ulp(x) = 2^(floor(log2 x) - 7))."""
    row_scale = torch.maximum(one.abs(), many.abs()).amax(dim=-1, keepdim=True)
    ulp = torch.exp2(torch.floor(torch.log2(row_scale.clamp_min(1e-30))) - 7)
    return float(((one - many).abs() / ulp).max())


# (workload, window, partition counts besides the plan's own; "max" = 32-position partitions)
SPLITS = [("gqa_bf16", 0, (2, 7, "max")), ("long_splitk_bf16", 0, (2, 7, "max")),
          ("swa_mtp_bf16", 128, (2, 7)), ("large_block_mtp_bf16", 4096, (2, 7)),
          ("gqa_f32", 0, (2, 7, "max"))]


@pytest.mark.parametrize("name,window,counts", SPLITS)
def test_one_partition_equals_many(name, window, counts):
    """One partition per sequence against NP = 2, 7, the most (32-position
    partitions) and the plan's own split, on the grid schedule and the
    automatic one.  Both compute the same function; they differ only in
    summation order and in the reference max each bf16-rounded softmax
    weight was taken against.  Each output is its fp32 value rounded to
    bf16 (half an ulp of its own), and the fp32 values differ by well under
    an ulp at the row's scale, so every gap stays within 2 bf16 ulps of its
    output row's largest magnitude (an element near 0 may differ by many of
    its own ulps: its value is a sum of terms of the row's size).  Measured:
    at most 1.5."""
    w = workloads.WORKLOADS[name]
    c = workloads.make_case(w, device="cuda", window=window)
    span = min(w.max_seq_len, window + w.query_len - 1) if window else w.max_seq_len
    one = run_gpu(c, part_size=((span + 31) // 32 + 1) * 32, schedule=pa.SCHED_GRID).float().clone()
    runs = [("plan", {})]
    for n in counts:
        # n partitions: ceil((span + 31) / n) positions each, in whole chunks
        P = 32 if n == "max" else -(-(-(-(span + 31) // n)) // 32) * 32
        runs.append((f"NP={n} P={P}", dict(part_size=P, schedule=pa.SCHED_GRID)))
    for label, o in runs:
        many = run_gpu(c, **o).float()
        if w.dtype == "f32":
            # fp32 throughout: only the summation order differs
            scale = torch.maximum(one.abs(), many.abs()).amax(dim=-1, keepdim=True)
            worst = float(((one - many).abs() / scale.clamp_min(1e-30)).max())
            say(f"[split] {name} {label}: max gap / row scale {worst:.3e}")
            assert worst <= 1e-5, (name, label, worst)
            continue
        worst = _split_gap(one, many)
        say(f"[split] {name} {label}: max gap {worst:.3f} bf16 ulps of the row scale")
        assert worst <= 2.0, (name, label, worst)


@pytest.mark.parametrize("sched", [pa.SCHED_GRID, pa.SCHED_PERSISTENT])
def test_load_forms_agree_bit_for_bit(sched):
    """Non-temporal and cached KV loads fetch the same bytes into the same
    registers: the outputs must be identical, on small MTP/window shapes and
    on the GQA workload (whose plan picks the non-temporal form itself)."""
    for win in (0, 5, 40):
        w = mtp_workload(seq_lens=(150, 77, 33), batch=3, query_len=2)
        c = workloads.make_case(w, device="cuda", window=win)
        for P in (0, 32):
            a = run_gpu(c, path=pa.PATH_MFMA, part_size=P, schedule=sched,
                        loads=pa.LOADS_CACHED).clone()
            b = run_gpu(c, path=pa.PATH_MFMA, part_size=P, schedule=sched,
                        loads=pa.LOADS_STREAMING)
            assert torch.equal(a, b), (sched, win, P)
    w = workloads.WORKLOADS["gqa_bf16"]
    c = workloads.make_case(w, device="cuda")
    a = run_gpu(c, schedule=sched, loads=pa.LOADS_CACHED).clone()
    assert torch.equal(run_gpu(c, schedule=sched), a)
    say(f"[loads] schedule={sched}: cached and non-temporal outputs identical")


@pytest.mark.parametrize("path,sched", KERNELS)
def test_timing_events_change_nothing(path, sched):
    """Timing events bound to the partition kernel's dispatch leave the
    output bits unchanged, and the interval they carry is positive and lies
    inside an interval recorded around the whole call."""
    w = workloads.WORKLOADS["gqa_bf16"]
    c = workloads.make_case(replace(w, batch=4), device="cuda", window=0)
    say(f"[case] timing events path={path} sched={sched}")
    plain = run_gpu(c, path=path, schedule=sched).clone()
    kb, ke, cb, ce = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    for e in (kb, ke):
        e.record()  # torch creates the HIP event on its first record
    torch.cuda.synchronize()
    cb.record()
    timed = run_gpu(c, path=path, schedule=sched, event_begin=kb, event_end=ke)
    ce.record()
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), timed.view(torch.int16))
    kern = kb.elapsed_time(ke)
    assert 0 < kern <= cb.elapsed_time(ce)
    assert cb.elapsed_time(kb) >= 0 and ke.elapsed_time(ce) >= 0


def test_concurrent_calls_from_threads():
    """Calls are reentrant: four host threads, each with its own stream, output
    and workspace, run the same calls (both schedules, several plans) at the
    same time and get bit-identical outputs to a single-threaded run."""
    import threading
    w = workloads.WORKLOADS["gqa_bf16"]
    c = workloads.make_case(replace(w, batch=6), device="cuda", window=0)
    plans = [dict(schedule=pa.SCHED_PERSISTENT), dict(schedule=pa.SCHED_GRID, part_size=256),
             dict(schedule=pa.SCHED_PERSISTENT, part_size=128), dict(path=pa.PATH_VALU)]
    ref_out = [run_gpu(c, **o).clone() for o in plans]
    results, errors = [None] * len(plans), []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                out = c.new_out()
                for _ in range(5):
                    pa.decode(out, c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                              c.query_lens, c.scale, 0, w.num_kv_heads, w.block_size,
                              max_seq_len=w.max_seq_len, max_query_len=1, stream=s, **plans[k])
                s.synchronize()
            results[k] = out
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(plans))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for k in range(len(plans)):
        assert torch.equal(results[k].view(torch.int16), ref_out[k].view(torch.int16)), plans[k]


@pytest.mark.parametrize("path,sched", KERNELS)
def test_window_at_least_context_equals_no_window(path, sched):
    """A window at least as long as every context sees what window 0 sees;
    the plans coincide, so the outputs are bit-identical."""
    w = mtp_workload()
    for big in (w.max_seq_len, w.max_seq_len + 7, 1 << 20):
        c0 = workloads.make_case(w, device="cuda", window=0)
        cw = workloads.make_case(w, device="cuda", window=big)
        a = run_gpu(c0, path=path, schedule=sched).clone()
        b = run_gpu(cw, path=path, schedule=sched)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (path, sched, big)


@pytest.mark.parametrize("window", [0, 5])
def test_mtp_row_equals_shorter_single_token_call(window):
    """Query token i of a q-token call equals a one-token call whose context
    ends at that token (L' = L - (q - 1 - i)), same cache and query vector."""
    w = mtp_workload(query_len=4, seq_lens=(150, 77))
    c = workloads.make_case(w, device="cuda", window=window)
    full = run_gpu(c).float()
    q_b = w.query_len
    for i in range(q_b):
        rows = [b * q_b + i for b in range(w.batch)]
        lens = torch.tensor([L - (q_b - 1 - i) for L in w.seq_lens], dtype=torch.int32, device="cuda")
        ones = torch.ones(w.batch, dtype=torch.int32, device="cuda")
        q1 = c.q[rows].contiguous()
        out1 = torch.empty_like(q1)
        pa.decode(out1, q1, c.k_cache, c.v_cache, c.block_tables, lens, ones, c.scale, window,
                  w.num_kv_heads, w.block_size, max_seq_len=w.max_seq_len, max_query_len=1)
        torch.cuda.synchronize()
        diff = (out1.float() - full[rows]).abs().max().item()
        assert diff <= 8e-3, (i, window, diff)


@pytest.mark.parametrize("path", PATHS)
def test_gqa_equals_mha_with_repeated_heads(path):
    """G = 4 query heads per KV head give bit for bit what G = 1 gives with
    each KV head repeated for its group (rows are computed independently;
    the same grid plan on both sides)."""
    w = mtp_workload(num_q_heads=8, num_kv_heads=2, query_len=2, seq_lens=(150, 77))
    c = workloads.make_case(w, device="cuda", window=0)
    gqa = run_gpu(c, path=path, schedule=pa.SCHED_GRID, part_size=64).clone()
    k8 = c.k_cache.repeat_interleave(4, dim=1).contiguous()
    v8 = c.v_cache.repeat_interleave(4, dim=1).contiguous()
    mha = torch.empty_like(gqa)
    pa.decode(mha, c.q, k8, v8, c.block_tables, c.seq_lens, c.query_lens, c.scale, 0, 8,
              w.block_size, max_seq_len=w.max_seq_len, max_query_len=w.query_len, path=path,
              schedule=pa.SCHED_GRID, part_size=64)
    torch.cuda.synchronize()
    assert torch.equal(gqa.view(torch.int16), mha.view(torch.int16))
