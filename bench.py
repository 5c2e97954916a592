"""Benchmark of one paged-attention decode call on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--window W]
                    [--no-cpu-baseline] [--no-side] [--reps N] [--flush]
                    [--path auto|mfma|valu] [--part-size P]
                    [--schedule auto|grid|persistent] [--loads auto|cached|streaming]

A step is one pa_decode call (partition kernel + LSE reduce) over the
workload's batch, inputs resident in HBM.  The default workload is the
largest configuration: the large-block MTP batch (128 sequences of 2048 to
65536 positions, 1024-slot blocks, 2 query tokens, 64/8 heads, head dim 128)
at window 0, about 17.7 GB of K/V per call.  Prints ONE JSON line: µs per
call (mean of K back-to-back calls, and median / p10 / p90 of individually
timed calls), achieved HBM GB/s of the partition kernel on algorithmic bytes
(HIP events the library binds to that kernel's dispatch, on its stream), the
roofline fraction of MI355X's 8 TB/s, the float64 CPU oracle timed on the
host's cores over a bounded sample of the same workload, and (``side``) the
other workloads' per-call figures measured in the same run: the GQA batch,
the single 131072-position sequence, the sliding-window MTP batch and the
GQA batch in fp32 (vector-ALU kernel) cold (flushed), and the large-block
batch at window 4096.

Algorithmic bytes per call (what the method must move): for every
(sequence, KV head) the K and V bytes of the union of its rows' visible
positions, plus Q read, output write, the block-table entries of blocks that
hold visible positions, and the two length arrays.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per paged-decode call + achieved HBM GB/s (fraction of MI355X peak)"
PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "large_block_mtp_bf16"   # the largest configuration, window 0 by default


def kernel_source_hash() -> str:
    """Fingerprint of the partition kernels' code, the plan and launch code
    (the part of pa_decode.hip before its extern "C" entry points) and the
    compile flags: what the roofline and traffic figures describe.  Comments
    and whitespace are left out: rewording a comment does not change the
    kernels the counters measured."""
    import re
    from decode_attention_pa_amd import build as b
    d = os.path.join(ROOT, "decode_attention_pa_amd", "csrc")
    h = hashlib.sha256()
    for f in ("pa_common.h", "pa_sched.h", "pa_mfma.h", "pa_valu.h", "pa_wave.h", "pa_launch.h",
              "pa_decode.hip",
              "pa_mfma_d64.hip", "pa_mfma_d128.hip", "pa_mfma_d256.hip", "pa_wave_kernels.hip"):
        src = open(os.path.join(d, f), encoding="utf-8").read()
        if f == "pa_decode.hip":
            src = src.split('extern "C" {')[0]
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(f.encode())
        h.update(" ".join(src.split()).encode())
    h.update(" ".join(a for a in b.command("x") if a.startswith("-")).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(case, one_shot: bool = False) -> dict:
    """Bytes the method must move for one call (see module docstring).
    ``partition_kernel``: the share of them the partition kernel moves.  On a
    one-shot plan it is the whole call (it writes the output rows itself);
    on a split plan the merge writes them, and the partition kernel's own
    writes are partial states, which the method does not need."""
    w = case.w
    s = 2 if w.dtype == "bf16" else 4
    skv = 1 if w.kv_dtype == "fp8" else s      # bytes per cached K / V element
    kv = 0
    tables = 0
    bs = w.block_size
    for L, q in zip(case.seq_lens_host, case.query_lens_host):
        if q <= 0:
            continue
        lo = 0 if case.window == 0 else max(0, L - q + 1 - case.window)
        kv += w.num_kv_heads * (L - lo) * w.head_dim * 2 * skv
        tables += 4 * ((L - 1) // bs - lo // bs + 1)
    T = sum(case.query_lens_host)
    qb = T * w.num_q_heads * w.head_dim * (1 if w.q_dtype == "fp8" else s)   # Q read
    ob = T * w.num_q_heads * w.head_dim * s                                   # out written
    lens = 8 * w.batch
    return dict(kv=kv, q=qb, out=ob, tables=tables, lens=lens,
                total=kv + qb + ob + tables + lens,
                partition_kernel=kv + qb + tables + lens + (ob if one_shot else 0))


CALIB_COPIES = 3  # plain 1 GiB device copies issued by --copy-calibration


def load_traffic(workload: str, window: int):
    """HBM traffic of the partition kernel from the committed rocprofv3 counter
    record, or None if absent or taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(f"{workload}:w{window}")
    if not rec or rec.get("kernel_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def _counter_rows(path):
    import csv
    for root, _, files in os.walk(path):
        for f in files:
            if f.endswith("counter_collection.csv"):
                yield from csv.DictReader(open(os.path.join(root, f)))


def counter_bytes(rows, name: str) -> dict:
    """HBM bytes per partition-kernel launch from one counter's rows
    ((dispatch id, kernel name, KiB) per dispatch, any order): the counter
    is scaled by what it reads for the plain 1 GiB device copies issued right
    before the first partition kernel (known to read and write 1 GiB each),
    and averaged over the partition dispatches after the first (cold) one."""
    gib_kib = float(1 << 20)
    rows = sorted(rows)
    is_part = lambda k: "pa::part_" in k      # part_mfma, part_mfma_ps, part_wave, part_valu
    part = [v for _, k, v in rows if is_part(k)]
    first_part = min((i for i, k, _ in rows if is_part(k)), default=0)
    # the calibration copies are the last CALIB_COPIES large copies before
    # the first partition kernel; earlier ones stage the workload's inputs
    # (of other sizes) and would skew the scale
    copy = [v for i, k, v in rows
            if "copyBuffer" in k and v > gib_kib / 8 and i < first_part][-CALIB_COPIES:]
    if not copy or not part:
        raise SystemExit(f"{name}: no calibration copy or partition kernel among the dispatches")
    calib = sum(copy) / len(copy)
    scale = gib_kib / calib
    per = sum(part[1:]) / max(len(part) - 1, 1) if len(part) > 1 else part[0]  # first is cold
    return {"copy_kib": round(calib, 2), "scale": round(scale, 5),
            "partition_kib_raw": round(per, 2),
            "partition_bytes": int(per * scale * 1024), "dispatches": len(part)}


def ingest_counters(workload: str, window: int, fetch_dir: str, write_dir: str,
                    command: str) -> dict:
    """Turns two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) of ``bench.py --copy-calibration`` into HBM bytes per launch of
    the partition kernel (``counter_bytes``) and writes the record into
    profiles/traffic.json."""
    rec = {"workload": workload, "window": window, "kernel_hash": kernel_source_hash(),
           "command": command}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [(int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
                for r in _counter_rows(d) if r["Counter_Name"] == name]
        rec[name] = counter_bytes(rows, name)
    rec["bytes_per_launch"] = rec["FETCH_SIZE"]["partition_bytes"] + rec["WRITE_SIZE"]["partition_bytes"]
    path = os.path.join(ROOT, "profiles", "traffic.json")
    allrec = json.load(open(path)) if os.path.exists(path) else {}
    allrec[f"{workload}:w{window}"] = rec
    json.dump(allrec, open(path, "w"), indent=1, sort_keys=True)
    return rec


def copy_ceiling(nbytes: int, flush_buf, reps: int = 10) -> dict:
    """A plain device copy moving the same number of HBM bytes as the
    partition kernel (half read, half written; capped at 4 GB moved), timed
    with events around each copy, flushed like the calls when they are: what
    a trivial kernel reaches at this size on this GPU."""
    import torch
    n = max(1, min(nbytes, 4 << 30) // 8)    # float32 elements per buffer
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        if flush_buf is not None:
            flush_buf.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    ts.sort()
    moved = 8 * n
    us = ts[len(ts) // 2]
    del src, dst
    torch.cuda.empty_cache()
    return {"kind": "device copy, read + write", "bytes": moved, "us": round(us, 2),
            "gbps": round(moved / us / 1e3, 1), "frac": round(moved / us / 1e3 / PEAK_GBPS, 4)}


def read_ceiling(pa, nbytes: int, flush_buf, reps: int = 10) -> dict:
    """A streaming read of as many HBM bytes as the partition kernel reads
    (capped at 4 GB) by the library's probe kernel (pa_stream_read: the
    partition kernels' 16-byte non-temporal loads, coalesced), timed with
    events around each read and flushed like the calls when they are; the
    best median over both read patterns and a few grid sizes.  The read rate
    a plain kernel reaches on this GPU at this size, beside the 8 TB/s peak."""
    import torch
    n = max(1, min(nbytes, 4 << 30) // 16) * 4   # int32 elements, whole 16-byte words
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    best = None
    for slab, grid in ((False, 256), (False, 2048), (False, 16384),
                       (True, 256), (True, 2048), (True, 16384)):
        sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
        pa.stream_read(src, sink, slab=slab)
        ts = []
        for _ in range(reps):
            if flush_buf is not None:
                flush_buf.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            wgs = pa.stream_read(src, sink, slab=slab)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        us = ts[len(ts) // 2]
        if best is None or us < best[0]:
            best = (us, wgs, slab)
    read = 4 * n
    us, wgs, slab = best
    del src
    torch.cuda.empty_cache()
    return {"kind": "streaming read (pa_stream_read)", "bytes": read, "workgroups": wgs,
            "pattern": "slab" if slab else "grid stride", "us": round(us, 2),
            "gbps": round(read / us / 1e3, 1), "frac": round(read / us / 1e3 / PEAK_GBPS, 4)}


def with_share(ceiling: dict, achieved_gbps: float) -> dict:
    """The ceiling record plus the partition kernel's achieved rate as a
    share of it."""
    return {**ceiling, "kernel_share": round(achieved_gbps / ceiling["gbps"], 3)}


def cpu_model() -> str:
    """CPU model string of this host (from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads(cap: int = 16) -> int:
    """Oracle worker threads: the cores this process may run on, at most
    ``cap`` (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, cap))


def cpu_baseline(case, out_gpu, budget_s: float) -> dict:
    """The float64 oracle, as it stands, on the host's cores: one worker
    thread per core (NumPy releases the interpreter lock in its array loops;
    one BLAS thread per worker), sequences handed out longest first in waves
    of one per thread, until ``budget_s`` of oracle wall time has passed or
    the whole batch is done; the time is scaled to one full call by
    algorithmic KV bytes.  Only the oracle calls are timed (copying the
    sampled blocks to the host is not).  Also checks the GPU output on the
    rows it computed."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    from oracle import paged_attention as ref
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from tests._gpu_util import oracle_inputs

    w = case.w
    s = 1 if w.kv_dtype == "fp8" else (2 if w.dtype == "bf16" else 4)   # bytes per K / V element

    def kv_bytes(b):
        L, q = case.seq_lens_host[b], case.query_lens_host[b]
        if q <= 0:
            return 0
        lo = 0 if case.window == 0 else max(0, L - q + 1 - case.window)
        return w.num_kv_heads * (L - lo) * w.head_dim * 2 * s

    order = sorted(range(w.batch), key=lambda b: -kv_bytes(b))
    nthr = host_threads()
    got_all = out_gpu.float().cpu().numpy().astype(np.float64)
    done, t_total, bytes_done, max_err, max_ref = 0, 0.0, 0, 0.0, 0.0
    with threadpool_limits(limits=1), ThreadPoolExecutor(nthr) as ex:
        for k in range(0, len(order), nthr):
            wave = order[k:k + nthr]
            inputs = [oracle_inputs(case, [b]) for b in wave]          # host copies, untimed
            t0 = time.perf_counter()
            results = list(ex.map(lambda ir: ref.decode(**ir[0]), inputs))
            t_total += time.perf_counter() - t0
            for (inp, rows), exp in zip(inputs, results):
                if rows:
                    max_err = max(max_err, float(np.abs(got_all[rows] - exp).max()))
                    max_ref = max(max_ref, float(np.abs(exp).max()))
            bytes_done += sum(kv_bytes(b) for b in wave)
            done += len(wave)
            del inputs, results
            if t_total >= budget_s:
                break
    kv_total = algorithmic_bytes(case)["kv"]
    scale = kv_total / max(bytes_done, 1)
    return dict(value=round(t_total * scale * 1e6, 1), unit="us/call", cores=nthr, kind="oracle",
                cpu_model=cpu_model(),
                sample=f"{done} of {w.batch} sequences, longest first ({bytes_done / 1e6:.1f} MB "
                       f"of {kv_total / 1e6:.1f} MB KV), float64 NumPy oracle on {nthr} worker "
                       f"threads (1 BLAS thread each), {t_total:.2f} s oracle wall time, "
                       f"scaled to one call by KV bytes",
                gbps=round(bytes_done / max(t_total, 1e-9) / 1e9, 3),
                parity_max_abs=max_err,
                parity_rel=(max_err / max_ref) if max_ref > 0 else None)


def pct(xs, p):
    """p-th percentile (nearest rank) of a sorted list."""
    return xs[min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))]


def make_call(pa, case, window, a, events=(None, None)):
    w = case.w
    path = {"auto": 0, "valu": pa.PATH_VALU, "mfma": pa.PATH_MFMA,
            "valu-lds": pa.PATH_VALU_LDS}[a.path]
    return pa.Prepared(case.new_out(), case.q, case.k_cache, case.v_cache, case.block_tables,
                       case.seq_lens, case.query_lens, case.scale, window, w.num_kv_heads,
                       w.block_size, max_seq_len=w.max_seq_len, max_query_len=w.query_len,
                       path=path, part_size=a.part_size, waves=a.waves,
                       schedule={"auto": 0, "grid": pa.SCHED_GRID,
                                 "persistent": pa.SCHED_PERSISTENT}[a.schedule],
                       loads={"auto": 0, "cached": pa.LOADS_CACHED,
                              "streaming": pa.LOADS_STREAMING}[a.loads],
                       k_scale=case.k_scale, v_scale=case.v_scale, q_scale=case.q_scale)


def timed_reps(call, reps, flush_buf):
    """Two passes of ``reps`` calls, the flush read (if any) before each call
    and outside its events: first each call bracketed by its own pair of
    events on the call's stream (the per-call time), then each call with
    HIP events the library binds to the partition kernel's own dispatch
    (that kernel's start and end, as a kernel trace reports it; binding them
    costs launch time, so they are kept out of the first pass).  Returns
    sorted per-call and per-kernel µs."""
    import torch
    stream = torch.cuda.current_stream()
    cb = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        if flush_buf is not None:
            flush_buf.sum()
        cb[i].record(stream)
        call()
        ce[i].record(stream)
    torch.cuda.synchronize()
    kb = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ke = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for e in kb + ke:
        e.record(stream)  # creates the HIP events; the library re-stamps them
    torch.cuda.synchronize()
    for i in range(reps):
        if flush_buf is not None:
            flush_buf.sum()
        call.set_events(kb[i], ke[i])
        call()
    torch.cuda.synchronize()
    call.set_events(None, None)
    kern = sorted(kb[i].elapsed_time(ke[i]) * 1e3 for i in range(reps))
    per = sorted(cb[i].elapsed_time(ce[i]) * 1e3 for i in range(reps))
    return per, kern


def summary(per, kern, nb) -> dict:
    med = pct(per, 50)
    kmed = pct(kern, 50)
    return {"reps": len(per),
            "call_us": {"median": round(med, 2), "p10": round(pct(per, 10), 2),
                        "p90": round(pct(per, 90), 2), "mean": round(sum(per) / len(per), 2)},
            "kernel_us": {"median": round(kmed, 2), "p10": round(pct(kern, 10), 2),
                          "p90": round(pct(kern, 90), 2), "mean": round(sum(kern) / len(kern), 2)},
            "gbps_per_call": round(nb["total"] / (med * 1e-6) / 1e9, 1),
            "frac_per_call": round(nb["total"] / (med * 1e-6) / 1e9 / PEAK_GBPS, 4),
            "kernel_frac": round(nb["partition_kernel"] / (kmed * 1e-6) / 1e9 / PEAK_GBPS, 4)}


# Other workloads timed in the same run, beside the headline: (workload,
# window, flush).  The small ones fit in the 256 MB MALL and are timed cold
# (a 1 GiB read before each call, outside its events), as a decode step over
# many layers meets them.
SIDE = (("gqa_bf16", 0, True), ("long_splitk_bf16", 0, True), ("swa_mtp_bf16", 128, True),
        ("large_block_mtp_bf16", 4096, False), ("gqa_f32", 0, True))


def side_line(pa, workloads, main_case, a, flush_buf, reps, name, window, flush) -> dict:
    import torch
    if name == main_case.w.name:
        c = main_case             # another window over the same cache
    else:
        c = workloads.make_case(workloads.WORKLOADS[name], device="cuda", window=window)
    c_win = workloads.Case(**{**c.__dict__, "window": window})
    call = make_call(pa, c_win, window, a)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    per, kern = timed_reps(call, reps, flush_buf if flush else None)
    nb = algorithmic_bytes(c_win, one_shot=bool(call.plan["one_shot"]))
    line = {"flush_between_calls": flush, "plan": call.plan, "algorithmic_bytes": nb["total"],
            **summary(per, kern, nb), "read_ceiling": None}
    rc = read_ceiling(pa, nb["partition_kernel"], flush_buf if flush else None)
    achieved = nb["partition_kernel"] / (line["kernel_us"]["median"] * 1e-6) / 1e9
    line["read_ceiling"] = with_share(rc, achieved)
    return line


def guarded(label, fn):
    """fn() for one of the figures reported beside the headline; an exception
    is printed to stderr and recorded in the line instead of losing the
    headline measured before it."""
    import traceback
    try:
        return fn()
    except Exception as e:  # reported, never silently dropped
        traceback.print_exc()
        print(f"bench: {label} failed: {e!r}", file=sys.stderr, flush=True)
        return {"error": f"{type(e).__name__}: {e}"}


def side_lines(pa, workloads, main_case, a, flush_buf, reps) -> dict:
    import torch
    res = {}
    for name, window, flush in SIDE:
        res[f"{name}:w{window}"] = guarded(
            f"side line {name} w={window}",
            lambda: side_line(pa, workloads, main_case, a, flush_buf, reps, name, window, flush))
        torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--window", type=int, default=None)
    ap.add_argument("--path", default="auto", choices=["auto", "mfma", "valu", "valu-lds"])
    ap.add_argument("--part-size", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--schedule", default="auto", choices=["auto", "grid", "persistent"])
    ap.add_argument("--loads", default="auto", choices=["auto", "cached", "streaming"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the other workloads timed beside the headline")
    ap.add_argument("--reps", type=int, default=50,
                    help="individually timed calls for the per-call percentiles")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--flush", action="store_true",
                    help="read a 1 GiB buffer before every call (outside the call's events); "
                         "the value is then the mean time between events around each call")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 1 GiB device copies (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="(no GPU) record rocprofv3 FETCH_SIZE/WRITE_SIZE runs of this "
                         "workload into profiles/traffic.json and exit")
    ap.add_argument("--ingest-command", default="", help="command line that produced them")
    ap.add_argument("--context", type=int, default=0,
                    help="every sequence of the workload this many positions long instead of "
                         "the workload's lengths (a context sweep; no traffic record applies)")
    a = ap.parse_args(argv)
    if a.ingest_counters:
        w = a.workload
        win = a.window if a.window is not None else __import__("workloads").WORKLOADS[w].windows[0]
        print(json.dumps(ingest_counters(w, win, *a.ingest_counters, a.ingest_command)))
        return 0
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this library has no "
              "multi-GPU path.", file=sys.stderr)
        return 2

    import torch

    import decode_attention_pa_amd as pa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    w = workloads.WORKLOADS[a.workload]
    if a.context:
        if a.context < w.query_len:
            print(f"--context {a.context} is shorter than the query length {w.query_len}",
                  file=sys.stderr)
            return 2
        w = workloads.with_context(w, a.context)
    window = w.windows[0] if a.window is None else a.window
    case = workloads.make_case(w, device="cuda", window=window)
    call = make_call(pa, case, window, a)
    out = call._keep[0]
    # flush = reading 1 GiB evicts the workload from L2 and the 256 MB MALL
    # with clean lines (a write would leave dirty lines behind to write back)
    need_flush = a.flush or (not a.no_side and any(f for _, _, f in SIDE))
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if need_flush else None
    if a.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(CALIB_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    nb = algorithmic_bytes(case, one_shot=bool(call.plan["one_shot"]))
    for _ in range(a.warmup):
        call()
    torch.cuda.synchronize()

    K = a.steps
    stream = torch.cuda.current_stream()
    # Pass 1 (the reported value): K calls back to back, bracketed by two
    # events and host synchronisation.  With --flush each call is preceded by
    # the flush read and bracketed by its own pair of events (the flush stays
    # outside them); nothing else is recorded inside a call.
    own_flush = flush_buf if a.flush else None
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    fb = [torch.cuda.Event(enable_timing=True) for _ in range(K)] if own_flush is not None else []
    fe = [torch.cuda.Event(enable_timing=True) for _ in range(K)] if own_flush is not None else []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        if own_flush is not None:
            own_flush.sum()
            fb[i].record(stream)
        call()
        if own_flush is not None:
            fe[i].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    flushed_ms = sorted(fb[i].elapsed_time(fe[i]) for i in range(K)) if fb else []

    # Pass 2: max(K, reps) calls, each bracketed by its own events, with HIP
    # events that the library binds to the partition kernel's dispatch
    # (stamped with that kernel's own start and end, as a kernel trace
    # reports it): per-call percentiles and the roofline's kernel time.
    per, kern = timed_reps(call, max(K, a.reps), own_flush)
    kern_avg = sum(kern) / len(kern)
    us_per_call = (sum(flushed_ms) / K if a.flush else total_ms / K) * 1e3
    achieved = nb["partition_kernel"] / (kern_avg * 1e-6) / 1e9
    call_gbps = nb["total"] / (us_per_call * 1e-6) / 1e9
    traffic = None if a.context else load_traffic(a.workload, window)
    stats = summary(per, kern, nb)

    res = {
        "metric": METRIC,
        "value": round(us_per_call, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(us_per_call / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8 QK, bf16 PV" if w.q_dtype == "fp8" else "bf16") if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "description": w.description, "window": window,
            "batch": w.batch, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "query_len": w.query_len,
            "kv_dtype": w.kv_dtype or w.dtype, "q_dtype": w.q_dtype or w.dtype,
            "realised_context_tokens": sum(case.seq_lens_host), "plan": call.plan,
            "flush_between_calls": bool(a.flush),
            "context_override": a.context or None,
        },
        "achieved_gbps_per_call": round(call_gbps, 1),
        "frac_of_peak_per_call": round(call_gbps / PEAK_GBPS, 4),
        "algorithmic_bytes": nb,
        "per_call": {"reps": stats["reps"], **stats["call_us"]},
        "kernel_us": {"partition_avg": round(kern_avg, 2),
                      "partition_median": stats["kernel_us"]["median"],
                      "partition_p10": stats["kernel_us"]["p10"],
                      "partition_p90": stats["kernel_us"]["p90"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic},
        "host_wall_s": round(wall, 3),
        # with --flush the timed pass also holds one 1 GiB flush read per call
        "ms_per_step_with_flush_reads": round(total_ms / K, 5) if a.flush else None,
        "copy_ceiling": copy_ceiling(nb["partition_kernel"], own_flush),
        "read_ceiling": with_share(read_ceiling(pa, nb["partition_kernel"], own_flush), achieved),
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = guarded("cpu_baseline", lambda: cpu_baseline(case, out, a.cpu_budget))
    if not a.no_side:
        del call
        res["side"] = side_lines(pa, workloads, case, a, flush_buf, a.reps)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
