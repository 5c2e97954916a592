"""Benchmark of one paged-attention decode call on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--window W]
                    [--no-cpu-baseline] [--flush] [--path auto|mfma|valu] [--part-size P]
                    [--schedule auto|grid|persistent] [--loads auto|cached|streaming]

A step is one pa_decode call (partition kernel + LSE reduce) over the
workload's batch, inputs resident in HBM.  Prints ONE JSON line: µs per call,
achieved HBM GB/s of the partition kernel on algorithmic bytes (HIP events
recorded by the library around that kernel, on its stream), the roofline
fraction of MI355X's 8 TB/s, and the float64 CPU oracle timed on a bounded
sample of the same workload.

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
DEFAULT_WORKLOAD = "gqa_bf16"


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
    for f in ("pa_common.h", "pa_mfma.h", "pa_valu.h", "pa_decode.hip"):
        src = open(os.path.join(d, f), encoding="utf-8").read()
        if f == "pa_decode.hip":
            src = src.split('extern "C" {')[0]
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(f.encode())
        h.update(" ".join(src.split()).encode())
    h.update(" ".join(a for a in b.command("x") if a.startswith("-")).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(case) -> dict:
    """Bytes the method must move for one call (see module docstring)."""
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
                partition_kernel=kv + qb + tables + lens)


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
    is_part = lambda k: "part_mfma" in k or "part_valu" in k
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


def cpu_baseline(case, out_gpu, budget_s: float, per_call_bytes: int) -> dict:
    """The float64 oracle, as it stands, on a bounded sample of the workload's
    sequences (host cores of this machine), scaled to µs per full call by
    algorithmic KV bytes.  Also checks the GPU output on the sampled rows."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import paged_attention as ref
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from tests._gpu_util import oracle_inputs

    w = case.w
    order = list(range(w.batch))
    done, t_total, bytes_done = [], 0.0, 0
    max_err = 0.0
    s = 1 if w.kv_dtype == "fp8" else (2 if w.dtype == "bf16" else 4)   # bytes per K / V element
    with threadpool_limits(limits=1):
        for b in order:
            inp, rows = oracle_inputs(case, [b])
            t0 = time.perf_counter()
            exp = ref.decode(**inp)
            t_total += time.perf_counter() - t0
            L, q = case.seq_lens_host[b], case.query_lens_host[b]
            lo = 0 if case.window == 0 else max(0, L - q + 1 - case.window)
            bytes_done += w.num_kv_heads * (L - lo) * w.head_dim * 2 * s
            got = out_gpu.float().cpu().numpy()[rows].astype(np.float64)
            max_err = max(max_err, float(np.abs(got - exp).max()))
            done.append(b)
            if t_total >= budget_s:
                break
    kv_total = algorithmic_bytes(case)["kv"]
    scale = kv_total / max(bytes_done, 1)
    return dict(value=round(t_total * scale * 1e6, 1), unit="us/call", cores=1, kind="oracle",
                sample=f"{len(done)} of {w.batch} sequences ({bytes_done / 1e6:.1f} MB of "
                       f"{kv_total / 1e6:.1f} MB KV), float64 NumPy, 1 BLAS thread, "
                       f"{t_total:.2f} s, scaled by KV bytes",
                gbps=round(bytes_done / max(t_total, 1e-9) / 1e9, 3),
                parity_max_abs=max_err)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--window", type=int, default=None)
    ap.add_argument("--path", default="auto", choices=["auto", "mfma", "valu"])
    ap.add_argument("--part-size", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--schedule", default="auto", choices=["auto", "grid", "persistent"])
    ap.add_argument("--loads", default="auto", choices=["auto", "cached", "streaming"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    window = w.windows[0] if a.window is None else a.window
    case = workloads.make_case(w, device="cuda", window=window)
    out = case.new_out()
    path = {"auto": 0, "valu": pa.PATH_VALU, "mfma": pa.PATH_MFMA}[a.path]
    call = pa.Prepared(out, case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
                       case.query_lens, case.scale, window, w.num_kv_heads, w.block_size,
                       max_seq_len=w.max_seq_len, max_query_len=w.query_len, path=path,
                       part_size=a.part_size, waves=a.waves,
                       schedule={"auto": 0, "grid": pa.SCHED_GRID,
                                 "persistent": pa.SCHED_PERSISTENT}[a.schedule],
                       loads={"auto": 0, "cached": pa.LOADS_CACHED,
                              "streaming": pa.LOADS_STREAMING}[a.loads],
                       k_scale=case.k_scale, v_scale=case.v_scale, q_scale=case.q_scale)
    # flush = reading 1 GiB evicts the workload from L2 and the 256 MB MALL
    # with clean lines (a write would leave dirty lines behind to write back)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if a.flush else None
    if a.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(CALIB_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    nb = algorithmic_bytes(case)
    for _ in range(a.warmup):
        call()
    torch.cuda.synchronize()

    K = a.steps
    stream = torch.cuda.current_stream()
    # Pass 1 (the reported value): K calls back to back, bracketed by two
    # events and host synchronisation.  With --flush each call is preceded by
    # the flush read and bracketed by its own pair of events (the flush stays
    # outside them); nothing else is recorded inside a call.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    fb = [torch.cuda.Event(enable_timing=True) for _ in range(K)] if flush_buf is not None else []
    fe = [torch.cuda.Event(enable_timing=True) for _ in range(K)] if flush_buf is not None else []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        if flush_buf is not None:
            flush_buf.sum()
            fb[i].record(stream)
        call()
        if flush_buf is not None:
            fe[i].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    flushed_ms = sorted(fb[i].elapsed_time(fe[i]) for i in range(K)) if fb else []

    # Pass 2: the same K calls with HIP events that the library binds to the
    # partition kernel's dispatch (stamped with that kernel's own start and
    # end, as a kernel trace reports it), plus events around each whole call.
    kb = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ke = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    cb = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for e in kb + ke:
        e.record(stream)  # creates the HIP events; the library re-stamps them
    torch.cuda.synchronize()
    for i in range(K):
        if flush_buf is not None:
            flush_buf.sum()
        call.set_events(kb[i], ke[i])
        cb[i].record(stream)
        call()
        ce[i].record(stream)
    torch.cuda.synchronize()
    call.set_events(None, None)
    kern_ms = sorted(kb[i].elapsed_time(ke[i]) for i in range(K))
    call_ms = sorted(cb[i].elapsed_time(ce[i]) for i in range(K))
    kern_avg = sum(kern_ms) / K
    call_avg = sum(call_ms) / K
    us_per_call = (sum(flushed_ms) / K if a.flush else total_ms / K) * 1e3
    achieved = nb["partition_kernel"] / (kern_avg * 1e-3) / 1e9
    call_gbps = nb["total"] / (us_per_call * 1e-6) / 1e9
    traffic = load_traffic(a.workload, window)

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
        },
        "achieved_gbps_per_call": round(call_gbps, 1),
        "frac_of_peak_per_call": round(call_gbps / PEAK_GBPS, 4),
        "algorithmic_bytes": nb,
        "kernel_us": {"partition_avg": round(kern_avg * 1e3, 2),
                      "partition_p10": round(kern_ms[K // 10] * 1e3, 2),
                      "partition_p90": round(kern_ms[(9 * K) // 10] * 1e3, 2),
                      "call_avg_with_kernel_events": round(call_avg * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic},
        "host_wall_s": round(wall, 3),
        # with --flush the timed pass also holds one 1 GiB flush read per call
        "ms_per_step_with_flush_reads": round(total_ms / K, 5) if a.flush else None,
        "copy_ceiling": copy_ceiling(nb["partition_kernel"], flush_buf),
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, out, a.cpu_budget, nb["total"])
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
