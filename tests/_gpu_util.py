"""Helpers for GPU parity tests: run the HIP path, and hand the oracle a
compact host copy of exactly the blocks it needs (data movement only)."""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

import decode_attention_pa_amd as pa
from oracle import paged_attention as ref

BF16_TOL = 2e-2   # max-abs bar for bf16 inputs with fp32 accumulation
F32_TOL = 1e-4    # max-abs bar for fp32 inputs

# Scale-free bars beside each max-abs bar.  Under N(0, 1) inputs an output
# row averages ~n visible values, so |out| ~ sqrt(e / n): ~0.007 at 65536
# positions, where a max-abs bar of 2e-2 alone would pass an all-zero output.
# With bf16 inputs the kernels round the softmax weights and the output to
# bf16 (relative steps of 2^-8 and 2^-9), which puts the measured errors at
# ~2-3e-3 of max|ref| and ~1e-3 in RMS; the bars below sit 5-10x above that
# and far below what a dropped term or a misnormalised row gives (>= 0.1).
# fp32 inputs take no reduced-precision step (errors ~1e-6 relative).
REL_BARS = {BF16_TOL: (2e-2, 1e-2), F32_TOL: (1e-3, 1e-4)}   # (max|d|/max|ref|, RMS ratio)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(case, out=None, **opts):
    """One pa_decode call on the case's tensors; returns the output tensor.
    FP8 cases pass their scales unless the caller overrides them."""
    if out is None:
        out = case.new_out().fill_(float("nan"))
    if case.k_scale is not None:
        opts.setdefault("k_scale", case.k_scale)
        opts.setdefault("v_scale", case.v_scale)
    if case.q_scale is not None:
        opts.setdefault("q_scale", case.q_scale)
    pa.decode(out, case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens,
              case.query_lens, case.scale, case.window, case.w.num_kv_heads, case.w.block_size,
              max_seq_len=case.w.max_seq_len, max_query_len=max(case.w.query_len,
                                                                   max(case.query_lens_host or [1])),
              **opts)
    torch.cuda.synchronize()
    return out


def oracle_inputs(case, seqs=None):
    """Compact oracle problem for sequences ``seqs`` (default all).

    Gathers only blocks that hold visible positions; table entries for other
    logical blocks point at a NaN block, so a wrong read would show.
    Returns (inputs dict, list of global q rows in compact order).
    """
    B = len(case.seq_lens_host)
    seqs = list(range(B)) if seqs is None else list(seqs)
    tables = case.tables_host.numpy()
    sp = ref.spans(tables, case.seq_lens_host, case.query_lens_host, case.window,
                   case.w.block_size)
    need = sorted(set(int(x) for b in seqs for x in sp[b]["blocks"] if x >= 0))
    remap = {p: i + 1 for i, p in enumerate(need)}
    ids = torch.tensor(need, dtype=torch.long, device=case.k_cache.device)
    k = _host_values(case.k_cache.index_select(0, ids), case.w.k_scale) if need else \
        np.zeros((0,) + tuple(case.k_cache.shape[1:]), np.float32)
    v = _host_values(case.v_cache.index_select(0, ids), case.w.v_scale) if need else \
        np.zeros((0,) + tuple(case.v_cache.shape[1:]), np.float32)
    k = np.concatenate([np.full((1,) + k.shape[1:], np.nan, np.float32), k])
    v = np.concatenate([np.full((1,) + v.shape[1:], np.nan, np.float32), v])
    ctab = np.zeros((len(seqs), tables.shape[1]), np.int64)
    rows = []
    for r, b in enumerate(seqs):
        for kk, p in enumerate(sp[b]["blocks"]):
            ctab[r, kk] = remap[int(p)] if p >= 0 else 0
        rows.extend(range(sp[b]["qoff"], sp[b]["qoff"] + case.query_lens_host[b]))
    qh = _host_values(case.q, case.w.q_scale)[rows] if rows else \
        np.zeros((0,) + tuple(case.q.shape[1:]))
    return dict(q=qh, k_cache=k, v_cache=v, block_tables=ctab,
                seq_lens=np.array([case.seq_lens_host[b] for b in seqs]),
                query_lens=np.array([case.query_lens_host[b] for b in seqs]),
                scale=case.scale, window=case.window, num_kv_heads=case.w.num_kv_heads,
                block_size=case.w.block_size), rows


def _host_values(t, scale):
    """Device values on the host: FP8 codes (caches, queries) dequantized by
    the oracle."""
    if t.dtype == torch.float8_e4m3fn:
        return ref.dequantize(t.view(torch.uint8).cpu().numpy(), scale)
    return t.float().cpu().numpy()


def sample_sequences(lens, nsample, seed):
    """``nsample`` seeded random sequences plus the longest and shortest
    (all of them when ``nsample`` is None), in increasing order."""
    B = len(lens)
    if nsample is None or nsample >= B:
        return list(range(B))
    lens = np.asarray(lens)
    r = np.random.default_rng(seed)
    pick = {int(lens.argmax()), int(lens.argmin())}
    pick |= set(int(x) for x in r.choice(B, size=nsample, replace=False))
    return sorted(pick)


def oracle_out(case, seqs=None):
    inp, rows = oracle_inputs(case, seqs)
    return ref.decode(**inp), rows


def compare(out_gpu, expect, rows, tol, label=""):
    got = out_gpu.float().cpu().numpy()[rows].astype(np.float64)
    assert got.shape == expect.shape
    assert np.all(np.isfinite(got)), f"{label}: non-finite GPU output"
    err = np.abs(got - expect)
    mx = float(err.max()) if err.size else 0.0
    scale = float(np.abs(expect).max()) if expect.size else 0.0
    rms_ratio = float(np.sqrt((err ** 2).mean() / max((expect ** 2).mean(), 1e-300))) if err.size else 0.0
    rel = mx / scale if scale > 0 else (0.0 if mx == 0 else float("inf"))
    rel_bar, rms_bar = REL_BARS[tol]
    say(f"[parity] {label}: max_abs={mx:.3e} max|ref|={scale:.3e} rel={rel:.3e} "
        f"rms_ratio={rms_ratio:.3e} tol={tol:g} rel_bar={rel_bar:g} rms_bar={rms_bar:g}")
    log = os.environ.get("PA_PARITY_LOG")
    if log:
        with open(log, "a", encoding="utf-8") as f:
            f.write(f"{label}\tmax_abs={mx:.3e}\tmax_ref={scale:.3e}\trel={rel:.3e}\t"
                    f"rms_ratio={rms_ratio:.3e}\n")
    assert mx <= tol, f"{label}: max-abs {mx:.3e} > {tol:g}"
    assert rel <= rel_bar, f"{label}: max-abs / max|ref| {rel:.3e} > {rel_bar:g}"
    assert rms_ratio <= rms_bar, f"{label}: RMS error / RMS ref {rms_ratio:.3e} > {rms_bar:g}"
    return mx, rms_ratio
