"""Scalar brute force for paged-attention decode (test infrastructure only).

Pure-Python loops, Python floats (IEEE double).  Deliberately written without
the range arithmetic of ``paged_attention``: it walks every position of the
context and tests visibility per position with the page's rule — gllm
"feat(backend): sliding-window PagedAttention" (#116), summary: a positive
window limits the query at position p to the last ``window`` positions up to
and including p, and a zero window leaves causal attention unlimited — i.e.
t is visible iff t <= p and, when a window is set, fewer than ``window``
positions separate t from p.  Only for tiny inputs.
"""

from __future__ import annotations

import math


def brute_decode(q, k_cache, v_cache, block_tables, seq_lens, query_lens,
                 scale, window, num_kv_heads, block_size):
    """Same contract and layouts as ``paged_attention.decode`` (nested
    lists or arrays indexed element by element).  Returns nested lists
    [T][H_q][D] of floats."""
    B = len(seq_lens)
    H_q = len(q[0]) if len(q) else 0
    D = len(q[0][0]) if len(q) else 0
    group = H_q // num_kv_heads
    vg = len(v_cache[0][0][0][0]) if len(v_cache) else 1   # V slot-group size
    sigma = float(_to_f32(scale))
    out = []
    row = 0
    for b in range(B):
        L = int(seq_lens[b])
        nq = int(query_lens[b])
        for i in range(nq):
            p = L - nq + i                     # this token's own position
            out_row = []
            for hq in range(H_q):
                kvh = hq // group
                logits = []
                where = []
                for t in range(L):
                    if t > p:
                        continue               # causal: nothing after p
                    if window != 0 and p - t >= window:
                        continue               # more than window-1 back
                    phys = int(block_tables[b][t // block_size])
                    off = t % block_size
                    dot = 0.0
                    for d in range(D):
                        dot += float(q[row][hq][d]) * _key(k_cache, phys, kvh, off, d)
                    logits.append(sigma * dot)
                    where.append((phys, off))
                top = max(logits)
                wts = [math.exp(x - top) for x in logits]
                tot = math.fsum(wts)
                vec = []
                for d in range(D):
                    acc = math.fsum(w * float(v_cache[phys][kvh][off // vg][d][off % vg])
                                    for w, (phys, off) in zip(wts, where))
                    vec.append(acc / tot)
                out_row.append(vec)
            out.append(out_row)
            row += 1
    return out


def _key(k_cache, phys, kvh, off, d):
    """Element d of slot ``off``'s key: a row per slot, or the tiled form
    (16-slot groups; slots 0-3 and 8-11 in half 0, 4-7 and 12-15 in half 1,
    dims in columns of 8 for bf16 or 16 for FP8)."""
    slab = k_cache[phys][kvh]
    if len(slab) and not hasattr(slab[0][0], "__len__"):     # [bs][D]
        return float(slab[off][d])
    width = len(slab[0][0][0][0])                           # dims per column
    grp, u = divmod(off, 16)
    if u < 4:
        half, place = 0, u
    elif u < 8:
        half, place = 1, u - 4
    elif u < 12:
        half, place = 0, u - 4
    else:
        half, place = 1, u - 8
    return float(slab[grp][half][d // width][place][d % width])


def _to_f32(x):
    import struct
    return struct.unpack("f", struct.pack("f", float(x)))[0]


def e4m3_value(code):
    """One OCP E4M3 code as a Python float, bit field by bit field."""
    sign = -1.0 if code & 0x80 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return math.nan
    if exponent == 0:
        return sign * mantissa * 2.0 ** -9           # subnormal: (m / 8) * 2^-6
    return sign * (8 + mantissa) * 2.0 ** (exponent - 10)   # (1 + m / 8) * 2^(e - 7)
