"""Float64 reference for paged-attention decode (test infrastructure only).

Nothing here is tuned: it is the definition written out, read against the
pages listed in ``oracle/__init__.py``.  Inputs are NumPy arrays (any float
dtype; they are widened to float64 exactly), in the layouts the library uses:

    q            [T, H_q, D]          T = sum(query_lens); sequence b owns rows
                                      qoff_b .. qoff_b + query_lens[b] - 1,
                                      qoff_b = query_lens[0] + ... + query_lens[b-1]
    k_cache      [num_blocks, H_kv, block_size, D]   (row per position), or
                 the library's tiled form [num_blocks, H_kv, block_size/16, 2,
                 D/E, 8, E] (E = 8 for bf16, 16 for FP8): within each group of
                 16 slots, slot s lies in half (s // 4) % 2 at place
                 s % 4 + 4 * (s // 8), and its dim d at column d // E,
                 element d % E of that place
    v_cache      [num_blocks, H_kv, block_size/g, D, g]   (positions grouped by
                 g: for each group of g consecutive slots, a [D, g] tile; the
                 library uses g = 8 for bf16 and g = 16 for FP8, tests with
                 blocks smaller than 8 use g = bs)
    block_tables [B, max_blocks_per_seq] int
    seq_lens     [B] int   context length, the query tokens included
    query_lens   [B] int   trailing query tokens of each context

The cache layouts are a reading: the pages name a paged KV cache with a block
size (aiter PR #2914 summary: "KV_BLOCK_SIZE=1024 path") but never its
physical layout.  FP8 caches use the same tiled forms with 16 one-byte
elements where bf16 has 8 two-byte ones (K columns of 16 dims, V groups of 16
slots); ``dequantize`` turns their codes into values first, and the gathers
below read the column and group widths from the array shapes.
"""

from __future__ import annotations

import math

import numpy as np


def decode_e4m3(codes):
    """Values of 8-bit floating-point codes in the OCP E4M3 format: sign bit,
    4 exponent bits (bias 7), 3 mantissa bits; exponent 0 holds the
    subnormals m/8 * 2^-6; the code with all exponent and mantissa bits set is
    NaN; there are no infinities.  Returns float64 (exact)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * val
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def dequantize(codes, scale):
    """An FP8 cache as float64 values: code value times the per-tensor scale
    (aiter PR #2914, review of ``pa_decode_gluon``: FP8 key and value caches
    come with key_scale / value_scale).  The layout is kept."""
    return decode_e4m3(codes) * float(np.float32(scale))


def row_position(seq_len: int, query_len: int, i: int) -> int:
    """Absolute position of query token ``i`` of a sequence.

    Reading: the query tokens are the last ``query_len`` positions of the
    ``seq_len``-position context (gllm #116 "Verification": its GPU test puts
    5 query tokens at the end of a context of 300 positions; aiter PR #2914:
    MTP decode), so their keys and values are already in the cache.
    """
    return seq_len - query_len + i


def visible_range(seq_len: int, query_len: int, i: int, window: int) -> tuple[int, int]:
    """Inclusive range [lo, p] of positions query token ``i`` attends to.

    gllm #116, summary: a positive window restricts the query at position p
    to the ``window`` positions ending at p itself; a zero window keeps causal
    attention unlimited.
    "What changes — CPU reference": its lower end is max(0, end - window)
    with end = p + 1.
    """
    p = row_position(seq_len, query_len, i)
    lo = 0 if window == 0 else max(0, p + 1 - window)
    return lo, p


def check_args(q, block_tables, seq_lens, query_lens, num_kv_heads, block_size, window):
    """Preconditions of the definition; the oracle raises where the GPU
    behaviour is undefined (query_len > seq_len, blocks missing)."""
    T, H_q, _ = q.shape
    if H_q % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if window < 0:
        raise ValueError("window must be >= 0")
    if int(np.sum(query_lens)) != T:
        raise ValueError("q rows must equal sum(query_lens)")
    for b in range(len(seq_lens)):
        L, qb = int(seq_lens[b]), int(query_lens[b])
        if qb < 0 or qb > L:
            raise ValueError(f"sequence {b}: need 0 <= query_len <= seq_len")
        if -(-L // block_size) > block_tables.shape[1]:
            raise ValueError(f"sequence {b}: block table too short")


def gather_keys(k_cache, table_row, positions, h, block_size):
    """K rows of positions t (slot s = t % bs of block table[t // bs]) -> [n, D]."""
    blocks = table_row[positions // block_size]
    offs = positions % block_size
    if k_cache.ndim == 4:
        return k_cache[blocks, h, offs, :].astype(np.float64)
    n = len(positions)
    grp, u = offs // 16, offs % 16
    half = (u // 4) % 2
    place = u % 4 + 4 * (u // 8)
    cols = k_cache[blocks, h, grp, half, :, place, :]        # [n, D/E columns, E]
    return cols.reshape(n, k_cache.shape[4] * k_cache.shape[6]).astype(np.float64)


def gather_values(v_cache, table_row, positions, h, block_size):
    """V rows of positions t: with slot s = t % bs and group size g,
    v_cache[table[t // bs], h, s // g, :, s % g] -> [n, D]."""
    g = v_cache.shape[-1]
    blocks = table_row[positions // block_size]
    offs = positions % block_size
    return v_cache[blocks, h, offs // g, :, offs % g].astype(np.float64)   # [n, D]


def decode(q, k_cache, v_cache, block_tables, seq_lens, query_lens,
           scale, window, num_kv_heads, block_size, rows=None):
    """Paged-attention decode output, float64 [T, H_q, D].

    For each sequence b, query token i and query head h_q:
      p = L_b - q_b + i; h = h_q // G with G = H_q // H_kv;
      visible positions V = [lo, p] (``visible_range``);
      s_t = scale * <q, k_t> for t in V; w = softmax(s); out = sum_t w_t v_t.
    ``scale`` is taken as the float32 value the library receives, widened.
    ``rows`` optionally restricts the work to a set of (b, i) pairs (used to
    sample very large workloads); other rows are left at NaN.
    """
    q = np.asarray(q)
    block_tables = np.asarray(block_tables)
    seq_lens = np.asarray(seq_lens)
    query_lens = np.asarray(query_lens)
    check_args(q, block_tables, seq_lens, query_lens, num_kv_heads, block_size, window)
    T, H_q, D = q.shape
    G = H_q // num_kv_heads
    sigma = float(np.float32(scale))
    out = np.full((T, H_q, D), np.nan if rows is not None else 0.0, dtype=np.float64)
    want = None if rows is None else set((int(b), int(i)) for b, i in rows)
    qoff = 0
    for b in range(len(seq_lens)):
        L, qb = int(seq_lens[b]), int(query_lens[b])
        for i in range(qb):
            if want is not None and (b, i) not in want:
                continue
            lo, p = visible_range(L, qb, i, window)
            pos = np.arange(lo, p + 1, dtype=np.int64)
            for h in range(num_kv_heads):
                K = gather_keys(k_cache, block_tables[b], pos, h, block_size)      # [n, D]
                V = gather_values(v_cache, block_tables[b], pos, h, block_size)    # [n, D]
                Q = q[qoff + i, h * G:(h + 1) * G, :].astype(np.float64)          # [G, D]
                s = sigma * (Q @ K.T)                                             # [G, n]
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                w = e / e.sum(axis=1, keepdims=True)
                assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-12)
                out[qoff + i, h * G:(h + 1) * G, :] = w @ V
        qoff += qb
    return out


def partial_state(s, V):
    """One partition's (max logit, exp-sum, normalised partial output).

    Split-K decode (executorch PR #18759, Copilot overview; aiter PR #2914
    workspace ``max_logits`` / ``exp_sums`` / ``temporary_output``).  A
    partition holding no visible position adds zero weight to the merge
    (gllm #116, "What changes", CUDA kernels: a split whose window leaves it
    no positions is left out of the combine): m = -inf, l = 0, o = 0.
    """
    if s.size == 0:
        return -math.inf, 0.0, np.zeros(V.shape[1])
    m = float(s.max())
    e = np.exp(s - m)
    l = float(e.sum())
    return m, l, (e @ V) / l


def merge_states(states):
    """Log-sum-exp merge of partition states into the final output.

    M = max over partitions with a finite max; each partition is weighted by
    exp(m_j - M) * l_j (zero for an empty one); out = weighted sum of the
    normalised partial outputs divided by the sum of weights.
    """
    finite = [m for m, _, _ in states if m != -math.inf]
    if not finite:
        raise ValueError("no partition holds a visible position")
    M = max(finite)
    num = 0.0
    den = 0.0
    for m, l, o in states:
        if m == -math.inf:
            continue
        a = math.exp(m - M) * l
        num = num + a * o
        den += a
    return num / den


def decode_split(q, k_cache, v_cache, block_tables, seq_lens, query_lens,
                 scale, window, num_kv_heads, block_size, boundaries):
    """Split-K decode in float64: partition, per-partition state, LSE merge.

    ``boundaries(b)`` returns the increasing absolute positions at which the
    context of sequence b is cut into partitions (any cut points; empty
    partitions allowed).  Must agree with ``decode`` up to rounding.
    """
    q = np.asarray(q)
    block_tables = np.asarray(block_tables)
    check_args(q, block_tables, seq_lens, query_lens, num_kv_heads, block_size, window)
    T, H_q, D = q.shape
    G = H_q // num_kv_heads
    sigma = float(np.float32(scale))
    out = np.zeros((T, H_q, D))
    qoff = 0
    for b in range(len(seq_lens)):
        L, qb = int(seq_lens[b]), int(query_lens[b])
        cuts = [0] + [int(c) for c in boundaries(b)] + [L]
        for i in range(qb):
            lo, p = visible_range(L, qb, i, window)
            for hq in range(H_q):
                h = hq // G
                qv = q[qoff + i, hq].astype(np.float64)
                states = []
                for a, z in zip(cuts[:-1], cuts[1:]):
                    pos = np.arange(max(a, lo), min(z, p + 1), dtype=np.int64)
                    K = gather_keys(k_cache, block_tables[b], pos, h, block_size)
                    V = gather_values(v_cache, block_tables[b], pos, h, block_size)
                    states.append(partial_state(sigma * (K @ qv), V))
                out[qoff + i, hq] = merge_states(states)
        qoff += qb
    return out


def spans(block_tables, seq_lens, query_lens, window, block_size):
    """Integer index facts the GPU must reproduce bit-exactly.

    Per sequence b: ``qoff`` (first q/out row), ``lo``/``hi`` (the union of
    its rows' visible ranges is [lo, hi), hi = seq_len), per query token the
    inclusive visible range (lo_i, p_i), and ``blocks``: for every logical
    block index k that holds a visible position, the physical block id
    block_tables[b][k]; -1 for logical blocks no row can see.
    """
    block_tables = np.asarray(block_tables)
    res = []
    qoff = 0
    for b in range(len(seq_lens)):
        L, qb = int(seq_lens[b]), int(query_lens[b])
        rows = [visible_range(L, qb, i, window) for i in range(qb)]
        blocks = np.full(block_tables.shape[1], -1, dtype=np.int64)
        if qb > 0:
            lo = min(r[0] for r in rows)
            hi = max(r[1] for r in rows) + 1
            for t in range(lo, hi):
                blocks[t // block_size] = block_tables[b, t // block_size]
        else:
            lo = hi = L
        res.append(dict(qoff=qoff, lo=lo, hi=hi, rows=rows, blocks=blocks))
        qoff += qb
    return res
