"""Seeded synthetic inputs for paged-attention decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the HIP path's tests/bench and the CPU oracle
can consume what it produces without sharing code.

Layouts (the library's contract):
    q, out        [T, H_q, D], T = sum(query_lens), packed in sequence order
    k_cache       [num_blocks, H_kv, block_size/16, 2, D/8, 8, 8]  (16-slot
                  groups; slot s of a group sits in half (s >> 2) & 1, at
                  place (s & 3) | ((s >> 3) << 2) of that half's [D/8][8][8]
                  tile of 8-dim columns).  Shapes the library does not take
                  (block_size < 16 or D not a multiple of 8, used only to pin
                  the oracle) keep one row per slot: [num_blocks, H_kv, bs, D]
    v_cache       [num_blocks, H_kv, block_size/8, D, 8]  (8-slot groups, each a
                  [D, 8] tile; blocks smaller than 8 use one group of bs)
    FP8 KV (kv_dtype "fp8"): OCP E4M3 codes (torch.float8_e4m3fn) with the same
                  tiles at 16 one-byte elements per 16 bytes: k_cache
                  [num_blocks, H_kv, bs/16, 2, D/16, 8, 16], v_cache
                  [num_blocks, H_kv, bs/16, D, 16]; value = code * k_scale
                  (v_scale), per-tensor float32 scales on the device
    FP8 queries (q_dtype "fp8"): q holds the E4M3 codes of the same N(0, 1)
                  draws (nearest code of x / q_scale); out stays bf16
    block_tables  int32 [B, max_blocks_per_seq]
    seq_lens      int32 [B]  (context length, query tokens included)
    query_lens    int32 [B]

Recipe: lengths and block tables come from a CPU
``torch.Generator`` seeded with the workload's seed; the pool holds
ceil(1.25 x needed) blocks unless the workload fixes it, and a seeded random
permutation of the pool is dealt out to the sequences in order.  Table
entries past a sequence's last block point at an unused pool block.  Q, K and
V are N(0, 1) drawn in float32 with a generator seeded from the same seed on
the target device, then rounded to the workload dtype (round-to-nearest-
even).  FP8 caches divide the N(0, 1) draws by the workload's scale, clamp
to the format's +-448 and round to the nearest E4M3 code.  With
``poison=True`` every pool block no table uses, and every slot at or past
seq_len in a sequence's last block, is filled with NaN, so any read of
memory outside the context shows up in the output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16" (q, k, v and out share it)
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    query_len: int
    windows: tuple
    scale: float
    seed: int
    max_blocks_per_seq: int
    max_seq_len: int           # host-known upper bound on seq_lens
    seq_lens: tuple = ()       # fixed lengths, or ...
    len_range: tuple = ()      # ... uniform integers in [lo, hi]
    query_lens: tuple = ()     # per-sequence query lengths (default: query_len each)
    pool: int = 0              # physical blocks; 0 = ceil(1.25 x needed)
    description: str = ""
    kv_dtype: str = ""         # "" = the workload dtype, "fp8" = OCP E4M3 codes + scales
    k_scale: float = 0.0123    # FP8 only: K value = code * k_scale
    v_scale: float = 0.0157    # FP8 only: V value = code * v_scale
    q_dtype: str = ""          # "" = the workload dtype, "fp8" = OCP E4M3 codes + q_scale
    q_scale: float = 0.0371    # FP8 query only: Q value = code * q_scale


WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", dtype="f32", batch=2, num_q_heads=4, num_kv_heads=1,
        head_dim=64, block_size=16, query_len=1, windows=(0, 5), scale=1.0 / 8.0,
        seed=1, max_blocks_per_seq=4, max_seq_len=50, seq_lens=(37, 50), pool=16,
        description="tiny fp32 paged decode: B=2, 4/1 heads, D=64, bs=16, "
                    "pool 16, context 37 and 50, q_len 1, window 0 and 5"),
    "gqa_bf16": Workload(
        name="gqa_bf16", dtype="bf16", batch=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, query_len=1, windows=(0,),
        scale=1.0 / math.sqrt(128.0), seed=2, max_blocks_per_seq=512,
        max_seq_len=8192, len_range=(512, 8192),
        description="GQA decode bf16: B=32, 32/8 heads, D=128, bs=16, "
                    "context U[512, 8192], q_len 1, window 0"),
    "swa_mtp_bf16": Workload(
        name="swa_mtp_bf16", dtype="bf16", batch=64, num_q_heads=64, num_kv_heads=8,
        head_dim=64, block_size=64, query_len=4, windows=(128,), scale=1.0 / 8.0,
        seed=3, max_blocks_per_seq=512, max_seq_len=32768, len_range=(1024, 32768),
        description="sliding-window MTP decode bf16: B=64, 64/8 heads, D=64, "
                    "bs=64, context U[1024, 32768], q_len 4, window 128"),
    "long_splitk_bf16": Workload(
        name="long_splitk_bf16", dtype="bf16", batch=1, num_q_heads=8, num_kv_heads=1,
        head_dim=128, block_size=16, query_len=1, windows=(0,),
        scale=1.0 / math.sqrt(128.0), seed=4, max_blocks_per_seq=8192,
        max_seq_len=131072, seq_lens=(131072,), pool=10240,
        description="single-KV-group long-context split-K decode bf16: B=1, "
                    "8/1 heads, D=128, bs=16, context 131072, q_len 1, window 0"),
    "gqa_f32": Workload(
        name="gqa_f32", dtype="f32", batch=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, query_len=1, windows=(0,),
        scale=1.0 / math.sqrt(128.0), seed=2, max_blocks_per_seq=512,
        max_seq_len=8192, len_range=(512, 8192),
        description="GQA decode fp32 (the GQA batch in float32): B=32, 32/8 heads, D=128, "
                    "bs=16, context U[512, 8192], q_len 1, window 0"),
    "gqa_fp8kv": Workload(
        name="gqa_fp8kv", dtype="bf16", kv_dtype="fp8", batch=32, num_q_heads=32,
        num_kv_heads=8, head_dim=128, block_size=16, query_len=1, windows=(0,),
        scale=1.0 / math.sqrt(128.0), seed=2, max_blocks_per_seq=512,
        max_seq_len=8192, len_range=(512, 8192),
        description="GQA decode, bf16 queries over an FP8 (E4M3) KV cache with "
                    "per-tensor scales: B=32, 32/8 heads, D=128, bs=16, "
                    "context U[512, 8192], q_len 1, window 0"),
    "gqa_fp8qkv": Workload(
        name="gqa_fp8qkv", dtype="bf16", kv_dtype="fp8", q_dtype="fp8", batch=32,
        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, query_len=1,
        windows=(0,), scale=1.0 / math.sqrt(128.0), seed=2, max_blocks_per_seq=512,
        max_seq_len=8192, len_range=(512, 8192),
        description="GQA decode, FP8 (E4M3) queries over an FP8 KV cache with "
                    "per-tensor scales, bf16 out: B=32, 32/8 heads, D=128, bs=16, "
                    "context U[512, 8192], q_len 1, window 0"),
    "d256_decode_bf16": Workload(
        name="d256_decode_bf16", dtype="bf16", batch=1, num_q_heads=16, num_kv_heads=2,
        head_dim=256, block_size=16, query_len=1, windows=(0,), scale=1.0 / 16.0, seed=6,
        max_blocks_per_seq=1024, max_seq_len=16384, seq_lens=(16384,), pool=1280,
        description="head-dim-256 decode bf16 (the split-K decode benchmark shape of "
                    "executorch PR #18759: B=1, 16/2 heads, D=256), bs=16, context 16384, "
                    "q_len 1"),
    "gqa_d256_bf16": Workload(
        name="gqa_d256_bf16", dtype="bf16", batch=32, num_q_heads=16, num_kv_heads=2,
        head_dim=256, block_size=16, query_len=1, windows=(0,), scale=1.0 / 16.0, seed=9,
        max_blocks_per_seq=512, max_seq_len=8192, len_range=(512, 8192),
        description="GQA decode bf16 at head dim 256: B=32, 16/2 heads, D=256, bs=16, "
                    "context U[512, 8192], q_len 1, window 0"),
    "prefill_chunk_bf16": Workload(
        name="prefill_chunk_bf16", dtype="bf16", batch=16, num_q_heads=32, num_kv_heads=4,
        head_dim=128, block_size=16, query_len=16, windows=(0,),
        scale=1.0 / math.sqrt(128.0), seed=7, max_blocks_per_seq=512, max_seq_len=8192,
        len_range=(2048, 8192),
        description="mixed-batch rows beyond one tile: B=16, 32/4 heads (G=8), D=128, "
                    "bs=16, 16 query tokens per sequence (128 packed rows per KV head), "
                    "context U[2048, 8192], window 0"),
    "large_block_mtp_bf16": Workload(
        name="large_block_mtp_bf16", dtype="bf16", batch=128, num_q_heads=64,
        num_kv_heads=8, head_dim=128, block_size=1024, query_len=2, windows=(0, 4096),
        scale=1.0 / math.sqrt(128.0), seed=5, max_blocks_per_seq=64,
        max_seq_len=65536, len_range=(2048, 65536),
        description="large-block mixed-window MTP decode bf16: B=128, 64/8 heads, "
                    "D=128, bs=1024, context U[2048, 65536], q_len 2, window 0 / 4096"),
}


def k_tiled(block_size: int, head_dim: int, elem_bytes: int = 2) -> bool:
    """True when the K cache takes the 16-slot tiled layout."""
    return block_size % 16 == 0 and head_dim % (16 // elem_bytes) == 0


def k_slot(slot):
    """(group, half, place) of block slot(s) ``slot`` in the tiled K layout."""
    u = slot % 16
    return slot // 16, (u // 4) % 2, u % 4 + 4 * (u // 8)


def read_k_row(k_cache, blk, h, slot):
    """Copy of the D elements of one slot's key, for either K layout."""
    if k_cache.dim() == 4:
        return k_cache[blk, h, slot].clone()
    c, half, j = k_slot(slot)
    return k_cache[blk, h, c, half, :, j, :].reshape(-1).clone()


def write_k_row(k_cache, blk, h, slot, row):
    """Stores the D-vector ``row`` as the key of one slot, for either K layout
    (``row`` already in the cache's element type)."""
    if k_cache.dim() == 4:
        k_cache[blk, h, slot] = row
    else:
        c, half, j = k_slot(slot)
        k_cache[blk, h, c, half, :, j, :] = row.reshape(-1, k_cache.shape[-1])


def to_e4m3(x: torch.Tensor, scale: float) -> torch.Tensor:
    """Nearest OCP E4M3 codes of x / scale, saturated at +-448."""
    return (x.float() / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclass
class Case:
    """One realised input set; tensors live on ``device``."""
    w: Workload
    window: int
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    query_lens: torch.Tensor
    seq_lens_host: list
    query_lens_host: list
    tables_host: torch.Tensor
    used_blocks: list           # per sequence, physical ids in logical order
    unused_blocks: list
    extra: dict = field(default_factory=dict)
    k_scale: torch.Tensor | None = None   # FP8 caches: float32 [1] on the device
    v_scale: torch.Tensor | None = None
    q_scale: torch.Tensor | None = None   # FP8 queries: float32 [1] on the device

    @property
    def scale(self) -> float:
        return self.w.scale

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    def new_out(self) -> torch.Tensor:
        return torch.empty(self.q.shape, dtype=torch_dtype(self.w.dtype), device=self.q.device)


def _lengths(w: Workload, g: torch.Generator) -> tuple[list, list]:
    if w.seq_lens:
        lens = [int(x) for x in w.seq_lens]
    else:
        lo, hi = w.len_range
        lens = [int(x) for x in torch.randint(lo, hi + 1, (w.batch,), generator=g)]
    if w.query_lens:
        qls = [int(x) for x in w.query_lens]
    else:
        qls = [w.query_len] * w.batch
    return lens, qls


def _fill_normal(t: torch.Tensor, gen: torch.Generator, chunk_elems: int = 1 << 28):
    """Fill ``t`` with N(0,1) drawn in float32 then rounded to t.dtype."""
    flat = t.view(-1)
    n = flat.numel()
    i = 0
    while i < n:
        m = min(chunk_elems, n - i)
        flat[i:i + m] = torch.randn(m, generator=gen, device=t.device, dtype=torch.float32)
        i += m


def make_case(w: Workload | str, device="cpu", window: int | None = None,
              poison: bool = True, q_gain: float = 1.0) -> Case:
    """Build the seeded inputs of workload ``w`` on ``device``.

    ``q_gain`` multiplies Q before rounding (a "peaked" variant with larger
    logits); ``window`` defaults to the workload's first window.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if window is None:
        window = w.windows[0]
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    lens, qls = _lengths(w, g)
    bs = w.block_size
    nblk = [-(-L // bs) for L in lens]
    needed = sum(nblk)
    pool = w.pool if w.pool else math.ceil(1.25 * needed)
    pool = max(pool, needed + 1)           # keep one unused block for table padding
    perm = torch.randperm(pool, generator=g).tolist()
    used, off = [], 0
    for n in nblk:
        used.append(perm[off:off + n])
        off += n
    unused = perm[needed:]
    if max(nblk, default=0) > w.max_blocks_per_seq:
        raise ValueError("max_blocks_per_seq too small for the drawn lengths")
    # row b holds its blocks' ids in order, then the padding id
    counts = np.asarray(nblk, dtype=np.int64)
    rows = np.repeat(np.arange(w.batch), counts)
    cols = np.arange(needed) - np.repeat(np.cumsum(counts) - counts, counts)
    tab = np.full((w.batch, w.max_blocks_per_seq), unused[0], dtype=np.int32)
    tab[rows, cols] = np.asarray(perm[:needed], dtype=np.int32)
    tables = torch.from_numpy(tab)

    dt = torch_dtype(w.dtype)
    dev = torch.device(device)
    vg = torch.Generator(device=dev).manual_seed(w.seed * 7919 + 17)
    T = sum(qls)
    q = torch.empty((T, w.num_q_heads, w.head_dim), dtype=dt, device=dev)
    _fill_normal(q, vg)
    if q_gain != 1.0:
        q.copy_((q.float() * q_gain).to(dt))
    if w.q_dtype == "fp8":
        q = to_e4m3(q, w.q_scale)
    D = w.head_dim
    fp8 = w.kv_dtype == "fp8"
    E = 16 if fp8 else 8                    # elements per 16-byte column / V group
    tiled = k_tiled(bs, D, 1 if fp8 else 2)
    kshape = (pool, w.num_kv_heads, bs // 16, 2, D // E, 8, E) if tiled else \
        (pool, w.num_kv_heads, bs, D)
    g = min(E, bs)
    vshape = (pool, w.num_kv_heads, bs // g, w.head_dim, g)
    if fp8:
        k = torch.empty(kshape, dtype=torch.float32, device=dev)
        v = torch.empty(vshape, dtype=torch.float32, device=dev)
        _fill_normal(k, vg)
        _fill_normal(v, vg)
        k = to_e4m3(k, w.k_scale)
        v = to_e4m3(v, w.v_scale)
    else:
        k = torch.empty(kshape, dtype=dt, device=dev)
        v = torch.empty(vshape, dtype=dt, device=dev)
        _fill_normal(k, vg)
        _fill_normal(v, vg)
    nan = float("nan")
    if poison:
        if unused:
            ids = torch.tensor(unused, dtype=torch.long, device=dev)
            if fp8:   # E4M3 NaN code 0x7F in every byte
                k.view(torch.uint8).index_fill_(0, ids, 0x7F)
                v.view(torch.uint8).index_fill_(0, ids, 0x7F)
            else:
                k.index_fill_(0, ids, nan)
                v.index_fill_(0, ids, nan)
        # slots past each sequence's end in its last block, all at once
        last, slot = [], []
        for b, L in enumerate(lens):
            tail = L % bs
            if tail and used[b]:
                last.append(np.full(bs - tail, used[b][-1], dtype=np.int64))
                slot.append(np.arange(tail, bs, dtype=np.int64))
        if last:
            blk = torch.from_numpy(np.concatenate(last)).to(dev)
            slots = torch.from_numpy(np.concatenate(slot)).to(dev)
            kb = k.view(torch.uint8) if fp8 else k
            vb = v.view(torch.uint8) if fp8 else v
            bad = 0x7F if fp8 else nan
            if tiled:
                c, half, j = k_slot(slots)
                kb[blk, :, c, half, :, j, :] = bad
            else:
                kb[blk, :, slots, :] = bad
            vb[blk, :, slots // g, :, slots % g] = bad
    return Case(
        w=w, window=int(window), q=q, k_cache=k, v_cache=v,
        block_tables=tables.to(dev), seq_lens=torch.tensor(lens, dtype=torch.int32, device=dev),
        query_lens=torch.tensor(qls, dtype=torch.int32, device=dev),
        seq_lens_host=lens, query_lens_host=qls, tables_host=tables,
        used_blocks=used, unused_blocks=unused,
        k_scale=torch.tensor([w.k_scale], dtype=torch.float32, device=dev) if fp8 else None,
        v_scale=torch.tensor([w.v_scale], dtype=torch.float32, device=dev) if fp8 else None,
        q_scale=torch.tensor([w.q_scale], dtype=torch.float32, device=dev)
        if w.q_dtype == "fp8" else None)


def with_context(w: Workload, L: int) -> Workload:
    """``w`` with every sequence exactly ``L`` positions long (its block
    tables sized for that, a fresh pool)."""
    return replace(w, seq_lens=(int(L),) * w.batch, len_range=(), max_seq_len=int(L),
                   max_blocks_per_seq=-(-int(L) // w.block_size) + 1, pool=0,
                   query_lens=())


def custom(name="custom", **kw) -> Workload:
    """A workload built from keyword overrides of the tiny fp32 one."""
    base = WORKLOADS["tiny_f32"]
    kw.setdefault("name", name)
    return replace(base, **kw)
