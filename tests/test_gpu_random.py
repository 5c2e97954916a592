"""GPU parity on seeded random shapes against the float64 oracle.

Each case draws a dtype (bf16, fp32, FP8 caches, FP8 queries), a head dim on
or off the matrix-core set, block size, GQA group, query lengths (zero
included), context lengths, window, and forced plan options (partition
size, schedule, load form, vector path), and compares every output row with
the oracle at the target tolerances.  Plans the library refuses (for
instance the persistent schedule on the vector path) are checked to be
refused before any launch and skipped.
"""

import numpy as np
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


def random_case(seed):
    r = np.random.default_rng(seed)
    dtype = "f32" if r.random() < 0.2 else "bf16"
    kv = "fp8" if (dtype == "bf16" and r.random() < 0.3) else ""
    qd = "fp8" if (kv == "fp8" and r.random() < 0.5) else ""
    D = int(r.choice([64, 128, 256] if kv else [64, 128, 256, 40, 66, 96, 200]))
    bs = int(r.choice([16, 32, 64, 128, 256, 1024]))
    hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 4, 5, 8]))
    ql = int(r.choice([1, 1, 2, 3, 4, 6, 12, 16]))
    B = int(r.integers(1, 5))
    hi = int(r.choice([40, 300, 1500, 3000]))
    lens = tuple(int(x) for x in r.integers(ql, hi + 1, size=B))
    qls = tuple(int(x) for x in r.integers(0 if r.random() < 0.2 else 1, ql + 1, size=B))
    mx = max(lens)
    w = workloads.custom(name=f"random{seed}", dtype=dtype, kv_dtype=kv, q_dtype=qd, batch=B,
                         num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D, block_size=bs,
                         query_len=ql, query_lens=qls, seq_lens=lens, max_seq_len=mx,
                         max_blocks_per_seq=-(-mx // bs) + int(r.integers(0, 3)), pool=0,
                         seed=5000 + seed, scale=float(1.0 / np.sqrt(D)), windows=(0,))
    win = int(r.choice([0, 0, 1, 2, 7, 33, 128, 1000, 100000]))
    opts = {}
    if r.random() < 0.4:
        opts["part_size"] = int(r.choice([32, 64, 96, 256, 512]))
    if r.random() < 0.3:
        opts["schedule"] = int(r.choice([pa.SCHED_GRID, pa.SCHED_PERSISTENT]))
    if r.random() < 0.2:
        opts["loads"] = int(r.choice([pa.LOADS_CACHED, pa.LOADS_STREAMING]))
    if r.random() < 0.15 and dtype == "bf16" and not kv:
        opts["path"] = pa.PATH_VALU
    return w, win, opts


@pytest.mark.parametrize("seed", range(400))
def test_random_shape(seed):
    w, win, opts = random_case(7000 + seed)
    dims = pa.make_dims(w.batch, w.num_q_heads, w.head_dim, w.query_len, w.max_seq_len,
                        w.max_blocks_per_seq, 1, pa.F32 if w.dtype == "f32" else pa.BF16,
                        pa.KV_FP8_E4M3 if w.kv_dtype else pa.KV_NATIVE,
                        pa.Q_FP8_E4M3 if w.q_dtype else pa.Q_NATIVE)
    try:
        pa.plan(dims, win, w.num_kv_heads, w.block_size, **opts)
    except pa.PaError as e:
        assert e.status == pa.ERR_UNSUPPORTED, e
        pytest.skip(f"refused as planned: {e}")
    c = workloads.make_case(w, device="cuda", window=win)
    say(f"[case] random seed={7000 + seed} {w.dtype} kv={w.kv_dtype} q={w.q_dtype} D={w.head_dim} "
        f"bs={w.block_size} H={w.num_q_heads}/{w.num_kv_heads} lens={w.seq_lens} "
        f"qls={w.query_lens} window={win} opts={opts}")
    exp, rows = oracle_out(c)
    compare(run_gpu(c, **opts), exp, rows, F32_TOL if w.dtype == "f32" else BF16_TOL,
            f"random {7000 + seed}")
