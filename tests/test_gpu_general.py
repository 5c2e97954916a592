"""GPU parity for general shapes: more than 64 packed rows per KV head (row
blocks), head dim 256 (matrix cores) and head dims off the 8-dim grid (the
vector kernel, K one row per slot), against the float64 oracle.

The mixed batch follows the GPU test of gllm "feat(backend): sliding-window
PagedAttention" (#116), "Verification": one sequence ends in 5 query tokens
at context length 300, the other decodes a single token at context length
40; windows 16, 100 and 4096; head dims 64 and 66.  Values are synthetic
(seeded N(0, 1)); the pages print none.
"""

from dataclasses import replace

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


def mixed_batch(D, dtype):
    return workloads.custom(
        name=f"gllm_mixed_d{D}_{dtype}", dtype=dtype, batch=2, num_q_heads=8, num_kv_heads=2,
        head_dim=D, block_size=16, query_len=5, query_lens=(5, 1), seq_lens=(300, 40),
        max_seq_len=300, max_blocks_per_seq=20, pool=0, seed=116,
        scale=float(1.0 / np.sqrt(D)), windows=(16,))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 66])
def test_gllm_mixed_batch(D, dtype):
    w = mixed_batch(D, dtype)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    paths = [pa.PATH_AUTO, pa.PATH_VALU] if (dtype == "bf16" and D == 64) else [pa.PATH_AUTO]
    for win in (16, 100, 4096, 0):
        c = workloads.make_case(w, device="cuda", window=win)
        exp, rows = oracle_out(c)
        for path in paths:
            for P in (0, 32, 96):
                say(f"[case] gllm mixed D={D} {dtype} window={win} path={path} P={P}")
                compare(run_gpu(c, path=path, part_size=P), exp, rows, tol,
                        f"gllm mixed D={D} {dtype} w={win} path={path} P={P}")


def many_rows(seed, D, dtype, kv="", G=8, ql=12):
    r = np.random.default_rng(seed)
    B = int(r.integers(1, 4))
    lens = tuple(int(x) for x in r.integers(ql, 900, size=B))
    qls = tuple(int(x) for x in r.integers(1, ql + 1, size=B))
    mx = max(lens)
    return workloads.custom(
        name=f"rows{seed}", dtype=dtype, kv_dtype=kv, batch=B, num_q_heads=2 * G, num_kv_heads=2,
        head_dim=D, block_size=int(r.choice([16, 64])), query_len=ql, query_lens=qls,
        seq_lens=lens, max_seq_len=mx, max_blocks_per_seq=mx // 16 + 2, pool=0,
        seed=3000 + seed, scale=float(1.0 / np.sqrt(D)), windows=(0,))


ROWS_CASES = [(64, "bf16", ""), (128, "bf16", ""), (128, "bf16", "fp8"), (256, "bf16", ""),
              (256, "bf16", "fp8"), (64, "f32", ""), (66, "bf16", ""), (200, "f32", "")]


@pytest.mark.parametrize("D,dtype,kv", ROWS_CASES,
                         ids=[f"d{d}-{t}{'-' + k if k else ''}" for d, t, k in ROWS_CASES])
@pytest.mark.parametrize("seed", range(3))
def test_more_than_64_rows(seed, D, dtype, kv):
    """G = 8 and up to 12 query tokens: up to 96 packed rows per KV head, so
    several row blocks per partition (also with ragged query_lens)."""
    w = many_rows(seed, D, dtype, kv)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    for win in (0, 7, 300):
        c = workloads.make_case(w, device="cuda", window=win)
        exp, rows = oracle_out(c)
        for P in (0, 64):
            plan = pa.plan(pa.dims_for(c.q, c.k_cache, c.block_tables, w.query_len, w.max_seq_len),
                           win, w.num_kv_heads, w.block_size, part_size=P)
            say(f"[case] rows seed={seed} D={D} {dtype} kv={kv} w={win} P={P} "
                f"row_blocks={plan['row_blocks']} row_tiles={plan['row_tiles']} path={plan['path']}")
            assert plan["row_blocks"] > 1
            compare(run_gpu(c, part_size=P), exp, rows, tol,
                    f"rows{seed} D={D} {dtype} kv={kv} w={win} P={P}")


@pytest.mark.parametrize("kv", ["", "fp8"])
@pytest.mark.parametrize("seed", range(4))
def test_head_dim_256_small(seed, kv):
    from tests.test_gpu_parity import small
    w = small(seed, head_dim=256, kv_dtype=kv)
    for win in (0, 5, 100000):
        c = workloads.make_case(w, device="cuda", window=win)
        exp, rows = oracle_out(c)
        for sched in (pa.SCHED_GRID, pa.SCHED_PERSISTENT):
            for P in (0, 32):
                if sched == pa.SCHED_PERSISTENT and (w.num_q_heads // w.num_kv_heads) * w.query_len > 16:
                    continue        # D = 256 keeps 16 rows per workgroup: grid only above that
                compare(run_gpu(c, part_size=P, schedule=sched), exp, rows, BF16_TOL,
                        f"d256 small{seed} kv={kv} w={win} sched={sched} P={P}")


@pytest.mark.parametrize("name", ["d256_decode_bf16", "gqa_d256_bf16", "prefill_chunk_bf16"])
def test_general_workloads(name):
    w = workloads.WORKLOADS[name]
    c = workloads.make_case(w, device="cuda")
    out = run_gpu(c)
    seqs = list(range(w.batch)) if w.batch <= 4 else [0, 5, 11, 15]
    exp, rows = oracle_out(c, seqs)
    compare(out, exp, rows, BF16_TOL, name)
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("D,dtype", [(66, "bf16"), (66, "f32"), (200, "f32")])
def test_vector_kernel_nan_poison(D, dtype):
    """Invisible blocks and tail slots hold NaN (K one row per slot at D = 66):
    output bit-identical to a clean run, with several row blocks."""
    w = many_rows(7, D, dtype)
    for win in (0, 9):
        for P in (0, 32):
            clean = run_gpu(workloads.make_case(w, device="cuda", window=win, poison=False),
                            part_size=P).clone()
            dirty = run_gpu(workloads.make_case(w, device="cuda", window=win, poison=True),
                            part_size=P)
            assert torch.equal(clean, dirty), (D, dtype, win, P)


MERGE_ODD = [(66, "bf16"), (200, "f32")]


@pytest.mark.parametrize("D,dtype", MERGE_ODD, ids=[f"d{d}-{t}" for d, t in MERGE_ODD])
def test_merge_lanes_with_partial_unit_blocks(D, dtype):
    """Merges with 16 and 32 lanes per output unit where the unit count per
    (sequence, KV head), rows x D / VEC, is not a multiple of a workgroup's
    units: the last workgroup holds lanes past the last row."""
    w = workloads.custom(
        name=f"merge_odd_d{D}_{dtype}", dtype=dtype, batch=2, num_q_heads=8, num_kv_heads=2,
        head_dim=D, block_size=16, query_len=3, query_lens=(3, 2), seq_lens=(9000, 70),
        max_seq_len=9000, max_blocks_per_seq=563, pool=0, seed=4242,
        scale=float(1.0 / np.sqrt(D)), windows=(0,))
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    for win in (0, 5000):
        c = workloads.make_case(w, device="cuda", window=win)
        exp, rows = oracle_out(c)
        for P in (32, 64):   # 282 / 141 partitions at window 0: 32- and 16-lane merges
            say(f"[case] merge odd units D={D} {dtype} w={win} P={P}")
            compare(run_gpu(c, part_size=P), exp, rows, tol,
                    f"merge odd D={D} {dtype} w={win} P={P}")


MAX_ROWS = [(64, "bf16", ""), (128, "bf16", ""), (256, "bf16", ""), (128, "bf16", "fp8"),
            (64, "f32", "")]


@pytest.mark.parametrize("D,dtype,kv", MAX_ROWS,
                         ids=[f"d{d}-{t}{'-' + k if k else ''}" for d, t, k in MAX_ROWS])
def test_maximum_rows(D, dtype, kv):
    """1024 packed rows per KV head, the most the library takes (G = 8 and 128
    query tokens): 16 to 64 row blocks per partition."""
    w = workloads.custom(
        name=f"rows1024_d{D}_{dtype}{kv}", dtype=dtype, kv_dtype=kv, batch=2, num_q_heads=16,
        num_kv_heads=2, head_dim=D, block_size=16, query_len=128, query_lens=(128, 77),
        seq_lens=(300, 150), max_seq_len=300, max_blocks_per_seq=20, pool=0, seed=1024 + D,
        scale=float(1.0 / np.sqrt(D)), windows=(0,))
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    for win in (0, 50):
        c = workloads.make_case(w, device="cuda", window=win)
        exp, rows = oracle_out(c)
        for P in (0, 64):
            say(f"[case] 1024 rows D={D} {dtype} kv={kv} w={win} P={P}")
            compare(run_gpu(c, part_size=P), exp, rows, tol, f"1024 rows D={D} {dtype} w={win} P={P}")
