"""GPU parity: the HIP path against the float64 oracle, element by element.

Small shapes (several 32-position chunks, ragged tails, shuffled blocks, GQA,
MTP, windows, forced partition sizes, both kernel families) are compared in
full; the full-size workloads are compared on sampled sequences, in the
launch configuration the bench times.  Tolerances: max-abs 2e-2 for bf16
inputs (fp32 accumulation), 1e-4 for fp32 inputs.
"""

import numpy as np
import pytest
import torch

import decode_attention_pa_amd as pa
import workloads
from oracle import paged_attention as ref
from tests._gpu_util import (BF16_TOL, F32_TOL, compare, oracle_out, run_gpu,
                             sample_sequences, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def small(seed, dtype="bf16", **over):
    r = np.random.default_rng(seed)
    D = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2, 3]))
    G = int(r.choice([1, 2, 4, 8]))
    ql = int(r.choice([1, 2, 3, 4]))
    while G * ql > 64:
        ql -= 1
    bs = int(r.choice([16, 32, 64, 256]))
    B = int(r.integers(1, 5))
    lens = tuple(int(x) for x in r.integers(ql, 700, size=B))
    mx = max(lens)
    kw = dict(name=f"small{seed}", dtype=dtype, batch=B, num_q_heads=G * hkv, num_kv_heads=hkv,
              head_dim=D, block_size=bs, query_len=ql, seq_lens=lens, max_seq_len=mx,
              max_blocks_per_seq=-(-mx // bs) + 1, pool=0, seed=1000 + seed,
              scale=float(1.0 / np.sqrt(D)), windows=(0,))
    kw.update(over)
    return workloads.custom(**kw)


@pytest.mark.parametrize("window", [0, 5])
def test_tiny_f32(window):
    c = workloads.make_case("tiny_f32", device="cuda", window=window)
    say(f"[case] tiny_f32 window={window}")
    exp, rows = oracle_out(c)
    compare(run_gpu(c), exp, rows, F32_TOL, f"tiny_f32 w={window}")
    for P in (32, 64):
        compare(run_gpu(c, part_size=P), exp, rows, F32_TOL, f"tiny_f32 w={window} P={P}")


KERNELS = [(pa.PATH_MFMA, pa.SCHED_GRID), (pa.PATH_MFMA, pa.SCHED_PERSISTENT),
           (pa.PATH_VALU, pa.SCHED_GRID), (pa.PATH_VALU, pa.SCHED_PERSISTENT),
           (pa.PATH_VALU_LDS, pa.SCHED_GRID)]


@pytest.mark.parametrize("path,sched", KERNELS)
@pytest.mark.parametrize("seed", range(10))
def test_small_bf16(seed, path, sched):
    w = small(seed)
    rows = (w.num_q_heads // w.num_kv_heads) * w.query_len
    if path == pa.PATH_VALU and sched == pa.SCHED_PERSISTENT and rows > 8:
        pytest.skip(f"{rows} rows per KV head: the vector kernels' persistent schedule takes "
                    "every row in one workgroup of at most 8")
    for win in (0, 1, 5, 37, 100000):
        c = workloads.make_case(w, device="cuda", window=win)
        say(f"[case] small seed={seed} path={path} schedule={sched} window={win} {w}")
        exp, rows = oracle_out(c)
        for P in (0, 32, 64):
            compare(run_gpu(c, path=path, part_size=P, schedule=sched), exp, rows, BF16_TOL,
                    f"small{seed} path={path} sched={sched} w={win} P={P}")


@pytest.mark.parametrize("path,sched", KERNELS[:3])
@pytest.mark.parametrize("scale", [-0.11, 0.0, 2.5])
def test_scale_sign_and_size(scale, path, sched):
    """Scales the decode call may get besides 1/sqrt(D): negative (the
    matrix-core kernels carry its sign in the query's sign bits), zero (every
    visible position weighs the same) and large (sharp weights)."""
    w = small(13, head_dim=128, num_q_heads=16, num_kv_heads=2, query_len=2, scale=scale)
    for win in (0, 7):
        c = workloads.make_case(w, device="cuda", window=win)
        say(f"[case] scale={scale} path={path} schedule={sched} window={win}")
        exp, rows = oracle_out(c)
        for P in (0, 64):
            compare(run_gpu(c, path=path, part_size=P, schedule=sched), exp, rows, BF16_TOL,
                    f"scale={scale} path={path} sched={sched} w={win} P={P}")


@pytest.mark.parametrize("seed", range(4))
def test_small_f32(seed):
    w = small(seed + 40, dtype="f32")
    for win in (0, 3, 64):
        c = workloads.make_case(w, device="cuda", window=win)
        say(f"[case] small f32 seed={seed} window={win}")
        exp, rows = oracle_out(c)
        for P in (0, 32, 96):
            compare(run_gpu(c, part_size=P), exp, rows, F32_TOL, f"small-f32 {seed} w={win} P={P}")


@pytest.mark.parametrize("sched", [pa.SCHED_GRID, pa.SCHED_PERSISTENT], ids=["grid", "ps"])
@pytest.mark.parametrize("waves", [1, 2, 4])
def test_mfma_waves(waves, sched):
    """Every workgroup size on both schedules (the persistent one keeps the
    lengths its prologue reads in shared memory with 2 or 4 waves and
    reloads them with one)."""
    w = small(7, head_dim=128, num_q_heads=8, num_kv_heads=2, query_len=2)  # R = 8: one row tile
    c = workloads.make_case(w, device="cuda", window=0)
    exp, rows = oracle_out(c)
    for P in (32, 96, 256):
        compare(run_gpu(c, path=pa.PATH_MFMA, waves=waves, part_size=P, schedule=sched), exp, rows,
                BF16_TOL, f"waves={waves} sched={sched} P={P}")


def test_max_rows_and_edge_lengths():
    """R = 64 (4 row tiles), contexts of 1, q == L, lengths at chunk edges, and
    sequences with no query tokens."""
    lens = (1, 4, 31, 32, 33, 64, 65, 700)
    qls = (1, 4, 4, 0, 2, 4, 0, 3)
    for D in (64, 128):
        w = small(3, head_dim=D, num_q_heads=16, num_kv_heads=1, query_len=4, batch=len(lens),
                  seq_lens=lens, query_lens=qls, block_size=32, max_seq_len=700,
                  max_blocks_per_seq=23)
        for win in (0, 2, 40):
            c = workloads.make_case(w, device="cuda", window=win)
            exp, rows = oracle_out(c)
            for path, sched in KERNELS:
                if path == pa.PATH_VALU and sched == pa.SCHED_PERSISTENT:
                    continue  # 64 rows: the vector kernels' persistent schedule takes at most 8
                for P in (0, 32):
                    compare(run_gpu(c, path=path, part_size=P, schedule=sched), exp, rows,
                            BF16_TOL, f"edges D={D} w={win} path={path} sched={sched} P={P}")


@pytest.mark.parametrize("B,sched", [(65, pa.SCHED_GRID), (130, pa.SCHED_AUTO),
                                     (1024, pa.SCHED_GRID), (1024, pa.SCHED_PERSISTENT),
                                     (1100, pa.SCHED_AUTO), (8192, pa.SCHED_AUTO),
                                     (65535, pa.SCHED_AUTO)])
def test_largest_batches(B, sched):
    """The persistent schedule's largest batch (1024 sequences, its prefix sums
    in shared memory) and larger ones, which the plan hands to the grid
    schedule with row offsets scanned once into the workspace.  Query
    lengths 0-3 make every row offset a long prefix sum; sampled sequences
    include the last ones; 65535 is the largest batch the library takes.
    Up to 1024 sequences on the grid schedule, each workgroup sums its row
    offset itself: one load per lane up to 64 sequences, all of a lane's
    loads at once beyond (sequences 63-65 sampled)."""
    r = np.random.default_rng(B)
    qls = tuple(int(x) for x in r.integers(0, 4, size=B))
    lens = tuple(int(q + x) for q, x in zip(qls, r.integers(1, 400 if B <= 8192 else 120, size=B)))
    w = small(5, batch=B, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
              query_len=3, seq_lens=lens, query_lens=qls, max_seq_len=max(lens),
              max_blocks_per_seq=-(-max(lens) // 16) + 1)
    pick = sorted(set(int(x) for x in r.choice(B, size=40, replace=False)) | {0, B - 2, B - 1}
                  | {k for k in (63, 64, 65) if k < B})
    for win in (0, 33):
        c = workloads.make_case(w, device="cuda", window=win)
        say(f"[case] batch {B} window={win} schedule={sched}")
        exp, rows = oracle_out(c, pick)
        # the larger batch is one-shot as planned; 64-position partitions
        # split it and send every sequence through the merge as well
        for P in ((0,) if sched == pa.SCHED_PERSISTENT else (0, 64)):
            out = run_gpu(c, schedule=sched, part_size=P)
            compare(out, exp, rows, BF16_TOL, f"batch {B} w={win} sched={sched} P={P}")
            assert torch.isfinite(out.float()).all()


def test_batch_without_query_tokens():
    """Every query_lens[b] = 0: no output rows (T = 0), and the call through the
    binding and a prepared call both return without error."""
    w = small(4, batch=3, seq_lens=(251, 40, 7), query_lens=(0, 0, 0), query_len=2,
              block_size=16, max_seq_len=251, max_blocks_per_seq=17)
    for win in (0, 5):
        c = workloads.make_case(w, device="cuda", window=win)
        assert c.q.shape[0] == 0
        out = run_gpu(c)
        assert out.shape[0] == 0
        call = pa.Prepared(out, c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                           c.query_lens, c.scale, win, w.num_kv_heads, w.block_size,
                           w.max_seq_len, w.query_len)
        call()
        torch.cuda.synchronize()


def test_debug_spans_bit_exact():
    for name in workloads.WORKLOADS:
        w = workloads.WORKLOADS[name]
        for win in w.windows:
            c = workloads.make_case(w, device="cuda", window=win, poison=False) if name in (
                "tiny_f32",) else _tables_only(w, win)
            _check_spans(c, win)
    for seed in range(6):
        w = small(seed)
        for win in (0, 1, 5, 37):
            _check_spans(workloads.make_case(w, device="cuda", window=win), win)


class _TablesOnly:
    pass


def _tables_only(w, win):
    """Lengths and tables of a workload without materialising its KV pool."""
    import math
    g = torch.Generator().manual_seed(w.seed)
    lens, qls = workloads._lengths(w, g)
    c = _TablesOnly()
    c.w = w
    c.window = win
    c.seq_lens_host, c.query_lens_host = lens, qls
    bs = w.block_size
    nblk = [-(-L // bs) for L in lens]
    pool = w.pool or math.ceil(1.25 * sum(nblk))
    perm = torch.randperm(max(pool, sum(nblk) + 1), generator=g).tolist()
    t = torch.full((w.batch, w.max_blocks_per_seq), perm[sum(nblk)], dtype=torch.int32)
    off = 0
    for b, n in enumerate(nblk):
        t[b, :n] = torch.tensor(perm[off:off + n], dtype=torch.int32)
        off += n
    c.tables_host = t
    c.block_tables = t.cuda()
    c.seq_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    c.query_lens = torch.tensor(qls, dtype=torch.int32, device="cuda")
    c.num_blocks = pool
    return c


def _check_spans(c, win):
    w = c.w
    dims = pa.make_dims(w.batch, w.num_q_heads, w.head_dim, max(w.query_len, max(c.query_lens_host)),
                        w.max_seq_len, w.max_blocks_per_seq, c.num_blocks,
                        pa.F32 if w.dtype == "f32" else pa.BF16)
    T = sum(c.query_lens_host)
    got = pa.debug_spans(c.block_tables, c.seq_lens, c.query_lens, win, w.num_kv_heads,
                         w.block_size, dims, T)
    torch.cuda.synchronize()
    sp = ref.spans(c.tables_host.numpy(), c.seq_lens_host, c.query_lens_host, win, w.block_size)
    si = got["seq_info"].cpu().numpy()
    ri = got["row_info"].cpu().numpy()
    bl = got["blocks"].cpu().numpy()
    parts = got["parts"].cpu().numpy()
    P = got["plan"]["part_size"]
    for b, s in enumerate(sp):
        assert si[b, 0] == s["qoff"], (w.name, b)
        if c.query_lens_host[b] > 0:
            assert (si[b, 1], si[b, 2]) == (s["lo"], s["hi"]), (w.name, b)
            np.testing.assert_array_equal(bl[b], s["blocks"])
            for i, (lo_i, p_i) in enumerate(s["rows"]):
                assert tuple(ri[s["qoff"] + i]) == (lo_i, p_i)
            # partitions tile [lo, hi) exactly, in order, none longer than P
            n = si[b, 3]
            assert n >= 1
            pr = parts[b, :n]
            assert pr[0, 0] == s["lo"] and pr[-1, 1] == s["hi"]
            assert np.all(pr[1:, 0] == pr[:-1, 1])
            assert np.all(pr[:, 1] > pr[:, 0]) and np.all(pr[:, 1] - pr[:, 0] <= P)
            assert np.all(parts[b, n:, 0] == parts[b, n:, 1])
        else:
            assert si[b, 3] == 0 and np.all(bl[b] == -1)
    say(f"[spans] {w.name} w={win}: bit-exact")


# (workload, window, sampled sequences or None for all).  Sampled workloads
# always include their longest and shortest sequences besides the draw.
FULL = [("gqa_bf16", 0, None), ("swa_mtp_bf16", 128, None), ("long_splitk_bf16", 0, None),
        ("large_block_mtp_bf16", 4096, 24), ("large_block_mtp_bf16", 0, 10)]


@pytest.mark.parametrize("sched", [pa.SCHED_AUTO, pa.SCHED_GRID])
@pytest.mark.parametrize("name,window,nsample", FULL)
def test_full_workload(name, window, nsample, sched):
    w = workloads.WORKLOADS[name]
    say(f"[case] full {name} window={window} schedule={sched}")
    c = workloads.make_case(w, device="cuda", window=window)
    out = run_gpu(c, schedule=sched)
    seqs = sample_sequences(c.seq_lens_host, nsample, w.seed)
    lens = [c.seq_lens_host[b] for b in seqs]
    say(f"[sample] {len(seqs)} sequences, lengths {min(lens)}..{max(lens)}")
    exp, rows = oracle_out(c, seqs)
    compare(out, exp, rows, BF16_TOL, f"{name} w={window} seqs={len(seqs)}")
    # rows not compared must still be finite and written
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("name,window,nsample", FULL)
def test_full_workload_peaked(name, window, nsample):
    """Every full-size workload with Q scaled by 3 (logits ~ N(0, 9)), in the
    launch configuration the bench times: the outputs are then of order
    0.3-1, so the max-abs bar bites at every context length, not only the
    scale-free ones."""
    w = workloads.WORKLOADS[name]
    say(f"[case] full peaked {name} window={window}")
    c = workloads.make_case(w, device="cuda", window=window, q_gain=3.0)
    out = run_gpu(c)
    seqs = sample_sequences(c.seq_lens_host, nsample, w.seed + 1)
    exp, rows = oracle_out(c, seqs)
    mx, _ = compare(out, exp, rows, BF16_TOL, f"{name} peaked w={window} seqs={len(seqs)}")
    assert float(np.abs(exp).max()) >= 0.1, "peaked outputs should be O(0.1-1)"
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("sched", [pa.SCHED_GRID, pa.SCHED_PERSISTENT])
@pytest.mark.parametrize("P", [32, 64, 256, 4096])
def test_reduce_lane_modes(P, sched):
    """Partition counts in every regime of the merge kernel (1, 16 or 32
    lanes per output unit): 3 sequences of up to 20000 positions."""
    w = small(11, head_dim=128, num_q_heads=16, num_kv_heads=2, query_len=2, batch=3,
              seq_lens=(20000, 4000, 129), block_size=32, max_seq_len=20000,
              max_blocks_per_seq=626)
    for win in (0, 3000):
        c = workloads.make_case(w, device="cuda", window=win)
        np_ = -(-(20000 + 31) // P) if win == 0 else -(-(win + 1 + 31) // P)
        say(f"[case] reduce modes P={P} window={win} partitions={np_}")
        exp, rows = oracle_out(c)
        compare(run_gpu(c, part_size=P, schedule=sched), exp, rows, BF16_TOL,
                f"reduce P={P} sched={sched} w={win}")


def _case_for_reuse():
    return workloads.make_case(small(21, head_dim=128, num_q_heads=16, num_kv_heads=2, query_len=2,
                                     batch=3, seq_lens=(9000, 3000, 129), block_size=32,
                                     max_seq_len=9000, max_blocks_per_seq=283), device="cuda")


REUSE_PLANS = [dict(part_size=32, schedule=pa.SCHED_GRID),      # 283 partitions: 32-lane merge
               dict(part_size=256, schedule=pa.SCHED_GRID),     # 36 partitions: 16-lane merge
               dict(part_size=512, schedule=pa.SCHED_PERSISTENT),
               dict(schedule=pa.SCHED_PERSISTENT),
               dict(path=pa.PATH_VALU, part_size=64)]


def test_workspace_contents_do_not_matter():
    """Every workspace value that enters a call's arithmetic was written by
    the same call (the merge requests a grid plan's first slots before it
    knows how many a unit uses, and drops the stale ones by select): a
    workspace full of random bytes, of NaN, or left behind by calls with
    other plans, gives the same output bits as a zeroed one."""
    c = _case_for_reuse()
    dims = pa.dims_for(c.q, c.k_cache, c.block_tables, 2, c.w.max_seq_len)
    need = max(pa.workspace_size(dims, 0, 2, 32, **o) for o in REUSE_PLANS)
    ref_out = []
    for o in REUSE_PLANS:
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        ref_out.append(run_gpu(c, workspace=ws, **o).clone())
    g = torch.Generator(device="cuda").manual_seed(5)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=g)
    for rep in range(2):
        for o, expect in zip(REUSE_PLANS, ref_out):
            assert torch.equal(run_gpu(c, workspace=ws, **o), expect), (rep, o)
    ws.fill_(255)  # every fp32 word 0xffffffff: a NaN
    for o, expect in zip(REUSE_PLANS, ref_out):
        assert torch.equal(run_gpu(c, workspace=ws, **o), expect), ("nan", o)
    say("[workspace] random, NaN and reused workspaces: identical outputs")


def test_graph_replays_match_eager():
    """A captured call (partition kernel + merge kernel) replays to the eager
    result every time, with eager calls on the same workspace in between."""
    c = _case_for_reuse()
    dims = pa.dims_for(c.q, c.k_cache, c.block_tables, 2, c.w.max_seq_len)
    for o in REUSE_PLANS[:2] + REUSE_PLANS[3:4]:
        ws = torch.zeros(pa.workspace_size(dims, 0, 2, 32, **o), dtype=torch.uint8, device="cuda")
        eager = run_gpu(c, workspace=ws, **o).clone()
        out_g = torch.full_like(eager, float("nan"))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            pa.decode(out_g, c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.query_lens,
                      c.scale, c.window, c.w.num_kv_heads, c.w.block_size,
                      max_seq_len=c.w.max_seq_len, max_query_len=2, workspace=ws, **o)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            pa.decode(out_g, c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.query_lens,
                      c.scale, c.window, c.w.num_kv_heads, c.w.block_size,
                      max_seq_len=c.w.max_seq_len, max_query_len=2, workspace=ws, **o)
        for rep in range(3):
            out_g.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_g, eager), (o, rep)
            assert torch.equal(run_gpu(c, workspace=ws, **o), eager), (o, rep)
        say(f"[graph] {o}: 3 replays identical to eager")


@pytest.mark.parametrize("sched", [pa.SCHED_GRID, pa.SCHED_PERSISTENT])
@pytest.mark.parametrize("D", [64, 128])
def test_two_tiles_four_waves(D, sched):
    """32 packed rows per KV head in one workgroup of 4 waves (each K/V load
    feeds both 16-row tiles), windowed and full, split and one-shot."""
    w = small(8, head_dim=D, num_q_heads=16, num_kv_heads=2, query_len=4, batch=3,
              seq_lens=(700, 129, 40), block_size=64, max_seq_len=700, max_blocks_per_seq=12)
    for win in (0, 5, 128):
        c = workloads.make_case(w, device="cuda", window=win)
        exp, rows = oracle_out(c)
        for P in (0, 64, 1024):
            compare(run_gpu(c, path=pa.PATH_MFMA, waves=4, part_size=P, schedule=sched), exp, rows,
                    BF16_TOL, f"2 tiles x 4 waves D={D} sched={sched} w={win} P={P}")


@pytest.mark.parametrize("name,nsample", [("gqa_f32", 8), ("long_splitk_bf16", None)])
def test_vector_kernel_full_size(name, nsample):
    """The register-resident vector kernel at full size, on both schedules:
    the fp32 GQA batch (its automatic path) at the fp32 bars, and the single
    131072-position bf16 sequence forced onto it."""
    w = workloads.WORKLOADS[name]
    c = workloads.make_case(w, device="cuda", window=0)
    seqs = sample_sequences(c.seq_lens_host, nsample, w.seed)
    exp, rows = oracle_out(c, seqs)
    for sched in (pa.SCHED_AUTO, pa.SCHED_GRID, pa.SCHED_PERSISTENT):
        out = run_gpu(c, path=pa.PATH_VALU, schedule=sched)
        compare(out, exp, rows, F32_TOL if w.dtype == "f32" else BF16_TOL,
                f"vector kernel {name} sched={sched} seqs={len(seqs)}")
        assert torch.isfinite(out.float()).all()
