"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
and its host logic (argument validation, launch plan, workspace size) behaves
as documented in include/pa_decode.h.  No call here touches a GPU."""

import ctypes
import math
import os
import re
import subprocess

import pytest

import decode_attention_pa_amd as pa
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa_decode.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.library_path()):
        pytest.fail("libpa_decode.so is not built (run python -m decode_attention_pa_amd.build)")
    return pa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(pa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code in range(5):
        assert lib.pa_status_string(code).decode().startswith("PA_")
    assert b"unknown" in lib.pa_status_string(99)


def dims_of(w: workloads.Workload, max_query_len=None, **over):
    d = dict(batch=w.batch, num_q_heads=w.num_q_heads, head_dim=w.head_dim,
             max_query_len=w.query_len if max_query_len is None else max_query_len, max_seq_len=w.max_seq_len,
             max_blocks_per_seq=w.max_blocks_per_seq, num_blocks=1000,
             dtype=pa.F32 if w.dtype == "f32" else pa.BF16,
             kv_format=pa.KV_FP8_E4M3 if w.kv_dtype == "fp8" else pa.KV_NATIVE,
             q_format=pa.Q_FP8_E4M3 if w.q_dtype == "fp8" else pa.Q_NATIVE)
    d.update(over)
    return pa.make_dims(**d)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_plan_covers_longest_span(lib, name):
    w = workloads.WORKLOADS[name]
    for win in w.windows:
        p = pa.plan(dims_of(w), win, w.num_kv_heads, w.block_size, num_cus=256)
        G = w.num_q_heads // w.num_kv_heads
        assert p["rows"] == G * w.query_len
        span = w.max_seq_len if win == 0 else min(w.max_seq_len, win + w.query_len - 1)
        assert p["span_max"] == span
        assert p["part_size"] % 32 == 0
        # every sequence's chunk-aligned span fits in the partition grid
        assert p["num_parts"] * p["part_size"] >= span + 31
        assert p["one_shot"] == (p["num_parts"] == 1)
        if p["one_shot"]:
            assert p["workspace_bytes"] == 0          # batches of at most 1024 sequences
        else:
            units = w.batch * w.num_kv_heads
            slots = p["ps_grid"] + units if p["persistent"] else units * p["num_parts"]
            states = slots * p["rows"]
            al = lambda x: (x + 255) // 256 * 256
            runs = al(8 * units) if p["persistent"] else 0
            assert p["workspace_bytes"] == 2 * al(4 * states) + al(4 * states * w.head_dim) + runs
            assert p["ps_grid"] > 0 if p["persistent"] else p["ps_grid"] == 0
        expect_path = pa.PATH_VALU if w.dtype == "f32" else pa.PATH_MFMA
        assert p["row_blocks"] == -(-p["rows"] // p["block_rows"])
        assert p["path"] == expect_path


def test_plan_forced_partition_size(lib):
    w = workloads.WORKLOADS["long_splitk_bf16"]
    p = pa.plan(dims_of(w), 0, 1, 16, part_size=4096)
    assert p["part_size"] == 4096 and p["num_parts"] == math.ceil((131072 + 31) / 4096)
    p1 = pa.plan(dims_of(w), 0, 1, 16, part_size=1 << 20)
    assert p1["num_parts"] == 1 and p1["one_shot"] == 1 and p1["workspace_bytes"] == 0


def test_plan_uses_more_partitions_on_more_cus(lib):
    w = workloads.WORKLOADS["long_splitk_bf16"]
    small = pa.plan(dims_of(w), 0, 1, 16, num_cus=64)
    big = pa.plan(dims_of(w), 0, 1, 16, num_cus=256)
    assert big["num_parts"] >= small["num_parts"]


def test_plan_window_bounds_the_span(lib):
    w = workloads.WORKLOADS["large_block_mtp_bf16"]
    p4096 = pa.plan(dims_of(w), 4096, 8, 1024)
    p0 = pa.plan(dims_of(w), 0, 8, 1024)
    assert p4096["span_max"] == 4097 and p0["span_max"] == 65536
    assert p4096["num_parts"] < p0["num_parts"]


BAD = [
    (dict(head_dim=257), pa.ERR_UNSUPPORTED),
    (dict(head_dim=0), pa.ERR_UNSUPPORTED),
    (dict(dtype=7), pa.ERR_INVALID_ARG),
    (dict(batch=-1), pa.ERR_INVALID_ARG),
    (dict(num_q_heads=6), pa.ERR_INVALID_ARG),          # not a multiple of 4 KV heads
    (dict(max_query_len=0), pa.ERR_INVALID_ARG),
    (dict(max_seq_len=0), pa.ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=3), pa.ERR_INVALID_ARG),   # 8192 / 16 needs 512
    (dict(num_blocks=0), pa.ERR_INVALID_ARG),
    (dict(max_query_len=257), pa.ERR_UNSUPPORTED),      # 4 * 257 rows > 1024
]


def test_general_rows_and_head_dims(lib):
    """More than 64 packed rows go in row blocks (16-row tiles: up to 64 rows
    per workgroup at D = 64, 32 at D = 128, 16 at D = 256, 16 on the vector
    path); head dims off the matrix-core set take the vector path."""
    w = workloads.WORKLOADS["gqa_bf16"]
    p = pa.plan(dims_of(w, max_query_len=17), 0, 8, 16)            # 68 rows, D = 128
    assert (p["path"], p["row_tiles"], p["row_blocks"], p["waves"]) == (pa.PATH_MFMA, 2, 3, 2)
    assert p["persistent"] == 0                                      # one block per workgroup only
    p = pa.plan(dims_of(w, max_query_len=16), 0, 8, 16)             # 64 rows fit one block
    assert (p["row_tiles"], p["row_blocks"]) == (4, 1)
    p = pa.plan(dims_of(w, max_query_len=256, head_dim=64), 0, 8, 16)   # 1024 rows
    assert (p["row_tiles"], p["row_blocks"], p["waves"]) == (4, 16, 1)
    p = pa.plan(dims_of(w, max_query_len=3, head_dim=256), 0, 8, 16)    # 12 rows, D = 256
    assert (p["path"], p["row_tiles"], p["row_blocks"], p["waves"]) == (pa.PATH_MFMA, 1, 1, 2)
    p = pa.plan(dims_of(w, max_query_len=5, head_dim=256), 0, 8, 16)    # 20 rows, D = 256
    assert (p["row_tiles"], p["row_blocks"]) == (1, 2)
    p = pa.plan(dims_of(w, head_dim=66), 0, 8, 16)                   # odd head dim: staged
    assert (p["path"], p["block_rows"], p["row_blocks"]) == (pa.PATH_VALU_LDS, 16, 1)
    p = pa.plan(dims_of(w, head_dim=66, max_query_len=9), 0, 8, 16)  # 36 rows
    assert p["row_blocks"] == 3
    # the register-resident vector kernel: 4 or 8 rows per workgroup
    f = dict(dtype=pa.F32)
    p = pa.plan(dims_of(w, **f), 0, 8, 16)                             # fp32, 4 rows
    assert (p["path"], p["block_rows"], p["row_blocks"]) == (pa.PATH_VALU, 4, 1)
    p = pa.plan(dims_of(w, max_query_len=9, **f), 0, 8, 16)            # fp32, 36 rows
    assert (p["path"], p["block_rows"], p["row_blocks"]) == (pa.PATH_VALU, 8, 5)
    p = pa.plan(dims_of(w, head_dim=64), 0, 8, 16, path=pa.PATH_VALU)  # bf16 on request
    assert (p["path"], p["block_rows"]) == (pa.PATH_VALU, 4)
    p = pa.plan(dims_of(w, head_dim=200, **f), 0, 8, 16, path=pa.PATH_VALU)  # no such kernel
    assert (p["path"], p["block_rows"]) == (pa.PATH_VALU_LDS, 16)
    p = pa.plan(dims_of(w, **f), 0, 8, 16, path=pa.PATH_VALU_LDS)      # staged on request
    assert (p["path"], p["block_rows"]) == (pa.PATH_VALU_LDS, 16)
    with pytest.raises(pa.PaError) as e:                             # no matrix-core kernel
        pa.plan(dims_of(w, head_dim=66), 0, 8, 16, path=pa.PATH_MFMA)
    assert e.value.status == pa.ERR_UNSUPPORTED
    with pytest.raises(pa.PaError) as e:                             # rows must fit one block
        pa.plan(dims_of(w, max_query_len=17), 0, 8, 16, schedule=pa.SCHED_PERSISTENT)
    assert e.value.status == pa.ERR_UNSUPPORTED
    with pytest.raises(pa.PaError) as e:                             # FP8 needs the matrix cores
        pa.plan(dims_of(w, head_dim=66, kv_format=pa.KV_FP8_E4M3), 0, 8, 16)
    assert e.value.status == pa.ERR_UNSUPPORTED


@pytest.mark.parametrize("over,code", BAD)
def test_plan_rejects_bad_dims(lib, over, code):
    w = workloads.WORKLOADS["gqa_bf16"]
    with pytest.raises(pa.PaError) as e:
        pa.plan(dims_of(w, **over), 0, 8 if "num_q_heads" not in over else 4, 16)
    assert e.value.status == code
    assert lib.pa_last_error().decode()


@pytest.mark.parametrize("bs,code", [(8, pa.ERR_UNSUPPORTED), (24, pa.ERR_UNSUPPORTED),
                                     (2048, pa.ERR_UNSUPPORTED), (0, pa.ERR_UNSUPPORTED)])
def test_plan_rejects_block_sizes(lib, bs, code):
    w = workloads.WORKLOADS["gqa_bf16"]
    with pytest.raises(pa.PaError) as e:
        pa.plan(dims_of(w, max_blocks_per_seq=100000), 0, 8, bs)
    assert e.value.status == code


def test_plan_rejects_negative_window_and_bad_options(lib):
    w = workloads.WORKLOADS["gqa_bf16"]
    for kw, win in [({}, -1), (dict(part_size=48), 0), (dict(part_size=-32), 0),
                    (dict(waves=3), 0), (dict(path=9), 0), (dict(schedule=3), 0),
                    (dict(loads=3), 0), (dict(loads=-1), 0)]:
        with pytest.raises(pa.PaError) as e:
            pa.plan(dims_of(w), win, 8, 16, **kw)
        assert e.value.status == pa.ERR_INVALID_ARG


def test_persistent_schedule_choice(lib):
    gqa = workloads.WORKLOADS["gqa_bf16"]
    assert pa.plan(dims_of(gqa), 0, 8, 16)["persistent"] == 1          # 256 units, split
    assert pa.plan(dims_of(gqa), 0, 8, 16, schedule=pa.SCHED_GRID)["persistent"] == 0
    long = workloads.WORKLOADS["long_splitk_bf16"]
    assert pa.plan(dims_of(long), 0, 1, 16)["persistent"] == 0         # one unit
    assert pa.plan(dims_of(long), 0, 1, 16, schedule=pa.SCHED_PERSISTENT)["persistent"] == 1
    tiny = workloads.WORKLOADS["tiny_f32"]
    # register-resident vector path: persistent when asked for (R <= 8 rows in
    # one workgroup); the staged vector kernel has the grid schedule only
    p = pa.plan(dims_of(tiny), 0, 1, 16, schedule=pa.SCHED_PERSISTENT)
    assert p["path"] == pa.PATH_VALU and p["persistent"] == 1 and p["ps_grid"] == 8 * 256
    assert pa.plan(dims_of(tiny), 0, 1, 16)["persistent"] == 0
    with pytest.raises(pa.PaError) as e:
        pa.plan(dims_of(tiny), 0, 1, 16, schedule=pa.SCHED_PERSISTENT, path=pa.PATH_VALU_LDS)
    assert e.value.status == pa.ERR_UNSUPPORTED
    with pytest.raises(pa.PaError) as e:                              # 16 rows in 2 blocks of 8
        pa.plan(dims_of(tiny, num_q_heads=16), 0, 1, 16, schedule=pa.SCHED_PERSISTENT)
    assert e.value.status == pa.ERR_UNSUPPORTED
    with pytest.raises(pa.PaError) as e:
        pa.plan(dims_of(gqa, batch=1025, max_blocks_per_seq=512), 0, 8, 16,
                schedule=pa.SCHED_PERSISTENT)
    assert e.value.status == pa.ERR_UNSUPPORTED


def test_streaming_loads_choice(lib):
    # Non-temporal KV loads on the matrix-core path unless row blocks re-read
    # K/V within the call; the options force either form.
    gqa = workloads.WORKLOADS["gqa_bf16"]
    for nb in (10899, 2000):                          # pool size does not matter
        assert pa.plan(dims_of(gqa, num_blocks=nb), 0, 8, 16)["streaming"] == 1
    assert pa.plan(dims_of(gqa, num_blocks=10899), 0, 8, 16,
                   loads=pa.LOADS_CACHED)["streaming"] == 0
    long = workloads.WORKLOADS["long_splitk_bf16"]
    assert pa.plan(dims_of(long, num_blocks=10240), 0, 1, 16)["streaming"] == 1
    assert pa.plan(dims_of(long, num_blocks=10240), 0, 1, 16,
                   loads=pa.LOADS_CACHED)["streaming"] == 0
    swa = workloads.WORKLOADS["swa_mtp_bf16"]         # one-shot, two tiles in one block
    p = pa.plan(dims_of(swa), 128, 8, 64)
    assert (p["row_blocks"], p["streaming"]) == (1, 1)
    p = pa.plan(dims_of(swa, num_q_heads=96), 128, 8, 64)   # 48 rows: one-tile blocks
    assert (p["row_blocks"], p["streaming"]) == (3, 0)
    pre = workloads.WORKLOADS["prefill_chunk_bf16"]   # 128 rows: four row blocks share K/V
    p = pa.plan(dims_of(pre), 0, 4, 16)
    assert p["row_blocks"] > 1 and p["streaming"] == 0
    assert pa.plan(dims_of(pre), 0, 4, 16, loads=pa.LOADS_STREAMING)["streaming"] == 1
    tiny = workloads.WORKLOADS["tiny_f32"]           # vector path: always cached
    assert pa.plan(dims_of(tiny), 0, 1, 16, loads=pa.LOADS_STREAMING)["streaming"] == 0


def test_plan_rejects_mfma_for_fp32(lib):
    w = workloads.WORKLOADS["tiny_f32"]
    with pytest.raises(pa.PaError) as e:
        pa.plan(dims_of(w), 0, 1, 16, path=pa.PATH_MFMA)
    assert e.value.status == pa.ERR_UNSUPPORTED


def test_decode_validates_before_touching_a_device(lib):
    """Invalid host arguments fail with a status before any HIP call, so this
    runs without a GPU."""
    w = workloads.WORKLOADS["gqa_bf16"]
    d = dims_of(w)
    P = ctypes.c_void_p
    good = P(4096)
    args = [good] * 7
    # (the pointers are fake: every call below must fail validation, so no
    # kernel is ever launched with them, on a machine with or without a GPU)
    st = lib.pa_decode(None, *args[1:7], ctypes.c_float(0.1), 0, 8, 16, ctypes.byref(d), None, 0, None)
    assert st == pa.ERR_INVALID_ARG
    st = lib.pa_decode(P(4097), *args[1:7], ctypes.c_float(0.1), 0, 8, 16, ctypes.byref(d), None, 0, None)
    assert st == pa.ERR_INVALID_ARG and b"aligned" in lib.pa_last_error()
    st = lib.pa_decode(*args[:7], ctypes.c_float(float("nan")), 0, 8, 16, ctypes.byref(d), None, 0, None)
    assert st == pa.ERR_INVALID_ARG and b"scale" in lib.pa_last_error()
    st = lib.pa_decode(*args[:7], ctypes.c_float(0.1), -2, 8, 16, ctypes.byref(d), None, 0, None)
    assert st == pa.ERR_INVALID_ARG
    st = lib.pa_decode(*args[:7], ctypes.c_float(0.1), 0, 8, 16, None, None, 0, None)
    assert st == pa.ERR_INVALID_ARG
    # an FP8 cache without its scales is refused (pa_decode has no way to pass
    # them; pa_decode_ex needs both, 4-byte aligned)
    d8 = dims_of(w, kv_format=pa.KV_FP8_E4M3)
    st = lib.pa_decode(*args[:7], ctypes.c_float(0.1), 0, 8, 16, ctypes.byref(d8), None, 0, None)
    assert st == pa.ERR_INVALID_ARG and b"k_scale" in lib.pa_last_error()
    for ks, vs in ((None, None), (P(4096), None), (None, P(4096)), (P(4098), P(4096))):
        o = pa.make_options()
        o.k_scale, o.v_scale = ks, vs
        st = lib.pa_decode_ex(*args[:7], ctypes.c_float(0.1), 0, 8, 16, ctypes.byref(d8), None, 0,
                              None, ctypes.byref(o))
        assert st == pa.ERR_INVALID_ARG, (ks, vs)


def test_fp8_kv_format_rules(lib):
    w = workloads.WORKLOADS["gqa_fp8kv"]
    p = pa.plan(dims_of(w, kv_format=pa.KV_FP8_E4M3), 0, 8, 16)
    assert p["path"] == pa.PATH_MFMA
    for over, kw, code in [(dict(kv_format=2), {}, pa.ERR_INVALID_ARG),
                           (dict(kv_format=pa.KV_FP8_E4M3, dtype=pa.F32), {}, pa.ERR_UNSUPPORTED),
                           (dict(kv_format=pa.KV_FP8_E4M3), dict(path=pa.PATH_VALU),
                            pa.ERR_UNSUPPORTED)]:
        with pytest.raises(pa.PaError) as e:
            pa.plan(dims_of(w, **over), 0, 8, 16, **kw)
        assert e.value.status == code, over
    # FP8 K/V takes the same load forms
    fp8 = dims_of(w, num_blocks=6000, kv_format=pa.KV_FP8_E4M3)
    assert pa.plan(fp8, 0, 8, 16)["streaming"] == 1
    assert pa.plan(fp8, 0, 8, 16, loads=pa.LOADS_CACHED)["streaming"] == 0


def test_empty_batch_is_a_no_op(lib):
    w = workloads.WORKLOADS["gqa_bf16"]
    d = dims_of(w, batch=0)
    P = ctypes.c_void_p
    st = lib.pa_decode(*([P(4096)] * 7), ctypes.c_float(0.1), 0, 8, 16, ctypes.byref(d), None, 0, None)
    assert st == pa.OK


def test_binding_rejects_cpu_tensors():
    import torch
    c = workloads.make_case("tiny_f32", device="cpu")
    with pytest.raises(pa.PaError):
        pa.decode(c.new_out(), c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                  c.query_lens, c.scale, 0, 1, 16, max_seq_len=50, max_query_len=1)


def test_grid_plans_with_few_waves(lib):
    # One-shot grid plans under 16 waves per CU run two row tiles as one
    # workgroup of 4 waves and more tiles as one-tile blocks of 4 waves; with
    # enough units, or waves forced, all rows stay in one workgroup of the
    # default waves.
    swa = workloads.WORKLOADS["swa_mtp_bf16"]        # 512 units x 32 rows, one-shot
    p = pa.plan(dims_of(swa), 128, 8, 64, num_cus=256)
    assert (p["one_shot"], p["row_tiles"], p["row_blocks"], p["waves"]) == (1, 2, 1, 4)
    p = pa.plan(dims_of(swa, num_q_heads=128), 128, 8, 64, num_cus=256)    # 64 rows
    assert (p["one_shot"], p["row_tiles"], p["row_blocks"], p["waves"]) == (1, 1, 4, 4)
    big = dims_of(swa, batch=1024)                   # 8192 units: plenty of waves
    p = pa.plan(big, 128, 8, 64, num_cus=256)
    assert (p["row_tiles"], p["row_blocks"], p["waves"]) == (2, 1, 2)
    p = pa.plan(dims_of(swa), 128, 8, 64, num_cus=256, waves=2)
    assert (p["row_tiles"], p["row_blocks"], p["waves"]) == (2, 1, 2)
    # head dim 256, one long sequence: 4-chunk partitions and 2 waves; a batch
    # on the persistent schedule takes 2 waves too
    d256 = workloads.WORKLOADS["d256_decode_bf16"]
    p = pa.plan(dims_of(d256), 0, 2, 16, num_cus=256)
    assert (p["part_size"], p["waves"], p["persistent"]) == (128, 2, 0)
    b256 = workloads.WORKLOADS["gqa_d256_bf16"]
    p = pa.plan(dims_of(b256), 0, 2, 16, num_cus=256)
    assert (p["waves"], p["persistent"]) == (2, 1)


def test_grid_splits_sized_by_loads_in_flight(lib):
    # One-tile grid splits size the grid for ~64 KB of K/V loads in flight
    # per CU if every unit had the longest span: 4 waves per CU at head dim
    # 128 in bf16 (one 16 KB chunk per wave), 4 over an FP8 cache too (two
    # 8 KB chunks per wave step), 8 at head dim 64, 2 at head dim 256; with
    # partitions rounded down to fill that many workgroups.
    def plan(B, hq, hkv, D, L, kv=pa.KV_NATIVE, q=1):
        d = pa.make_dims(batch=B, num_q_heads=hq, head_dim=D, max_query_len=q, max_seq_len=L,
                         max_blocks_per_seq=L // 16 + 1, num_blocks=B * (L // 16 + 1),
                         dtype=pa.BF16, kv_format=kv)
        return pa.plan(d, 0, hkv, 16, num_cus=256)
    long = plan(1, 8, 1, 128, 131072)                     # 256 workgroups x 4 waves
    assert (long["part_size"], long["num_parts"], long["waves"], long["persistent"]) == (512, 257, 4, 0)
    assert plan(4, 32, 8, 128, 32768)["part_size"] == 4096   # 32 units: 8 partitions each
    assert plan(2, 16, 2, 128, 65536)["part_size"] == 1024   # 4 units: 64 partitions each
    assert plan(4, 32, 8, 128, 32768, kv=pa.KV_FP8_E4M3)["part_size"] == 4096
    assert plan(1, 8, 1, 128, 131072, kv=pa.KV_FP8_E4M3)["part_size"] == 512
    assert plan(2, 64, 8, 64, 16384)["part_size"] == 512     # head dim 64: 2 workgroups per CU
    assert plan(1, 16, 2, 256, 16384)["part_size"] == 128    # head dim 256: 2 waves per CU
    assert plan(1, 8, 1, 128, 32768)["part_size"] == 256     # floor of 8 chunks
    # two row tiles keep the ~8-workgroups-per-CU split (a longer partition
    # for the states' sake would leave fewer than two workgroups per CU)
    r32 = plan(8, 32, 1, 128, 16384)
    assert (r32["row_tiles"], r32["part_size"]) == (2, 256)
    # 128 rows per unit: partitions long enough that their states stay near
    # 1/6 of the K/V they read (24 R (D + 2) / (D s) = 1560 -> 49 chunks)
    r128 = plan(16, 32, 4, 128, 8192, q=16)
    assert (r128["row_blocks"], r128["part_size"], r128["num_parts"]) == (4, 1568, 6)


def test_fp8_query_format_rules(lib):
    w = workloads.WORKLOADS["gqa_fp8qkv"]
    d = dims_of(w, kv_format=pa.KV_FP8_E4M3, q_format=pa.Q_FP8_E4M3)
    p = pa.plan(d, 0, 8, 16)
    assert p["path"] == pa.PATH_MFMA and p["persistent"] == 1
    # the same plan as bf16 queries over the same cache
    assert p == pa.plan(dims_of(w, kv_format=pa.KV_FP8_E4M3, q_format=pa.Q_NATIVE), 0, 8, 16)
    for over, kw, code in [(dict(q_format=2), {}, pa.ERR_INVALID_ARG),
                           (dict(kv_format=pa.KV_NATIVE, q_format=pa.Q_FP8_E4M3), {},
                            pa.ERR_UNSUPPORTED),
                           (dict(kv_format=pa.KV_FP8_E4M3, q_format=pa.Q_FP8_E4M3),
                            dict(path=pa.PATH_VALU), pa.ERR_UNSUPPORTED),
                           (dict(kv_format=pa.KV_FP8_E4M3, q_format=pa.Q_FP8_E4M3, head_dim=96),
                            {}, pa.ERR_UNSUPPORTED)]:
        with pytest.raises(pa.PaError) as e:
            pa.plan(dims_of(w, **over), 0, 8, 16, **kw)
        assert e.value.status == code, over


def test_check_inputs_rejects_null_pointers(lib):
    d = pa.make_dims(2, 4, 64, 1, 64, 4, 16, pa.BF16)
    z = ctypes.c_void_p(16)
    for args in ((None, z, z, z), (z, None, z, z), (z, z, None, z), (z, z, z, None)):
        st = lib.pa_check_inputs(args[0], args[1], args[2], 0, 1, 16, ctypes.byref(d), args[3], None)
        assert st == pa.ERR_INVALID_ARG


def test_stream_read_rejects_bad_arguments_before_any_launch(lib):
    """Host-side validation of pa_stream_read (no device touched)."""
    P = ctypes.c_void_p
    n = ctypes.c_int32(-7)

    def call(src=P(4096), nbytes=4096, sink=P(1 << 20), sink_len=64, layout=0, wg=ctypes.byref(n)):
        return lib.pa_stream_read(src, nbytes, sink, sink_len, layout, wg, None)

    assert call(src=None) == pa.ERR_INVALID_ARG
    assert call(sink=None) == pa.ERR_INVALID_ARG
    assert call(wg=None) == pa.ERR_INVALID_ARG
    assert call(src=P(4104)) == pa.ERR_INVALID_ARG        # not 16-byte aligned
    assert call(nbytes=4100) == pa.ERR_INVALID_ARG        # not whole 16-byte words
    assert call(sink=P((1 << 20) + 2)) == pa.ERR_INVALID_ARG
    assert call(sink_len=0) == pa.ERR_INVALID_ARG
    assert call(layout=2) == pa.ERR_INVALID_ARG
    assert n.value == -7                                  # nothing launched, nothing written


def test_pack_rejects_bad_arguments_before_any_launch(lib):
    """Host-side validation of pa_pack_kv_cache (no device touched)."""
    P = ctypes.c_void_p
    MB = 1 << 20

    def call(k=P(4096), v=P(4096 + 64 * MB), kc=P(4096 + 128 * MB), vc=P(4096 + 192 * MB),
             ids=None, n=0, nb=4, h=2, bs=16, D=128, dtype=pa.BF16, fmt=pa.KV_NATIVE):
        return lib.pa_pack_kv_cache(k, v, kc, vc, ids, n, nb, h, bs, D, dtype, fmt, None)

    assert call(k=None) == pa.ERR_INVALID_ARG
    assert call(k=P(4100)) == pa.ERR_INVALID_ARG                  # misaligned
    assert call(kc=P(4096 + 1024)) == pa.ERR_INVALID_ARG          # overlaps k_rows
    assert call(dtype=5) == pa.ERR_INVALID_ARG
    assert call(fmt=3) == pa.ERR_INVALID_ARG
    assert call(bs=8) == pa.ERR_UNSUPPORTED
    assert call(D=300) == pa.ERR_UNSUPPORTED
    assert call(nb=0) == pa.ERR_INVALID_ARG
    assert call(ids=P(4096 + 256 * MB), n=-1) == pa.ERR_INVALID_ARG
    assert call(ids=P(4096 + 256 * MB), n=0) == pa.OK               # nothing listed: no launch


def test_large_batches_scan_row_offsets(lib):
    """Above 1024 sequences the workspace also holds the scanned row offsets
    (4 bytes per sequence), one-shot plans included."""
    w = workloads.WORKLOADS["gqa_bf16"]
    al = lambda x: (x + 255) // 256 * 256
    small = pa.plan(dims_of(w, batch=1024, max_seq_len=64, max_blocks_per_seq=4), 0, 8, 16)
    big = pa.plan(dims_of(w, batch=5000, max_seq_len=64, max_blocks_per_seq=4), 0, 8, 16)
    assert small["one_shot"] and big["one_shot"]
    assert small["workspace_bytes"] == 0 and big["workspace_bytes"] == al(4 * 5000)
    split = pa.plan(dims_of(w, batch=5000, max_seq_len=64, max_blocks_per_seq=4), 0, 8, 16,
                    part_size=32, schedule=pa.SCHED_GRID)
    states = 5000 * 8 * split["num_parts"] * split["rows"]
    assert split["workspace_bytes"] == (2 * al(4 * states) + al(4 * states * 128)
                                        + al(4 * 5000))


def test_binding_rejects_tensors_and_streams_of_another_device():
    """The binding keeps one call on one GPU: a tensor or a stream on another
    device than the call's tensors is refused before the library is called."""
    import torch
    with pytest.raises(pa.PaError) as e:
        pa._same_device(torch.device("cuda", 0), workspace=torch.empty(4))
    assert e.value.status == pa.ERR_INVALID_ARG and "workspace" in str(e.value)
    pa._same_device(torch.device("cpu"), workspace=torch.empty(4), k_scale=None)

    class FakeStream:
        device = torch.device("cuda", 1)
        cuda_stream = 0

    with pytest.raises(pa.PaError) as e:
        pa._stream_handle(FakeStream(), torch.device("cuda", 0))
    assert e.value.status == pa.ERR_INVALID_ARG
    assert pa._stream_handle(FakeStream(), torch.device("cuda", 1)).value is None


def _align256(n):
    return (n + 255) // 256 * 256


# (row tiles, waves) instantiated for the matrix-core kernels at head dims 64 / 128
MFMA_SHAPES = {(1, 1), (1, 2), (1, 4), (2, 1), (2, 2), (2, 4), (3, 1), (4, 1)}


def test_plan_invariants_on_random_shapes(lib):
    """What the kernels take for granted about a plan, over seeded random
    shapes, windows, CU counts and forced options: partitions cover the
    windowed span on the 32-position grid, row blocks cover the rows, only
    instantiated (row tiles, waves) pairs, the persistent schedule only where
    it exists, and the workspace bytes the header documents."""
    import numpy as np
    r = np.random.default_rng(2024)
    planned = refused = 0
    for _ in range(4000):
        dtype = pa.F32 if r.random() < 0.2 else pa.BF16
        kv = pa.KV_FP8_E4M3 if dtype == pa.BF16 and r.random() < 0.25 else pa.KV_NATIVE
        qf = pa.Q_FP8_E4M3 if kv == pa.KV_FP8_E4M3 and r.random() < 0.4 else pa.Q_NATIVE
        D = int(r.choice([64, 128, 256, 40, 66, 96, 200]))
        hkv = int(r.choice([1, 2, 4, 8]))
        G = int(r.choice([1, 2, 4, 5, 8, 16]))
        ql = int(r.choice([1, 2, 4, 16, 64, 128]))
        bs = int(r.choice([16, 32, 64, 256, 1024]))
        B = int(r.choice([0, 1, 3, 32, 128, 1100, 5000]))
        L = int(r.choice([ql, 100, 4096, 65536, 131072]))
        L = max(L, ql)
        win = int(r.choice([0, 0, 1, 7, 128, 4096, 100000]))
        cus = int(r.choice([256, 80, 304, 1]))
        opts = {}
        if r.random() < 0.3:
            opts["part_size"] = int(r.choice([32, 64, 192, 1024, 4096]))
        if r.random() < 0.2:
            opts["schedule"] = int(r.choice([pa.SCHED_GRID, pa.SCHED_PERSISTENT]))
        if r.random() < 0.15:
            opts["waves"] = int(r.choice([1, 2, 4]))
        dims = pa.make_dims(B, G * hkv, D, ql, L, -(-L // bs), 1000, dtype, kv, qf)
        try:
            p = pa.plan(dims, win, hkv, bs, num_cus=cus, **opts)
        except pa.PaError as e:
            assert e.status in (pa.ERR_UNSUPPORTED, pa.ERR_INVALID_ARG), e
            refused += 1
            continue
        planned += 1
        R = G * ql
        span = min(L, win + ql - 1) if win else L
        assert p["rows"] == R and p["span_max"] == span, p
        P = p["part_size"]
        assert P >= 32 and P % 32 == 0, p
        assert p["num_parts"] == -(-(span + 31) // P) or (p["num_parts"] == 1 and P >= span + 31), p
        assert p["one_shot"] == (p["num_parts"] == 1), p
        assert p["row_blocks"] * p["block_rows"] >= R > (p["row_blocks"] - 1) * p["block_rows"], p
        assert p["waves"] in (1, 2, 4), p
        if kv == pa.KV_FP8_E4M3:
            assert p["path"] == pa.PATH_MFMA, p
        if dtype == pa.F32:
            assert p["path"] != pa.PATH_MFMA, p
        if p["path"] == pa.PATH_MFMA:
            assert D in (64, 128, 256) and p["block_rows"] == 16 * p["row_tiles"], p
            pair = (p["row_tiles"], p["waves"])
            assert pair in (MFMA_SHAPES if D != 256 else {(1, 1), (1, 2), (1, 4)}), p
        else:
            assert p["streaming"] == 0, p
        if p["persistent"]:
            assert p["path"] in (pa.PATH_MFMA, pa.PATH_VALU) and B <= 1024, p
            assert p["row_blocks"] == 1 and p["ps_grid"] > 0, p
        else:
            assert p["ps_grid"] == 0, p
        # workspace: 256-byte aligned regions of maxima, exp-sums, outputs,
        # run records (persistent) and row offsets (batches above 1024)
        units = B * hkv
        slots = 0 if p["one_shot"] else (p["ps_grid"] + units if p["persistent"] else units * p["num_parts"])
        S = slots * R
        ws = 2 * _align256(S * 4) + _align256(S * D * 4)
        ws += _align256(units * 8) if p["persistent"] and not p["one_shot"] else 0
        ws += _align256(B * 4) if B > 1024 else 0
        assert p["workspace_bytes"] == ws, (p, ws)
    assert planned > 2000 and refused > 0, (planned, refused)
