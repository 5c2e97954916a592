"""pa_pack_kv_cache: row-layout caches [num_blocks, H_kv, block_size, D]
repacked on the GPU into the tiled layouts must equal, byte for byte, the
tiled caches the seeded input generator lays out directly (workloads.py), for
bf16, fp32 and FP8 elements, head dims on and off the column grid, and block
sizes 16-1024; a listed subset of blocks changes only those blocks; and a
decode over the repacked caches gives the same output bits."""

from dataclasses import replace

import pytest
import torch

import decode_attention_pa_amd as pa
import workloads
from tests._gpu_util import run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def rows_of(case):
    """The case's tiled caches rearranged to one row per slot (test-side
    indexing from the layout description; no library code)."""
    k, v = case.k_cache, case.v_cache
    nb, hkv = k.shape[:2]
    bs, D = case.w.block_size, case.w.head_dim
    s = torch.arange(bs, device=k.device)
    if k.dim() == 4:
        kr = k.clone()
    else:
        grp, half, place = workloads.k_slot(s)
        kr = k[:, :, grp, half, :, place, :]            # [bs, nb, hkv, D/E, E]
        kr = kr.permute(1, 2, 0, 3, 4).reshape(nb, hkv, bs, D).contiguous()
    E = v.shape[-1]
    vr = v[:, :, s // E, :, s % E]                       # [bs, nb, hkv, D]
    vr = vr.permute(1, 2, 0, 3).contiguous()
    return kr, vr


def raw(t):
    return t.contiguous().view(torch.uint8)


SHAPES = [
    dict(name="gqa_bf16", batch=3),                                     # bf16 D=128 bs=16
    dict(name="swa_mtp_bf16", batch=3),                                 # bf16 D=64 bs=64
    dict(name="gqa_fp8kv", batch=3),                                    # FP8 D=128 bs=16
    dict(name="large_block_mtp_bf16", batch=2, len_range=(2048, 5000)),  # bs=1024
    dict(name="tiny_f32"),                                              # fp32 D=64
    dict(name="tiny_f32", head_dim=66, block_size=32, max_blocks_per_seq=2),  # fp32, K rows
    dict(name="gqa_bf16", batch=2, head_dim=200, num_q_heads=16, num_kv_heads=8),  # bf16 D=200
    dict(name="gqa_d256_bf16", batch=2),                                # bf16 D=256
    dict(name="tiny_f32", pool=70000),            # more blocks than 65536 (one grid dimension)
]


@pytest.mark.parametrize("over", SHAPES, ids=lambda o: "-".join(f"{k}{v}" for k, v in o.items()))
def test_pack_matches_generator_layout(over):
    w = replace(workloads.WORKLOADS[over["name"]], **{k: v for k, v in over.items() if k != "name"})
    c = workloads.make_case(w, device="cuda", window=w.windows[0])
    kr, vr = rows_of(c)
    say(f"[case] pack {w.name} D={w.head_dim} bs={w.block_size} {c.k_cache.dtype} "
        f"k_cache={tuple(c.k_cache.shape)}")
    k2, v2 = pa.pack_kv_cache(kr, vr)
    torch.cuda.synchronize()
    assert k2.shape == c.k_cache.shape and v2.shape == c.v_cache.shape
    assert torch.equal(raw(k2), raw(c.k_cache))
    assert torch.equal(raw(v2), raw(c.v_cache))


def test_pack_listed_blocks_only():
    w = replace(workloads.WORKLOADS["gqa_bf16"], batch=4)
    c = workloads.make_case(w, device="cuda")
    kr, vr = rows_of(c)
    nb = c.k_cache.shape[0]
    ids = [0, 5, nb - 1, 7]
    k2 = torch.full_like(c.k_cache, 3.0)
    v2 = torch.full_like(c.v_cache, 3.0)
    sel = torch.tensor(ids + [nb, -1], dtype=torch.int32, device="cuda")   # two ids out of range
    pa.pack_kv_cache(kr, vr, k2, v2, block_ids=sel)
    torch.cuda.synchronize()
    listed = torch.zeros(nb, dtype=torch.bool, device="cuda")
    listed[ids] = True
    assert torch.equal(raw(k2[listed]), raw(c.k_cache[listed]))
    assert torch.equal(raw(v2[listed]), raw(c.v_cache[listed]))
    assert bool((k2[~listed] == 3.0).all()) and bool((v2[~listed] == 3.0).all())


@pytest.mark.parametrize("name,window", [("gqa_bf16", 0), ("swa_mtp_bf16", 128)])
def test_decode_over_repacked_caches(name, window):
    w = replace(workloads.WORKLOADS[name], batch=8)
    c = workloads.make_case(w, device="cuda", window=window)
    expect = run_gpu(c).clone()
    kr, vr = rows_of(c)
    c.k_cache, c.v_cache = pa.pack_kv_cache(kr, vr)
    assert torch.equal(run_gpu(c), expect)
