"""Pins for the CPU oracle: it is checked against things other than itself.

* brute force (``oracle.brute``) on tiny shuffled-block GQA / MTP cases;
* the textbook reduction: ``torch.nn.functional.scaled_dot_product_attention``
  in float64 on the gathered, contiguous K/V with an explicit mask and torch's
  own GQA head mapping;
* hand-derived visible sets (``tests/golden/visible_sets.json``);
* closed forms (equal keys give the mean of the visible values; two logits
  ln 3 apart give weights 1/4 and 3/4; a dominant logit returns its value);
* identities the pages fix: window 0 == window >= context, one partition ==
  any split (float64 LSE merge), window 1 returns the token's own value,
  constant V returns the constant, MTP row i == a single-token call over the
  shorter context, GQA == MHA with repeated KV heads.
All CPU, seconds.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import brute
from oracle import paged_attention as pa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _values(cache, scale):
    """Cache tensor as float64 values (FP8 codes dequantized by the oracle)."""
    if cache.dtype == torch.float8_e4m3fn:
        return pa.dequantize(cache.view(torch.uint8).numpy(), scale)
    return cache.float().numpy().astype(np.float64)


def as_np(case):
    return dict(
        q=case.q.float().numpy().astype(np.float64),
        k_cache=_values(case.k_cache, case.w.k_scale),
        v_cache=_values(case.v_cache, case.w.v_scale),
        block_tables=case.block_tables.numpy().astype(np.int64),
        seq_lens=np.array(case.seq_lens_host), query_lens=np.array(case.query_lens_host),
        scale=case.scale, window=case.window,
        num_kv_heads=case.w.num_kv_heads, block_size=case.w.block_size)


def tiny_random(seed, **over):
    """Random tiny workload: B<=3, G in {1,2,4}, q in {1,2,4}, bs in {1,2,16}."""
    r = np.random.default_rng(seed)
    B = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 4]))
    hkv = int(r.choice([1, 2]))
    ql = int(r.choice([1, 2, 4]))
    bs = int(r.choice([1, 2, 16]))
    lens = tuple(int(x) for x in r.integers(ql, 40, size=B))
    D = int(r.choice([4, 8]))
    w = workloads.custom(
        name=f"tiny{seed}", batch=B, num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D,
        block_size=bs, query_len=ql, seq_lens=lens, max_seq_len=max(lens),
        max_blocks_per_seq=-(-max(lens) // bs) + 2, pool=0, seed=100 + seed,
        scale=float(r.choice([1.0, 0.5, 0.125])))
    w = workloads.replace(w, **over) if over else w
    return w


def windows_for(lens):
    L = max(lens)
    return [0, 1, 2, 5, L, L + 3]


@pytest.mark.parametrize("seed", range(12))
def test_matches_brute_force(seed):
    w = tiny_random(seed)
    for win in windows_for(w.seq_lens):
        a = as_np(workloads.make_case(w, window=win, poison=False))
        ref = pa.decode(**a)
        bf = np.array(brute.brute_decode(**a))
        assert ref.shape == bf.shape
        assert np.max(np.abs(ref - bf)) <= 1e-12, (seed, win)


@pytest.mark.parametrize("window", [0, 5])
def test_tiny_workload_matches_brute_force(window):
    a = as_np(workloads.make_case("tiny_f32", window=window, poison=True))
    ref = pa.decode(**a)
    bf = np.array(brute.brute_decode(**a))
    assert np.all(np.isfinite(ref))
    assert np.max(np.abs(ref - bf)) <= 1e-12


def _k_rows(k):
    """Any K cache as rows [num_blocks, H_kv, bs, D]: the tiled form
    (16-slot groups, two halves of 8 places, dims in columns of 8 or 16)
    undone slot by slot."""
    if k.ndim == 4:
        return k
    nb, H, ngrp, _, ncol, _, width = k.shape
    rows = np.empty((nb, H, ngrp * 16, ncol * width), k.dtype)
    for s in range(ngrp * 16):
        u = s % 16
        half = 1 if u % 8 >= 4 else 0
        place = u % 4 + (4 if u >= 8 else 0)
        rows[:, :, s, :] = k[:, :, s // 16, half, :, place, :].reshape(nb, H, ncol * width)
    return rows


def _k_tiled(rows):
    """Rows [num_blocks, H_kv, bs, D] into the tiled form, slot by slot."""
    nb, H, bs, D = rows.shape
    k = np.full((nb, H, bs // 16, 2, D // 8, 8, 8), np.nan)
    for s in range(bs):
        u = s % 16
        half = 1 if u % 8 >= 4 else 0
        place = u % 4 + (4 if u >= 8 else 0)
        k[:, :, s // 16, half, :, place, :] = rows[:, :, s, :].reshape(nb, H, D // 8, 8)
    return k


def _sdpa_reference(a):
    """Gather each sequence's context contiguously and call torch SDPA (float64)."""
    out = []
    qoff = 0
    bs = a["block_size"]
    Hkv = a["num_kv_heads"]
    for b, (L, ql) in enumerate(zip(a["seq_lens"], a["query_lens"])):
        L, ql = int(L), int(ql)
        t = np.arange(L)
        blk = a["block_tables"][b][t // bs]
        K = _k_rows(a["k_cache"])[blk, :, t % bs, :]           # [L, Hkv, D]
        g = a["v_cache"].shape[-1]
        V = np.stack([a["v_cache"][blk[j], :, (t[j] % bs) // g, :, (t[j] % bs) % g]
                      for j in range(L)])                      # [L, Hkv, D]
        Q = a["q"][qoff:qoff + ql]                             # [ql, Hq, D]
        i = np.arange(ql)[:, None]
        p = L - ql + i
        win = a["window"]
        mask = (t[None, :] <= p) & ((win == 0) | (t[None, :] > p - win))
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q).permute(1, 0, 2)[None],
            torch.from_numpy(K).permute(1, 0, 2)[None],
            torch.from_numpy(V).permute(1, 0, 2)[None],
            attn_mask=torch.from_numpy(mask)[None, None],
            scale=float(np.float32(a["scale"])), enable_gqa=Hkv != Q.shape[1])
        out.append(o[0].permute(1, 0, 2).numpy())
        qoff += ql
    return np.concatenate(out, 0)


@pytest.mark.parametrize("seed", range(8))
def test_matches_torch_sdpa(seed):
    w = tiny_random(seed + 50)
    for win in windows_for(w.seq_lens):
        a = as_np(workloads.make_case(w, window=win, poison=False))
        assert np.max(np.abs(pa.decode(**a) - _sdpa_reference(a))) <= 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_tiled_key_layout_is_the_row_layout(seed):
    """The library's tiled K form holds the same keys as one row per slot:
    converting a row-layout cache slot by slot gives identical oracle and
    brute-force outputs, and the generator's tiled caches read back as rows
    agree with the oracle's own gather."""
    r = np.random.default_rng(300 + seed)
    bs = int(r.choice([16, 32]))
    w = tiny_random(seed + 70, block_size=bs, head_dim=int(r.choice([8, 16])),
                    max_blocks_per_seq=-(-40 // bs) + 2)
    for win in (0, 3):
        a = as_np(workloads.make_case(w, window=win, poison=False))
        assert a["k_cache"].ndim == 7                       # generator made the tiled form
        rows = dict(a, k_cache=_k_rows(a["k_cache"]))
        np.testing.assert_array_equal(pa.decode(**a), pa.decode(**rows))
        np.testing.assert_array_equal(np.array(brute.brute_decode(**a)),
                                      np.array(brute.brute_decode(**rows)))
        back = dict(a, k_cache=_k_tiled(rows["k_cache"]))
        np.testing.assert_array_equal(back["k_cache"], a["k_cache"])
        # the generator's slot accessors agree with the slot-by-slot reading
        kt = torch.from_numpy(a["k_cache"].copy())
        for slot in range(bs):
            np.testing.assert_array_equal(workloads.read_k_row(kt, 1, 0, slot).numpy(),
                                          rows["k_cache"][1, 0, slot])
            workloads.write_k_row(kt, 1, 0, slot, torch.full((kt.shape[4] * 8,), float(slot)))
        assert np.all(_k_rows(kt.numpy())[1, 0] == np.arange(bs)[:, None])
        for b in range(len(a["seq_lens"])):
            t = np.arange(int(a["seq_lens"][b]))
            blk = a["block_tables"][b][t // bs]
            for h in range(a["num_kv_heads"]):
                np.testing.assert_array_equal(
                    pa.gather_keys(a["k_cache"], a["block_tables"][b], t, h, bs),
                    rows["k_cache"][blk, h, t % bs, :])


@pytest.mark.parametrize("window", [0, 5])
def test_tiny_workload_matches_torch_sdpa(window):
    a = as_np(workloads.make_case("tiny_f32", window=window, poison=True))
    assert np.max(np.abs(pa.decode(**a) - _sdpa_reference(a))) <= 1e-12


def test_golden_visible_sets():
    g = json.load(open(os.path.join(GOLDEN, "visible_sets.json")))
    for c in g["cases"]:
        got = [list(pa.visible_range(c["seq_len"], c["query_len"], i, c["window"]))
               for i in range(c["query_len"])]
        assert got == c["rows"], c["why"]


def test_golden_visible_sets_through_outputs():
    """Equal keys and one-hot values: the output row is 1/n on exactly the
    visible positions, for the oracle and for the brute force."""
    g = json.load(open(os.path.join(GOLDEN, "visible_sets.json")))
    for c in g["cases"]:
        L, ql, win = c["seq_len"], c["query_len"], c["window"]
        if L > 64:
            continue
        bs = 4
        nb = -(-L // bs)
        D = L
        k = np.ones((nb, 1, bs, D))
        v = np.zeros((nb, 1, 1, D, bs))            # one slot group per block
        for t in range(L):
            v[t // bs, 0, 0, t, t % bs] = 1.0
        a = dict(q=np.ones((ql, 1, D)), k_cache=k, v_cache=v,
                 block_tables=np.arange(nb)[None, :], seq_lens=np.array([L]),
                 query_lens=np.array([ql]), scale=1.0, window=win, num_kv_heads=1, block_size=bs)
        for out in (pa.decode(**a), np.array(brute.brute_decode(**a))):
            for i, (lo, hi) in enumerate(c["rows"]):
                expect = np.zeros(D)
                expect[lo:hi + 1] = 1.0 / (hi - lo + 1)
                assert np.max(np.abs(out[i, 0] - expect)) <= 1e-15, c["why"]


def _one_seq(q, K, V, window=0, scale=1.0, bs=2, ql=1):
    """Wrap per-position K [L, D] and V [L, D] into a shuffled paged cache."""
    L, D = K.shape
    nb = -(-L // bs)
    perm = np.random.default_rng(7).permutation(nb + 3)
    k = np.full((nb + 3, 1, bs, D), np.nan)
    v = np.full((nb + 3, 1, 1, D, bs), np.nan)     # one slot group per block
    for t in range(L):
        k[perm[t // bs], 0, t % bs, :] = K[t]
        v[perm[t // bs], 0, 0, :, t % bs] = V[t]
    return dict(q=np.asarray(q, float).reshape(ql, 1, D), k_cache=k, v_cache=v,
                block_tables=perm[None, :nb], seq_lens=np.array([L]), query_lens=np.array([ql]),
                scale=scale, window=window, num_kv_heads=1, block_size=bs)


def test_closed_form_two_logits():
    # logits 0 and ln 3 -> weights 1/4, 3/4 -> 0.25*4 + 0.75*8 = 7
    K = np.array([[5.0], [0.0], [math.log(3.0)]])
    V = np.array([[100.0], [4.0], [8.0]])
    a = _one_seq([1.0], K, V, window=2)
    assert abs(pa.decode(**a)[0, 0, 0] - 7.0) <= 4e-15
    assert abs(brute.brute_decode(**a)[0][0][0] - 7.0) <= 4e-15


def test_closed_form_dominant_logit():
    # one logit 1000 above the rest: every other weight underflows to 0
    r = np.random.default_rng(3)
    K = r.normal(size=(11, 4))
    V = r.normal(size=(11, 4))
    q = np.array([1.0, 0, 0, 0])
    K[6] = [1000.0, 0, 0, 0]
    a = _one_seq(q, K, V)
    np.testing.assert_array_equal(pa.decode(**a)[0, 0], V[6])


def test_closed_form_equal_keys_mean():
    r = np.random.default_rng(4)
    K = np.tile(r.normal(size=(1, 8)), (13, 1))
    V = r.normal(size=(13, 8))
    for win, lo in [(0, 0), (4, 9), (13, 0)]:
        a = _one_seq(r.normal(size=8), K, V, window=win, scale=0.3)
        np.testing.assert_allclose(pa.decode(**a)[0, 0], V[lo:].mean(0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(6))
def test_window_zero_equals_window_at_least_context(seed):
    w = tiny_random(seed + 200)
    L = max(w.seq_lens)
    a0 = as_np(workloads.make_case(w, window=0, poison=False))
    for win in (L, L + 1, 10 * L):
        a = dict(a0, window=win)
        np.testing.assert_array_equal(pa.decode(**a0), pa.decode(**a))


@pytest.mark.parametrize("seed", range(6))
def test_one_partition_equals_any_split(seed):
    w = tiny_random(seed + 300)
    r = np.random.default_rng(seed)
    for win in windows_for(w.seq_lens):
        a = as_np(workloads.make_case(w, window=win, poison=False))
        ref = pa.decode(**a)
        for _ in range(3):
            cuts = {b: sorted(set(int(x) for x in r.integers(0, int(L) + 1, size=r.integers(0, 6))))
                    for b, L in enumerate(a["seq_lens"])}
            got = pa.decode_split(**a, boundaries=lambda b: cuts[b])
            assert np.max(np.abs(got - ref)) <= 1e-13


def test_split_with_empty_partitions_contributes_nothing():
    w = tiny_random(400)
    a = as_np(workloads.make_case(w, window=2, poison=False))
    # many cut points inside the window's dead zone: most partitions are empty
    got = pa.decode_split(**a, boundaries=lambda b: list(range(1, int(a["seq_lens"][b]))))
    assert np.max(np.abs(got - pa.decode(**a))) <= 1e-13


def test_window_one_returns_own_value():
    w = tiny_random(500, query_len=2, seq_lens=(9, 17), batch=2)
    a = as_np(workloads.make_case(w, window=1, poison=False))
    out = pa.decode(**a)
    G = w.num_q_heads // w.num_kv_heads
    row = 0
    for b, (L, ql) in enumerate(zip(a["seq_lens"], a["query_lens"])):
        for i in range(ql):
            p = L - ql + i
            blk = a["block_tables"][b][p // w.block_size]
            for hq in range(w.num_q_heads):
                g = a["v_cache"].shape[-1]
                s = p % w.block_size
                np.testing.assert_array_equal(out[row, hq], a["v_cache"][blk, hq // G, s // g, :, s % g])
            row += 1


def test_constant_values_return_constant():
    w = tiny_random(600)
    for win in windows_for(w.seq_lens):
        a = as_np(workloads.make_case(w, window=win, poison=False))
        a["v_cache"] = np.full_like(a["v_cache"], -0.3125)
        assert np.max(np.abs(pa.decode(**a) + 0.3125)) <= 1e-15


@pytest.mark.parametrize("win", [0, 1, 3, 7])
def test_mtp_row_equals_single_token_call_over_shorter_context(win):
    w = tiny_random(700, query_len=4, seq_lens=(23, 30), batch=2)
    a = as_np(workloads.make_case(w, window=win, poison=False))
    out = pa.decode(**a)
    row = 0
    for b, (L, ql) in enumerate(zip(a["seq_lens"], a["query_lens"])):
        for i in range(ql):
            one = dict(a, q=a["q"][row:row + 1], seq_lens=np.array([L - (ql - 1 - i)]),
                       query_lens=np.array([1]), block_tables=a["block_tables"][b:b + 1])
            assert np.max(np.abs(pa.decode(**one)[0] - out[row])) <= 1e-15
            row += 1


def test_gqa_equals_mha_with_repeated_kv_heads():
    w = tiny_random(800, num_q_heads=4, num_kv_heads=2)
    a = as_np(workloads.make_case(w, window=3, poison=False))
    G = 2
    mha = dict(a, k_cache=np.repeat(a["k_cache"], G, axis=1),
               v_cache=np.repeat(a["v_cache"], G, axis=1), num_kv_heads=4)
    # same arithmetic, only the BLAS call shape differs: rounding-level agreement
    assert np.max(np.abs(pa.decode(**a) - pa.decode(**mha))) <= 1e-15


def test_spans_match_visible_ranges_and_tables():
    w = tiny_random(900, query_len=2, seq_lens=(5, 33, 2), batch=3, block_size=4,
                    max_blocks_per_seq=12)
    c = workloads.make_case(w, window=6, poison=False)
    sp = pa.spans(c.tables_host.numpy(), c.seq_lens_host, c.query_lens_host, 6, 4)
    assert [s["qoff"] for s in sp] == [0, 2, 4]
    assert (sp[1]["lo"], sp[1]["hi"]) == (26, 33)     # rows at 31, 32; window 6 -> 26..32
    assert sp[1]["rows"] == [(26, 31), (27, 32)]
    expect = np.full(12, -1)
    expect[6:9] = c.tables_host.numpy()[1, 6:9]       # positions 26..32 live in blocks 6, 7, 8
    np.testing.assert_array_equal(sp[1]["blocks"], expect)
    assert (sp[2]["lo"], sp[2]["hi"]) == (0, 2)


def test_oracle_rejects_query_longer_than_context():
    w = tiny_random(901, query_len=2, seq_lens=(5,), batch=1)
    a = as_np(workloads.make_case(w, window=0, poison=False))
    a["seq_lens"] = np.array([1])
    with pytest.raises(ValueError):
        pa.decode(**a)


def test_poisoned_tail_and_unused_blocks_are_not_visible():
    """Workload poison (NaN past seq_len and in unused blocks) never reaches
    the oracle's output: it only reads visible positions."""
    for win in (0, 5):
        a = as_np(workloads.make_case("tiny_f32", window=win, poison=True))
        assert np.isnan(a["k_cache"]).any()
        assert np.all(np.isfinite(pa.decode(**a)))



def test_e4m3_decoding_matches_the_format():
    """All 256 codes: the oracle's vectorised decoder, the brute-force bit-field
    decoder and torch's float8_e4m3fn conversion agree (NaN for 0x7F / 0xFF);
    and a few values fixed by the format: 448 is the largest finite value,
    2^-6 the smallest normal, 2^-9 the smallest subnormal."""
    codes = np.arange(256, dtype=np.uint8)
    mine = pa.decode_e4m3(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    bits = np.array([brute.e4m3_value(int(c)) for c in codes])
    np.testing.assert_array_equal(mine, lib)
    np.testing.assert_array_equal(mine, bits)
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and np.isfinite(mine[0x7E])
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9 and mine[0x07] == 7 * 2.0 ** -9
    assert mine[0x38] == 1.0 and mine[0xB8] == -1.0 and mine[0x00] == 0.0
    assert np.nanmax(mine) == 448.0 and np.count_nonzero(np.isnan(mine)) == 2
    # dequantize multiplies by the float32 value of the scale
    assert pa.dequantize(np.array([0x38], np.uint8), 0.1)[0] == float(np.float32(0.1))


@pytest.mark.parametrize("seed", range(6))
def test_fp8_caches_match_brute_force_and_rows(seed):
    """FP8 tiled caches (K columns of 16 dims, V groups of 16 slots): the
    oracle on dequantized codes equals the brute force, equals the oracle on
    the same values laid out one row per slot, and equals torch SDPA."""
    r = np.random.default_rng(400 + seed)
    bs = int(r.choice([16, 32]))
    w = tiny_random(seed + 90, block_size=bs, head_dim=int(r.choice([16, 32])), dtype="bf16",
                    kv_dtype="fp8", max_blocks_per_seq=-(-40 // bs) + 2)
    for win in (0, 4):
        case = workloads.make_case(w, window=win, poison=False)
        assert case.k_cache.dtype == torch.float8_e4m3fn and case.k_cache.shape[-1] == 16
        a = as_np(case)
        ref = pa.decode(**a)
        assert np.max(np.abs(ref - np.array(brute.brute_decode(**a)))) <= 1e-12
        rows = dict(a, k_cache=_k_rows(a["k_cache"]))
        np.testing.assert_array_equal(ref, pa.decode(**rows))
        assert np.max(np.abs(ref - _sdpa_reference(a))) <= 1e-12
        # the cached values are the codes times the scales, not the codes
        assert np.nanmax(np.abs(a["k_cache"])) <= 448 * float(np.float32(w.k_scale))
