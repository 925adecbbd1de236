"""Continuing sequences over the retained segmented state (decode) through the C ABI, on the CPU
(host-only tables): rk_seg_tables_advance against the integer oracle's replay (bit-exact page ids and
free lists) and the hand-derived golden fixture; the split-KV decode items against a brute-force
scan of the decode query's visible keys (page "小红书把 KV Cache 按「头」拆了…" (zhichai.net), section
事件内容: GLOBAL heads read every context page, LOCAL heads only sink plus recent-window pages)."""
import json
import os

import numpy as np
import pytest

from head_aware_paged_prefill_amd import rk_seg
from oracle import attention, paging

from test_abi_host import fake_pool, _status

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _export(t, nl, Hkv, B, P):
    out = {}
    for l in range(nl):
        for g in range(Hkv):
            for b in range(B):
                segs, ids = rk_seg.rk_seg_tables_export(t, l, g, b)
                logical = [tb // P + i for tb, n, _ in segs for i in range(n)]
                out[(l, g, b)] = dict(zip(logical, ids))
    return out


def _golden_tables(d):
    return {tuple(int(x) for x in k.split(",")): {int(p): v for p, v in t.items()} for k, t in d.items()}


def test_golden_advance_through_the_abi():
    gd = json.load(open(os.path.join(GOLDEN, "advance_small.json")))
    P = gd["page_size"]
    pool = fake_pool(gd["num_pages"], None, 1, 2, 64, P)
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, 2, gd["build"]["q_starts"], gd["build"]["kv_lens"], gd["head_class"],
                                   gd["sink"], gd["window"], device=False)
    assert _export(t, 1, 2, 1, P) == _golden_tables(gd["tables_after_build"])
    assert rk_seg.rk_seg_pool_free_list(pool) == gd["free_after_build"]
    rk_seg.rk_seg_tables_trim(t)
    for st in gd["steps"]:
        rk_seg.rk_seg_tables_advance(t, st["n_new"], device=False)
        assert _export(t, 1, 2, 1, P) == _golden_tables(st["tables"])
        assert rk_seg.rk_seg_pool_free_list(pool) == st["free"]
        assert rk_seg.rk_seg_tables_stats(t)["total_q"] == sum(st["n_new"])
    before = (_export(t, 1, 2, 1, P), rk_seg.rk_seg_pool_free_list(pool))
    assert _status(lambda: rk_seg.rk_seg_tables_advance(t, gd["out_of_pages"]["n_new"], device=False)) == \
        rk_seg.RK_ERR_OUT_OF_PAGES
    assert (_export(t, 1, 2, 1, P), rk_seg.rk_seg_pool_free_list(pool)) == before
    rk_seg.rk_seg_tables_destroy(t)
    assert sorted(rk_seg.rk_seg_pool_free_list(pool)) == list(range(gd["num_pages"]))
    rk_seg.rk_seg_pool_destroy(pool)


@pytest.mark.parametrize("seed", range(16))
def test_advance_matches_integer_oracle_bit_exact(seed):
    rng = np.random.Generator(np.random.PCG64(4200 + seed))
    nl, Hkv = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    P = int(rng.choice([16, 32, 64]))
    B = int(rng.integers(1, 4))
    S, W = int(rng.choice([0, 4, 17])), int(rng.choice([1, 16, 50, 300]))
    hc = rng.integers(0, 2, size=(nl, Hkv)).astype(np.uint8)
    kv = [int(x) for x in rng.integers(1, 400, size=B)]
    qs = [int(rng.integers(0, L + 1)) for L in kv]
    N = 3000
    order = rng.permutation(N).tolist()
    pool = fake_pool(N, order, nl, Hkv, 64, P)
    replay = paging.PoolReplay(N, order)
    t = rk_seg.rk_seg_build_tables(pool, 0, nl, Hkv, qs, kv, hc, S, W, device=False)
    want = replay.build(0, nl, hc, qs, kv, S, W, P)
    if rng.random() < 0.5:
        rk_seg.rk_seg_tables_trim(t)
        want = replay.trim(want, hc, kv, S, W, P)
    for step in range(5):
        n_new = [int(x) for x in rng.integers(0, 3 if step % 2 else 70, size=B)]
        rk_seg.rk_seg_tables_advance(t, n_new, device=False)
        want, kv = replay.advance(want, hc, kv, n_new, S, W, P)
        assert _export(t, nl, Hkv, B, P) == want
        assert rk_seg.rk_seg_pool_free_list(pool) == list(replay.free)
        st = rk_seg.rk_seg_tables_stats(t)
        assert st["total_q"] == sum(n_new)
        assert st["pages_held"] == sum(len(x) for x in want.values())
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


def _decode_case(rng, long=False):
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 4, 8, 16]))
    P = int(rng.choice([16, 64]))
    B = int(rng.integers(1, 5))
    # long: the layer may reach 65536 visible keys, where the larger minimum chunk applies
    kv = [int(x) for x in rng.integers(20000, 70000, size=B)] if long else [int(x) for x in rng.integers(1, 5000, size=B)]
    S, W = int(rng.choice([0, 4, 40])), int(rng.choice([1, 64, 700, 3000]))
    hc = rng.integers(0, 2, size=(1, Hkv)).astype(np.uint8)
    return dict(Hkv=Hkv, G=G, P=P, kv=kv, S=S, W=W, hc=hc)


def _ranges(cls, L, S, W):
    """Visible key ranges of the query at L - 1, counted from the mask (runs of visible keys)."""
    vis = attention.visibility_mask(cls, np.array([L - 1]), L, S, W)[0].astype(np.int8)
    edges = np.flatnonzero(np.diff(np.concatenate([[0], vis, [0]])))
    return list(zip(edges[::2], edges[1::2]))


@pytest.mark.parametrize("seed", range(16))
def test_decode_items_cover_the_visible_keys_once(seed):
    rng = np.random.Generator(np.random.PCG64(4400 + seed))
    c = _decode_case(rng, long=seed >= 12)
    B, Hkv = len(c["kv"]), c["Hkv"]
    # one query row per sequence, except a sequence that does not advance (no row)
    n_new = [1 if rng.random() < 0.8 else 0 for _ in range(B)]
    n_new[0] = 1
    pre = [L - n for L, n in zip(c["kv"], n_new)]
    N = sum(Hkv * (L // c["P"] + 2) for L in c["kv"]) + 8
    pool = fake_pool(N, None, 1, Hkv, 64, c["P"])
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, c["G"] * Hkv, pre, pre, c["hc"], c["S"], c["W"], device=False)
    rk_seg.rk_seg_tables_advance(t, n_new, device=False)
    items, comb = rk_seg.rk_seg_tables_decode_schedule(t, 0)
    assert comb is not None and comb[-1] == len(items) and list(comb) == sorted(comb)
    chunk = None
    for b in range(B):
        L = c["kv"][b]
        for g in range(Hkv):
            mine = items[comb[b * Hkv + g]:comb[b * Hkv + g + 1]]
            assert (mine[:, 0] == b).all() and (mine[:, 1] == g).all()
            if not n_new[b]:
                assert len(mine) == 0
                continue
            # four items per workgroup, all of one (seq, kv head): empty items (0, 0) pad the last group
            assert len(mine) % 4 == 0 and comb[b * Hkv + g] % 4 == 0
            real = mine[mine[:, 3] > mine[:, 2]]
            pad = mine[len(real):]
            assert (pad[:, 2:] == 0).all() and len(pad) < 4, "padding only closes the group"
            vis = attention.visibility_mask(int(c["hc"][0, g]), np.array([L - 1]), L, c["S"], c["W"])[0]
            cover = np.zeros(L, np.int64)
            for _, _, k0, k1 in real.tolist():
                assert 0 <= k0 < k1 <= L
                cover[k0:k1] += 1
            assert (cover == vis.astype(np.int64)).all(), "items must cover each visible key exactly once"
            ks = real[:, 2:].tolist()
            assert ks == sorted(ks)
    # one key chunk, aiming the layer at 8192 items: a multiple of 32, at least 128 (192 from 65536
    # visible keys on); no item crosses
    # a multiple of it
    keys = sum(int(attention.visibility_mask(int(c["hc"][0, g]), np.array([L - 1]), L, c["S"], c["W"]).sum())
               for b, L in enumerate(c["kv"]) if n_new[b] for g in range(Hkv))
    ranges = sum(len(_ranges(int(c["hc"][0, g]), L, c["S"], c["W"])) for b, L in enumerate(c["kv"]) if n_new[b]
                 for g in range(Hkv))
    room = max(8192 // 4, 8192 - 2 * ranges)
    chunk = max(192 if keys >= 65536 else 128, -(-(-(-keys // room)) // 32) * 32)
    real = items[items[:, 3] > items[:, 2]]
    assert len(real) <= 8192 or room == 8192 // 4
    for _, _, k0, k1 in real.tolist():
        assert k0 // chunk == (k1 - 1) // chunk
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


def test_prefill_shaped_tables_have_no_decode_items():
    pool = fake_pool(64, None, 1, 2, 64, 16)
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, 4, [0], [100], [[1, 0]], 4, 16, device=False)
    items, comb = rk_seg.rk_seg_tables_decode_schedule(t, 0)
    assert len(items) == 0 and comb is None
    rk_seg.rk_seg_tables_advance(t, [1], device=False)
    items, comb = rk_seg.rk_seg_tables_decode_schedule(t, 0)
    assert len(items) >= 4 and len(items) % 4 == 0 and comb[-1] == len(items)
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


def test_advance_rejects_bad_input_and_keeps_state():
    pool = fake_pool(64, None, 1, 2, 64, 16)
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, 4, [0, 5], [100, 30], [[1, 0]], 4, 16, device=False)
    before = (_export(t, 1, 2, 2, 16), rk_seg.rk_seg_pool_free_list(pool))
    assert _status(lambda: rk_seg.rk_seg_tables_advance(t, [1, -1], device=False)) == rk_seg.RK_ERR_INVALID_ARG
    assert (_export(t, 1, 2, 2, 16), rk_seg.rk_seg_pool_free_list(pool)) == before
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


def test_advance_workspace_bound_does_not_depend_on_head_classes():
    pool = fake_pool(4000, None, 2, 4, 64, 16)
    sizes = set()
    for hc in (np.zeros((2, 4), np.uint8), np.ones((2, 4), np.uint8), np.array([[1, 0, 0, 1], [0, 1, 0, 0]], np.uint8)):
        t = rk_seg.rk_seg_build_tables(pool, 0, 2, 32, [0, 0], [3000, 900], hc, 4, 256, device=False)
        sizes.add(rk_seg.rk_seg_tables_advance_workspace_bytes(t, [1, 1]))
        rk_seg.rk_seg_tables_destroy(t)
    assert len(sizes) == 1
    rk_seg.rk_seg_pool_destroy(pool)
