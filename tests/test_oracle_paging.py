"""Pins of the integer oracle: brute force from the dense mask, closed forms, a hand-derived replay."""
import json
import os

import numpy as np
import pytest

from oracle import attention, paging
from oracle.paging import GLOBAL, LOCAL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_held_pages_are_exactly_the_pages_some_query_sees():
    """Brute force: the pages touched by the union of the call's visible sets (dense mask scan)."""
    rng = np.random.Generator(np.random.PCG64(7))
    for _ in range(400):
        L = int(rng.integers(1, 300))
        qs = int(rng.integers(0, L))
        S = int(rng.choice([0, 1, 4, 20, 400]))
        W = int(rng.choice([1, 2, 16, 33, 128, 1000]))
        P = int(rng.choice([1, 4, 16, 64]))
        for cls in (GLOBAL, LOCAL):
            m = attention.visibility_mask(cls, np.arange(qs, L), L, S, W)
            seen = np.flatnonzero(m.any(axis=0))
            want = sorted(set((seen // P).tolist()))
            assert paging.held_pages(cls, qs, L, S, W, P) == want


def test_visible_intervals_closed_form():
    L = 90
    for S, W in [(0, 1), (4, 10), (12, 10), (3, 1), (0, 200)]:
        for cls in (GLOBAL, LOCAL):
            m = attention.visibility_mask(cls, np.arange(L), L, S, W)
            for i in range(L):
                got = paging.visible_intervals(m[i])
                if cls == GLOBAL:
                    want = [(0, i + 1)]
                else:
                    w0 = max(0, i - W + 1)
                    want = [(0, i + 1)] if min(S, i + 1) >= w0 else \
                        ([(0, min(S, i + 1))] if S > 0 else []) + [(w0, i + 1)]
                assert got == want, (cls, S, W, i)


def test_pair_count_closed_forms():
    for L, qs, S, W in [(512, 0, 4, 128), (300, 120, 0, 7), (77, 76, 5, 3), (1000, 10, 4, 1024)]:
        mg = attention.visibility_mask(GLOBAL, np.arange(qs, L), L, S, W)
        ml = attention.visibility_mask(LOCAL, np.arange(qs, L), L, S, W)
        assert paging.pair_count(mg) == sum(i + 1 for i in range(qs, L))
        assert paging.pair_count(ml) == sum(min(i + 1, W) + min(S, max(0, i + 1 - W)) for i in range(qs, L))


def test_tiny_config_page_counts():
    """L=512, P=16, S=4, W=128: 32 pages each during prefill; the local head keeps 9 (0 and 24..31)."""
    assert paging.held_pages(GLOBAL, 0, 512, 4, 128, 16) == list(range(32))
    assert paging.held_pages(LOCAL, 0, 512, 4, 128, 16) == list(range(32))
    assert paging.retained_pages(LOCAL, 512, 4, 128, 16) == [0] + list(range(24, 32))
    assert paging.retained_pages(GLOBAL, 512, 4, 128, 16) == list(range(32))


def test_reused_prefix_local_head_page_count():
    """8K queries after a 120K reused prefix, P=64, S=4, W=4096: sink page 0 plus pages 1856..2047.

    The first query (position 122880) sees keys down to 122880 - 4095 = 118785, which lies in page 1856.
    """
    pages = paging.held_pages(LOCAL, 122880, 131072, 4, 4096, 64)
    assert pages == [0] + list(range(1856, 2048))
    assert len(pages) == 193
    assert paging.segments(pages, 64) == [(0, 1, 0), (1856 * 64, 192, 1)]


def test_segments_merge_touching_runs():
    assert paging.segments([0, 1, 2, 5, 6, 9], 16) == [(0, 3, 0), (80, 2, 3), (144, 1, 5)]
    # sink and window pages that touch merge into one segment
    assert paging.segments(paging.held_pages(LOCAL, 40, 60, 16, 30, 16), 16) == [(0, 4, 0)]


def test_allocator_replay_matches_hand_derivation():
    gd = json.load(open(os.path.join(GOLDEN, "alloc_tiny.json")))
    hc = np.array(gd["head_class"], np.uint8)
    pool = paging.PoolReplay(gd["num_pages"], gd["free_order"])
    t = pool.build(0, 1, hc, gd["q_starts"], gd["kv_lens"], gd["sink"], gd["window"], gd["page_size"])
    as_json = {"%d,%d,%d" % k: {str(p): i for p, i in v.items()} for k, v in t.items()}
    assert as_json == gd["tables_after_build"]
    for key, segs in gd["segments_after_build"].items():
        k = tuple(int(x) for x in key.split(","))
        assert [list(s) for s in paging.segments(sorted(t[k]), gd["page_size"])] == segs
    assert list(pool.free) == gd["free_after_build"]
    t2 = pool.trim(t, hc, gd["kv_lens"], gd["sink"], gd["window"], gd["page_size"])
    assert {"%d,%d,%d" % k: {str(p): i for p, i in v.items()} for k, v in t2.items()} == gd["tables_after_trim"]
    assert list(pool.free) == gd["free_after_trim"]
    pool.release(t2)
    assert list(pool.free) == gd["free_after_release"]


def test_allocator_invariants_and_transactional_failure():
    rng = np.random.Generator(np.random.PCG64(3))
    for trial in range(30):
        Hkv = int(rng.integers(1, 5))
        nl = int(rng.integers(1, 3))
        hc = rng.integers(0, 2, size=(nl, Hkv)).astype(np.uint8)
        B = int(rng.integers(1, 4))
        kv = [int(x) for x in rng.integers(0, 200, size=B)]
        qs = [int(rng.integers(0, L + 1)) for L in kv]
        need = sum(len(paging.held_pages(int(hc[l, g]), q, L, 3, 40, 16))
                   for l in range(nl) for g in range(Hkv) for q, L in zip(qs, kv))
        N = need + int(rng.integers(0, 5))
        pool = paging.PoolReplay(N, rng.permutation(N))
        t = pool.build(0, nl, hc, qs, kv, 3, 40, 16)
        ids = [i for v in t.values() for i in v.values()]
        assert len(ids) == len(set(ids)) == need == pool.used
        assert all(0 <= i < N for i in ids)
        assert pool.used + len(pool.free) == N
        before = list(pool.free)
        if len(pool.free) < need:
            with pytest.raises(paging.OutOfPages):
                pool.build(0, nl, hc, qs, kv, 3, 40, 16)
            assert list(pool.free) == before
        pool.release(t)
        assert pool.used == 0


def test_empty_and_zero_length_sequences():
    assert paging.held_token_ranges(GLOBAL, 0, 0, 4, 8) == []
    assert paging.held_pages(LOCAL, 0, 0, 4, 8, 16) == []
    # no queries (q_start == kv_len): a local head still holds what its next query would see
    assert paging.held_token_ranges(LOCAL, 50, 50, 4, 8) == [(0, 4), (43, 50)]


def test_held_token_ranges_are_the_runs_of_the_visible_union():
    """Brute force: held token ranges equal the runs of keys that some query of the call sees."""
    rng = np.random.Generator(np.random.PCG64(11))
    for _ in range(300):
        L = int(rng.integers(1, 200))
        qs = int(rng.integers(0, L))
        S = int(rng.choice([0, 1, 4, 9, 300]))
        W = int(rng.choice([1, 3, 6, 50, 500]))
        for cls in (GLOBAL, LOCAL):
            m = attention.visibility_mask(cls, np.arange(qs, L), L, S, W)
            assert paging.held_token_ranges(cls, qs, L, S, W) == paging.visible_intervals(m.any(axis=0))


def _golden_tables(d):
    return {tuple(int(x) for x in k.split(",")): {int(p): v for p, v in t.items()} for k, t in d.items()}


def test_golden_advance_replay():
    # hand-derived: pages that stay held keep their ids, released pages are pushed first, new pages
    # are taken from the head after, both in (layer, kv head, seq, logical page) order
    g = json.load(open(os.path.join(GOLDEN, "advance_small.json")))
    hc = np.array(g["head_class"], np.uint8)
    pool = paging.PoolReplay(g["num_pages"])
    t = pool.build(0, 1, hc, g["build"]["q_starts"], g["build"]["kv_lens"], g["sink"], g["window"], g["page_size"])
    assert t == _golden_tables(g["tables_after_build"])
    kv = g["build"]["kv_lens"]
    t = pool.trim(t, hc, kv, g["sink"], g["window"], g["page_size"])
    for st in g["steps"]:
        t, kv = pool.advance(t, hc, kv, st["n_new"], g["sink"], g["window"], g["page_size"])
        assert kv == st["kv_lens"]
        assert t == _golden_tables(st["tables"])
        assert list(pool.free) == st["free"]
    before = (dict(t), list(pool.free))
    with pytest.raises(paging.OutOfPages):
        pool.advance(t, hc, kv, g["out_of_pages"]["n_new"], g["sink"], g["window"], g["page_size"])
    assert (dict(t), list(pool.free)) == before


@pytest.mark.parametrize("seed", range(8))
def test_advance_holds_exactly_the_pages_of_the_visible_keys(seed):
    # after any sequence of advances, a (kv head, seq) holds the pages of the keys some query of the
    # latest call sees (brute force over the dense mask), and no id is held twice
    rng = np.random.Generator(np.random.PCG64(3100 + seed))
    Hkv, P = 3, int(rng.choice([4, 8, 16]))
    S, W = int(rng.choice([0, 1, 5])), int(rng.choice([1, 3, 17, 40]))
    hc = rng.integers(0, 2, size=(1, Hkv)).astype(np.uint8)
    kv = [int(x) for x in rng.integers(1, 60, size=2)]
    qs = [int(rng.integers(0, L)) for L in kv]
    pool = paging.PoolReplay(4000)
    t = pool.build(0, 1, hc, qs, kv, S, W, P)
    for _ in range(6):
        n_new = [int(x) for x in rng.integers(0, 9, size=2)]
        old = kv
        t, kv = pool.advance(t, hc, kv, n_new, S, W, P)
        ids = [pid for tt in t.values() for pid in tt.values()]
        assert len(ids) == len(set(ids)) and len(ids) + len(pool.free) == 4000
        for (l, g, b), tt in t.items():
            if kv[b] == 0:
                assert tt == {}
                continue
            pos = np.arange(old[b], kv[b])
            m = attention.visibility_mask(int(hc[0, g]), pos, kv[b], S, W) if len(pos) else np.zeros((0, kv[b]), bool)
            want = sorted(set((np.flatnonzero(m.any(axis=0)) // P).tolist()))
            if not len(pos):  # no query: the retained state, what a query at kv_len would see
                m = attention.visibility_mask(int(hc[0, g]), np.array([kv[b]]), kv[b] + 1, S, W)[:, :kv[b]]
                want = sorted(set((np.flatnonzero(m[0]) // P).tolist()))
            assert sorted(tt) == want
