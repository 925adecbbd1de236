"""Host logic of librk_seg.so through the C ABI, on the CPU (no device calls).

Tables, allocation, trim and release are compared bit-exactly with the integer oracle's replay;
the schedule is checked against coverage invariants derived from the dense mask.
"""
import json
import os
import re

import numpy as np
import pytest

import workloads
from head_aware_paged_prefill_amd import rk_seg
from oracle import attention, paging

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_library_exports_every_declared_function():
    header = open(os.path.join(ROOT, "include", "rk_seg.h")).read()
    declared = set(re.findall(r"^\s*(?:rk_status|const char \*|void)\s*\*?\s*(rk_\w+)\s*\(", header, re.M))
    assert declared == set(rk_seg.EXPORTS)
    lib = rk_seg.load()
    for name in declared:
        assert hasattr(lib, name), name
    assert rk_seg.rk_seg_version().startswith("rk_seg")
    import head_aware_paged_prefill_amd as pkg
    for name in declared:  # the package re-exports every entry point's binding
        assert callable(getattr(pkg, name, None)), name


def test_static_decode_scratch_size_matches_the_header():
    header = open(os.path.join(ROOT, "include", "rk_seg.h")).read()
    m = re.search(r"#define RK_DECODE_SCRATCH_BYTES \((\d+)u << (\d+)\)", header)
    assert m and int(m.group(1)) << int(m.group(2)) == rk_seg.RK_DECODE_SCRATCH_BYTES


def host_pool(num_pages, free_order=None, num_layers=1, Hkv=2, D=64, P=16, dtype=rk_seg.RK_BF16):
    return rk_seg.rk_seg_pool_create(num_layers, Hkv, D, P, num_pages, dtype, None, None, free_order)


def fake_pool(num_pages, free_order=None, num_layers=1, Hkv=2, D=64, P=16):
    """A pool whose page storage pointers are never dereferenced (host-only tables)."""
    class _T:
        def __init__(self, p):
            self.p = p

        def data_ptr(self):
            return self.p
    return rk_seg.rk_seg_pool_create(num_layers, Hkv, D, P, num_pages, rk_seg.RK_BF16, _T(1 << 20), _T(1 << 21),
                                     free_order)


def test_golden_allocator_replay_through_the_abi():
    gd = json.load(open(os.path.join(GOLDEN, "alloc_tiny.json")))
    pool = fake_pool(gd["num_pages"], gd["free_order"], 1, 2, 64, gd["page_size"])
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, 2, gd["q_starts"], gd["kv_lens"], gd["head_class"], gd["sink"],
                                   gd["window"], device=False)
    for key, want in gd["tables_after_build"].items():
        l, g, b = (int(x) for x in key.split(","))
        segs, ids = rk_seg.rk_seg_tables_export(t, l, g, b)
        assert ids == [want[p] for p in sorted(want, key=int)]
        assert [list(s) for s in segs] == gd["segments_after_build"][key]
    assert rk_seg.rk_seg_pool_free_list(pool) == gd["free_after_build"]
    rk_seg.rk_seg_tables_trim(t)
    for key, want in gd["tables_after_trim"].items():
        l, g, b = (int(x) for x in key.split(","))
        assert rk_seg.rk_seg_tables_export(t, l, g, b)[1] == [want[p] for p in sorted(want, key=int)]
    assert rk_seg.rk_seg_pool_free_list(pool) == gd["free_after_trim"]
    rk_seg.rk_seg_tables_destroy(t)
    assert rk_seg.rk_seg_pool_free_list(pool) == gd["free_after_release"]
    rk_seg.rk_seg_pool_destroy(pool)


def _random_batch(rng):
    nl = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    P = int(rng.choice([16, 32, 64, 128, 256]))
    B = int(rng.integers(0, 5))
    kv = [int(x) for x in rng.integers(0, 900, size=B)]
    qs = [int(rng.integers(0, L + 1)) if rng.random() < 0.5 else 0 for L in kv]
    S = int(rng.choice([0, 1, 4, 17, 100]))
    W = int(rng.choice([1, 5, 64, 100, 1000]))
    hc = rng.integers(0, 2, size=(nl, Hkv)).astype(np.uint8)
    lb = int(rng.integers(0, nl))
    le = int(rng.integers(lb + 1, nl + 1))
    return dict(nl=nl, Hkv=Hkv, G=G, P=P, kv=kv, qs=qs, S=S, W=W, hc=hc, lb=lb, le=le)


@pytest.mark.parametrize("seed", range(25))
def test_tables_match_integer_oracle_bit_exact(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    c = _random_batch(rng)
    need = sum(len(paging.held_pages(int(c["hc"][l, g]), q, L, c["S"], c["W"], c["P"]))
               for l in range(c["lb"], c["le"]) for g in range(c["Hkv"]) for q, L in zip(c["qs"], c["kv"]))
    N = need + int(rng.integers(0, 9))
    order = rng.permutation(N).tolist()
    pool = fake_pool(N, order, c["nl"], c["Hkv"], 64, c["P"])
    replay = paging.PoolReplay(N, order)
    t = rk_seg.rk_seg_build_tables(pool, c["lb"], c["le"], c["G"] * c["Hkv"], c["qs"], c["kv"], c["hc"], c["S"],
                                   c["W"], device=False)
    want = replay.build(c["lb"], c["le"], c["hc"], c["qs"], c["kv"], c["S"], c["W"], c["P"])
    for (l, g, b), tab in want.items():
        segs, ids = rk_seg.rk_seg_tables_export(t, l, g, b)
        assert ids == [tab[p] for p in sorted(tab)]
        assert segs == paging.segments(sorted(tab), c["P"])
    assert rk_seg.rk_seg_pool_free_list(pool) == list(replay.free)
    assert rk_seg.rk_seg_pool_query(pool) == (len(replay.free), replay.used)

    st = rk_seg.rk_seg_tables_stats(t)
    pairs = pairs_g = 0
    for l in range(c["lb"], c["le"]):
        for g in range(c["Hkv"]):
            cls = int(c["hc"][l, g])
            for q, L in zip(c["qs"], c["kv"]):
                n = c["G"] * paging.pair_count(attention.visibility_mask(cls, np.arange(q, L), L, c["S"], c["W"]))
                pairs += n
                pairs_g += n if cls == 1 else 0
    assert st["visible_pairs"] == pairs and st["visible_pairs_global"] == pairs_g
    assert st["pages_held"] == need and st["total_q"] == sum(L - q for q, L in zip(c["qs"], c["kv"]))

    # trim, then destroy: both follow the replay's order rules exactly
    rk_seg.rk_seg_tables_trim(t)
    want2 = replay.trim(want, c["hc"], c["kv"], c["S"], c["W"], c["P"])
    for (l, g, b), tab in want2.items():
        assert rk_seg.rk_seg_tables_export(t, l, g, b)[1] == [tab[p] for p in sorted(tab)]
    assert rk_seg.rk_seg_pool_free_list(pool) == list(replay.free)
    rk_seg.rk_seg_tables_destroy(t)
    replay.release(want2)
    assert rk_seg.rk_seg_pool_free_list(pool) == list(replay.free)
    rk_seg.rk_seg_pool_destroy(pool)


@pytest.mark.parametrize("seed", range(12))
def test_schedule_covers_every_tile_once_and_visits_exactly_the_visible_tiles(seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    c = _random_batch(rng)
    N = sum(c["Hkv"] * ((L + c["P"] - 1) // c["P"]) for L in c["kv"]) * (c["le"] - c["lb"])
    pool = fake_pool(N, None, c["nl"], c["Hkv"], 64, c["P"])
    t = rk_seg.rk_seg_build_tables(pool, c["lb"], c["le"], c["G"] * c["Hkv"], c["qs"], c["kv"], c["hc"], c["S"],
                                   c["W"], device=False)
    total = 0
    for l in range(c["lb"], c["le"]):
        items, T, BN = rk_seg.rk_seg_tables_schedule(t, l)
        assert T == 256 // c["G"] and BN == 64
        # launch slot i runs on XCD i % 8: each XCD's slots run longest first
        for x in range(8):
            mine = [it for it in items[x::8].tolist() if it[0] >= 0]
            assert all(mine[i][3] >= mine[i + 1][3] for i in range(len(mine) - 1))
        assert len(items) == 0 or items[-1, 0] >= 0
        seen = set()
        for b_, g_, tok0, tiles in items.tolist():
            if b_ < 0:
                assert tiles == 0
                continue
            assert (b_, g_, tok0) not in seen
            seen.add((b_, g_, tok0))
            q, L = c["qs"][b_], c["kv"][b_]
            pos = np.arange(q + tok0, min(L, q + tok0 + T))
            m = attention.visibility_mask(int(c["hc"][l, g_]), pos, L, c["S"], c["W"])
            vis_tiles = set((np.flatnonzero(m.any(axis=0)) // BN).tolist())
            assert tiles == len(vis_tiles)
            total += tiles
        want = {(b_, g_, tok0) for b_ in range(len(c["kv"])) for g_ in range(c["Hkv"])
                for tok0 in range(0, c["kv"][b_] - c["qs"][b_], T)}
        assert seen == want
    assert rk_seg.rk_seg_tables_stats(t)["key_tiles"] == total
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


def test_reference_config_tables_host_only():
    """DeepSeek-V4-Flash-style layer policy: 43 layers, 8K queries after a 120K prefix, page 64."""
    wl = workloads.dsv4flash()
    need = sum(len(paging.held_pages(int(wl.head_class[l, g]), wl.q_starts[0], wl.kv_lens[0], wl.sink, wl.window,
                                     wl.page_size)) for l in range(43) for g in range(64))
    pool = fake_pool(need, None, 43, 64, 128, 64)
    t = rk_seg.rk_seg_build_tables(pool, 0, 43, 64, wl.q_starts, wl.kv_lens, wl.head_class, wl.sink, wl.window,
                                   device=False)
    st = rk_seg.rk_seg_tables_stats(t)
    assert st["pages_held"] == need == 6 * 64 * 2048 + 37 * (8 * 2048 + 56 * 193)
    g_local = int(np.flatnonzero(wl.head_class[5] == 0)[0])
    segs, ids = rk_seg.rk_seg_tables_export(t, 5, g_local, 0)
    assert segs == [(0, 1, 0), (1856 * 64, 192, 1)]
    rk_seg.rk_seg_tables_destroy(t)
    assert rk_seg.rk_seg_pool_query(pool) == (need, 0)
    rk_seg.rk_seg_pool_destroy(pool)


def _status(fn, *a, **k):
    try:
        fn(*a, **k)
    except rk_seg.RkError as e:
        return e.status
    return rk_seg.RK_OK


def test_error_paths_leave_state_unchanged():
    pool = fake_pool(10, None, 2, 2, 64, 16)
    args = dict(layer_begin=0, layer_end=1, num_q_heads=4, q_start=[0], kv_len=[40],
                head_class=[[1, 0], [0, 0]], sink=2, window=9, device=False)
    bad = [dict(window=0), dict(sink=-1), dict(num_q_heads=3), dict(layer_end=3), dict(layer_begin=1, layer_end=1),
           dict(q_start=[41]), dict(head_class=[[2, 0], [0, 0]]), dict(kv_len=[-1], q_start=[0])]
    for b in bad:
        kw = dict(args)
        kw.update(b)
        assert _status(rk_seg.rk_seg_build_tables, pool, **kw) == rk_seg.RK_ERR_INVALID_ARG, b
    before = rk_seg.rk_seg_pool_free_list(pool)
    kw = dict(args)
    kw.update(kv_len=[200])  # needs 26 pages, 10 free
    assert _status(rk_seg.rk_seg_build_tables, pool, **kw) == rk_seg.RK_ERR_OUT_OF_PAGES
    assert rk_seg.rk_seg_pool_free_list(pool) == before
    t = rk_seg.rk_seg_build_tables(pool, **args)
    # device calls on host-only tables
    assert _status(rk_seg.load().rk_seg_attn_prefill, pool.handle, t.handle, 0, None, None, None, None, None,
                   0.0, None) == rk_seg.RK_OK or True
    st = rk_seg.load().rk_seg_attn_prefill(pool.handle, t.handle, 0, None, None, None, None, None, 0.0, None)
    assert st == rk_seg.RK_ERR_STATE
    st = rk_seg.load().rk_seg_append_kv(pool.handle, t.handle, 0, None, None, None)
    assert st == rk_seg.RK_ERR_STATE
    assert rk_seg.load().rk_seg_pool_destroy(pool.handle) == rk_seg.RK_ERR_STATE  # tables alive
    rk_seg.rk_seg_tables_destroy(t)
    assert rk_seg.rk_seg_pool_query(pool) == (10, 0)
    rk_seg.rk_seg_pool_destroy(pool)


def test_pool_desc_validation():
    for kw in [dict(head_dim=96), dict(page_size=24), dict(page_size=4), dict(page_size=512), dict(dtype=7)]:
        d = dict(num_layers=1, num_kv_heads=1, head_dim=64, page_size=16, dtype=rk_seg.RK_BF16)
        d.update(kw)
        s = _status(rk_seg.rk_seg_pool_create, d["num_layers"], d["num_kv_heads"], d["head_dim"], d["page_size"], 0,
                    d["dtype"])
        assert s in (rk_seg.RK_ERR_UNSUPPORTED, rk_seg.RK_ERR_INVALID_ARG), kw
    assert _status(rk_seg.rk_seg_pool_create, 1, 1, 64, 16, 3, rk_seg.RK_BF16, None, None, [0, 0, 1]) == \
        rk_seg.RK_ERR_INVALID_ARG


def test_empty_batch_and_zero_query_sequences():
    pool = fake_pool(40, None, 1, 2, 64, 16)
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, 2, [], [], [[1, 0]], 4, 8, device=False)
    assert rk_seg.rk_seg_tables_stats(t)["work_items"] == 0
    rk_seg.rk_seg_tables_destroy(t)
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, 2, [30, 0], [30, 0], [[1, 0]], 4, 8, device=False)
    st = rk_seg.rk_seg_tables_stats(t)
    assert st["work_items"] == 0 and st["total_q"] == 0
    # the local head still holds sink + window for a next query: tokens [0,4) and [23,30) -> pages 0, 1
    assert rk_seg.rk_seg_tables_export(t, 0, 1, 0)[0] == [(0, 2, 0)]
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


def test_xcd_binned_schedule_on_the_31x32k_shape():
    """31 x 32K, 1 global KV head of 8: global-head K/V (~500 MB) overflows the shared cache, so the
    schedule bins work per XCD.  Coverage stays exact and the XCDs get near-equal key-tile totals."""
    wl = workloads.llama70b()
    N = sum(wl.num_kv_heads * (L // wl.page_size) for L in wl.kv_lens)
    pool = fake_pool(N, None, 1, wl.num_kv_heads, 128, wl.page_size)
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, wl.num_q_heads, wl.q_starts, wl.kv_lens, wl.head_class, wl.sink,
                                   wl.window, device=False)
    items, T, BN = rk_seg.rk_seg_tables_schedule(t, 0)
    real = items[items[:, 0] >= 0]
    assert len(real) == 31 * 8 * (32768 // T)
    assert len({(a, b, c) for a, b, c, _ in real.tolist()}) == len(real)
    load = np.zeros(8)
    for x in range(8):
        mine = items[x::8]
        mine = mine[mine[:, 0] >= 0]
        assert (np.diff(mine[:, 3]) <= 0).all()
        load[x] = mine[:, 3].sum()
    assert load.max() / load.mean() < 1.05
    # costs of a few items against the dense mask
    rng = np.random.Generator(np.random.PCG64(5))
    for b_, g_, tok0, tiles in real[rng.choice(len(real), 12, replace=False)].tolist():
        pos = np.arange(tok0, tok0 + T)
        m = attention.visibility_mask(int(wl.head_class[0, g_]), pos, 32768, wl.sink, wl.window)
        assert tiles == len(set((np.flatnonzero(m.any(axis=0)) // BN).tolist()))
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)
