"""Head-ragged query ranges through the C ABI, on the CPU (host-only tables): GLOBAL heads start at
q_start_global, LOCAL heads at q_start (EXECUTE's split; page "RedKnot - Xiaohongshuが開発した…",
section 使い方, EXECUTE item).  Schedules and counters are checked against the dense mask and the
integer oracle's replay."""
import numpy as np
import pytest

from head_aware_paged_prefill_amd import rk_seg
from oracle import attention, paging

from test_abi_host import fake_pool, _status


def _split_batch(rng):
    nl = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.choice([16, 32, 64]))
    B = int(rng.integers(1, 5))
    kv = [int(x) for x in rng.integers(0, 700, size=B)]
    qs = [int(rng.integers(0, L + 1)) for L in kv]
    qg = [0 if rng.random() < 0.6 else int(rng.integers(0, q + 1)) for q in qs]
    S = int(rng.choice([0, 1, 4, 17]))
    W = int(rng.choice([1, 5, 64, 100]))
    hc = rng.integers(0, 2, size=(nl, Hkv)).astype(np.uint8)
    return dict(nl=nl, Hkv=Hkv, G=G, P=P, kv=kv, qs=qs, qg=qg, S=S, W=W, hc=hc)


def _build(c, qg="split"):
    N = sum(c["Hkv"] * ((L + c["P"] - 1) // c["P"]) for L in c["kv"]) * c["nl"]
    pool = fake_pool(N, None, c["nl"], c["Hkv"], 64, c["P"])
    t = rk_seg.rk_seg_build_tables(pool, 0, c["nl"], c["G"] * c["Hkv"], c["qs"], c["kv"], c["hc"], c["S"], c["W"],
                                   device=False, q_start_global=c["qg"] if qg == "split" else qg)
    return pool, t


def _start(c, cls, b):
    return c["qg"][b] if cls == 1 else c["qs"][b]


@pytest.mark.parametrize("seed", range(16))
def test_split_schedule_covers_each_class_range(seed):
    c = _split_batch(np.random.Generator(np.random.PCG64(700 + seed)))
    pool, t = _build(c)
    total = 0
    for l in range(c["nl"]):
        items, T, BN = rk_seg.rk_seg_tables_schedule(t, l)
        seen = set()
        for b_, g_, tok0, tiles in items.tolist():
            if b_ < 0:
                continue
            assert (b_, g_, tok0) not in seen
            seen.add((b_, g_, tok0))
            cls = int(c["hc"][l, g_])
            qb, L = c["qg"][b_], c["kv"][b_]
            # rows are packed from the GLOBAL start; a head's items begin at its class start
            assert qb + tok0 >= _start(c, cls, b_)
            pos = np.arange(qb + tok0, min(L, qb + tok0 + T))
            m = attention.visibility_mask(cls, pos, L, c["S"], c["W"])
            assert tiles == len(set((np.flatnonzero(m.any(axis=0)) // BN).tolist()))
            total += tiles
        want = set()
        for b_ in range(len(c["kv"])):
            for g_ in range(c["Hkv"]):
                a = _start(c, int(c["hc"][l, g_]), b_)
                want |= {(b_, g_, a - c["qg"][b_] + k) for k in range(0, c["kv"][b_] - a, T)}
        assert seen == want
    assert rk_seg.rk_seg_tables_stats(t)["key_tiles"] == total
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


@pytest.mark.parametrize("seed", range(16))
def test_split_counters_match_the_dense_mask_and_the_replay(seed):
    c = _split_batch(np.random.Generator(np.random.PCG64(800 + seed)))
    pool, t = _build(c)
    st = rk_seg.rk_seg_tables_stats(t)
    assert st["total_q"] == sum(L - g for L, g in zip(c["kv"], c["qg"]))
    pairs = pairs_g = 0
    for l in range(c["nl"]):
        for g_ in range(c["Hkv"]):
            cls = int(c["hc"][l, g_])
            for b_, L in enumerate(c["kv"]):
                pos = np.arange(_start(c, cls, b_), L)
                n = c["G"] * paging.pair_count(attention.visibility_mask(cls, pos, L, c["S"], c["W"]))
                pairs += n
                pairs_g += n if cls == 1 else 0
    assert st["visible_pairs"] == pairs and st["visible_pairs_global"] == pairs_g
    # held pages do not depend on the GLOBAL start: LOCAL windows follow q_start, GLOBAL heads hold all
    rp = paging.PoolReplay(1 << 20)
    tb = rp.build(0, c["nl"], c["hc"], c["qs"], c["kv"], c["S"], c["W"], c["P"])
    assert st["pages_held"] == sum(len(v) for v in tb.values())
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


def test_equal_starts_give_the_plain_tables():
    c = _split_batch(np.random.Generator(np.random.PCG64(901)))
    c["qg"] = list(c["qs"])
    pool, t = _build(c)
    pool2, t2 = _build(c, qg=None)
    assert rk_seg.rk_seg_tables_stats(t) == rk_seg.rk_seg_tables_stats(t2)
    for l in range(c["nl"]):
        np.testing.assert_array_equal(rk_seg.rk_seg_tables_schedule(t, l)[0], rk_seg.rk_seg_tables_schedule(t2, l)[0])
    for x, p in ((t, pool), (t2, pool2)):
        rk_seg.rk_seg_tables_destroy(x)
        rk_seg.rk_seg_pool_destroy(p)


def test_split_validation():
    pool = fake_pool(64)
    hc = np.array([[1, 0]], np.uint8)
    args = (pool, 0, 1, 4, [10], [40], hc, 4, 8)
    assert _status(rk_seg.rk_seg_build_tables, *args, device=False, q_start_global=[11]) == rk_seg.RK_ERR_INVALID_ARG
    assert _status(rk_seg.rk_seg_build_tables, *args, device=False, q_start_global=[-1]) == rk_seg.RK_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        rk_seg.rk_seg_build_tables(*args, device=False, q_start_global=[0, 0])
    assert rk_seg.rk_seg_pool_query(pool)[1] == 0  # nothing allocated by the failed builds
    t = rk_seg.rk_seg_build_tables(*args, device=False, q_start_global=[0])
    assert rk_seg.rk_seg_tables_stats(t)["total_q"] == 40
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)
