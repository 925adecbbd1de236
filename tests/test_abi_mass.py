"""Work units of the per-key attention mass pass through the C ABI, on the CPU (host-only tables).

The mass of key j for q head h is the sum over the call's queries of that head of the attention
weight of (query, j): the routing score of the sparse FFN (page "小红书把 KV Cache 按「头」拆了…",
section 事件内容, item 2).  The pass is split into units (seq, kv head, key block, query chunk); the
exported list must hold exactly the units with a visible (query, key) pair, each once, under the
visibility rule of the oracle (global: causal; local: sink plus window)."""
import numpy as np
import pytest

from head_aware_paged_prefill_amd import rk_seg
from oracle import attention

from test_abi_host import fake_pool


def _mass_batch(rng):
    nl = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 3, 4, 8, 12, 16]))
    P = int(rng.choice([16, 64]))
    B = int(rng.integers(1, 4))
    kv = [int(x) for x in rng.integers(0, 2600, size=B)]
    qs = [int(rng.integers(0, L + 1)) if rng.random() < 0.7 else 0 for L in kv]
    qg = [0 if rng.random() < 0.5 else int(rng.integers(0, q + 1)) for q in qs]
    S = int(rng.choice([0, 4, 300]))
    W = int(rng.choice([1, 64, 500]))
    hc = rng.integers(0, 2, size=(nl, Hkv)).astype(np.uint8)
    return dict(nl=nl, Hkv=Hkv, G=G, P=P, kv=kv, qs=qs, qg=qg, S=S, W=W, hc=hc)


def _build(c):
    N = sum(c["Hkv"] * ((L + c["P"] - 1) // c["P"]) for L in c["kv"]) * c["nl"]
    pool = fake_pool(N, None, c["nl"], c["Hkv"], 64, c["P"])
    t = rk_seg.rk_seg_build_tables(pool, 0, c["nl"], c["G"] * c["Hkv"], c["qs"], c["kv"], c["hc"], c["S"], c["W"],
                                   device=False, q_start_global=c["qg"])
    return pool, t


def _expected_units(c, l, T, K, S):
    """Brute force: every (seq, kv head, key block, query chunk) holding a visible pair."""
    want = set()
    for b, L in enumerate(c["kv"]):
        for g in range(c["Hkv"]):
            cls = int(c["hc"][l, g])
            start = c["qg"][b] if cls == attention.GLOBAL else c["qs"][b]
            if L <= start:
                continue
            pos = np.arange(start, L)
            m = attention.visibility_mask(cls, pos, L, c["S"], c["W"])
            qi, kj = np.nonzero(m)
            chunk = (qi // T) // S  # qi = token - start
            for kb, qc in set(zip((kj // K).tolist(), chunk.tolist())):
                want.add((b, g, kb, qc))
    return want


@pytest.mark.parametrize("seed", range(12))
def test_mass_units_are_exactly_the_visible_blocks(seed):
    c = _mass_batch(np.random.Generator(np.random.PCG64(900 + seed)))
    pool, t = _build(c)
    try:
        for l in range(c["nl"]):
            units, K, T, S = rk_seg.rk_seg_tables_mass_schedule(t, l)
            # a workgroup of 8 waves holds 64 keys per wave (32 when G > 8, to fit the LDS sums);
            # a step stages 256 query rows of whole 16-row halves per head
            assert K == (512 if c["G"] <= 8 else 256) and S >= 1
            assert T % 16 == 0 and c["G"] * T <= 256 and c["G"] * (T + 16) > 256
            real = [tuple(u) for u in units.tolist() if u[0] >= 0]
            assert len(real) == len(set(real)), "a unit is listed twice"
            assert set(real) == _expected_units(c, l, T, K, S)
            if len(units):
                assert units[-1][0] >= 0, "trailing padding"
    finally:
        rk_seg.rk_seg_tables_destroy(t)
        rk_seg.rk_seg_pool_destroy(pool)


def test_mass_units_group_key_blocks_of_one_query_chunk_on_one_xcd():
    # one long global sequence: many key blocks read the same query chunk; runs of them stay on one
    # XCD (launch position i runs on XCD i % 8) in ascending key-block order
    c = dict(nl=1, Hkv=2, G=8, P=16, kv=[20000], qs=[0], qg=[0], S=4, W=64, hc=np.array([[1, 0]], np.uint8))
    pool, t = _build(c)
    try:
        units, K, T, S = rk_seg.rk_seg_tables_mass_schedule(t, 0)
        for x in range(8):
            bin_ = [tuple(u) for u in units[x::8].tolist() if u[0] >= 0]
            runs, cur = [], []
            for u in bin_:
                if cur and u[:2] + u[3:] != cur[-1][:2] + cur[-1][3:]:
                    runs.append(cur)
                    cur = []
                cur.append(u)
            if cur:
                runs.append(cur)
            for r in runs:
                kbs = [u[2] for u in r]
                assert kbs == sorted(kbs)
            # the bin holds few switches between (seq, head, chunk): runs of up to 16 blocks
            assert len(runs) <= max(1, len(bin_) // 4)
        real = units[units[:, 0] >= 0]
        counts = np.bincount(np.flatnonzero(units[:, 0] >= 0) % 8, minlength=8)
        assert counts.max() - counts.min() <= 16  # runs spread evenly over the XCDs
        assert len(real) == len(set(map(tuple, real.tolist())))
    finally:
        rk_seg.rk_seg_tables_destroy(t)
        rk_seg.rk_seg_pool_destroy(pool)


def test_mass_units_empty_when_no_query():
    c = dict(nl=1, Hkv=1, G=4, P=16, kv=[300, 0], qs=[300, 0], qg=[300, 0], S=4, W=8, hc=np.array([[1]], np.uint8))
    pool, t = _build(c)
    try:
        units, _, _, _ = rk_seg.rk_seg_tables_mass_schedule(t, 0)
        assert len(units) == 0
    finally:
        rk_seg.rk_seg_tables_destroy(t)
        rk_seg.rk_seg_pool_destroy(pool)


def test_workspace_size_does_not_depend_on_head_classes():
    # one workspace serves every layer: its size is a bound over the head classes
    c = _mass_batch(np.random.Generator(np.random.PCG64(77)))
    c["kv"] = [3000, 1200]
    c["qs"], c["qg"] = [1000, 0], [0, 0]
    N = sum(c["Hkv"] * ((L + c["P"] - 1) // c["P"]) for L in c["kv"]) * c["nl"]
    pool = fake_pool(N, None, c["nl"], c["Hkv"], 64, c["P"])
    try:
        sizes = set()
        for fill in (0, 1, None):
            hc = c["hc"] if fill is None else np.full_like(c["hc"], fill)
            sizes.add(rk_seg.rk_seg_tables_workspace_bytes(pool, 0, c["nl"], c["G"] * c["Hkv"], c["qs"], c["kv"], hc,
                                                           c["S"], c["W"], c["qg"]))
        assert len(sizes) == 1
    finally:
        rk_seg.rk_seg_pool_destroy(pool)


@pytest.mark.parametrize("G", [17, 32, 256])
def test_groups_above_sixteen_have_no_mass_units(G):
    # the mass pass supports at most 16 q heads per KV head: tables still build, with an empty unit list
    pool = fake_pool(64, None, 1, 1, 64, 16)
    ws = rk_seg.rk_seg_tables_workspace_bytes(pool, 0, 1, G, [0], [100], [[1]], 4, 16)
    assert ws > 0
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, G, [0], [100], [[1]], 4, 16, device=False)
    try:
        units, K, T, S = rk_seg.rk_seg_tables_mass_schedule(t, 0)
        assert len(units) == 0
    finally:
        rk_seg.rk_seg_tables_destroy(t)
        rk_seg.rk_seg_pool_destroy(pool)
