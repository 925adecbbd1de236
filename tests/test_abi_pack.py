"""Byte ledger of the page hand-off through the C ABI, on the CPU (host-only tables), against the
integer oracle: the pages a hand-off moves (the held pages: every page of a GLOBAL head, the sink and
window pages of a LOCAL head; page "小红书把 KV Cache 按「头」拆了…" (zhichai.net), section 事件内容)
and the dense per-head layout that keeps every token of every head."""
import numpy as np
import pytest

from head_aware_paged_prefill_amd import rk_seg
from oracle import paging

from test_abi_host import fake_pool, _status


def _want(hc, qs, kv, S, W, P, D, elem, seqs, layers, trimmed):
    w = dict(pages=0, pages_global=0, pages_local=0, tokens=0, dense_tokens=0)
    for b in seqs:
        L = kv[b]
        q = L if trimmed else qs[b]
        for l in layers:
            for g in range(hc.shape[1]):
                cls = int(hc[l, g])
                pages = paging.retained_pages(cls, L, S, W, P) if trimmed else paging.held_pages(cls, q, L, S, W, P)
                w["pages"] += len(pages)
                w["pages_global" if cls == paging.GLOBAL else "pages_local"] += len(pages)
                held = np.zeros(L, bool)
                for a, e in paging.held_token_ranges(cls, q, L, S, W):
                    held[a:e] = True
                w["tokens"] += int(held.sum())
                w["dense_tokens"] += L
    w["packed_bytes"] = w["pages"] * 2 * P * D * elem
    w["token_bytes"] = w["tokens"] * 2 * D * elem
    w["dense_bytes"] = w["dense_tokens"] * 2 * D * elem
    return w


def test_ledger_small_by_hand():
    # 1 layer, KV head 0 GLOBAL, 1 LOCAL; kv_len 40, page 16, sink 4, window 20, D 64, bf16 (2 bytes):
    # GLOBAL pages 0,1,2 and 40 tokens; LOCAL (queries from 0) pages 0,1,2 and 40 tokens.  After trim
    # the LOCAL head keeps sink [0,4) and [21,40): 23 tokens, still pages 0,1,2.
    pool = fake_pool(12, None, 1, 2, 64, 16)
    t = rk_seg.rk_seg_build_tables(pool, 0, 1, 2, [0], [40], [[1, 0]], 4, 20, device=False)
    page = 16 * 64 * 2
    assert rk_seg.rk_seg_pack_ledger(t) == dict(pages=6, pages_global=3, pages_local=3, packed_bytes=6 * 2 * page,
                                                tokens=80, token_bytes=80 * 2 * 64 * 2, dense_tokens=80,
                                                dense_bytes=80 * 2 * 64 * 2)
    rk_seg.rk_seg_tables_trim(t)
    led = rk_seg.rk_seg_pack_ledger(t)
    assert (led["pages"], led["tokens"], led["dense_tokens"]) == (6, 40 + 23, 80)
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


@pytest.mark.parametrize("seed", range(16))
def test_ledger_matches_integer_oracle(seed):
    rng = np.random.Generator(np.random.PCG64(5200 + seed))
    nl, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    P = int(rng.choice([16, 32, 64]))
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 5))
    S, W = int(rng.choice([0, 4, 17])), int(rng.choice([1, 16, 100, 1000]))
    hc = rng.integers(0, 2, size=(nl, Hkv)).astype(np.uint8)
    kv = [int(x) for x in rng.integers(0, 2000, size=B)]
    qs = [int(rng.integers(0, L + 1)) for L in kv]
    lb = int(rng.integers(0, nl))
    le = int(rng.integers(lb + 1, nl + 1))
    pool = fake_pool(200000, None, nl, Hkv, D, P)
    t = rk_seg.rk_seg_build_tables(pool, lb, le, Hkv, qs, kv, hc, S, W, device=False)
    for trimmed in (False, True):
        if trimmed:
            rk_seg.rk_seg_tables_trim(t)
        for seq in [-1] + list(range(B)):
            seqs = range(B) if seq < 0 else [seq]
            assert rk_seg.rk_seg_pack_ledger(t, seq) == _want(hc, qs, kv, S, W, P, D, 2, seqs, range(lb, le), trimmed)
    assert _status(lambda: rk_seg.rk_seg_pack_ledger(t, B)) == rk_seg.RK_ERR_INVALID_ARG
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)


def test_ledger_after_advance_by_zero_is_the_retained_state():
    # advancing a trimmed call by 0 tokens holds exactly the retained pages and tokens
    rng = np.random.Generator(np.random.PCG64(5300))
    hc = rng.integers(0, 2, size=(2, 3)).astype(np.uint8)
    kv, qs = [900, 1333, 17], [0, 500, 3]
    pool = fake_pool(20000, None, 2, 3, 128, 16)
    t = rk_seg.rk_seg_build_tables(pool, 0, 2, 24, qs, kv, hc, 4, 256, device=False)
    rk_seg.rk_seg_tables_trim(t)
    a = rk_seg.rk_seg_pack_ledger(t)
    rk_seg.rk_seg_tables_advance(t, [0, 0, 0], device=False)
    assert rk_seg.rk_seg_pack_ledger(t) == a == _want(hc, qs, kv, 4, 256, 16, 128, 2, range(3), range(2), True)
    rk_seg.rk_seg_tables_destroy(t)
    rk_seg.rk_seg_pool_destroy(pool)
