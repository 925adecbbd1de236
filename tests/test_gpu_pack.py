"""Page hand-off on the GPU through the C ABI: pack the held pages of the retained state, unpack them
into another pool's tables of the same state, and decode there.

Bars: bit-exact.  The packed buffer must equal the pool's pages that the integer oracle's replay names,
in hand-off order (sequence, layer, KV head, logical page; K page then V page); the decode on the
receiving pool must equal the sender's decode bit for bit (same kernel, same bytes, same schedule) and
the fp64 oracle's decode row within the attention bars (page "小红书把 KV Cache 按「头」拆了…"
(zhichai.net), section 事件内容: only the pages a head keeps are transferred)."""
import numpy as np
import pytest
import torch

import workloads
from head_aware_paged_prefill_amd import rk_seg
from head_aware_paged_prefill_amd.runner import PrefillRunner
from oracle import decode, paging, reference

from test_gpu_parity import check, say, to_dev

pytestmark = pytest.mark.gpu


def _prefill_retained(wl, num_pages):
    """Prefill call, trim, advance by 0 tokens: the retained state with a device view."""
    inp = workloads.make_inputs(wl, num_pages=num_pages)
    dinp = to_dev(inp)
    r = PrefillRunner(wl, free_order=inp.free_order, poison=True)
    r.build()
    r.import_docs(dinp.docs)
    r.attend(dinp.q, dinp.k_new, dinp.v_new)
    r.trim()
    r.advance([0] * wl.num_seqs)
    torch.cuda.synchronize()
    return inp, r


def _replay_ids(wl, inp):
    """Physical pages of the retained state in hand-off order, from the integer oracle's replay of
    build, trim and advance by 0 tokens."""
    pool = paging.PoolReplay(len(inp.free_order), inp.free_order.tolist())
    hc = wl.head_class
    # held sets follow the LOCAL heads' start (GLOBAL heads hold everything)
    t = pool.build(wl.layer, wl.layer + 1, hc, wl.q_starts, wl.kv_lens, wl.sink, wl.window, wl.page_size)
    t = pool.trim(t, hc, wl.kv_lens, wl.sink, wl.window, wl.page_size)
    t, _ = pool.advance(t, hc, wl.kv_lens, [0] * wl.num_seqs, wl.sink, wl.window, wl.page_size)
    ids = []
    for b in range(wl.num_seqs):
        for g in range(wl.num_kv_heads):
            tab = t[(wl.layer, g, b)]
            ids.extend(tab[p] for p in sorted(tab))
    return ids


def _packed_from_pool(r, ids):
    idx = torch.tensor(ids, dtype=torch.long, device="cuda")
    k = r.k_pages.index_select(0, idx).reshape(len(ids), -1).view(torch.uint8)
    v = r.v_pages.index_select(0, idx).reshape(len(ids), -1).view(torch.uint8)
    return torch.cat([k, v], dim=1).reshape(-1)


CASES = [("tiny", lambda: workloads.tiny(torch.bfloat16)),
         ("random-small 2", lambda: workloads.random_small(2, torch.bfloat16, allow_reuse=False)),
         ("random-small 5", lambda: workloads.random_small(5, torch.bfloat16, allow_reuse=False))]


@pytest.mark.parametrize("name,make", CASES)
def test_pack_is_the_retained_pages_bit_exact(name, make):
    wl = make()
    say("pack %s: kv_lens=%s q_starts=%s Hkv=%d P=%d S=%d W=%d" % (name, wl.kv_lens, wl.q_starts, wl.num_kv_heads,
                                                                 wl.page_size, wl.sink, wl.window))
    inp, r = _prefill_retained(wl, workloads.pool_pages_needed_hint(wl) + wl.pool_slack)
    try:
        led = rk_seg.rk_seg_pack_ledger(r.tables)
        dst = torch.full((led["packed_bytes"] + 64,), 0xA5, dtype=torch.uint8, device="cuda")
        rk_seg.rk_seg_pack_pages(r.tables, -1, dst)
        torch.cuda.synchronize()
        ids = _replay_ids(wl, inp)
        assert len(ids) == led["pages"]
        assert torch.equal(dst[:led["packed_bytes"]], _packed_from_pool(r, ids))
        assert (dst[led["packed_bytes"]:] == 0xA5).all(), "pack wrote past the ledger's bytes"
        # per sequence: consecutive slices of the whole, in sequence order
        off = 0
        for b in range(wl.num_seqs):
            lb = rk_seg.rk_seg_pack_ledger(r.tables, b)
            one = torch.empty((lb["packed_bytes"],), dtype=torch.uint8, device="cuda")
            rk_seg.rk_seg_pack_pages(r.tables, b, one)
            torch.cuda.synchronize()
            assert torch.equal(one, dst[off:off + lb["packed_bytes"]])
            off += lb["packed_bytes"]
        assert off == led["packed_bytes"]
    finally:
        r.close()


@pytest.mark.parametrize("name,make", CASES + [("random-split 1", lambda: workloads.random_split(1, torch.bfloat16))])
def test_handoff_to_another_pool_then_decode(name, make):
    wl = make()
    B, H, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    pages = workloads.pool_pages_needed_hint(wl) + wl.pool_slack + 2 * B * Hkv
    say("hand-off %s: kv_lens=%s q_starts=%s qg=%s H=%d Hkv=%d P=%d" % (name, wl.kv_lens, wl.q_starts,
                                                                      wl.q_starts_global, H, Hkv, wl.page_size))
    inp, ra = _prefill_retained(wl, pages)
    order_b = np.random.Generator(np.random.PCG64(77)).permutation(pages + 9).astype(np.int32)
    rb = PrefillRunner(wl, free_order=order_b, poison=True)
    try:
        led = rk_seg.rk_seg_pack_ledger(ra.tables)
        buf = torch.empty((led["packed_bytes"],), dtype=torch.uint8, device="cuda")
        rk_seg.rk_seg_pack_pages(ra.tables, -1, buf)
        # receiver: tables of the same state (no queries: q_start = kv_len holds the retained pages)
        rb.tables = rk_seg.rk_seg_build_tables(rb.pool, wl.layer, wl.layer + 1, H, wl.kv_lens, wl.kv_lens,
                                               wl.head_class, wl.sink, wl.window, device=True)
        rb.workspace = rb.tables.workspace
        assert rk_seg.rk_seg_pack_ledger(rb.tables) == led
        rk_seg.rk_seg_unpack_pages(rb.tables, -1, buf)
        back = torch.empty_like(buf)
        rk_seg.rk_seg_pack_pages(rb.tables, -1, back)
        torch.cuda.synchronize()
        assert torch.equal(back, buf), "the receiving pool's pages differ from the packed ones"
        with pytest.raises(rk_seg.RkError) as ei:
            rk_seg.rk_seg_unpack_pages(rb.tables, -1, buf[:-16])
        assert ei.value.status == rk_seg.RK_ERR_INVALID_ARG
        kv_class = wl.head_class[wl.layer]
        hist = {b: [list(reference.head_kv(inp, b, g)) for g in range(Hkv)] for b in range(B)}
        for s in range(3):
            q, k, v = workloads.decode_inputs(wl, s, B)
            outs = []
            for r in (ra, rb):
                r.advance([1] * B)
                outs.append(r.decode(q.cuda(), k.cuda(), v.cuda()))
            torch.cuda.synchronize()
            oa, ob = outs[0][0].float(), outs[1][0].float()
            assert torch.isfinite(oa).all() and torch.isfinite(ob).all(), "%s step %d: non-finite decode (%s, %s)" % (
                name, s, bool(torch.isfinite(oa).all()), bool(torch.isfinite(ob).all()))
            assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), \
                "%s step %d: the receiving pool decodes differently (max |do| %.3g, rows %s)" % (
                    name, s, (oa - ob).abs().max().item(), torch.nonzero((oa - ob).abs().amax(dim=2))[:8].tolist())
            o_ref = np.zeros((B, H, D))
            lse_ref = np.zeros((H, B))
            for b in range(B):
                for g in range(Hkv):
                    hist[b][g][0] = np.vstack([hist[b][g][0], k[b, g].double().numpy()[None]])
                    hist[b][g][1] = np.vstack([hist[b][g][1], v[b, g].double().numpy()[None]])
                o_ref[b], lse_ref[:, b] = decode.decode_step(q[b].double().numpy(), [x[0] for x in hist[b]],
                                                             [x[1] for x in hist[b]], kv_class, wl.sink, wl.window)
            check(outs[1][0], outs[1][1], o_ref, lse_ref, wl.dtype, "%s hand-off decode step %d" % (name, s))
    finally:
        ra.close()
        rb.close()


def test_pack_needs_a_device_view():
    wl = workloads.tiny(torch.bfloat16)
    inp = to_dev(workloads.make_inputs(wl))
    r = PrefillRunner(wl, free_order=inp.free_order)
    try:
        r.build()
        r.import_docs(inp.docs)
        r.attend(inp.q, inp.k_new, inp.v_new)
        r.trim()
        dst = torch.empty((1 << 20,), dtype=torch.uint8, device="cuda")
        with pytest.raises(rk_seg.RkError) as ei:
            rk_seg.rk_seg_pack_pages(r.tables, -1, dst)
        assert ei.value.status == rk_seg.RK_ERR_STATE
    finally:
        r.close()


def test_pack_roundtrip_fp32_pool_bit_exact():
    # the hand-off moves bytes: an fp32 pool packs and unpacks bit for bit as well
    wl = workloads.random_small(6, torch.float32, allow_reuse=False)
    say("pack fp32 %s: kv_lens=%s P=%d" % (wl.name, wl.kv_lens, wl.page_size))
    inp, ra = _prefill_retained(wl, workloads.pool_pages_needed_hint(wl) + wl.pool_slack)
    order_b = np.random.Generator(np.random.PCG64(91)).permutation(len(inp.free_order) + 5).astype(np.int32)
    rb = PrefillRunner(wl, free_order=order_b, poison=True)
    try:
        led = rk_seg.rk_seg_pack_ledger(ra.tables)
        buf = torch.empty((led["packed_bytes"],), dtype=torch.uint8, device="cuda")
        rk_seg.rk_seg_pack_pages(ra.tables, -1, buf)
        torch.cuda.synchronize()
        assert torch.equal(buf, _packed_from_pool(ra, _replay_ids(wl, inp)))
        rb.tables = rk_seg.rk_seg_build_tables(rb.pool, wl.layer, wl.layer + 1, wl.num_q_heads, wl.kv_lens, wl.kv_lens,
                                               wl.head_class, wl.sink, wl.window, device=True)
        rk_seg.rk_seg_unpack_pages(rb.tables, -1, buf)
        back = torch.empty_like(buf)
        rk_seg.rk_seg_pack_pages(rb.tables, -1, back)
        torch.cuda.synchronize()
        assert torch.equal(back, buf)
    finally:
        ra.close()
        rb.close()
