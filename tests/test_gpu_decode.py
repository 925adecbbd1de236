"""Decode over the retained segmented state on the GPU, through the C ABI, against the fp64 oracle.

A prefill call fills the pool; trim leaves what the next query can see; then each step advances the
tables by one token per sequence (rk_seg_tables_advance) and runs rk_seg_attn_decode (append, split-KV
attention, combine).  The oracle's row is the masked softmax attention of the new token over the
sequence's whole K/V history (oracle.decode.decode_step), so a LOCAL head that lost a page it still
needed, a window that slid wrong, or a split whose partials merge wrong all fail.  Bars: those of the
attention parity tests (bf16 max-abs 2e-2, mean-abs 2e-3, lse 1e-3 * max(1, |lse|))."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from head_aware_paged_prefill_amd import rk_seg
from head_aware_paged_prefill_amd.runner import PrefillRunner
from oracle import decode, reference

from test_gpu_parity import check, say, to_dev

pytestmark = pytest.mark.gpu


def _to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _poison_free_pages(r):
    """NaN into every page on the free list, so that a page taken later holds no stale finite data:
    a kernel that loads a slot nothing wrote then fails the check instead of passing by luck."""
    free = rk_seg.rk_seg_pool_free_list(r.pool)
    if free:
        idx = torch.tensor(free, dtype=torch.long, device="cuda")
        r.k_pages.index_fill_(0, idx, float("nan"))
        r.v_pages.index_fill_(0, idx, float("nan"))


def decode_parity(wl, steps, what, pattern=None, device_inputs=False, seqs=None):
    """Prefill, trim, then `steps` decode steps.  pattern(step) -> n_new per sequence (default all 1).
    seqs: the sequences whose rows are checked (default all)."""
    B, H, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    extra = B * Hkv * (steps // wl.page_size + 2)
    num_pages = workloads.pool_pages_needed_hint(wl) + wl.pool_slack + extra
    say("%s: kv_lens=%s q_starts=%s qg=%s H=%d Hkv=%d D=%d P=%d S=%d W=%d steps=%d" % (
        what, wl.kv_lens if B <= 8 else "%d x %d" % (B, wl.kv_lens[0]), wl.q_starts if B <= 8 else "...",
        wl.q_starts_global, H, Hkv, D, wl.page_size, wl.sink, wl.window, steps))
    inp = workloads.make_inputs(wl, device="cuda" if device_inputs else "cpu", num_pages=num_pages)
    dinp = inp if device_inputs else to_dev(inp)
    r = PrefillRunner(wl, free_order=inp.free_order, poison=True)
    try:
        r.build()
        r.import_docs(dinp.docs)
        r.attend(dinp.q, dinp.k_new, dinp.v_new)
        r.trim()
        _poison_free_pages(r)
        seqs = range(B) if seqs is None else list(seqs)
        hist = {b: [list(reference.head_kv(inp, b, g)) for g in range(Hkv)] for b in seqs}
        kv_class = wl.head_class[wl.layer]
        for s in range(steps):
            n_new = [1] * B if pattern is None else pattern(s)
            active = [b for b in range(B) if n_new[b]]
            r.advance(n_new)
            _poison_free_pages(r)
            q, k, v = workloads.decode_inputs(wl, s, len(active))
            o, lse = r.decode(q.cuda(), k.cuda(), v.cuda())
            torch.cuda.synchronize()
            rows = [i for i, b in enumerate(active) if b in hist]
            o_ref = np.zeros((len(rows), H, D))
            lse_ref = np.zeros((H, len(rows)))
            for j, i in enumerate(rows):
                b = active[i]
                for g in range(Hkv):
                    hist[b][g][0] = np.vstack([hist[b][g][0], _to64(k[i, g])[None]])
                    hist[b][g][1] = np.vstack([hist[b][g][1], _to64(v[i, g])[None]])
                o_ref[j], lse_ref[:, j] = decode.decode_step(_to64(q[i]), [x[0] for x in hist[b]],
                                                             [x[1] for x in hist[b]], kv_class, wl.sink, wl.window)
            idx = torch.tensor(rows, dtype=torch.long, device="cuda")
            check(o.index_select(0, idx), lse.index_select(1, idx), o_ref, lse_ref, wl.dtype,
                  "%s step %d" % (what, s))
    finally:
        r.close()


def test_tiny_decode_crosses_pages_and_slides_the_window():
    # 40 steps at page 16 cross two page boundaries; the LOCAL head's window (128) slides past pages
    decode_parity(workloads.tiny(torch.bfloat16), 40, "decode tiny")


@pytest.mark.parametrize("seed", range(6))
def test_random_small_decode(seed):
    decode_parity(workloads.random_small(seed, torch.bfloat16), 12, "decode random-small %d" % seed)


@pytest.mark.parametrize("seed", range(3))
def test_random_split_decode(seed):
    # after EXECUTE's head-ragged prefill (GLOBAL heads recomputed the prefix)
    decode_parity(workloads.random_split(seed, torch.bfloat16), 6, "decode random-split %d" % seed)


@pytest.mark.parametrize("G", [1, 3, 16])
def test_decode_group_sizes(G):
    wl = workloads.random_small(7, torch.bfloat16)
    wl = dataclasses.replace(wl, num_q_heads=G * wl.num_kv_heads, name="decode G=%d" % G)
    decode_parity(wl, 8, wl.name)


def test_decode_with_sequences_that_do_not_advance():
    wl = workloads.random_small(9, torch.bfloat16)
    wl = dataclasses.replace(wl, kv_lens=[300, 41, 520], q_starts=[0, 0, 100], doc_len=50,
                             name="decode ragged advance")
    decode_parity(wl, 8, wl.name, pattern=lambda s: [1, s % 2, 1 if s % 3 else 0])


def test_decode_long_context_splits_and_combines():
    # many split-KV items per GLOBAL head, LOCAL window wider than a chunk: the combine merges them
    wl = workloads.Workload(name="decode 2 x ~6K 32q/4kv D=128", config_id=410, num_layers=1, layer=0,
                            kv_lens=[6000, 4111], q_starts=[0, 3000], num_q_heads=32, num_kv_heads=4, head_dim=128,
                            page_size=16, sink=4, window=700, dtype=torch.bfloat16,
                            head_class=np.array([[1, 0, 0, 1]], np.uint8), pool_slack=7, doc_len=1000,
                            rope_base=1.0e4)
    decode_parity(wl, 4, wl.name)


@pytest.mark.parametrize("G,D,P", [(16, 64, 16), (8, 64, 256), (2, 128, 128), (4, 64, 8), (16, 128, 8)])
def test_decode_shapes(G, D, P):
    wl = workloads.random_small(4, torch.bfloat16)
    wl = dataclasses.replace(wl, num_q_heads=G * wl.num_kv_heads, head_dim=D, page_size=P,
                             name="decode G=%d D=%d P=%d" % (G, D, P))
    decode_parity(wl, 6, wl.name)


def test_decode_page_64():
    wl = workloads.random_small(3, torch.bfloat16)
    wl = dataclasses.replace(wl, page_size=64, head_dim=128, kv_lens=[700, 1300], q_starts=[0, 650], doc_len=200,
                             name="decode P=64")
    decode_parity(wl, 70, wl.name)


def test_decode_single_long_sequence_takes_the_large_chunk():
    # one 72K-token sequence: at least 65536 visible keys, so 192-key items; the GLOBAL heads' rows merge
    # ~95 workgroup partials each in the combine, the LOCAL heads' window slides across page boundaries
    wl = workloads.Workload(name="decode 1 x 72K 32q/4kv D=128", config_id=412, num_layers=1, layer=0,
                            kv_lens=[72000], q_starts=[0], num_q_heads=32, num_kv_heads=4, head_dim=128,
                            page_size=64, sink=4, window=3000, dtype=torch.bfloat16,
                            head_class=np.array([[1, 0, 1, 0]], np.uint8), pool_slack=8)
    decode_parity(wl, 3, wl.name, device_inputs=True)


def test_llama70b_shape_decode_sampled():
    # the full 31 x 32K state; three sequences' rows checked against the oracle
    wl = workloads.llama70b()
    decode_parity(wl, 2, "decode Llama-3.3-70B-shaped", device_inputs=True, seqs=[0, 15, 30])


def test_decode_rejects_unsupported_and_prefill_shaped_tables():
    wl = workloads.random_small(1, torch.float32)
    inp = to_dev(workloads.make_inputs(wl, num_pages=workloads.pool_pages_needed_hint(wl) + 64))
    r = PrefillRunner(wl, free_order=inp.free_order)
    try:
        r.build()
        r.import_docs(inp.docs)
        r.attend(inp.q, inp.k_new, inp.v_new)
        r.advance([1] * wl.num_seqs)
        q, k, v = workloads.decode_inputs(wl, 0, wl.num_seqs)
        with pytest.raises(rk_seg.RkError) as ei:
            r.decode(q.cuda(), k.cuda(), v.cuda())
        assert ei.value.status == rk_seg.RK_ERR_UNSUPPORTED
    finally:
        r.close()
    wl = workloads.random_small(1, torch.bfloat16)
    inp = to_dev(workloads.make_inputs(wl))
    r = PrefillRunner(wl, free_order=inp.free_order)
    try:
        r.build()
        q, k, v = workloads.decode_inputs(wl, 0, wl.num_seqs)
        if max(L - s for L, s in zip(wl.kv_lens, wl.q_starts)) > 1:
            with pytest.raises(rk_seg.RkError) as ei:
                r.decode(q.cuda(), k.cuda(), v.cuda())
            assert ei.value.status == rk_seg.RK_ERR_STATE
    finally:
        r.close()


@pytest.mark.parametrize("seed", [11, 23, 14])  # LOCAL W=16 < P=32; mixed, W=1, sink 4; mixed, P=64
def test_decode_appending_itself_matches_explicit_append_bit_for_bit(seed):
    """rk_seg_attn_decode given k_new / v_new appends the token inside the decode kernel; with k_new =
    v_new = NULL it skips the append.  After rk_seg_append_kv of the same tokens the NULL call must
    return the bits of the call that appends itself, step after step across page boundaries, and the
    pool pages (with the append's clearing of slots past kv_len and, with a window shorter than a page,
    below a LOCAL head's window) must end bit-identical too."""
    wl = workloads.random_small(seed, torch.bfloat16, allow_reuse=False)
    steps = 2 * wl.page_size + 3
    say("decode self-append vs explicit: kv_lens=%s G=%d P=%d W=%d steps=%d" % (
        wl.kv_lens, wl.group, wl.page_size, wl.window, steps))
    B = wl.num_seqs
    inp = workloads.make_inputs(wl, num_pages=workloads.pool_pages_needed_hint(wl) + wl.pool_slack
                                + 4 * B * wl.num_kv_heads * (steps // wl.page_size + 2))
    dinp = to_dev(inp)
    outs = []
    for explicit in (False, True):
        r = PrefillRunner(wl, free_order=inp.free_order, poison=True)
        run = []
        try:
            r.build()
            r.attend(dinp.q, dinp.k_new, dinp.v_new)
            r.trim()
            for st in range(steps):
                r.advance([1] * B)
                _poison_free_pages(r)
                q, k, v = (t.cuda() for t in workloads.decode_inputs(wl, st, B))
                o = torch.empty((B, wl.num_q_heads, wl.head_dim), dtype=wl.dtype, device="cuda")
                lse = torch.empty((wl.num_q_heads, B), dtype=torch.float32, device="cuda")
                if explicit:
                    rk_seg.rk_seg_append_kv(r.tables, wl.layer, k, v)
                    rk_seg.rk_seg_attn_decode(r.tables, wl.layer, q, None, None, o, lse)
                else:
                    rk_seg.rk_seg_attn_decode(r.tables, wl.layer, q, k, v, o, lse)
                torch.cuda.synchronize()
                assert torch.isfinite(o.float()).all(), "step %d" % st
                run.append((o.cpu(), lse.cpu()))
            with pytest.raises(rk_seg.RkError) as ei:  # one of the two missing is an error
                rk_seg.rk_seg_attn_decode(r.tables, wl.layer, q, k, None, o, lse)
            assert ei.value.status == rk_seg.RK_ERR_INVALID_ARG
            held = torch.tensor(sorted(set(range(r.num_pages)) - set(rk_seg.rk_seg_pool_free_list(r.pool))),
                                dtype=torch.long, device="cuda")
            outs.append((run, r.k_pages.index_select(0, held).cpu(), r.v_pages.index_select(0, held).cpu()))
        finally:
            r.close()
    for st, ((o0, l0), (o1, l1)) in enumerate(zip(outs[0][0], outs[1][0])):
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), "o differs at step %d" % st
        assert torch.equal(l0, l1), "lse differs at step %d" % st
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16)), "K pages differ"
    assert torch.equal(outs[0][2].view(torch.int16), outs[1][2].view(torch.int16)), "V pages differ"
