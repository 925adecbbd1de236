"""Head-ragged query ranges on the GPU (EXECUTE's split: GLOBAL heads recompute from q_start_global,
LOCAL heads query from q_start; page "RedKnot - Xiaohongshuが開発した…", section 使い方, EXECUTE item),
through the C ABI against the fp64 oracle.  Same bars as the other parity tests; rows a LOCAL head
does not compute must keep whatever the output buffers held."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from head_aware_paged_prefill_amd import rk_seg
from head_aware_paged_prefill_amd.runner import PrefillRunner
from oracle import paging, reference, rope

from test_gpu_parity import TOL, bf16_ulp, check, cleared_below_window, say, to_dev

pytestmark = pytest.mark.gpu

O_SENTINEL, LSE_SENTINEL = 7.0, -3.0


def run_split(inp, fill=float("nan"), free_order=None):
    wl = inp.wl
    r = PrefillRunner(wl, free_order=inp.free_order if free_order is None else free_order, poison=False)
    r.k_pages.fill_(fill)
    r.v_pages.fill_(fill)
    r.build()
    r.import_docs(inp.docs)
    o = torch.full((wl.total_q, wl.num_q_heads, wl.head_dim), O_SENTINEL, dtype=wl.dtype, device="cuda")
    lse = torch.full((wl.num_q_heads, wl.total_q), LSE_SENTINEL, dtype=torch.float32, device="cuda")
    r.attend(inp.q, inp.k_new, inp.v_new, o=o, lse=lse)
    torch.cuda.synchronize()
    return r, o, lse


def check_split(o, lse, o_ref, lse_ref, dtype, what):
    """Compare the rows each head computes (finite in the oracle); the others keep the sentinels."""
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    done = np.isfinite(lse_ref)                     # [H][rows]
    assert done.any(), what + ": nothing computed"
    assert (lse[~done] == LSE_SENTINEL).all(), what + ": lse written outside the head's rows"
    assert (o.transpose(1, 0, 2)[~done] == O_SENTINEL).all(), what + ": o written outside the head's rows"
    check(o.transpose(1, 0, 2)[done], lse[done], o_ref.transpose(1, 0, 2)[done], lse_ref[done], dtype, what)


def split_parity(wl, what):
    inp = workloads.make_inputs(wl)
    o_ref, lse_ref = reference.prefill(inp)
    say("%s  kv_lens=%s q_starts=%s q_starts_global=%s H=%d Hkv=%d D=%d P=%d S=%d W=%d classes=%s dtype=%s" % (
        what, wl.kv_lens, wl.q_starts, wl.q_starts_global, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
        wl.page_size, wl.sink, wl.window, wl.head_class.tolist(), wl.dtype))
    r, o, lse = run_split(to_dev(inp))
    try:
        check_split(o, lse, o_ref, lse_ref, wl.dtype, what)
    finally:
        r.close()


@pytest.mark.parametrize("seed", range(12))
def test_random_split_bf16(seed):
    split_parity(workloads.random_split(seed, torch.bfloat16), "random-split bf16 %d" % seed)


@pytest.mark.parametrize("seed", range(4))
def test_random_split_f32(seed):
    split_parity(workloads.random_split(seed, torch.float32), "random-split f32 %d" % seed)


def test_tiny_split():
    wl = workloads.execute_split(dataclasses.replace(workloads.tiny(torch.bfloat16), q_starts=[384], doc_len=100),
                                 [0])
    split_parity(wl, "tiny split")


@pytest.mark.parametrize("seed", [1, 6])
def test_split_poison_and_permutation_do_not_change_a_bit(seed):
    wl = workloads.random_split(seed, torch.bfloat16)
    inp = to_dev(workloads.make_inputs(wl))
    say("split poison/permutation seed %d" % seed)
    r1, o1, l1 = run_split(inp, fill=float("nan"))
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(len(inp.free_order)).astype(np.int32)
    r2, o2, l2 = run_split(inp, fill=float("inf"), free_order=perm)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    r1.close()
    r2.close()


@pytest.mark.parametrize("seed", [0, 2, 9])
def test_split_pages_hold_recomputed_and_reused_kv(seed):
    """GLOBAL heads' pages hold the call's new K/V from q_start_global on (bit-exact); LOCAL heads'
    pages hold the re-rotated reused keys below q_start (within one bf16 ulp of the exact rotation)."""
    wl = workloads.random_split(seed, torch.bfloat16)
    inp = workloads.make_inputs(wl)
    say("split page contents %s" % wl.name)
    r, o, lse = run_split(to_dev(inp))
    for b in range(wl.num_seqs):
        for g in range(wl.num_kv_heads):
            cls = int(wl.head_class[0, g])
            k_ref, v_ref = reference.head_kv(inp, b, g)
            start = wl.q_start_of(b, cls)
            exact = k_ref.copy()
            for d in inp.docs:  # exact rotation below the head's start (the kernel rounds once)
                if d.seq == b:
                    lo, hi = d.tok_begin, min(d.tok_begin + d.n_tok, start)
                    if hi > lo:
                        kk = rope.rotate(reference.to64(d.k_off[g]), d.delta, wl.rope_base)
                        exact[lo:hi] = kk[:hi - lo]
            kg, vg, toks = r.page_contents(0, g, b)
            toks = np.array(toks)
            sel = toks < wl.kv_lens[b]
            t = toks[sel]
            kg, vg = kg.double().numpy()[sel], vg.double().numpy()[sel]
            want = paging.pages_of_ranges(paging.held_token_ranges(cls, wl.q_starts[b], wl.kv_lens[b], wl.sink,
                                                                    wl.window), wl.page_size)
            assert sorted(set((t // wl.page_size).tolist())) == want
            z = cleared_below_window(t, cls, start, wl.kv_lens[b], wl.sink, wl.window, wl.page_size)
            assert (kg[z] == 0).all() and (vg[z] == 0).all(), "slots below a LOCAL window not cleared"
            kg, vg, t = kg[~z], vg[~z], t[~z]
            new = t >= start
            assert np.array_equal(kg[new], k_ref[t[new]]), "new keys not written bit-exactly"
            assert (np.abs(kg[~new] - exact[t[~new]]) <= bf16_ulp(exact[t[~new]])).all()
            assert np.array_equal(vg, v_ref[t])
    r.close()


def test_dsv4flash_split_sampled():
    """DeepSeek-V4-Flash-style mixed layer under EXECUTE: 8 GLOBAL heads recompute all 131,072 positions,
    56 LOCAL heads query the last 8,192 over their reused sink + window KV.  Sampled rows."""
    wl = workloads.dsv4flash_split(3)
    what = "DeepSeek-V4-Flash-style EXECUTE split"
    say("%s: generating inputs on the GPU" % what)
    inp = workloads.make_inputs(wl, device="cuda")
    say("%s: running the call" % what)
    r, o, lse = run_split(inp)
    rng = np.random.Generator(np.random.PCG64(3))
    cls_row = wl.head_class[wl.layer]
    heads = []
    for c in (1, 0):
        for g in np.flatnonzero(cls_row == c)[:2]:
            heads.append(int(g) * wl.group)
    n_q = wl.q_lens[0]
    n = 0
    for h in heads:
        c = int(cls_row[h // wl.group])
        lo = wl.q_start_of(0, c) - wl.q_begin(0)
        rows = np.unique(np.concatenate([[lo, lo + 1, n_q - 1, (lo + n_q) // 2, lo + wl.sink, lo + wl.window],
                                         rng.integers(lo, n_q, size=10)]))
        rows = rows[(rows >= lo) & (rows < n_q)]
        o_ref, lse_ref = reference.prefill_rows(inp, 0, h, rows)
        idx = torch.from_numpy(rows).cuda()
        check(o[idx, h], lse[h, idx], o_ref, lse_ref, wl.dtype, "%s head %d" % (what, h))
        if c == 0 and lo > 0:  # the LOCAL head's rows before its start stay untouched
            assert (lse[h, :lo] == LSE_SENTINEL).all()
        n += len(rows)
    assert n > 0
    r.close()


@pytest.mark.parametrize("seed", range(3))
def test_import_stops_at_each_heads_class_start(seed):
    # the reuse import alone (no append): below a head's class start its held slots hold the re-rotated
    # document keys (within a bf16 ulp of the exact rotation) and the document values; from the class
    # start on (a GLOBAL head's recomputed prefix) nothing is written -- the slots keep their poison
    wl = workloads.random_split(seed, torch.bfloat16)
    inp = workloads.make_inputs(wl)
    dinp = to_dev(inp)
    say("import stops at the class start: %s q_starts=%s qg=%s classes=%s" % (
        wl.name, wl.q_starts, wl.q_starts_global, wl.head_class.tolist()))
    r = PrefillRunner(wl, free_order=inp.free_order, poison=True)
    try:
        r.build()
        r.import_docs(dinp.docs)
        torch.cuda.synchronize()
        for b in range(wl.num_seqs):
            ref_k = np.full((wl.num_kv_heads, wl.kv_lens[b], wl.head_dim), np.nan)
            ref_v = np.full_like(ref_k, np.nan)
            for d in inp.docs:
                if d.seq == b:
                    ref_k[:, d.tok_begin:d.tok_begin + d.n_tok] = rope.rotate(reference.to64(d.k_off), d.delta,
                                                                               wl.rope_base)
                    ref_v[:, d.tok_begin:d.tok_begin + d.n_tok] = reference.to64(d.v_off)
            for g in range(wl.num_kv_heads):
                cls = int(wl.head_class[wl.layer, g])
                start = wl.q_start_of(b, cls)
                kg, vg, toks = r.page_contents(wl.layer, g, b)
                t = np.array(toks)
                kg, vg = kg.double().numpy(), vg.double().numpy()
                doc = np.zeros(len(t), bool)
                for d in inp.docs:
                    if d.seq == b:
                        doc |= (t >= d.tok_begin) & (t < d.tok_begin + d.n_tok)
                below = doc & (t < start)
                above = doc & (t >= start)
                assert np.isnan(kg[above]).all() and np.isnan(vg[above]).all(), \
                    "seq %d head %d: the import wrote tokens from the class start %d on" % (b, g, start)
                kr, vr = ref_k[g, t[below]], ref_v[g, t[below]]
                assert (np.abs(kg[below] - kr) <= bf16_ulp(kr)).all(), "re-rotated keys off by more than a bf16 ulp"
                assert np.array_equal(vg[below], vr)
        # the source head stride must keep 16-byte rows: a stride 3 elements past n_tok * D is rejected on
        # the host, before any device access
        d = dinp.docs[0]
        Hkv, D = wl.num_kv_heads, wl.head_dim
        if Hkv > 1:
            st = d.n_tok * D + 3
            buf = torch.zeros((Hkv * st,), dtype=wl.dtype, device="cuda")
            odd = torch.as_strided(buf, (Hkv, d.n_tok, D), (st, D, 1))
            with pytest.raises(rk_seg.RkError) as ei:
                rk_seg.rk_seg_reuse_rerotate(r.tables, wl.layer, d.seq, d.tok_begin, odd, odd, d.delta, wl.rope_base)
            assert ei.value.status == rk_seg.RK_ERR_INVALID_ARG
    finally:
        r.close()
