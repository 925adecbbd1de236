"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on an MI355X.

Bars: bf16 output max-abs <= 2e-2 and mean-abs <= 2e-3 over all compared elements, row LSE within
1e-3 * max(1, |lse|); fp32 storage max-abs 1e-4, mean-abs 1e-5, LSE 1e-5 * max(1, |lse|).  The LSE
bar is asserted as two bars: the relative error over rows with |lse| >= 1, and the absolute error over
the near-zero rows below (row 0's lse is ~0, where a relative error is meaningless).  Integer
work (page tables, visible-key counts) is compared bit-exactly.  Re-rotated keys: within one bf16 ulp
of the oracle's exact value.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import workloads
from head_aware_paged_prefill_amd import rk_seg
from head_aware_paged_prefill_amd.runner import PrefillRunner
from oracle import attention, paging, reference, rope

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (2e-2, 2e-3, 1e-3), torch.float32: (1e-4, 1e-5, 1e-5)}


def say(msg):
    print("[gpu case] " + msg, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    docs = [dataclasses.replace(d, k_off=d.k_off.cuda(), v_off=d.v_off.cuda()) for d in inp.docs]
    return dataclasses.replace(inp, q=inp.q.cuda(), k_new=inp.k_new.cuda(), v_new=inp.v_new.cuda(), docs=docs)


def cleared_below_window(t, cls, start, kv_len, sink, window, page_size):
    """Tokens of a LOCAL head's held pages that the append clears to zero: on its first written page
    (the page of its first query, when the call has queries), those below its window and above its
    sink -- no query of the call or of a later one sees them, and a page newly taken when the window
    moved on would otherwise hold unwritten bits there."""
    t = np.asarray(t)
    if cls == paging.GLOBAL or kv_len <= start:
        return np.zeros(len(t), bool)
    p0 = (start // page_size) * page_size
    return (t >= max(p0, sink)) & (t < min(start, start - window + 1))


def run_call(inp, free_order=None, fill=float("nan"), rope_style=rk_seg.RK_ROPE_ROTATE_HALF):
    wl = inp.wl
    fo = inp.free_order if free_order is None else free_order
    r = PrefillRunner(wl, free_order=fo, poison=False)
    r.k_pages.fill_(fill)
    r.v_pages.fill_(fill)
    r.build()
    r.import_docs(inp.docs, rope_style=rope_style)
    o, lse = r.attend(inp.q, inp.k_new, inp.v_new)
    torch.cuda.synchronize()
    return r, o, lse


def check(o, lse, o_ref, lse_ref, dtype, what=""):
    mx_tol, mean_tol, lse_tol = TOL[dtype]
    o = o.float().cpu().double().numpy() if isinstance(o, torch.Tensor) else o
    lse = lse.cpu().double().numpy() if isinstance(lse, torch.Tensor) else lse
    assert np.isfinite(o).all(), what + ": non-finite output"
    err = np.abs(o - o_ref)
    assert err.max() <= mx_tol, "%s: max-abs %.3g" % (what, err.max())
    assert err.mean() <= mean_tol, "%s: mean-abs %.3g" % (what, err.mean())
    d, a = np.abs(lse - lse_ref), np.abs(lse_ref)
    big = a >= 1.0
    if big.any():  # rows with |lse| >= 1: the true relative error
        rel = (d[big] / a[big]).max()
        assert rel <= lse_tol, "%s: lse relative error %.3g (rows with |lse| >= 1)" % (what, rel)
    if (~big).any():  # near-zero rows (row 0's lse is ~0): an absolute bound of the same size
        ab = d[~big].max()
        assert ab <= lse_tol, "%s: lse absolute error %.3g (rows with |lse| < 1)" % (what, ab)


def full_parity(wl, what):
    inp = workloads.make_inputs(wl)
    o_ref, lse_ref = reference.prefill(inp)
    say("%s  kv_lens=%s q_starts=%s H=%d Hkv=%d D=%d P=%d S=%d W=%d dtype=%s" % (
        what, wl.kv_lens, wl.q_starts, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.sink,
        wl.window, wl.dtype))
    r, o, lse = run_call(to_dev(inp))
    try:
        check(o, lse, o_ref, lse_ref, wl.dtype, what)
    finally:
        r.close()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_tiny_config_full_parity(dtype):
    full_parity(workloads.tiny(dtype), "tiny")


@pytest.mark.parametrize("seed", range(24))
def test_random_small_bf16(seed):
    full_parity(workloads.random_small(seed, torch.bfloat16), "random-small bf16 %d" % seed)


@pytest.mark.parametrize("seed", range(8))
def test_random_small_f32(seed):
    full_parity(workloads.random_small(seed, torch.float32), "random-small f32 %d" % seed)


@pytest.mark.parametrize("seed", range(6))
def test_random_many_items_per_workgroup_bf16(seed):
    """Hundreds of items: every persistent workgroup runs a chain of them (one-step items included),
    so each item's first tiles come from the stream of the item before it."""
    full_parity(workloads.random_many(seed, torch.bfloat16), "random-many bf16 %d" % seed)


@pytest.mark.parametrize("seed", range(2))
def test_random_many_items_per_workgroup_f32(seed):
    full_parity(workloads.random_many(seed, torch.float32), "random-many f32 %d" % seed)


@pytest.mark.parametrize("factor", [8.0, 24.0])
def test_late_outlier_keys_take_the_rescale_path(factor):
    """Key rows scaled up deep into a row lift its scores far above the running max taken so far
    (8x: ~35, 24x: ~100 log2 units at the top, past the kernel's 2^20 rescale bound), so the rescale
    path runs in the middle and at the end of rows of both head classes."""
    wl = workloads.Workload(name="late outliers", config_id=950, num_layers=1, layer=0, kv_lens=[1500, 2100],
                            q_starts=[0, 0], num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, sink=4,
                            window=600, dtype=torch.bfloat16, head_class=np.array([[1, 0]], np.uint8), pool_slack=7)
    inp = workloads.make_inputs(wl)
    cu = wl.cu_q()
    for b, L in enumerate(wl.kv_lens):
        for pos in (700, 1400, L - 5):
            inp.k_new[cu[b] + pos] = (inp.k_new[cu[b] + pos].float() * factor).to(wl.dtype)
    full_parity_of(inp, "late outliers x%g" % factor)


def full_parity_of(inp, what):
    o_ref, lse_ref = reference.prefill(inp)
    say(what)
    r, o, lse = run_call(to_dev(inp))
    try:
        check(o, lse, o_ref, lse_ref, inp.wl.dtype, what)
    finally:
        r.close()


def test_all_global_and_window_covering_local_equal_each_other():
    """The dense reference (every head GLOBAL) and LOCAL heads whose window covers the sequence agree."""
    wl = workloads.tiny(torch.bfloat16)
    wl_g = wl.with_classes(np.ones_like(wl.head_class))
    wl_l = dataclasses.replace(wl.with_classes(np.zeros_like(wl.head_class)), window=10 ** 6)
    inp = to_dev(workloads.make_inputs(wl_g))
    say("all-global vs wide-window local")
    r1, o1, l1 = run_call(inp)
    r2, o2, l2 = run_call(dataclasses.replace(inp, wl=wl_l))
    o_ref, lse_ref = reference.prefill(workloads.make_inputs(wl_g))
    check(o1, l1, o_ref, lse_ref, wl.dtype, "all-global")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    r1.close()
    r2.close()


@pytest.mark.parametrize("seed", [0, 3, 7])
def test_nan_poison_and_page_permutation_do_not_change_a_bit(seed):
    wl = workloads.random_small(seed, torch.bfloat16)
    inp = to_dev(workloads.make_inputs(wl))
    say("poison/permutation seed %d" % seed)
    r1, o1, l1 = run_call(inp, fill=float("nan"))
    r2, o2, l2 = run_call(inp, fill=0.0)
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(len(inp.free_order)).astype(np.int32)
    r3, o3, l3 = run_call(inp, free_order=perm, fill=float("inf"))
    r4, o4, l4 = run_call(inp, fill=float("nan"))
    assert torch.isfinite(o1.float()).all()
    for o, l in ((o2, l2), (o3, l3), (o4, l4)):
        assert torch.equal(o1, o), "output depends on never-written slots, page ids or the run"
        assert torch.equal(l1, l)
    for r in (r1, r2, r3, r4):
        r.close()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("seed", range(6))
def test_visible_count_probe(dtype, seed):
    """q = 0 makes every visible key weigh the same: exp(lse) = |V(i)|, bit-exact after rounding.
    With fp32 storage and v_j[0] = j, o[0] * |V(i)| = sum of visible positions (exact)."""
    wl = workloads.random_small(seed, dtype, allow_reuse=False)
    inp = workloads.make_inputs(wl)
    inp.q.zero_()
    cu = wl.cu_q()
    if dtype == torch.float32:
        for b in range(wl.num_seqs):
            inp.v_new[cu[b]:cu[b + 1], :, 0] = torch.arange(wl.kv_lens[b], dtype=torch.float32)[:, None]
    say("count probe %s seed %d" % (dtype, seed))
    r, o, lse = run_call(to_dev(inp))
    lse = lse.cpu().double().numpy()
    o = o.float().cpu().double().numpy()
    for b in range(wl.num_seqs):
        L = wl.kv_lens[b]
        for h in range(wl.num_q_heads):
            cls = int(wl.head_class[0, h // wl.group])
            m = attention.visibility_mask(cls, np.arange(L), L, wl.sink, wl.window)
            cnt = m.sum(axis=1)
            got = np.rint(np.exp(lse[h, cu[b]:cu[b + 1]])).astype(np.int64)
            assert (got == cnt).all(), (b, h)
            if dtype == torch.float32:
                sums = (m * np.arange(L)[None, :]).sum(axis=1)
                assert (np.rint(o[cu[b]:cu[b + 1], h, 0] * cnt).astype(np.int64) == sums).all(), (b, h)
    r.close()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


@pytest.mark.parametrize("seed,style", [(1, rope.ROTATE_HALF), (2, rope.ROTATE_HALF), (4, rope.ROTATE_HALF),
                                        (9, rope.ROTATE_HALF), (11, rope.ROTATE_HALF), (1, rope.INTERLEAVED),
                                        (9, rope.INTERLEAVED)])
def test_pages_hold_rerotated_prefix_and_appended_tokens(seed, style):
    wl = None
    s = seed
    while wl is None or all(q == 0 for q in wl.q_starts):  # need a reused prefix
        wl = workloads.random_small(s, torch.bfloat16)
        s += 100
    inp = workloads.make_inputs(wl)
    say("page contents %s style %d" % (wl.name, style))
    kstyle = rk_seg.RK_ROPE_ROTATE_HALF if style == rope.ROTATE_HALF else rk_seg.RK_ROPE_INTERLEAVED
    r, o, lse = run_call(to_dev(inp), rope_style=kstyle)
    # the call's attention over the pages, against the oracle with the same pairing
    o_ref, lse_ref = reference.prefill(inp, rope_style=style)
    check(o, lse, o_ref, lse_ref, wl.dtype, "page contents %s style %d" % (wl.name, style))
    held = set()
    for b in range(wl.num_seqs):
        k_ref, v_ref = reference.sequence_kv(inp, b, style)
        # exact rotation, not rounded: the kernel rounds once
        for d in inp.docs:
            if d.seq == b:
                k_ref[:, d.tok_begin:d.tok_begin + d.n_tok] = rope.rotate(reference.to64(d.k_off), d.delta,
                                                                           wl.rope_base, style)
        for g in range(wl.num_kv_heads):
            kg, vg, toks = r.page_contents(0, g, b)
            _, ids = rk_seg.rk_seg_tables_export(r.tables, 0, g, b)
            held.update(ids)
            toks = np.array(toks)
            sel = toks < wl.kv_lens[b]
            kg = kg.double().numpy()[sel]
            vg = vg.double().numpy()[sel]
            t = toks[sel]
            want = paging.pages_of_ranges(paging.held_token_ranges(int(wl.head_class[0, g]), wl.q_starts[b],
                                                                    wl.kv_lens[b], wl.sink, wl.window), wl.page_size)
            assert sorted(set((t // wl.page_size).tolist())) == want
            z = cleared_below_window(t, int(wl.head_class[0, g]), wl.q_starts[b], wl.kv_lens[b], wl.sink, wl.window,
                                     wl.page_size)
            assert (kg[z] == 0).all() and (vg[z] == 0).all(), "slots below a LOCAL window not cleared"
            kg, vg, t = kg[~z], vg[~z], t[~z]
            kr, vr = k_ref[g, t], v_ref[g, t]
            assert (np.abs(kg - kr) <= bf16_ulp(kr)).all(), "re-rotated keys off by more than one bf16 ulp"
            zero_delta = np.zeros(len(t), bool)
            for d in inp.docs:
                if d.seq == b and d.delta == 0:
                    zero_delta |= (t >= d.tok_begin) & (t < d.tok_begin + d.n_tok)
            new = t >= wl.q_starts[b]
            assert np.array_equal(kg[new | zero_delta], kr[new | zero_delta])
            assert np.array_equal(vg, vr)
    # pages nobody holds keep their poison
    free = sorted(set(range(r.num_pages)) - held)
    if free:
        idx = torch.tensor(free, device="cuda")
        assert torch.isnan(r.k_pages.index_select(0, idx).float()).all()
        assert torch.isnan(r.v_pages.index_select(0, idx).float()).all()
    r.close()


# ------------------------------------------------------------------------------------------------
# full-size configurations, sampled rows (the oracle computes them one by one)
# ------------------------------------------------------------------------------------------------

def sample_rows(n_q, q_start, sink, window, rng, k=12):
    rows = {0, 1, n_q - 1, n_q // 2}
    for pos in (sink - 1, sink, window - 1, window, window + 1, sink + window):
        if 0 <= pos - q_start < n_q:
            rows.add(pos - q_start)
    rows.update(rng.integers(0, n_q, size=k).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n_q))


def sampled_parity(wl, seqs, heads, what, seed=0):
    say("%s: generating inputs on the GPU" % what)
    inp = workloads.make_inputs(wl, device="cuda")
    say("%s: running the call" % what)
    r, o, lse = run_call(inp)
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = wl.cu_q()
    errs, n = [], 0
    for b in seqs:
        rows = sample_rows(wl.q_lens[b], wl.q_starts[b], wl.sink, wl.window, rng)
        for h in heads:
            o_ref, lse_ref = reference.prefill_rows(inp, b, h, rows)
            idx = torch.from_numpy(cu[b] + rows).cuda()
            check(o[idx, h], lse[h, idx], o_ref, lse_ref, wl.dtype, "%s seq %d head %d" % (what, b, h))
            n += len(rows)
    r.close()
    del inp, o, lse
    torch.cuda.empty_cache()
    return n


def heads_of_both_classes(wl, per_class=2):
    cls = wl.head_class[wl.layer]
    out = []
    for c in (1, 0):
        kv = np.flatnonzero(cls == c)
        for g in kv[:per_class]:
            out.append(int(g) * wl.group + (wl.group - 1 if len(out) % 2 else 0))
    return out


def test_mistral7b_shape_sampled():
    wl = workloads.mistral7b()
    assert sampled_parity(wl, range(4), heads_of_both_classes(wl), "Mistral-7B-shaped") > 0


def test_mistral7b_shape_all_global_sampled():
    wl = workloads.mistral7b()
    wl = wl.with_classes(np.ones_like(wl.head_class), wl.name + " all-global")
    assert sampled_parity(wl, [1, 3], [0, 31], "Mistral-7B-shaped all-global") > 0


def test_llama70b_shape_sampled():
    wl = workloads.llama70b()
    assert sampled_parity(wl, [0, 15, 30], heads_of_both_classes(wl), "Llama-3.3-70B-shaped") > 0


def test_qwen32b_shape_sampled():
    wl = workloads.qwen32b()
    assert sampled_parity(wl, [0], heads_of_both_classes(wl, 3), "Qwen3-32B-shaped 128K") > 0


def test_dsv4flash_layer_with_reuse_sampled():
    wl = workloads.dsv4flash(layer=3)
    assert sampled_parity(wl, [0], heads_of_both_classes(wl, 2), "DeepSeek-V4-Flash-style reuse") > 0


@pytest.mark.parametrize("seed,P,G,D", [(2, 8, 2, 64), (5, 128, 4, 128), (6, 256, 1, 128), (12, 16, 3, 64),
                                        (13, 32, 16, 128), (14, 64, 5, 64), (15, 256, 8, 64), (3, 8, 8, 128),
                                        (7, 8, 1, 128)])
def test_edge_shapes(seed, P, G, D):
    wl = workloads.random_small(seed, torch.bfloat16)
    wl = dataclasses.replace(wl, page_size=P, num_q_heads=G * wl.num_kv_heads, head_dim=D,
                             name="edge P=%d G=%d D=%d seed %d" % (P, G, D, seed))
    full_parity(wl, wl.name)


@pytest.mark.parametrize("G,D,dtype", [(32, 128, torch.bfloat16), (64, 64, torch.bfloat16), (100, 128, torch.bfloat16),
                                       (256, 64, torch.bfloat16), (48, 64, torch.float32)])
def test_large_groups(G, D, dtype):
    # up to 256 q heads per KV head (T = 256 / G tokens per work item, down to one); a GLOBAL and a LOCAL
    # KV head, reused prefix on the second sequence
    wl = workloads.Workload(name="G=%d D=%d %s" % (G, D, str(dtype).split(".")[-1]), config_id=430 + G, num_layers=1,
                            layer=0, kv_lens=[300, 77], q_starts=[0, 40], num_q_heads=2 * G, num_kv_heads=2, head_dim=D,
                            page_size=16, sink=4, window=100, dtype=dtype, head_class=np.array([[1, 0]], np.uint8),
                            pool_slack=7, doc_len=50, rope_base=1.0e4)
    full_parity(wl, wl.name)


def test_empty_batch_and_zero_query_sequence():
    wl = workloads.random_small(4, torch.bfloat16, allow_reuse=False)
    # a sequence whose queries were all served earlier sits next to a normal one
    wl0 = dataclasses.replace(wl, kv_lens=[40, 300], q_starts=[0, 0], doc_len=0, name="with zero-query seq")
    inp = workloads.make_inputs(wl0)
    # turn seq 0 into a zero-query sequence: q_start = kv_len, its prefix imported as one document
    wl1 = dataclasses.replace(wl0, q_starts=[40, 0])
    cu = wl0.cu_q()
    docs = [workloads.Document(0, 0, 40, 0, inp.k_new[cu[0]:cu[1]].transpose(0, 1).contiguous(),
                               inp.v_new[cu[0]:cu[1]].transpose(0, 1).contiguous())]
    inp1 = dataclasses.replace(inp, wl=wl1, q=inp.q[cu[1]:], k_new=inp.k_new[cu[1]:], v_new=inp.v_new[cu[1]:],
                               docs=docs)
    o_ref, lse_ref = reference.prefill(inp1)
    say("zero-query sequence")
    r, o, lse = run_call(to_dev(inp1))
    check(o, lse, o_ref, lse_ref, wl.dtype, "zero-query seq")
    r.close()
    wl2 = dataclasses.replace(wl0, kv_lens=[], q_starts=[], name="empty")
    inp2 = workloads.make_inputs(wl2)
    say("empty batch")
    r, o, lse = run_call(to_dev(inp2))
    assert o.numel() == 0 and lse.numel() == 0
    r.close()
