"""Per-key attention mass on the GPU through the C ABI, against the fp64 oracle.

Bars: fed the oracle's lse, the kernel's mass is within 1e-4 * max(1, mass) of the oracle (the only
differences are fp32 accumulation of the same bf16 products and exp2); with the GPU's own lse (which
the attention parity tests bound), within 2e-3 * max(1, mass).  Every head's masses sum to its
number of query rows.  At full size, sampled key columns are recomputed in fp64 from the GPU lse."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from head_aware_paged_prefill_amd import rk_seg
from head_aware_paged_prefill_amd.runner import PrefillRunner
from oracle import reference

from test_gpu_parity import say, to_dev

pytestmark = pytest.mark.gpu


def run_with_mass(inp, lse_for_mass=None):
    wl = inp.wl
    r = PrefillRunner(wl, free_order=inp.free_order, poison=True)
    r.build()
    r.import_docs(inp.docs)
    o, lse = r.attend(inp.q, inp.k_new, inp.v_new)
    mass = r.key_mass(inp.q, lse if lse_for_mass is None else lse_for_mass)
    torch.cuda.synchronize()
    return r, o, lse, mass


def rel_err(a, b):
    return np.abs(a - b) / np.maximum(1.0, np.abs(b))


def row_counts(wl):
    n = np.zeros(wl.num_q_heads)
    off = reference.kv_offsets(wl)
    out = []
    for b in range(wl.num_seqs):
        per = np.array([wl.kv_lens[b] - wl.q_start_of(b, int(wl.head_class[wl.layer, h // wl.group]))
                        for h in range(wl.num_q_heads)], np.float64)
        out.append((off[b], off[b + 1], per))
    return out


def mass_parity(wl, what):
    inp = workloads.make_inputs(wl)
    want = reference.key_mass(inp)
    _, lse_ref = reference.prefill(inp)
    say("%s kv_lens=%s q_starts=%s qg=%s H=%d Hkv=%d D=%d P=%d S=%d W=%d" % (
        what, wl.kv_lens, wl.q_starts, wl.q_starts_global, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
        wl.page_size, wl.sink, wl.window))
    dinp = to_dev(inp)
    # kernel alone: the oracle's lse (rows a LOCAL head does not compute carry NaN there and are not read)
    lse_in = torch.from_numpy(np.nan_to_num(lse_ref, nan=0.0)).float().cuda()
    r, o, lse, mass = run_with_mass(dinp, lse_in)
    m = mass.double().cpu().numpy()
    assert np.isfinite(m).all()
    e = rel_err(m, want)
    assert e.max() <= 1e-4, "%s: kernel-only mass rel err %.3g" % (what, e.max())
    # end to end: the GPU's own lse
    m2 = r.key_mass(dinp.q, lse).double().cpu().numpy()
    e2 = rel_err(m2, want)
    assert e2.max() <= 2e-3, "%s: end-to-end mass rel err %.3g" % (what, e2.max())
    for a, b, per in row_counts(wl):
        np.testing.assert_allclose(m2[:, a:b].sum(axis=1), per, rtol=1e-3)
    r.close()


@pytest.mark.parametrize("seed", range(10))
def test_random_small_mass(seed):
    mass_parity(workloads.random_small(seed, torch.bfloat16), "mass random-small %d" % seed)


@pytest.mark.parametrize("seed", range(6))
def test_random_split_mass(seed):
    mass_parity(workloads.random_split(seed, torch.bfloat16), "mass random-split %d" % seed)


def test_tiny_mass():
    mass_parity(workloads.tiny(torch.bfloat16), "mass tiny")


@pytest.mark.parametrize("G", [3, 5, 12, 16])
def test_mass_odd_and_large_groups(G):
    wl = workloads.random_small(2, torch.bfloat16)
    wl = dataclasses.replace(wl, num_q_heads=G * wl.num_kv_heads, name="mass G=%d" % G)
    mass_parity(wl, wl.name)


@pytest.mark.parametrize("P,D", [(8, 64), (8, 128), (256, 128)])
def test_mass_page_sizes(P, D):
    # 8-key pages (the smallest the pool takes) and 256-key pages: the kernel looks up each key's page
    wl = workloads.random_small(4, torch.bfloat16)
    wl = dataclasses.replace(wl, page_size=P, head_dim=D, name="mass P=%d D=%d" % (P, D))
    mass_parity(wl, wl.name)


@pytest.mark.parametrize("G", [8, 16])
def test_mass_multi_chunk(G):
    # several key blocks and query chunks per head, so that the partial sums of many work units meet
    # in one output; a LOCAL head with a window wider than a key block, and EXECUTE's split
    wl = workloads.Workload(name="mass multi-chunk G=%d" % G, config_id=400 + G, num_layers=1, layer=0,
                            kv_lens=[2600, 1100], q_starts=[900, 300], num_q_heads=2 * G, num_kv_heads=2,
                            head_dim=128, page_size=16, sink=4, window=700, dtype=torch.bfloat16,
                            head_class=np.array([[1, 0]], np.uint8), pool_slack=7, doc_len=200, rope_base=1.0e4,
                            q_starts_global=[0, 300])
    mass_parity(wl, wl.name)


def test_mass_rejects_unsupported():
    wl = workloads.random_small(1, torch.float32)
    inp = to_dev(workloads.make_inputs(wl))
    r = PrefillRunner(wl, free_order=inp.free_order)
    r.build()
    r.import_docs(inp.docs)
    o, lse = r.attend(inp.q, inp.k_new, inp.v_new)
    with pytest.raises(rk_seg.RkError) as ei:
        r.key_mass(inp.q, lse)
    assert ei.value.status == rk_seg.RK_ERR_UNSUPPORTED
    r.close()


def _sampled_full(wl, what, keys_per_head=10, seed=0):
    say("%s: generating inputs on the GPU" % what)
    inp = workloads.make_inputs(wl, device="cuda")
    say("%s: attention and mass" % what)
    r, o, lse, mass = run_with_mass(inp)
    m = mass.double().cpu().numpy()
    assert np.isfinite(m).all()
    for a, b, per in row_counts(wl):
        np.testing.assert_allclose(m[:, a:b].sum(axis=1), per, rtol=1e-3)
    rng = np.random.Generator(np.random.PCG64(seed))
    cls_row = wl.head_class[wl.layer]
    heads = [int(g) * wl.group for c in (1, 0) for g in np.flatnonzero(cls_row == c)[:2]]
    lse_c = lse.double().cpu().numpy()
    cu = wl.cu_q()
    scale = 1.0 / np.sqrt(wl.head_dim)
    for b in range(wl.num_seqs)[:2]:
        L, qb = wl.kv_lens[b], wl.q_begin(b)
        off = reference.kv_offsets(wl)[b]
        for h in heads:
            g = h // wl.group
            c = int(cls_row[g])
            start = wl.q_start_of(b, c)
            k, _ = reference.head_kv(inp, b, g)
            keys = np.unique(np.concatenate([[0, wl.sink - 1, wl.sink, L - 1, max(0, start - wl.window),
                                              max(0, start - wl.window + 1), start, (start + L) // 2],
                                             rng.integers(0, L, size=keys_per_head)]))
            keys = keys[(keys >= 0) & (keys < L)]
            pos = np.arange(start, L)
            q = reference.to64(inp.q[cu[b] + start - qb:cu[b + 1], h])
            li = lse_c[h, cu[b] + start - qb:cu[b + 1]]
            # visibility of the sampled keys only (a dense [queries][L] mask would not fit at 128K)
            kj = keys[None, :]
            pp = pos[:, None]
            vis = (kj <= pp) & ((c == 1) | (kj < wl.sink) | (kj > pp - wl.window))
            s = scale * (q @ k[keys].T)
            want = np.where(vis, np.exp(s - li[:, None]), 0.0).sum(axis=0)
            got = m[h, off + keys]
            e = rel_err(got, want)
            assert e.max() <= 1e-3, "%s seq %d head %d: rel err %.3g" % (what, b, h, e.max())
    r.close()


def test_qwen32b_mass_sampled():
    _sampled_full(workloads.qwen32b(), "Qwen3-32B-shaped 128K mass")


def test_dsv4flash_split_mass_sampled():
    _sampled_full(workloads.dsv4flash_split(3), "DeepSeek-V4-Flash-style EXECUTE split mass")


def test_mass_with_no_query_rows_writes_zeros():
    """A call whose sequences have keys but no query row (q_start = kv_len): every mass entry is
    written, and each is 0 (no query sees any key).  The output starts as a sentinel."""
    wl = workloads.Workload(name="mass without queries", config_id=431, num_layers=1, layer=0,
                            kv_lens=[300, 77], q_starts=[300, 77], num_q_heads=8, num_kv_heads=2, head_dim=128,
                            page_size=16, sink=4, window=64, dtype=torch.bfloat16,
                            head_class=np.array([[1, 0]], np.uint8), pool_slack=3)
    say(wl.name)
    r = PrefillRunner(wl, num_pages=workloads.pool_pages_needed_hint(wl) + 8)
    try:
        r.build()
        mass = torch.full((wl.num_q_heads, sum(wl.kv_lens)), 7.0, dtype=torch.float32, device="cuda")
        rk_seg.rk_seg_key_mass(r.tables, wl.layer, None, None, mass)
        torch.cuda.synchronize()
        assert torch.equal(mass, torch.zeros_like(mass))
    finally:
        r.close()
