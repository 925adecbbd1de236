"""Pins of the oracle's head-ragged query ranges (EXECUTE's split: GLOBAL heads recompute from an
earlier position than LOCAL heads; page "RedKnot - Xiaohongshuが開発した…", section 使い方, EXECUTE
item).  Each pin ties the split call to something other than itself: the plain call on the same
inputs, or explicit loops over the definition of masked softmax attention."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import reference


def _split_wl(qs, qg, L, dtype=torch.float64, D=8):
    hc = np.array([[workloads.GLOBAL, workloads.LOCAL]], np.uint8)
    wl = workloads.Workload(name="split pin", config_id=950, num_layers=1, layer=0, kv_lens=L, q_starts=qs,
                            num_q_heads=4, num_kv_heads=2, head_dim=D, page_size=8, sink=3, window=6,
                            dtype=dtype, head_class=hc, doc_len=7, rope_base=1.0e4)
    return workloads.execute_split(wl, qg)


@pytest.mark.parametrize("qg", [[0, 0], [10, 3]])
def test_split_matches_brute_force(qg):
    """fp64 inputs; every computed row against loops over keys, exp and sums written from the definition."""
    wl = _split_wl([25, 12], qg, [40, 19])
    inp = workloads.make_inputs(wl)
    o, lse = reference.prefill(inp)
    cu = wl.cu_q()
    scale = 1.0 / math.sqrt(wl.head_dim)
    checked = 0
    for b in range(wl.num_seqs):
        k, v = reference.sequence_kv(inp, b)
        qb, L = wl.q_begin(b), wl.kv_lens[b]
        for h in range(wl.num_q_heads):
            g = h // wl.group
            cls = int(wl.head_class[0, g])
            start = qg[b] if cls == workloads.GLOBAL else wl.q_starts[b]
            for r in range(L - qb):
                i = qb + r
                row_o, row_l = o[cu[b] + r, h], lse[h, cu[b] + r]
                if i < start:
                    assert np.isnan(row_o).all() and np.isnan(row_l)
                    continue
                qv = inp.q[cu[b] + r, h].double().numpy()
                keys = [j for j in range(L) if j <= i and (cls == workloads.GLOBAL or j < wl.sink or j > i - wl.window)]
                sc = [scale * sum(qv[d] * k[g, j, d] for d in range(wl.head_dim)) for j in keys]
                m = max(sc)
                den = sum(math.exp(x - m) for x in sc)
                exp_l = m + math.log(den)
                exp_o = [sum(math.exp(sc[t] - exp_l) * v[g, j, d] for t, j in enumerate(keys)) for d in range(wl.head_dim)]
                assert abs(row_l - exp_l) <= 1e-12 * max(1.0, abs(exp_l))
                assert np.allclose(row_o, exp_o, rtol=0, atol=1e-12)
                checked += 1
    assert checked > 0


def test_split_global_rows_equal_plain_call_from_global_start():
    """GLOBAL heads: identical to a plain call whose every head starts at q_start_global (same packed rows)."""
    wl = workloads.random_split(3)
    inp = workloads.make_inputs(wl)
    o, lse = reference.prefill(inp)
    wl2 = dataclasses.replace(wl, q_starts=list(wl.q_starts_global), q_starts_global=None)
    o2, lse2 = reference.prefill(dataclasses.replace(inp, wl=wl2))
    heads = [h for h in range(wl.num_q_heads) if wl.head_class[0, h // wl.group] == workloads.GLOBAL]
    assert heads
    np.testing.assert_allclose(o[:, heads], o2[:, heads], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[heads], lse2[heads], rtol=0, atol=1e-12)


def test_split_local_rows_equal_plain_call_on_trailing_rows():
    """LOCAL heads: identical to a plain call from q_start on the sequences' trailing rows, the reused
    documents supplying everything below q_start."""
    wl = workloads.random_split(5)
    inp = workloads.make_inputs(wl)
    o, lse = reference.prefill(inp)
    cu = wl.cu_q()
    keep = np.concatenate([np.arange(cu[b] + wl.q_starts[b] - wl.q_begin(b), cu[b + 1]) for b in range(wl.num_seqs)])
    wl3 = dataclasses.replace(wl, q_starts_global=None)
    sel = torch.from_numpy(keep)
    inp3 = dataclasses.replace(inp, wl=wl3, q=inp.q[sel], k_new=inp.k_new[sel], v_new=inp.v_new[sel])
    o3, lse3 = reference.prefill(inp3)
    heads = [h for h in range(wl.num_q_heads) if wl.head_class[0, h // wl.group] == workloads.LOCAL]
    assert heads
    np.testing.assert_allclose(o[keep][:, heads], o3[:, heads], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[heads][:, keep], lse3[heads], rtol=0, atol=1e-12)


def test_equal_starts_reduce_to_the_plain_call():
    wl = workloads.random_small(7)
    inp = workloads.make_inputs(wl)
    o, lse = reference.prefill(inp)
    wl_s = workloads.execute_split(wl, list(wl.q_starts))
    o_s, lse_s = reference.prefill(dataclasses.replace(inp, wl=wl_s))
    np.testing.assert_array_equal(o, o_s)
    np.testing.assert_array_equal(lse, lse_s)


def test_prefill_rows_matches_prefill_on_a_split_call():
    wl = workloads.random_split(8)
    inp = workloads.make_inputs(wl)
    o, lse = reference.prefill(inp)
    cu = wl.cu_q()
    for b in range(wl.num_seqs):
        for h in range(wl.num_q_heads):
            cls = int(wl.head_class[0, h // wl.group])
            lo = wl.q_start_of(b, cls) - wl.q_begin(b)
            rows = np.arange(lo, wl.q_lens[b])
            if len(rows) == 0:
                continue
            orr, lr = reference.prefill_rows(inp, b, h, rows)
            np.testing.assert_allclose(orr, o[cu[b] + rows, h], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lr, lse[h, cu[b] + rows], rtol=0, atol=1e-12)
