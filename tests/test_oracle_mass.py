"""Pins of the oracle's per-key attention mass (column sums of the attention weights over the call's
queries, per q head): explicit loops, torch softmax with independently built masks, and the
row-normalisation identity (a head's masses sum to its number of query rows)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import reference


def _wl(qs, qg, L, classes=(1, 0), D=8, S=3, W=6, G=2):
    hc = np.array([classes], np.uint8)
    wl = workloads.Workload(name="mass pin", config_id=960, num_layers=1, layer=0, kv_lens=L, q_starts=qs,
                            num_q_heads=G * len(classes), num_kv_heads=len(classes), head_dim=D, page_size=8,
                            sink=S, window=W, dtype=torch.float64, head_class=hc, doc_len=5, rope_base=1.0e4)
    return wl if qg is None else workloads.execute_split(wl, qg)


@pytest.mark.parametrize("qg", [None, [0, 2]])
def test_mass_matches_loops(qg):
    wl = _wl([9, 4], qg, [23, 11])
    inp = workloads.make_inputs(wl)
    mass = reference.key_mass(inp)
    off = reference.kv_offsets(wl)
    cu = wl.cu_q()
    scale = 1.0 / math.sqrt(wl.head_dim)
    for b in range(wl.num_seqs):
        k, _ = reference.sequence_kv(inp, b)
        L, qb = wl.kv_lens[b], wl.q_begin(b)
        for h in range(wl.num_q_heads):
            g = h // wl.group
            cls = int(wl.head_class[0, g])
            start = wl.q_start_of(b, cls)
            want = [0.0] * L
            for i in range(start, L):
                qv = inp.q[cu[b] + i - qb, h].numpy()
                keys = [j for j in range(L) if j <= i and (cls == 1 or j < wl.sink or j > i - wl.window)]
                sc = {j: scale * sum(qv[d] * k[g, j, d] for d in range(wl.head_dim)) for j in keys}
                m = max(sc.values())
                den = sum(math.exp(x - m) for x in sc.values())
                for j in keys:
                    want[j] += math.exp(sc[j] - m) / den
            np.testing.assert_allclose(mass[h, off[b]:off[b] + L], want, rtol=1e-12, atol=1e-14)


def test_mass_matches_torch_softmax_with_independent_masks():
    """Masks built with torch.tril / triu (causal, and causal minus the band beyond the window, plus sink
    columns); weights by torch.softmax; column sums by torch.sum."""
    wl = _wl([0], None, [40], classes=(1, 0), D=16, S=2, W=7)
    inp = workloads.make_inputs(wl)
    mass = reference.key_mass(inp)
    L = wl.kv_lens[0]
    k, _ = reference.sequence_kv(inp, 0)
    causal = torch.tril(torch.ones(L, L, dtype=torch.bool))
    band = causal & ~torch.tril(torch.ones(L, L, dtype=torch.bool), diagonal=-wl.window)
    sinkc = causal.clone()
    sinkc[:, wl.sink:] = False
    masks = {1: causal, 0: band | sinkc}
    for h in range(wl.num_q_heads):
        g = h // wl.group
        q = inp.q[:, h].to(torch.float64)
        s = (q @ torch.from_numpy(k[g]).T) / math.sqrt(wl.head_dim)
        s = s.masked_fill(~masks[int(wl.head_class[0, g])], float("-inf"))
        want = torch.softmax(s, dim=-1).sum(dim=0).numpy()
        np.testing.assert_allclose(mass[h], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed", [0, 4, 11])
def test_mass_sums_to_the_number_of_query_rows(seed):
    wl = workloads.random_split(seed, torch.float32) if seed % 2 == 0 else workloads.random_small(seed, torch.float32)
    inp = workloads.make_inputs(wl)
    mass = reference.key_mass(inp)
    off = reference.kv_offsets(wl)
    for b in range(wl.num_seqs):
        for h in range(wl.num_q_heads):
            cls = int(wl.head_class[0, h // wl.group])
            n = wl.kv_lens[b] - wl.q_start_of(b, cls)
            assert abs(mass[h, off[b]:off[b + 1]].sum() - n) <= 1e-9 * max(1, n)
