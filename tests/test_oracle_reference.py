"""Pins of the oracle's assembly of one prefill call (packing, reuse import, head map)."""
import math

import numpy as np
import torch

import workloads
from oracle import reference


def complex_rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """RoPE of x [..., n, D] at positions pos [n], as a complex multiplication of rotate-half pairs."""
    D = x.shape[-1]
    th = base ** (-np.arange(D // 2) * 2.0 / D)
    z = (x[..., : D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * pos[:, None] * th)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_packed_call_matches_per_head_loops():
    """Unpacking [total_q][H][D] into per-head rows: checked with explicit loops over (seq, head, row)."""
    wl = workloads.random_small(3, torch.float32, allow_reuse=False)
    inp = workloads.make_inputs(wl)
    o, lse = reference.prefill(inp)
    cu = wl.cu_q()
    G = wl.group
    for b in range(wl.num_seqs):
        L = wl.kv_lens[b]
        for h in range(wl.num_q_heads):
            g = h // G
            cls = int(wl.head_class[0, g])
            for t in range(0, L, max(1, L // 7)):
                qv = inp.q[cu[b] + t, h].double().numpy()
                ks = inp.k_new[cu[b]:cu[b] + L, g].double().numpy()
                vs = inp.v_new[cu[b]:cu[b] + L, g].double().numpy()
                vis = [j for j in range(L) if j <= t and (cls == 1 or j < wl.sink or j > t - wl.window)]
                s = ks[vis] @ qv / math.sqrt(wl.head_dim)
                mx = s.max()
                p = np.exp(s - mx)
                assert abs(lse[h, cu[b] + t] - (mx + math.log(p.sum()))) < 1e-10
                np.testing.assert_allclose(o[cu[b] + t, h], p @ vs[vis] / p.sum(), rtol=0, atol=1e-10)


def test_reused_keys_equal_direct_rope_at_actual_position():
    """Offline keys = RoPE(raw, offline pos); after import they must equal RoPE(raw, actual pos)."""
    wl = workloads.Workload(name="reuse pin", config_id=900, num_layers=1, layer=0, kv_lens=[96], q_starts=[64],
                            num_q_heads=2, num_kv_heads=2, head_dim=16, page_size=16, sink=2, window=8,
                            dtype=torch.float32, head_class=np.array([[1, 0]], np.uint8), doc_len=32,
                            rope_base=1e4)
    inp = workloads.make_inputs(wl)
    raw = {}
    for d in inp.docs:
        r = np.random.Generator(np.random.PCG64(d.tok_begin)).standard_normal((2, d.n_tok, 16))
        off_pos = d.offline_start + np.arange(d.n_tok)
        d.k_off = torch.from_numpy(complex_rope(r, off_pos, wl.rope_base)).float()
        raw[d.tok_begin] = r
    k, v = reference.sequence_kv(inp, 0)
    for d in inp.docs:
        want = complex_rope(raw[d.tok_begin], d.tok_begin + np.arange(d.n_tok), wl.rope_base)
        np.testing.assert_allclose(k[:, d.tok_begin:d.tok_begin + d.n_tok], want, rtol=0, atol=2e-5)
        assert d.delta != 0
    np.testing.assert_array_equal(k[:, 64:], inp.k_new.double().numpy().transpose(1, 0, 2))


def test_per_head_rows_equal_whole_call():
    wl = workloads.random_small(5, torch.float32)
    inp = workloads.make_inputs(wl)
    o, lse = reference.prefill(inp)
    cu = wl.cu_q()
    for b in range(wl.num_seqs):
        n = wl.q_lens[b]
        if n == 0:
            continue
        rows = np.unique(np.array([0, n - 1, n // 2]))
        for h in (0, wl.num_q_heads - 1):
            ob, lb = reference.prefill_rows(inp, b, h, rows)
            np.testing.assert_allclose(ob, o[cu[b] + rows, h], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lb, lse[h, cu[b] + rows], rtol=0, atol=1e-12)


def _golden_rows(name):
    import os
    rows = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", name)):
        if line.startswith("#") or not line.strip():
            continue
        a, b = line.split()[:2]
        rows.append((float.fromhex(a), math.inf if b == "inf" else float.fromhex(b)))
    return rows


def test_round_store_bf16_hand_worked_values():
    """The cache's bf16 rounding: ties to even, one rounding of the exact value (the case just above a
    tie, where fp64 -> fp32 -> bf16 would land on the even neighbour below), subnormals, overflow."""
    rows = _golden_rows("round_bf16.txt")
    x = np.array([r[0] for r in rows])
    want = np.array([r[1] for r in rows])
    got = reference.round_store(x, torch.bfloat16)
    np.testing.assert_array_equal(got, want)
    # the double rounding the oracle does not do, for contrast
    dbl = torch.tensor([1.0 + 2.0 ** -8 + 2.0 ** -40], dtype=torch.float64).float().to(torch.bfloat16).double()
    assert float(dbl[0]) == 1.0 and reference.round_store(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]),
                                                          torch.bfloat16)[0] == 1.0 + 2.0 ** -7


def test_round_store_bf16_equals_torch_on_fp32_values():
    """For values an fp32 holds exactly, one rounding to bf16 is torch's fp32 -> bf16 conversion
    (nearest even): 200k random fp32 values over the whole exponent range, including ties."""
    rng = np.random.Generator(np.random.PCG64(31))
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ties = (rng.integers(0, 2 ** 16, size=5000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32).view(np.float32)
    f = np.concatenate([f, ties[np.isfinite(ties)]])
    want = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    got = reference.round_store(f.astype(np.float64), torch.bfloat16)
    np.testing.assert_array_equal(got, want)


def test_round_store_f32_is_nearest_even():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 1.0 + 2.0 ** -24 + 2.0 ** -40])
    np.testing.assert_array_equal(reference.round_store(x, torch.float32),
                                  [1.0, 1.0 + 2.0 ** -22, 1.0 + 2.0 ** -23])
