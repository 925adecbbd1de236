"""Pins of the fp64 attention oracle against things other than itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped sink term, a
window off by one, a wrong GQA head map, a transposed operand, a missing scale
or a wrong LSE) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention
from oracle.attention import GLOBAL, LOCAL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def closed_form_count(cls, i, S, W):
    """|V(i)| written from the class definitions: i+1 (global); window plus sink tokens left of it (local)."""
    if cls == GLOBAL:
        return i + 1
    return min(i + 1, W) + min(S, max(0, i + 1 - W))


def test_mask_matches_hand_written_golden():
    want = np.loadtxt(os.path.join(GOLDEN, "mask_L8_S2_W3.txt"), dtype=int).astype(bool)
    got = attention.visibility_mask(LOCAL, np.arange(8), 8, sink=2, window=3)
    assert (got == want).all()


def test_mask_global_is_lower_triangle_and_local_band_is_numpy_band():
    L = 37
    assert (attention.visibility_mask(GLOBAL, np.arange(L), L, 4, 5) == np.tril(np.ones((L, L), bool))).all()
    for W in (1, 2, 7, 36, 37, 100):
        band = np.tril(np.triu(np.ones((L, L), bool), -(W - 1)))
        assert (attention.visibility_mask(LOCAL, np.arange(L), L, 0, W) == band).all()


@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 2), (4, 1)])
def test_all_global_equals_torch_sdpa_causal(G, Hkv):
    H, L, D = G * Hkv, 70, 16
    q, k, v = rnd(1, H, L, D), rnd(2, Hkv, L, D), rnd(3, Hkv, L, D)
    o, lse = attention.attention_heads(q, k, v, np.full(Hkv, GLOBAL), 0, 4, 8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=True, enable_gqa=True)[0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_local_sink0_equals_sdpa_with_numpy_band_mask():
    H, L, D, W = 2, 50, 8, 9
    q, k, v = rnd(4, H, L, D), rnd(5, H, L, D), rnd(6, H, L, D)
    o, _ = attention.attention_heads(q, k, v, np.full(H, LOCAL), 0, 0, W)
    band = torch.from_numpy(np.tril(np.triu(np.ones((L, L), bool), -(W - 1))))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=band).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_lse_equals_scipy_logsumexp_and_rows_sum_to_one():
    L, D, S, W = 40, 8, 3, 6
    q, k, v = rnd(7, L, D), rnd(8, L, D), rnd(9, L, D)
    scale = 1 / math.sqrt(D)
    for cls in (GLOBAL, LOCAL):
        m = attention.visibility_mask(cls, np.arange(L), L, S, W)
        _, lse = attention.masked_attention(q, k, v, m, scale)
        s = scale * q @ k.T
        want = np.array([scipy.special.logsumexp(s[i][m[i]]) for i in range(L)])
        np.testing.assert_allclose(lse, want, rtol=0, atol=1e-12)
        p = attention.softmax_rows(q, k, m, scale)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        assert (p[~m] == 0).all()


@pytest.mark.parametrize("S,W", [(0, 64), (3, 64), (64, 5), (200, 1)])
def test_wide_window_or_sink_makes_local_equal_global(S, W):
    L, D = 64, 8
    q, k, v = rnd(10, 1, L, D), rnd(11, 1, L, D), rnd(12, 1, L, D)
    og, lg = attention.attention_heads(q, k, v, np.array([GLOBAL]), 0, S, W)
    ol, ll = attention.attention_heads(q, k, v, np.array([LOCAL]), 0, S, W)
    np.testing.assert_array_equal(og, ol)
    np.testing.assert_array_equal(lg, ll)


def test_sink0_window1_closed_form():
    L, D = 30, 8
    q, k, v = rnd(13, 1, L, D), rnd(14, 1, L, D), rnd(15, 1, L, D)
    o, lse = attention.attention_heads(q, k, v, np.array([LOCAL]), 0, 0, 1)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    s_diag = np.einsum("id,id->i", q[0], k[0]) / math.sqrt(D)
    np.testing.assert_allclose(lse[0], s_diag, rtol=0, atol=1e-13)


def test_row0_attends_only_key0():
    L, D = 10, 8
    q, k, v = rnd(16, 2, L, D), rnd(17, 2, L, D), rnd(18, 2, L, D)
    o, _ = attention.attention_heads(q, k, v, np.array([GLOBAL, LOCAL]), 0, 2, 3)
    np.testing.assert_allclose(o[:, 0], v[:, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("cls,S,W", [(GLOBAL, 0, 1), (LOCAL, 3, 5), (LOCAL, 0, 4), (LOCAL, 7, 2)])
def test_identical_keys_give_mean_of_visible_values(cls, S, W):
    L, D = 25, 8
    q, v = rnd(19, 1, L, D), rnd(20, 1, L, D)
    k = np.tile(rnd(21, 1, 1, D), (1, L, 1))
    o, lse = attention.attention_heads(q, k, v, np.array([cls]), 0, S, W)
    for i in range(L):
        vis = [j for j in range(L) if j <= i and (cls == GLOBAL or j < S or j > i - W)]
        assert len(vis) == closed_form_count(cls, i, S, W)
        np.testing.assert_allclose(o[0, i], v[0, vis].mean(axis=0), rtol=0, atol=1e-13)
        s = q[0, i] @ k[0, 0] / math.sqrt(D)
        assert abs(lse[0, i] - (s + math.log(len(vis)))) < 1e-12


def test_gqa_equals_mha_with_replicated_kv_heads():
    G, Hkv, L, D = 3, 2, 33, 8
    q, k, v = rnd(22, G * Hkv, L, D), rnd(23, Hkv, L, D), rnd(24, Hkv, L, D)
    cls = np.array([GLOBAL, LOCAL])
    o1, l1 = attention.attention_heads(q, k, v, cls, 0, 2, 5)
    o2, l2 = attention.attention_heads(q, np.repeat(k, G, 0), np.repeat(v, G, 0), np.repeat(cls, G), 0, 2, 5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_chunked_queries_equal_single_shot_rows():
    H, L, D, qs = 2, 45, 8, 19
    q, k, v = rnd(25, H, L, D), rnd(26, H, L, D), rnd(27, H, L, D)
    cls = np.array([LOCAL, GLOBAL])
    o_full, l_full = attention.attention_heads(q, k, v, cls, 0, 3, 7)
    o_chunk, l_chunk = attention.attention_heads(q[:, qs:], k, v, cls, qs, 3, 7)
    np.testing.assert_array_equal(o_chunk, o_full[:, qs:])
    np.testing.assert_array_equal(l_chunk, l_full[:, qs:])


def test_brute_force_scalar_loops_tiny():
    """Second, loop-by-loop evaluation of the definition on a tiny case."""
    H, Hkv, L, D, S, W, qs = 4, 2, 9, 4, 2, 3, 2
    q, k, v = rnd(28, H, L - qs, D), rnd(29, Hkv, L, D), rnd(30, Hkv, L, D)
    cls = [LOCAL, GLOBAL]
    o, lse = attention.attention_heads(q, k, v, np.array(cls), qs, S, W, scale=0.37)
    for h in range(H):
        g = h // (H // Hkv)
        for t in range(L - qs):
            i = qs + t
            vis = [j for j in range(L) if j <= i and (cls[g] == GLOBAL or j < S or j > i - W)]
            sc = [0.37 * sum(q[h, t, d] * k[g, j, d] for d in range(D)) for j in vis]
            mx = max(sc)
            den = sum(math.exp(x - mx) for x in sc)
            assert abs(lse[h, t] - (mx + math.log(den))) < 1e-12
            for d in range(D):
                num = sum(math.exp(x - mx) * v[g, j, d] for x, j in zip(sc, vis))
                assert abs(o[h, t, d] - num / den) < 1e-12


def test_tiny_workload_pair_count_closed_form():
    """Tiny config: L=512, KV0 global, KV1 local (S=4, W=128), 2 q heads each -> 380,532 visible pairs."""
    L, S, W = 512, 4, 128
    cnt = 0
    for cls in (GLOBAL, LOCAL):
        m = attention.visibility_mask(cls, np.arange(L), L, S, W)
        assert m.sum() == sum(closed_form_count(cls, i, S, W) for i in range(L))
        cnt += 2 * int(m.sum())
    assert cnt == 380532


def test_row_without_visible_key_is_rejected():
    with pytest.raises(ValueError):
        attention.masked_attention(np.zeros((1, 2)), np.zeros((1, 2)), np.zeros((1, 2)),
                                   np.zeros((1, 1), bool), 1.0)
    with pytest.raises(ValueError):
        attention.visibility_mask(LOCAL, np.arange(3), 3, 0, 0)
