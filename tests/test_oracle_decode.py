"""Pins of the oracle's decode row and split-KV combine: torch's scaled_dot_product_attention with an
independent boolean mask, closed forms (one key; equal keys give uniform weights over the visible
count, counted from the sink/window definition by hand), and the combine's partition identity against
the unsplit row with scipy's logsumexp."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention, decode


def _case(rng, L, Hkv=2, G=3, D=16):
    q = rng.standard_normal((Hkv * G, D))
    k = [rng.standard_normal((L, D)) for _ in range(Hkv)]
    v = [rng.standard_normal((L, D)) for _ in range(Hkv)]
    return q, k, v


@pytest.mark.parametrize("seed", range(6))
def test_decode_step_matches_torch_sdpa(seed):
    rng = np.random.Generator(np.random.PCG64(6100 + seed))
    L = int(rng.integers(1, 90))
    S, W = int(rng.choice([0, 2, 7])), int(rng.choice([1, 5, 30]))
    cls = rng.integers(0, 2, size=2).astype(np.uint8)
    q, k, v = _case(rng, L)
    o, lse = decode.decode_step(q, k, v, cls, S, W)
    G = q.shape[0] // 2
    for h in range(q.shape[0]):
        g = h // G
        j = np.arange(L)
        vis = j <= L - 1
        if cls[g] == attention.LOCAL:
            vis = vis & ((j < S) | (j > L - 1 - W))
        qt = torch.from_numpy(q[h][None, None]).double()
        kt = torch.from_numpy(k[g][None]).double()
        vt = torch.from_numpy(v[g][None]).double()
        want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(vis)[None, None])
        np.testing.assert_allclose(o[h], want[0, 0].numpy(), rtol=1e-12, atol=1e-12)
        s = (q[h] @ k[g].T) / np.sqrt(q.shape[1])
        np.testing.assert_allclose(lse[h], logsumexp(s[vis]), rtol=1e-12, atol=1e-12)


def test_decode_step_single_key():
    rng = np.random.Generator(np.random.PCG64(6200))
    q, k, v = _case(rng, 1)
    o, lse = decode.decode_step(q, k, v, np.array([0, 1], np.uint8), 0, 1)
    G = q.shape[0] // 2
    for h in range(q.shape[0]):
        np.testing.assert_allclose(o[h], v[h // G][0], rtol=0, atol=1e-15)
        assert abs(lse[h] - q[h] @ k[h // G][0] / 4.0) < 1e-12


@pytest.mark.parametrize("L,S,W", [(100, 4, 16), (100, 0, 16), (19, 4, 16), (20, 4, 16), (21, 4, 16), (5, 4, 16),
                                   (100, 4, 1), (100, 30, 80)])
def test_decode_step_equal_keys_give_uniform_weights(L, S, W):
    # all keys equal: every visible key has the same weight, so o is the mean of the visible values and
    # lse = s + ln(n).  LOCAL: keys j < S or j > L - 1 - W, i.e. min(S, L) sink keys plus the last W
    # keys, counted once where they overlap; GLOBAL: all L keys.
    rng = np.random.Generator(np.random.PCG64(6300 + L + S + W))
    D = 8
    q = rng.standard_normal((2, D))
    kk = rng.standard_normal(D)
    k = [np.tile(kk, (L, 1)), np.tile(kk, (L, 1))]
    v = [rng.standard_normal((L, D)), rng.standard_normal((L, D))]
    o, lse = decode.decode_step(q, k, v, np.array([0, 1], np.uint8), S, W)
    last = list(range(max(0, L - W), L))
    local = sorted(set(range(min(S, L))) | set(last))
    for h, keys in ((0, local), (1, list(range(L)))):
        np.testing.assert_allclose(o[h], v[h][keys].mean(axis=0), rtol=1e-12, atol=1e-12)
        assert abs(lse[h] - (q[h] @ kk / np.sqrt(D) + np.log(len(keys)))) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_combine_of_a_partition_equals_the_unsplit_row(seed):
    rng = np.random.Generator(np.random.PCG64(6400 + seed))
    L, D = int(rng.integers(2, 300)), 16
    q = rng.standard_normal(D)
    k = rng.standard_normal((L, D)) * 2.0
    v = rng.standard_normal((L, D))
    s = k @ q / np.sqrt(D)
    cuts = sorted(set(rng.integers(1, L, size=int(rng.integers(1, 6))).tolist()))
    bounds = [0] + cuts + [L]
    o_parts, lse_parts = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        w = np.exp(s[a:b] - logsumexp(s[a:b]))
        o_parts.append(w @ v[a:b])
        lse_parts.append(logsumexp(s[a:b]))
    o, lse = decode.combine_partials(np.array(o_parts), np.array(lse_parts))
    w = np.exp(s - logsumexp(s))
    np.testing.assert_allclose(o, w @ v, rtol=1e-12, atol=1e-12)
    assert abs(lse - logsumexp(s)) < 1e-12
