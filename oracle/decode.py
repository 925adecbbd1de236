"""Decode over the retained segmented state, computed by the oracle.

After a prefill call the pool keeps, per (layer, KV head, sequence), what the next
query can see: every page of a GLOBAL head, the sink and recent-window pages of a
LOCAL head ([BJ] 二 ③; [SS] 核心特点: far more long-context sessions per GPU).  A
decode step adds one token per sequence; its query, at position L - 1 of the
L tokens now held, attends like any prefill row: masked softmax attention over
the visible keys (`attention.visibility_mask`, `attention.masked_attention`).

The split-KV combine (this library's decode runs the visible keys in parts and
merges them; the pages describe no decode kernel) is written out as its plain
definition: for parts s with normalised outputs o_s and log-sum-exps lse_s,
lse = log sum_s e^{lse_s} and o = sum_s e^{lse_s - lse} o_s.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import attention


def decode_step(q: np.ndarray, k_hist: Sequence[np.ndarray], v_hist: Sequence[np.ndarray], kv_class: np.ndarray,
                sink: int, window: int, scale: Optional[float] = None):
    """One sequence's decode row: o [H][D], lse [H] (fp64, natural log).

    q: [H][D] the new token's queries; k_hist[g], v_hist[g]: [L][D] the keys and values of KV head g
    for positions 0 .. L - 1, the new token's included; kv_class: [Hkv].  Query head h reads KV head
    h // (H / Hkv) and sees key j when j <= L - 1 and (GLOBAL, or j < sink, or j > L - 1 - window)."""
    q = np.asarray(q, np.float64)
    H, D = q.shape
    Hkv = len(k_hist)
    G = H // Hkv
    L = k_hist[0].shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros((H, D))
    lse = np.zeros(H)
    for h in range(H):
        g = h // G
        mask = attention.visibility_mask(int(kv_class[g]), np.array([L - 1]), L, sink, window)
        oh, lh = attention.masked_attention(q[h][None], k_hist[g], v_hist[g], mask, scale)
        o[h], lse[h] = oh[0], lh[0]
    return o, lse


def combine_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge S partial results of one row: o_parts [S][D] (each normalised over its own keys),
    lse_parts [S].  lse = log sum_s e^{lse_s}; o = sum_s e^{lse_s - lse} o_s."""
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    m = lse_parts.max()
    lse = m + np.log(np.exp(lse_parts - m).sum())
    w = np.exp(lse_parts - lse)
    return (w[:, None] * o_parts).sum(axis=0), lse
