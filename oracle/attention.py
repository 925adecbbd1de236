"""Dense masked attention in fp64: the plain definition that SegPagedAttention reaches.

The pages state that today's KV cache is a dense [B, H, L, D] tensor in which
every head is stored, moved and computed together ([ZC] 事件内容; [AB] 技術原則,
first item), and that a token-level system expresses per-head sparsity with an
attn_mask on that dense layout ([AB] comparison table, rows on storage layout
and kernel efficiency).  SegPagedAttention gets the same result without
building a mask: global heads attend over the whole context, local heads only
over sink tokens plus a recent window ([BJ] 二 ③; [AB] 使い方, EXECUTE item).
So the oracle is that dense layout with an explicit per-head mask, in fp64.

Readings where the pages are silent (each is listed in the design notes):
  * window of W keys including the query itself: j in (i - W, i];
  * sink = the first S absolute token positions of the sequence;
  * causality is bottom-right aligned: a query at absolute position i sees j <= i;
  * classes are per (layer, KV head); q head h reads KV head h // G;
  * scale 1/sqrt(D), natural-log LSE.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

LOCAL = 0
GLOBAL = 1


def visibility_mask(head_class: int, q_pos: np.ndarray, kv_len: int, sink: int, window: int) -> np.ndarray:
    """bool [len(q_pos)][kv_len]: key j is visible to the query at absolute position i.

    Global heads see the full causal context; local heads see the sink tokens and
    the recent window ([BJ] 二 ③: global heads read every context page, local
    heads keep only sink plus recent-window pages; [SS] 核心特点 1: local heads
    only look at a local window).  M[i][j] = j <= i and (global or j < S or j > i - W).
    """
    if window < 1:
        raise ValueError("window must be >= 1")
    i = np.asarray(q_pos, dtype=np.int64)[:, None]
    j = np.arange(kv_len, dtype=np.int64)[None, :]
    causal = j <= i
    if head_class == GLOBAL:
        return causal
    return causal & ((j < sink) | (j > i - window))


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float):
    """One head: o, lse for fp64 q [n][D], k [L][D], v [L][D] and bool mask [n][L].

    s = scale * q k^T; lse_i = log sum_{visible j} exp(s_ij); p = mask * exp(s - lse); o = p v.
    Every row must have at least one visible key.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = scale * (q @ k.T)
    s_masked = np.where(mask, s, -np.inf)
    m = s_masked.max(axis=1)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key")
    lse = m + np.log(np.exp(s_masked - m[:, None]).sum(axis=1))
    p = np.where(mask, np.exp(s - lse[:, None]), 0.0)
    o = p @ v
    return o, lse


def attention_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_class: np.ndarray, q_start: int,
                    sink: int, window: int, scale: float | None = None, rows: np.ndarray | None = None):
    """One sequence, all heads.

    q: [H][n_q][D] for queries at absolute positions q_start .. q_start + n_q - 1
    k, v: [Hkv][L][D] with L = kv_len; kv_class: [Hkv] 0 LOCAL / 1 GLOBAL
    rows: optional subset of query indices (0-based within the call) to evaluate
    returns o [H][len(rows)][D] fp64, lse [H][len(rows)] fp64
    """
    H, n_q, D = q.shape
    Hkv, L, _ = k.shape
    G = H // Hkv
    if H != G * Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        rows = np.arange(n_q)
    rows = np.asarray(rows, np.int64)
    q_pos = q_start + rows
    o = np.empty((H, len(rows), D), np.float64)
    lse = np.empty((H, len(rows)), np.float64)
    masks = {}
    for h in range(H):
        g = h // G  # contiguous GQA groups
        c = int(kv_class[g])
        if c not in masks:
            masks[c] = visibility_mask(c, q_pos, L, sink, window)
        o[h], lse[h] = masked_attention(q[h, rows], k[g], v[g], masks[c], scale)
    return o, lse


def softmax_rows(q: np.ndarray, k: np.ndarray, mask: np.ndarray, scale: float) -> np.ndarray:
    """The normalised attention weights p [n][L] of one head (used by the row-sum invariant)."""
    s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    s_masked = np.where(mask, s, -np.inf)
    m = s_masked.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(s_masked - m), 0.0)
    return e / e.sum(axis=1, keepdims=True)
