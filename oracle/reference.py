"""One SegPagedAttention prefill call of a synthetic workload, computed by the oracle.

Data flow, as the pages describe it: reused document keys are rotated from
their offline to their actual position and stored in the request's cache ([SS]
技术原理 2; [AB] 使い方, BUILDSTATE and SELECTVISIBLESTATE items); the new tokens'
keys and values are written into the online cache; then global heads attend
over the full context and local heads over their paged sink + window KV ([AB]
使い方, EXECUTE item).  Here the cache is a dense [Hkv][L][D] array per
sequence, and attention is the dense masked definition of `attention`.

The cache stores keys in the storage dtype, so a re-rotated key is rounded once
to that dtype before attention reads it (`round_store`).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import attention, rope


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def round_store(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Round fp64 values to the cache's storage dtype (nearest-even) and back to fp64."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(dtype).to(torch.float64).numpy()


def rerotated_keys(doc, head_dim: int, base: float, style: int, dtype: Optional[torch.dtype]):
    """fp64 [Hkv][n][D] keys of one reused document at their actual positions."""
    k = rope.rotate(to64(doc.k_off), doc.delta, base, style)
    return round_store(k, dtype) if dtype is not None else k


def sequence_kv(inp, seq: int, rope_style: int = rope.ROTATE_HALF):
    """Dense fp64 K, V [Hkv][kv_len][D] of one sequence after reuse import and append."""
    wl = inp.wl
    L, qs = wl.kv_lens[seq], wl.q_starts[seq]
    Hkv, D = wl.num_kv_heads, wl.head_dim
    k = np.full((Hkv, L, D), np.nan)
    v = np.full((Hkv, L, D), np.nan)
    for doc in inp.docs:
        if doc.seq != seq:
            continue
        sl = slice(doc.tok_begin, doc.tok_begin + doc.n_tok)
        k[:, sl] = rerotated_keys(doc, D, wl.rope_base, rope_style, wl.dtype)
        v[:, sl] = to64(doc.v_off)
    cu = wl.cu_q()
    k[:, qs:L] = to64(inp.k_new[cu[seq]:cu[seq + 1]]).transpose(1, 0, 2)
    v[:, qs:L] = to64(inp.v_new[cu[seq]:cu[seq + 1]]).transpose(1, 0, 2)
    if np.isnan(k).any() or np.isnan(v).any():
        raise ValueError("sequence %d has prefix tokens that no reused document covers" % seq)
    return k, v


def prefill_seq(inp, seq: int, rows: Optional[Sequence[int]] = None, scale: Optional[float] = None,
                rope_style: int = rope.ROTATE_HALF):
    """o [H][n][D], lse [H][n] (fp64) for the given query rows (0-based within the sequence's queries)."""
    wl = inp.wl
    cu = wl.cu_q()
    k, v = sequence_kv(inp, seq, rope_style)
    q = to64(inp.q[cu[seq]:cu[seq + 1]]).transpose(1, 0, 2)
    kv_class = wl.head_class[wl.layer]
    return attention.attention_heads(q, k, v, kv_class, wl.q_starts[seq], wl.sink, wl.window, scale,
                                     None if rows is None else np.asarray(rows))


def prefill(inp, scale: Optional[float] = None, rope_style: int = rope.ROTATE_HALF):
    """The whole call: o [total_q][H][D] and lse [H][total_q], fp64."""
    wl = inp.wl
    H, D = wl.num_q_heads, wl.head_dim
    o = np.empty((wl.total_q, H, D))
    lse = np.empty((H, wl.total_q))
    cu = wl.cu_q()
    for b in range(wl.num_seqs):
        if cu[b + 1] == cu[b]:
            continue
        ob, lb = prefill_seq(inp, b, None, scale, rope_style)
        o[cu[b]:cu[b + 1]] = ob.transpose(1, 0, 2)
        lse[:, cu[b]:cu[b + 1]] = lb
    return o, lse


def head_kv(inp, seq: int, kv_head: int, rope_style: int = rope.ROTATE_HALF):
    """Dense fp64 K, V [kv_len][D] of one (sequence, KV head): the slice of `sequence_kv` for that head."""
    wl = inp.wl
    L, qs = wl.kv_lens[seq], wl.q_starts[seq]
    D = wl.head_dim
    k = np.full((L, D), np.nan)
    v = np.full((L, D), np.nan)
    for doc in inp.docs:
        if doc.seq != seq:
            continue
        sl = slice(doc.tok_begin, doc.tok_begin + doc.n_tok)
        kk = rope.rotate(to64(doc.k_off[kv_head]), doc.delta, wl.rope_base, rope_style)
        k[sl] = round_store(kk, wl.dtype)
        v[sl] = to64(doc.v_off[kv_head])
    cu = wl.cu_q()
    k[qs:L] = to64(inp.k_new[cu[seq]:cu[seq + 1], kv_head])
    v[qs:L] = to64(inp.v_new[cu[seq]:cu[seq + 1], kv_head])
    if np.isnan(k).any() or np.isnan(v).any():
        raise ValueError("sequence %d has prefix tokens that no reused document covers" % seq)
    return k, v


def prefill_rows(inp, seq: int, q_head: int, rows, scale: Optional[float] = None,
                 rope_style: int = rope.ROTATE_HALF):
    """o [n][D], lse [n] (fp64) of one q head for the given query rows of one sequence."""
    wl = inp.wl
    g = q_head // wl.group
    k, v = head_kv(inp, seq, g, rope_style)
    rows = np.asarray(rows, np.int64)
    cu = wl.cu_q()
    q = to64(inp.q[cu[seq] + torch.from_numpy(rows).to(inp.q.device), q_head])
    if scale is None:
        scale = 1.0 / np.sqrt(wl.head_dim)
    cls = int(wl.head_class[wl.layer, g])
    mask = attention.visibility_mask(cls, wl.q_starts[seq] + rows, wl.kv_lens[seq], wl.sink, wl.window)
    return attention.masked_attention(q, k, v, mask, scale)
