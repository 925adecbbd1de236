"""One SegPagedAttention prefill call of a synthetic workload, computed by the oracle.

Data flow, as the pages describe it: reused document keys are rotated from
their offline to their actual position and stored in the request's cache ([SS]
技术原理 2; [AB] 使い方, BUILDSTATE and SELECTVISIBLESTATE items); the new tokens'
keys and values are written into the online cache; then global heads attend
over the full context and local heads over their paged sink + window KV ([AB]
使い方, EXECUTE item).  Here the cache is a dense [Hkv][L][D] array per
sequence, and attention is the dense masked definition of `attention`.

Head-ragged query ranges (EXECUTE's split, same item): a workload may give the
GLOBAL heads an earlier first query position than the LOCAL heads.  GLOBAL heads
then recompute those positions and write their new KV from there; LOCAL heads
keep the reused KV below their own start and query only from it.  A sequence's
packed rows begin at the earlier start.

The cache stores keys in the storage dtype, so a re-rotated key is rounded once
to that dtype before attention reads it (`round_store`).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import attention, rope

LOCAL, GLOBAL = 0, 1


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


# largest finite bfloat16: (2 - 2^-7) * 2^127
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values rounded once to bfloat16 (8 significant bits, the exponent range of fp32), to
    nearest with ties to even, returned as fp64.  Written from the format's definition: the value is
    scaled so that its bf16 quantum becomes 1, rounded half-to-even by np.rint, and scaled back (both
    scalings are exact powers of two).  Below 2^-126 the quantum stays 2^-133 (subnormals); past the
    largest finite value the result is +-inf."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                        # x = m 2^e with 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)               # exponent of the quantum: 8 significant bits
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    big = np.abs(y) > _BF16_MAX
    return np.where(big, np.copysign(np.inf, x), np.where(x == 0, x, y))


def round_store(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """fp64 values as the cache stores them: rounded once, to nearest even, to the storage dtype, and
    returned as fp64.  One rounding of the exact value (not fp64 -> fp32 -> bf16, which differs from it
    just above a bf16 tie)."""
    if dtype == torch.bfloat16:
        return round_bf16(x)
    if dtype == torch.float32:
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == torch.float64:
        return np.asarray(x, dtype=np.float64)
    raise ValueError("storage dtype %s" % dtype)


def _new_rows(inp, seq: int, kv_head: int):
    """(first position, fp64 K rows, fp64 V rows) that the call writes for one (sequence, KV head):
    from the head's class start to kv_len.  The packed rows of a sequence begin at q_begin."""
    wl = inp.wl
    cls = int(wl.head_class[wl.layer, kv_head])
    a, L = wl.q_start_of(seq, cls), wl.kv_lens[seq]
    cu = wl.cu_q()
    r0 = cu[seq] + (a - wl.q_begin(seq))
    return a, to64(inp.k_new[r0:cu[seq + 1], kv_head]), to64(inp.v_new[r0:cu[seq + 1], kv_head])


def head_kv(inp, seq: int, kv_head: int, rope_style: int = rope.ROTATE_HALF):
    """Dense fp64 K, V [kv_len][D] of one (sequence, KV head) after reuse import and append.

    Reused documents fill their token ranges with re-rotated keys; then the call's new keys and values
    overwrite the positions from the head's class start on.  Under EXECUTE's split ([AB] 使い方,
    EXECUTE item) a GLOBAL head recomputes from its own, earlier start and so writes the online KV
    there too, while a LOCAL head keeps the reused KV below its start."""
    wl = inp.wl
    L, D = wl.kv_lens[seq], wl.head_dim
    k = np.full((L, D), np.nan)
    v = np.full((L, D), np.nan)
    for doc in inp.docs:
        if doc.seq != seq:
            continue
        sl = slice(doc.tok_begin, doc.tok_begin + doc.n_tok)
        kk = rope.rotate(to64(doc.k_off[kv_head]), doc.delta, wl.rope_base, rope_style)
        k[sl] = round_store(kk, wl.dtype)
        v[sl] = to64(doc.v_off[kv_head])
    a, kn, vn = _new_rows(inp, seq, kv_head)
    k[a:L] = kn
    v[a:L] = vn
    if np.isnan(k).any() or np.isnan(v).any():
        raise ValueError("sequence %d has prefix tokens that no reused document covers" % seq)
    return k, v


def sequence_kv(inp, seq: int, rope_style: int = rope.ROTATE_HALF):
    """Dense fp64 K, V [Hkv][kv_len][D] of one sequence: `head_kv` for every KV head."""
    wl = inp.wl
    kv = [head_kv(inp, seq, g, rope_style) for g in range(wl.num_kv_heads)]
    return np.stack([x[0] for x in kv]), np.stack([x[1] for x in kv])


def prefill_seq(inp, seq: int, rows: Optional[Sequence[int]] = None, scale: Optional[float] = None,
                rope_style: int = rope.ROTATE_HALF):
    """o [H][n][D], lse [H][n] (fp64) for the given rows of the sequence's packed queries (row r is
    position q_begin + r).  A head computes the rows from its class start on; a LOCAL head's rows
    below its start (EXECUTE's split) are not part of the call and come back as NaN."""
    wl = inp.wl
    cu = wl.cu_q()
    k, v = sequence_kv(inp, seq, rope_style)
    q = to64(inp.q[cu[seq]:cu[seq + 1]]).transpose(1, 0, 2)
    n = q.shape[1]
    rows = np.arange(n) if rows is None else np.asarray(rows, np.int64)
    kv_class = wl.head_class[wl.layer]
    qb = wl.q_begin(seq)
    if scale is None:
        scale = 1.0 / np.sqrt(wl.head_dim)
    o = np.full((wl.num_q_heads, len(rows), wl.head_dim), np.nan)
    lse = np.full((wl.num_q_heads, len(rows)), np.nan)
    masks = {}
    for h in range(wl.num_q_heads):
        g = h // wl.group
        cls = int(kv_class[g])
        if cls not in masks:
            sel = np.nonzero(rows >= wl.q_start_of(seq, cls) - qb)[0]
            masks[cls] = (sel, attention.visibility_mask(cls, qb + rows[sel], wl.kv_lens[seq], wl.sink, wl.window))
        sel, mask = masks[cls]
        if len(sel):
            o[h, sel], lse[h, sel] = attention.masked_attention(q[h, rows[sel]], k[g], v[g], mask, scale)
    return o, lse


def prefill(inp, scale: Optional[float] = None, rope_style: int = rope.ROTATE_HALF):
    """The whole call: o [total_q][H][D] and lse [H][total_q], fp64 (NaN where a LOCAL head's rows
    precede its start)."""
    wl = inp.wl
    H, D = wl.num_q_heads, wl.head_dim
    o = np.full((wl.total_q, H, D), np.nan)
    lse = np.full((H, wl.total_q), np.nan)
    cu = wl.cu_q()
    for b in range(wl.num_seqs):
        if cu[b + 1] == cu[b]:
            continue
        ob, lb = prefill_seq(inp, b, None, scale, rope_style)
        o[cu[b]:cu[b + 1]] = ob.transpose(1, 0, 2)
        lse[:, cu[b]:cu[b + 1]] = lb
    return o, lse


def prefill_rows(inp, seq: int, q_head: int, rows, scale: Optional[float] = None,
                 rope_style: int = rope.ROTATE_HALF):
    """o [n][D], lse [n] (fp64) of one q head for the given packed rows of one sequence (rows at or
    after the head's class start)."""
    wl = inp.wl
    g = q_head // wl.group
    k, v = head_kv(inp, seq, g, rope_style)
    rows = np.asarray(rows, np.int64)
    cls = int(wl.head_class[wl.layer, g])
    if len(rows) and rows.min() < wl.q_start_of(seq, cls) - wl.q_begin(seq):
        raise ValueError("row before the head's class start")
    cu = wl.cu_q()
    q = to64(inp.q[cu[seq] + torch.from_numpy(rows).to(inp.q.device), q_head])
    if scale is None:
        scale = 1.0 / np.sqrt(wl.head_dim)
    mask = attention.visibility_mask(cls, wl.q_begin(seq) + rows, wl.kv_lens[seq], wl.sink, wl.window)
    return attention.masked_attention(q, k, v, mask, scale)


def kv_offsets(wl):
    """Start of each sequence's keys in the packed per-key output: cumulative kv_len."""
    out = [0]
    for L in wl.kv_lens:
        out.append(out[-1] + L)
    return out


def key_mass(inp, scale: Optional[float] = None, rope_style: int = rope.ROTATE_HALF):
    """Per-key attention mass: mass [H][sum kv_len] (fp64), mass[h][off_b + j] = the sum, over the call's
    queries i of head h (from its class start), of the attention weight p_ij of key j.

    This is the attention-score signal by which the pages route tokens: the dense FFN runs only on the
    top-k tokens by attention score, the rest take the residual path ([ZC] 事件内容, item 2; [SS]
    RedKnot技术原理, 3. 稀疏FFN动态调度).  Which statistic of the scores ranks a token is not stated;
    the plainest reading is the attention a token receives as a key, per head.  Each row of p sums
    to one, so a head's masses sum to its number of query rows."""
    wl = inp.wl
    if scale is None:
        scale = 1.0 / np.sqrt(wl.head_dim)
    off = kv_offsets(wl)
    mass = np.zeros((wl.num_q_heads, off[-1]))
    cu = wl.cu_q()
    kv_class = wl.head_class[wl.layer]
    for b in range(wl.num_seqs):
        L, qb = wl.kv_lens[b], wl.q_begin(b)
        q = to64(inp.q[cu[b]:cu[b + 1]])  # [rows][H][D]
        kv = [head_kv(inp, b, g, rope_style) for g in range(wl.num_kv_heads)]
        for h in range(wl.num_q_heads):
            g = h // wl.group
            cls = int(kv_class[g])
            a = wl.q_start_of(b, cls)
            if a >= L:
                continue
            pos = np.arange(a, L)
            p = attention.softmax_rows(q[a - qb:, h], kv[g][0], attention.visibility_mask(cls, pos, L, wl.sink,
                                                                                          wl.window), scale)
            mass[h, off[b]:off[b] + L] = p.sum(axis=0)
    return mass
