"""Integer oracle: held tokens, page sets, allocator replay, visible intervals, pair counts.

SegPagedAttention organises KV pages per (layer, head, segment): global heads
read every context page, local heads physically store only sink plus recent
window pages ([BJ] 二 ③).  The storage is per (layer, head) ([SS] 技术原理 1),
pages sit in global/local pools by head ([AB] 使い方, BUILDSTATE item), and a
head only loads the tokens it needs ([SS] 技术原理 1, second item).

Readings where the pages are silent:
  * classes are per (layer, KV head);
  * a LOCAL head of a sequence with queries [q_start, kv_len) holds tokens
    [0, min(S, kv_len)) and [max(0, q_start - W + 1), kv_len) -- exactly the keys
    some query of the call can see; a GLOBAL head holds [0, kv_len);
  * held tokens are expanded to whole pages; page runs that overlap or touch merge;
  * allocator policy (ours, the pages give none): one free list seeded from the
    caller's permutation (or ascending ids); pages are taken from its head in
    ascending (layer, kv head, seq, logical page) order; freed pages are pushed on
    its head in ascending (layer, kv head, seq, logical page) order (LIFO reuse);
    a build that does not fit takes nothing (transactional);
  * trimming after the call keeps, for LOCAL heads, the sink pages and the pages
    covering [max(0, kv_len - W + 1), kv_len) -- what the next query would see;
  * the next call on the same sequences (decode) keeps every still-held page in
    place, frees the others first and then allocates the missing ones, both in the
    (layer, kv head, seq, logical page) order.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import collections
from typing import Dict, List, Sequence, Tuple

import numpy as np

LOCAL = 0
GLOBAL = 1


class OutOfPages(Exception):
    pass


def held_token_ranges(cls: int, q_start: int, kv_len: int, sink: int, window: int) -> List[Tuple[int, int]]:
    """Token ranges [a, b) a (layer, kv head, seq) holds during a call with queries [q_start, kv_len)."""
    if kv_len <= 0:
        return []
    if cls == GLOBAL:
        return [(0, kv_len)]
    out = []
    if sink > 0:
        out.append((0, min(sink, kv_len)))
    out.append((max(0, q_start - window + 1), kv_len))
    out = [r for r in out if r[1] > r[0]]
    merged: List[Tuple[int, int]] = []
    for a, b in sorted(out):
        if merged and a <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(merged[-1][1], b))
        else:
            merged.append((a, b))
    return merged


def pages_of_ranges(ranges: Sequence[Tuple[int, int]], page_size: int) -> List[int]:
    """Sorted logical pages that contain at least one token of the ranges."""
    pages = set()
    for a, b in ranges:
        pages.update(range(a // page_size, (b - 1) // page_size + 1))
    return sorted(pages)


def held_pages(cls: int, q_start: int, kv_len: int, sink: int, window: int, page_size: int) -> List[int]:
    return pages_of_ranges(held_token_ranges(cls, q_start, kv_len, sink, window), page_size)


def retained_pages(cls: int, kv_len: int, sink: int, window: int, page_size: int) -> List[int]:
    """Pages kept after the call: all for GLOBAL; sink + [kv_len - W + 1, kv_len) for LOCAL."""
    return held_pages(cls, kv_len, kv_len, sink, window, page_size) if cls == LOCAL else \
        held_pages(cls, 0, kv_len, sink, window, page_size)


def segments(pages: Sequence[int], page_size: int) -> List[Tuple[int, int, int]]:
    """Runs of consecutive logical pages as (tok_begin, n_pages, page_off)."""
    out: List[Tuple[int, int, int]] = []
    off = 0
    for p in pages:
        if out and p == out[-1][0] // page_size + out[-1][1]:
            t, n, o = out[-1]
            out[-1] = (t, n + 1, o)
        else:
            out.append((p * page_size, 1, off))
        off += 1
    return out


class PoolReplay:
    """Replays the allocator policy; tables map (layer, kv_head, seq) -> {logical page: physical id}."""

    def __init__(self, num_pages: int, free_order: Sequence[int] | None = None):
        self.num_pages = int(num_pages)
        order = list(range(num_pages)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_pages)):
            raise ValueError("free order must be a permutation of the pool's pages")
        self.free = collections.deque(order)

    @property
    def used(self) -> int:
        return self.num_pages - len(self.free)

    def build(self, layer_begin: int, layer_end: int, head_class: np.ndarray, q_starts: Sequence[int],
              kv_lens: Sequence[int], sink: int, window: int, page_size: int) -> Dict:
        plan = []
        for l in range(layer_begin, layer_end):
            for g in range(head_class.shape[1]):
                for b, (qs, L) in enumerate(zip(q_starts, kv_lens)):
                    plan.append(((l, g, b), held_pages(int(head_class[l, g]), qs, L, sink, window, page_size)))
        need = sum(len(p) for _, p in plan)
        if need > len(self.free):
            raise OutOfPages(need)
        tables = {}
        for key, pages in plan:
            tables[key] = {p: self.free.popleft() for p in pages}
        return tables

    def _push(self, page_ids: Sequence[int]) -> None:
        for pid in page_ids:
            self.free.appendleft(pid)

    def trim(self, tables: Dict, head_class: np.ndarray, kv_lens: Sequence[int], sink: int, window: int,
             page_size: int) -> Dict:
        freed = []
        out = {}
        for key in sorted(tables):
            l, g, b = key
            keep = set(retained_pages(int(head_class[l, g]), kv_lens[b], sink, window, page_size))
            t = tables[key]
            out[key] = {p: t[p] for p in sorted(t) if p in keep}
            freed.extend(t[p] for p in sorted(t) if p not in keep)
        self._push(freed)
        return out

    def advance(self, tables: Dict, head_class: np.ndarray, kv_lens: Sequence[int], n_new: Sequence[int], sink: int,
                window: int, page_size: int):
        """The next call on the same sequences (decode, or a further chunk): sequence b gains n_new[b]
        tokens, which are its queries, so q_start becomes the old kv_len.  Each (layer, kv head, seq)
        then holds held_pages(class, old kv_len, new kv_len); a logical page it held before keeps its
        physical page (and contents), the pages it no longer holds are freed first, the missing ones
        allocated after, both in ascending (layer, kv head, seq, logical page) order.  Transactional.
        Returns (tables, new kv_lens)."""
        new_kv = [int(L) + int(n) for L, n in zip(kv_lens, n_new)]
        plan = {}
        for key in sorted(tables):
            l, g, b = key
            plan[key] = held_pages(int(head_class[l, g]), int(kv_lens[b]), new_kv[b], sink, window, page_size)
        freed = [tables[key][p] for key in sorted(tables) for p in sorted(tables[key]) if p not in set(plan[key])]
        fresh = [(key, p) for key in sorted(plan) for p in plan[key] if p not in tables[key]]
        if len(fresh) > len(self.free) + len(freed):
            raise OutOfPages(len(fresh))
        self._push(freed)
        out = {key: {p: tables[key][p] for p in plan[key] if p in tables[key]} for key in plan}
        for key, p in fresh:
            out[key][p] = self.free.popleft()
        out = {key: dict(sorted(t.items())) for key, t in out.items()}
        return out, new_kv

    def release(self, tables: Dict) -> None:
        freed = []
        for key in sorted(tables):
            t = tables[key]
            freed.extend(t[p] for p in sorted(t))
        self._push(freed)


def visible_intervals(mask_row: np.ndarray) -> List[Tuple[int, int]]:
    """Runs [a, b) of visible keys in one mask row, found by scanning the row."""
    out = []
    j, L = 0, len(mask_row)
    while j < L:
        if mask_row[j]:
            a = j
            while j < L and mask_row[j]:
                j += 1
            out.append((a, j))
        else:
            j += 1
    return out


def pair_count(mask: np.ndarray) -> int:
    """Visible (query, key) pairs of one head, counted off the dense mask."""
    return int(np.count_nonzero(mask))
