"""Seeded synthetic workloads: shapes, sizes and random draws only.

This module is shared by the fp64 oracle (tests) and the HIP path (tests, bench,
smoke).  It holds none of the method's arithmetic: no masks, no softmax, no
rotation, no paging.  It only says which sizes a workload has and draws its
random inputs from fixed seeds.

Shapes follow the workloads the RedKnot pages measure on: long-context QA/RAG
prefill from 2K to 128K tokens on GQA models with one global KV head in eight
(page "小红书把 KV Cache 按「头」拆了", section 事件内容, items 1 and 3: 12-15 %
global heads, 8K-128K contexts) and a DeepSeek-V4-Flash layer policy with
boundary layers fully global and 8 of 64 heads global in between (page
"为什么长上下文推理这么慢？RedKnot…", section 二 ①).  No dataset is used: every
value is N(0, 1) from a seeded generator, rounded once to the storage dtype.

Seed streams: seed = 10 * config_id + {0: q, 1: k, 2: v, 3: pool permutation,
4: class choice, 5: boosted key rows, 6: document offsets}.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

LOCAL = 0
GLOBAL = 1

SEED_Q, SEED_K, SEED_V, SEED_POOL, SEED_CLASS, SEED_BOOST, SEED_DOC = range(7)


@dataclasses.dataclass
class Workload:
    """One prefill call's sizes.  Heads are GQA-grouped: q head h reads KV head h // (H // Hkv)."""

    name: str
    config_id: int
    num_layers: int
    layer: int                    # the layer the call runs on
    kv_lens: List[int]            # per sequence, total context length after the call
    q_starts: List[int]           # per sequence, first query position (prefix below it is reused)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    sink: int
    window: int
    dtype: torch.dtype
    head_class: np.ndarray        # uint8 [num_layers][num_kv_heads], 0 LOCAL / 1 GLOBAL
    boost_frac: float = 0.0       # fraction of key rows per KV head multiplied by 4 (concentrated attention)
    doc_len: int = 0              # reused prefix is cut into documents of this many tokens (0: no reuse)
    rope_base: float = 1.0e6
    num_pages: int = 0            # pool size; 0 -> exactly what the call holds
    pool_slack: int = 0           # extra pages on top of what the call holds
    # per sequence, first query position of the GLOBAL heads (None: q_starts).  GLOBAL heads then
    # recompute queries from here while LOCAL heads query from q_starts (<= those, per sequence).
    q_starts_global: Optional[List[int]] = None

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_seqs(self) -> int:
        return len(self.kv_lens)

    def q_begin(self, seq: int) -> int:
        """First query position of the sequence's packed rows (the earlier of the two class starts)."""
        return self.q_starts[seq] if self.q_starts_global is None else self.q_starts_global[seq]

    def q_start_of(self, seq: int, cls: int) -> int:
        """First query position of a head of class cls."""
        return self.q_begin(seq) if cls == GLOBAL else self.q_starts[seq]

    @property
    def q_lens(self) -> List[int]:
        return [L - self.q_begin(b) for b, L in enumerate(self.kv_lens)]

    @property
    def total_q(self) -> int:
        return sum(self.q_lens)

    def cu_q(self) -> List[int]:
        out = [0]
        for n in self.q_lens:
            out.append(out[-1] + n)
        return out

    def seed(self, stream: int) -> int:
        return 10 * self.config_id + stream

    def with_classes(self, head_class: np.ndarray, name: Optional[str] = None) -> "Workload":
        return dataclasses.replace(self, head_class=np.ascontiguousarray(head_class, dtype=np.uint8),
                                   name=name or self.name)


def _class_map_one_global(num_layers: int, num_kv: int, seed: int) -> np.ndarray:
    """One seeded KV head per layer is global; the rest are local."""
    rng = np.random.Generator(np.random.PCG64(seed))
    hc = np.zeros((num_layers, num_kv), np.uint8)
    for l in range(num_layers):
        hc[l, rng.integers(0, num_kv)] = GLOBAL
    return hc


def _class_map_dsv4(seed: int) -> np.ndarray:
    """43 layers x 64 heads: layers 0-2 and 40-42 all global, 3-39 with a seeded 8 of 64 global."""
    rng = np.random.Generator(np.random.PCG64(seed))
    hc = np.zeros((43, 64), np.uint8)
    hc[:3] = GLOBAL
    hc[40:] = GLOBAL
    for l in range(3, 40):
        hc[l, rng.choice(64, size=8, replace=False)] = GLOBAL
    return hc


def tiny(dtype: torch.dtype = torch.bfloat16) -> Workload:
    """1 layer, B=1, L=512, 4 q heads / 2 KV heads, D=64; KV head 0 global, 1 local (sink 4, window 128); page 16."""
    return Workload(name="tiny L=512 4q/2kv D=64", config_id=1, num_layers=1, layer=0, kv_lens=[512],
                    q_starts=[0], num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, sink=4,
                    window=128, dtype=dtype, head_class=np.array([[GLOBAL, LOCAL]], np.uint8),
                    pool_slack=32)


def mistral7b() -> Workload:
    """B=4, L={2K,4K,6K,8K}, 32 q / 8 KV heads, D=128, bf16; 1 of 8 KV heads global; sink 4, window 1024; page 16."""
    return Workload(name="Mistral-7B-shaped 4 seqs 2K-8K 32q/8kv", config_id=2, num_layers=1, layer=0,
                    kv_lens=[2048, 4096, 6144, 8192], q_starts=[0, 0, 0, 0], num_q_heads=32, num_kv_heads=8,
                    head_dim=128, page_size=16, sink=4, window=1024, dtype=torch.bfloat16,
                    head_class=_class_map_one_global(1, 8, 10 * 2 + SEED_CLASS))


def llama70b(num_seqs: int = 31) -> Workload:
    """31 x 32K, 64 q / 8 KV heads, D=128, bf16; 1 global KV head; sink 4, window 2048; page 16."""
    return Workload(name="Llama-3.3-70B-shaped single-GPU share %d x 32K 64q/8kv" % num_seqs, config_id=3,
                    num_layers=1, layer=0, kv_lens=[32768] * num_seqs, q_starts=[0] * num_seqs,
                    num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=16, sink=4, window=2048,
                    dtype=torch.bfloat16, head_class=_class_map_one_global(1, 8, 10 * 3 + SEED_CLASS))


def qwen32b() -> Workload:
    """B=1, L=128K, 64 q / 8 KV heads, D=128, bf16; 1 global KV head; sink 4, window 4096; page 64; 5 % keys x4."""
    return Workload(name="Qwen3-32B-shaped 1 x 128K 64q/8kv", config_id=4, num_layers=1, layer=0,
                    kv_lens=[131072], q_starts=[0], num_q_heads=64, num_kv_heads=8, head_dim=128,
                    page_size=64, sink=4, window=4096, dtype=torch.bfloat16,
                    head_class=_class_map_one_global(1, 8, 10 * 4 + SEED_CLASS), boost_frac=0.05)


def dsv4flash(layer: int = 3) -> Workload:
    """43 layers, 64 heads (MHA), D=128, bf16, L=128K; prefix 120K reused (15 docs x 8K), 8K queries; page 64."""
    return Workload(name="DeepSeek-V4-Flash-style layer %d, 8K queries over 128K, 64 heads MHA" % layer,
                    config_id=5, num_layers=43, layer=layer, kv_lens=[131072], q_starts=[122880],
                    num_q_heads=64, num_kv_heads=64, head_dim=128, page_size=64, sink=4, window=4096,
                    dtype=torch.bfloat16, head_class=_class_map_dsv4(10 * 5 + SEED_CLASS), doc_len=8192)


def execute_split(wl: Workload, q_starts_global: Optional[Sequence[int]] = None, name: Optional[str] = None) -> Workload:
    """The same call with EXECUTE's head-ragged query ranges: GLOBAL heads recompute from
    q_starts_global (default 0: the whole prefix), LOCAL heads query from q_starts."""
    qg = [0] * wl.num_seqs if q_starts_global is None else [int(x) for x in q_starts_global]
    if any(g < 0 or g > s for g, s in zip(qg, wl.q_starts)):
        raise ValueError("need 0 <= q_start_global <= q_start")
    return dataclasses.replace(wl, q_starts_global=qg, name=name or wl.name + ", global heads recompute")


def dsv4flash_split(layer: int = 3) -> Workload:
    """DeepSeek-V4-Flash-style mixed layer under EXECUTE: the 8 GLOBAL heads recompute all 128K positions,
    the 56 LOCAL heads query the last 8K over their reused sink + window KV."""
    return execute_split(dsv4flash(layer), [0],
                         name="DeepSeek-V4-Flash-style layer %d, EXECUTE split: global heads 128K queries, "
                              "local heads 8K, 64 heads MHA" % layer)


CONFIGS = {"tiny": tiny, "mistral7b": mistral7b, "llama70b": llama70b, "qwen32b": qwen32b,
           "dsv4flash": dsv4flash, "dsv4flash_split": dsv4flash_split}


def random_small(seed: int, dtype: torch.dtype = torch.bfloat16, allow_reuse: bool = True) -> Workload:
    """Seeded random small shape: B in [1,4], L in [1,700], G in {1,2,4,8}, D in {64,128}, P in {16,32,64}."""
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    B = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 4))
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64]))
    kv_lens = [int(x) for x in rng.integers(1, 701, size=B)]
    q_starts = []
    for L in kv_lens:
        if allow_reuse and rng.random() < 0.4 and L > 1:
            q_starts.append(int(rng.integers(1, L)))
        else:
            q_starts.append(0)
    S = int(rng.choice([0, 1, 4, 17]))
    W = int(rng.choice([1, 16, 64, 100, 257, 1024]))
    hc = rng.integers(0, 2, size=(1, Hkv)).astype(np.uint8)
    doc_len = int(rng.choice([0, 50, 200]))  # 0: the prefix is one document with delta 0 (chunked prefill)
    return Workload(name="random-small seed %d" % seed, config_id=100 + seed, num_layers=1, layer=0,
                    kv_lens=kv_lens, q_starts=q_starts, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                    page_size=P, sink=S, window=W, dtype=dtype, head_class=hc, pool_slack=7, doc_len=doc_len,
                    rope_base=float(rng.choice([1.0e4, 1.0e6])))


def random_split(seed: int, dtype: torch.dtype = torch.bfloat16) -> Workload:
    """A random small shape with reuse and EXECUTE's head-ragged query ranges: every sequence has a
    reused prefix; GLOBAL heads recompute from 0 (most sequences) or from a point inside the prefix."""
    rng = np.random.Generator(np.random.PCG64(5000 + seed))
    wl = random_small(seed, dtype, allow_reuse=True)
    qs = [int(rng.integers(1, L)) if L > 1 else 0 for L in wl.kv_lens]
    qg = [0 if rng.random() < 0.7 or s == 0 else int(rng.integers(0, s + 1)) for s in qs]
    hc = wl.head_class.copy()
    if wl.num_kv_heads > 1:  # both classes present
        hc[0, 0], hc[0, 1] = GLOBAL, LOCAL
    wl = dataclasses.replace(wl, q_starts=qs, head_class=hc, name="random-split seed %d" % seed,
                             config_id=300 + seed)
    return execute_split(wl, qg, name=wl.name)


def random_many(seed: int, dtype: torch.dtype = torch.bfloat16) -> Workload:
    """Seeded random batch of many short sequences: B in [48, 96], L in [1, 700] (a third of them up to
    64 tokens, so one key tile), G in {4, 8}, Hkv in {2, 3}, D in {64, 128}, P in {8, 16, 64}, with
    reuse and both head classes: several hundred work items, so every attention workgroup runs a chain
    of items of every length, one-step items included."""
    rng = np.random.Generator(np.random.PCG64(9000 + seed))
    B = int(rng.integers(48, 97))
    G = int(rng.choice([4, 8]))
    Hkv = int(rng.integers(2, 4))
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([8, 16, 64]))
    kv_lens = [int(rng.integers(1, 65)) if rng.random() < 1 / 3 else int(rng.integers(65, 701)) for _ in range(B)]
    q_starts = [int(rng.integers(1, L)) if L > 1 and rng.random() < 0.3 else 0 for L in kv_lens]
    S = int(rng.choice([0, 4, 17]))
    W = int(rng.choice([16, 100, 257]))
    hc = np.zeros((1, Hkv), np.uint8)
    hc[0, int(rng.integers(0, Hkv))] = GLOBAL
    return Workload(name="random-many seed %d" % seed, config_id=600 + seed, num_layers=1, layer=0,
                    kv_lens=kv_lens, q_starts=q_starts, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                    page_size=P, sink=S, window=W, dtype=dtype, head_class=hc, pool_slack=7, doc_len=0)


# ----------------------------------------------------------------------------------------------
# random draws
# ----------------------------------------------------------------------------------------------

def _normal_host(seed: int, shape: Sequence[int]) -> torch.Tensor:
    rng = np.random.Generator(np.random.PCG64(seed))
    return torch.from_numpy(rng.standard_normal(size=tuple(shape), dtype=np.float32))


def _normal_dev(seed: int, shape: Sequence[int], device: torch.device, dtype: torch.dtype) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(tuple(shape), dtype=dtype, device=device)
    # draw in slabs so that fp32 temporaries stay small on 100+ GB inputs
    flat = out.view(-1)
    slab = 1 << 28
    for s in range(0, flat.numel(), slab):
        e = min(flat.numel(), s + slab)
        flat[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def normal(seed: int, shape: Sequence[int], dtype: torch.dtype, device: str | torch.device = "cpu") -> torch.Tensor:
    """N(0,1) draws rounded once to `dtype` (round-to-nearest-even).  CPU draws use numpy PCG64."""
    device = torch.device(device)
    if device.type == "cpu":
        return _normal_host(seed, shape).to(dtype)
    return _normal_dev(seed, shape, device, dtype)


def boosted_rows(wl: Workload, seq: int) -> np.ndarray:
    """bool [Hkv][kv_len]: for each KV head, floor(frac * L) key rows drawn without replacement."""
    L = wl.kv_lens[seq]
    out = np.zeros((wl.num_kv_heads, L), bool)
    if wl.boost_frac <= 0:
        return out
    rng = np.random.Generator(np.random.PCG64(wl.seed(SEED_BOOST) * 1000 + seq))
    n = int(np.floor(wl.boost_frac * L))
    for g in range(wl.num_kv_heads):
        out[g, rng.choice(L, size=n, replace=False)] = True
    return out


@dataclasses.dataclass
class Document:
    """A reused slice of a sequence's prefix: tokens [tok_begin, tok_begin + n_tok) whose keys were
    computed offline at positions starting at offline_start.  delta = tok_begin - offline_start."""

    seq: int
    tok_begin: int
    n_tok: int
    offline_start: int
    k_off: torch.Tensor   # [Hkv][n_tok][D] storage dtype, keys at their offline positions
    v_off: torch.Tensor   # [Hkv][n_tok][D]

    @property
    def delta(self) -> int:
        return self.tok_begin - self.offline_start


def document_layout(wl: Workload, seq: int) -> List[tuple]:
    """(tok_begin, n_tok, offline_start) for each reused document of a sequence's prefix [0, q_start)."""
    qs = wl.q_starts[seq]
    if qs == 0:
        return []
    dl = wl.doc_len if wl.doc_len > 0 else qs
    rng = np.random.Generator(np.random.PCG64(wl.seed(SEED_DOC) * 1000 + seq))
    out = []
    t = 0
    while t < qs:
        n = min(dl, qs - t)
        hi = max(0, wl.kv_lens[seq] - n)
        off = int(rng.integers(0, hi + 1)) if wl.doc_len > 0 else t
        out.append((t, n, off))
        t += n
    return out


@dataclasses.dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor        # [total_q][H][D]
    k_new: torch.Tensor    # [total_q][Hkv][D]
    v_new: torch.Tensor    # [total_q][Hkv][D]
    docs: List[Document]   # reused prefix documents (k_off/v_off already boosted where boosted)
    free_order: np.ndarray  # int32 permutation of the pool's pages
    boost: List[np.ndarray]  # per seq bool [Hkv][kv_len]


def decode_inputs(wl: Workload, step: int, rows: int, device: str | torch.device = "cpu"):
    """The new token of each decoding sequence at decode step `step`: q [rows][H][D], k, v
    [rows][Hkv][D], seeded normal draws in the workload's dtype."""
    base = wl.seed(SEED_Q) * 104729 + 7 * step
    q = normal(base + 1, (rows, wl.num_q_heads, wl.head_dim), wl.dtype, device)
    k = normal(base + 2, (rows, wl.num_kv_heads, wl.head_dim), wl.dtype, device)
    v = normal(base + 3, (rows, wl.num_kv_heads, wl.head_dim), wl.dtype, device)
    return q, k, v


def pool_pages_needed_hint(wl: Workload) -> int:
    """An upper bound on the pages one call holds: every (kv head, seq) holding its whole context."""
    P = wl.page_size
    return sum(wl.num_kv_heads * ((L + P - 1) // P) for L in wl.kv_lens)


def make_inputs(wl: Workload, device: str | torch.device = "cpu", num_pages: Optional[int] = None) -> Inputs:
    """Draw every input of one call.  Documents with offline offsets are drawn when q_start > 0."""
    H, Hkv, D = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    T = wl.total_q
    q = normal(wl.seed(SEED_Q), (T, H, D), wl.dtype, device)
    k_new = normal(wl.seed(SEED_K), (T, Hkv, D), wl.dtype, device)
    v_new = normal(wl.seed(SEED_V), (T, Hkv, D), wl.dtype, device)
    boost = [boosted_rows(wl, b) for b in range(wl.num_seqs)]
    cu = wl.cu_q()
    if wl.boost_frac > 0:
        for b in range(wl.num_seqs):
            qs = wl.q_begin(b)
            rows = torch.from_numpy(boost[b][:, qs:].T.copy()).to(k_new.device)  # [q_len][Hkv]
            blk = k_new[cu[b]:cu[b + 1]]
            blk[rows] = blk[rows] * 4
    docs = []
    for b in range(wl.num_seqs):
        for di, (t0, n, off) in enumerate(document_layout(wl, b)):
            s = 100000 * (b + 1) + di
            k_off = normal(wl.seed(SEED_K) * 7919 + s, (Hkv, n, D), wl.dtype, device)
            v_off = normal(wl.seed(SEED_V) * 7919 + s, (Hkv, n, D), wl.dtype, device)
            if wl.boost_frac > 0:
                rows = torch.from_numpy(boost[b][:, t0:t0 + n].copy()).to(k_off.device)
                k_off[rows] = k_off[rows] * 4
            docs.append(Document(b, t0, n, off, k_off, v_off))
    if num_pages is None:
        num_pages = wl.num_pages or (pool_pages_needed_hint(wl) + wl.pool_slack)
    rng = np.random.Generator(np.random.PCG64(wl.seed(SEED_POOL)))
    free_order = rng.permutation(num_pages).astype(np.int32)
    return Inputs(wl, q, k_new, v_new, docs, free_order, boost)
