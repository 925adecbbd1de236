"""Drive one SegPagedAttention prefill call through the C ABI.

A call is: build tables (classes, held pages, allocation, schedule, upload) -> import the reused
documents with RoPE re-rotation -> append the new tokens' K/V and attend -> trim local heads to
sink + window -> destroy.  Device buffers are torch tensors; every step runs in librk_seg.so.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import rk_seg

_DT = {torch.bfloat16: rk_seg.RK_BF16, torch.float32: rk_seg.RK_F32}


def pages_needed(wl) -> int:
    """Pages one call of the workload holds (upper bound: every (kv head, seq) holding all of its context)."""
    P = wl.page_size
    return sum(wl.num_kv_heads * ((L + P - 1) // P) for L in wl.kv_lens)


class PrefillRunner:
    """Owns a pool sized for a workload's call and runs the call's steps."""

    def __init__(self, wl, free_order=None, num_pages: Optional[int] = None, poison: bool = True,
                 device: str = "cuda"):
        self.wl = wl
        self.device = device
        n = num_pages if num_pages is not None else (len(free_order) if free_order is not None else pages_needed(wl))
        self.num_pages = int(n)
        dt = wl.dtype
        self.k_pages = torch.empty((self.num_pages, wl.page_size, wl.head_dim), dtype=dt, device=device)
        self.v_pages = torch.empty((self.num_pages, wl.head_dim, wl.page_size), dtype=dt, device=device)
        if poison:  # slots nobody writes must never reach the output
            self.k_pages.fill_(float("nan"))
            self.v_pages.fill_(float("nan"))
        self.pool = rk_seg.rk_seg_pool_create(wl.num_layers, wl.num_kv_heads, wl.head_dim, wl.page_size,
                                              self.num_pages, _DT[dt], self.k_pages, self.v_pages, free_order)
        self.tables = None
        self.workspace = None

    def build(self, layer_begin: Optional[int] = None, layer_end: Optional[int] = None, stream=None):
        wl = self.wl
        lb = wl.layer if layer_begin is None else layer_begin
        le = lb + 1 if layer_end is None else layer_end
        if self.workspace is None:
            nbytes = rk_seg.rk_seg_tables_workspace_bytes(self.pool, lb, le, wl.num_q_heads, wl.q_starts, wl.kv_lens,
                                                          wl.head_class, wl.sink, wl.window, wl.q_starts_global)
            self.workspace = torch.empty(max(256, nbytes), dtype=torch.uint8, device=self.device)
        self.tables = rk_seg.rk_seg_build_tables(self.pool, lb, le, wl.num_q_heads, wl.q_starts, wl.kv_lens,
                                                 wl.head_class, wl.sink, wl.window, device=True,
                                                 workspace=self.workspace, stream=stream,
                                                 q_start_global=wl.q_starts_global)
        return self.tables

    def import_docs(self, docs, layer: Optional[int] = None, rope_style: int = rk_seg.RK_ROPE_ROTATE_HALF, stream=None):
        layer = self.wl.layer if layer is None else layer
        for d in docs:
            rk_seg.rk_seg_reuse_rerotate(self.tables, layer, d.seq, d.tok_begin, d.k_off, d.v_off, d.delta,
                                         self.wl.rope_base, rope_style, stream)

    def attend(self, q, k_new, v_new, o=None, lse=None, layer: Optional[int] = None, scale: float = 0.0,
               stream=None):
        wl = self.wl
        layer = wl.layer if layer is None else layer
        if o is None:
            o = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=wl.dtype, device=self.device)
        if lse is None:
            lse = torch.empty((wl.num_q_heads, wl.total_q), dtype=torch.float32, device=self.device)
        rk_seg.rk_seg_attn_prefill(self.tables, layer, q, k_new, v_new, o, lse, scale, stream)
        return o, lse

    def key_mass(self, q, lse, mass=None, layer: Optional[int] = None, scale: float = 0.0, stream=None):
        """Per-key attention mass [H][sum kv_len] fp32 of the call attended last (same q, its lse)."""
        wl = self.wl
        layer = wl.layer if layer is None else layer
        if mass is None:
            mass = torch.empty((wl.num_q_heads, sum(wl.kv_lens)), dtype=torch.float32, device=self.device)
        rk_seg.rk_seg_key_mass(self.tables, layer, q, lse, mass, scale, stream)
        return mass

    def trim(self):
        """After the call: LOCAL heads keep only what the next query sees (sink + window pages)."""
        rk_seg.rk_seg_tables_trim(self.tables)

    def advance(self, n_new, stream=None):
        """The next call on the same sequences: sequence b gains n_new[b] tokens (its queries).  The
        device view is rebuilt in the runner's workspace (grown when it is too small)."""
        rk_seg.rk_seg_tables_advance(self.tables, n_new, device=True, workspace=self.workspace, stream=stream)
        self.workspace = self.tables.workspace
        return self.tables

    def decode(self, q, k_new, v_new, o=None, lse=None, layer: Optional[int] = None, scale: float = 0.0,
               stream=None):
        """Decode on decode-shaped tables: q, k_new, v_new one row per sequence with a query
        ([rows][H][D], [rows][Hkv][D]); returns o [rows][H][D] and lse [H][rows]."""
        wl = self.wl
        layer = wl.layer if layer is None else layer
        rows = q.shape[0]
        if o is None:
            o = torch.empty((rows, wl.num_q_heads, wl.head_dim), dtype=wl.dtype, device=self.device)
        if lse is None:
            lse = torch.empty((wl.num_q_heads, rows), dtype=torch.float32, device=self.device)
        rk_seg.rk_seg_attn_decode(self.tables, layer, q, k_new, v_new, o, lse, scale, stream)
        return o, lse

    def release(self, trim: bool = True):
        if self.tables is not None:
            if trim:
                rk_seg.rk_seg_tables_trim(self.tables)
            rk_seg.rk_seg_tables_destroy(self.tables)
            self.tables = None

    def close(self):
        self.release(trim=False)
        if self.pool is not None and self.pool.handle is not None:
            rk_seg.rk_seg_pool_destroy(self.pool)
        self.pool = None

    def page_contents(self, layer: int, kv_head: int, seq: int):
        """(K [n_tok][D], V [n_tok][D]) of a (layer, kv head, seq)'s held pages, token-major, on the host,
        together with the token index of each row."""
        segs, ids = rk_seg.rk_seg_tables_export(self.tables, layer, kv_head, seq)
        P = self.wl.page_size
        ids_t = torch.tensor(ids, dtype=torch.long, device=self.k_pages.device)
        k = self.k_pages.index_select(0, ids_t).cpu()                     # [n][P][D]
        v = self.v_pages.index_select(0, ids_t).cpu().transpose(1, 2)     # [n][P][D]
        toks = []
        for tb, npg, off in segs:
            toks.extend(range(tb, tb + npg * P))
        return k.reshape(-1, self.wl.head_dim), v.reshape(-1, self.wl.head_dim), toks
