"""ctypes binding of librk_seg.so.  Argument marshalling only: every step runs in the library.

Functions carry the names of the C entry points declared in include/rk_seg.h.  Device buffers are
torch tensors (used for device memory and streams only); the library reads and writes them through
their data pointers on the current HIP stream unless a stream is given.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# RK_SEG_LIB selects another build of the same library, e.g. the sanitizer build
# (`python -m head_aware_paged_prefill_amd.build --checked` -> librk_seg_checked.so)
LIB_PATH = os.environ.get("RK_SEG_LIB") or os.path.join(_HERE, "librk_seg.so")

RK_OK = 0
RK_ERR_INVALID_ARG = -1
RK_ERR_OUT_OF_PAGES = -2
RK_ERR_WORKSPACE_TOO_SMALL = -3
RK_ERR_UNSUPPORTED = -4
RK_ERR_HIP = -5
RK_ERR_STATE = -6
RK_ERR_INTERNAL = -7
RK_LOCAL, RK_GLOBAL = 0, 1
RK_BF16, RK_F32 = 0, 1
RK_ROPE_ROTATE_HALF, RK_ROPE_INTERLEAVED = 0, 1

# every function include/rk_seg.h declares
EXPORTS = [
    "rk_seg_pool_create", "rk_seg_pool_destroy", "rk_seg_pool_query", "rk_seg_pool_free_list",
    "rk_seg_tables_workspace_bytes", "rk_seg_build_tables", "rk_seg_tables_export", "rk_seg_tables_schedule",
    "rk_seg_tables_mass_schedule", "rk_seg_tables_stats", "rk_seg_tables_trim", "rk_seg_tables_destroy", "rk_seg_reuse_rerotate",
    "rk_seg_append_kv", "rk_seg_attn_prefill", "rk_seg_key_mass", "rk_seg_tables_advance_workspace_bytes",
    "rk_seg_tables_advance", "rk_seg_tables_decode_schedule", "rk_seg_attn_decode", "rk_seg_attn_decode_noalloc",
    "rk_seg_pack_ledger",
    "rk_seg_pack_pages", "rk_seg_unpack_pages", "rk_status_string",
    "rk_last_error", "rk_seg_version",
]


class RkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_status_name(status), msg))
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("initial_free_order", ctypes.POINTER(ctypes.c_int32))]


class BatchDesc(ctypes.Structure):
    _fields_ = [("layer_begin", ctypes.c_int32), ("layer_end", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("q_start", ctypes.POINTER(ctypes.c_int32)),
                ("kv_len", ctypes.POINTER(ctypes.c_int32)), ("head_class", ctypes.POINTER(ctypes.c_uint8)),
                ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("q_start_global", ctypes.POINTER(ctypes.c_int32))]


class TablesStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("pages_held", "total_q", "visible_pairs", "visible_pairs_global",
                                              "work_items", "key_tiles", "workspace_bytes")]


class PackLedger(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("pages", "pages_global", "pages_local", "packed_bytes", "tokens",
                                              "token_bytes", "dense_tokens", "dense_bytes")]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library; raises when it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("librk_seg.so not found at %s: build it with "
                           "`python -m head_aware_paged_prefill_amd.build`" % path)
    L = ctypes.CDLL(path)
    P, I32, I64, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "rk_seg_pool_create": [P(PoolDesc), P(VP)],
        "rk_seg_pool_destroy": [VP],
        "rk_seg_pool_query": [VP, P(I64), P(I64)],
        "rk_seg_pool_free_list": [VP, P(I32), I64, P(I64)],
        "rk_seg_tables_workspace_bytes": [VP, P(BatchDesc), P(ctypes.c_size_t)],
        "rk_seg_build_tables": [VP, P(BatchDesc), VP, ctypes.c_size_t, VP, P(VP)],
        "rk_seg_tables_export": [VP, I32, I32, I32, P(I32), P(I32), I32, P(I32), P(I32), I32, P(I32)],
        "rk_seg_tables_schedule": [VP, I32, P(I32), I64, P(I64), P(I32), P(I32)],
        "rk_seg_tables_mass_schedule": [VP, I32, P(I32), I64, P(I64), P(I32), P(I32), P(I32)],
        "rk_seg_tables_stats": [VP, P(TablesStats)],
        "rk_seg_tables_trim": [VP, VP],
        "rk_seg_tables_destroy": [VP, VP],
        "rk_seg_reuse_rerotate": [VP, VP, I32, I32, I32, I32, VP, VP, I64, I64, ctypes.c_double, I32, VP],
        "rk_seg_append_kv": [VP, VP, I32, VP, VP, VP],
        "rk_seg_attn_prefill": [VP, VP, I32, VP, VP, VP, VP, VP, ctypes.c_float, VP],
        "rk_seg_key_mass": [VP, VP, I32, VP, VP, VP, ctypes.c_float, VP],
        "rk_seg_tables_advance_workspace_bytes": [VP, VP, P(I32), P(ctypes.c_size_t)],
        "rk_seg_tables_advance": [VP, VP, P(I32), VP, ctypes.c_size_t, VP],
        "rk_seg_tables_decode_schedule": [VP, I32, P(I32), I64, P(I64), P(I32), I64],
        "rk_seg_attn_decode": [VP, VP, I32, VP, VP, VP, VP, VP, ctypes.c_float, VP],
        "rk_seg_attn_decode_noalloc": [VP, VP, I32, VP, VP, VP, VP, VP, ctypes.c_float, VP],
        "rk_seg_pack_ledger": [VP, I32, P(PackLedger)],
        "rk_seg_pack_pages": [VP, VP, I32, VP, ctypes.c_size_t, VP],
        "rk_seg_unpack_pages": [VP, VP, I32, VP, ctypes.c_size_t, VP],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = I32
    for name in ("rk_status_string",):
        getattr(L, name).argtypes = [I32]
        getattr(L, name).restype = ctypes.c_char_p
    for name in ("rk_last_error", "rk_seg_version"):
        getattr(L, name).argtypes = []
        getattr(L, name).restype = ctypes.c_char_p
    _lib = L
    return L


def _status_name(s: int) -> str:
    return load().rk_status_string(s).decode()


def _check(s: int) -> None:
    if s != RK_OK:
        raise RkError(s, load().rk_last_error().decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------------------------------------------
# pool
# ------------------------------------------------------------------------------------------------

class Pool:
    """A page pool: library handle plus the torch tensors that hold the pages.

    k_pages: [num_pages][page_size][head_dim]; v_pages: [num_pages][head_dim][page_size].
    """

    def __init__(self, handle: int, desc: PoolDesc, k_pages, v_pages):
        self.handle = handle
        self.desc = desc
        self.k_pages = k_pages
        self.v_pages = v_pages

    @property
    def num_pages(self) -> int:
        return int(self.desc.num_pages)


def rk_seg_pool_create(num_layers: int, num_kv_heads: int, head_dim: int, page_size: int, num_pages: int,
                       dtype: int, k_pages=None, v_pages=None, free_order: Optional[Sequence[int]] = None) -> Pool:
    """Create a pool over k_pages / v_pages (torch tensors of the documented layout; may be None when
    num_pages is 0 or for host-only use)."""
    L = load()
    d = PoolDesc(num_layers, num_kv_heads, head_dim, page_size, dtype, 0, num_pages, _ptr(k_pages), _ptr(v_pages),
                 None)
    fo = None
    if free_order is not None:
        fo = _i32(free_order)
        d.initial_free_order = fo.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    h = ctypes.c_void_p()
    _check(L.rk_seg_pool_create(ctypes.byref(d), ctypes.byref(h)))
    d.initial_free_order = None
    return Pool(h.value, d, k_pages, v_pages)


def rk_seg_pool_destroy(pool: Pool) -> None:
    _check(load().rk_seg_pool_destroy(pool.handle))
    pool.handle = None


def rk_seg_pool_query(pool: Pool) -> Tuple[int, int]:
    f, u = ctypes.c_int64(), ctypes.c_int64()
    _check(load().rk_seg_pool_query(pool.handle, ctypes.byref(f), ctypes.byref(u)))
    return f.value, u.value


def rk_seg_pool_free_list(pool: Pool) -> List[int]:
    n = ctypes.c_int64()
    _check(load().rk_seg_pool_free_list(pool.handle, None, 0, ctypes.byref(n)))
    out = np.empty(max(1, n.value), np.int32)
    _check(load().rk_seg_pool_free_list(pool.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value,
                                        ctypes.byref(n)))
    return out[:n.value].tolist()


# ------------------------------------------------------------------------------------------------
# tables
# ------------------------------------------------------------------------------------------------

class Tables:
    def __init__(self, handle: int, pool: Pool, batch_arrays, workspace):
        self.handle = handle
        self.pool = pool
        self._keep = batch_arrays
        self.workspace = workspace


def _batch(pool: Pool, layer_begin, layer_end, num_q_heads, q_start, kv_len, head_class, sink, window,
           q_start_global=None):
    qs, kl = _i32(q_start), _i32(kv_len)
    hc = np.ascontiguousarray(np.asarray(head_class, dtype=np.uint8).reshape(-1))
    qg = None if q_start_global is None else _i32(q_start_global)
    if qg is not None and len(qg) != len(qs):
        raise ValueError("q_start_global needs one entry per sequence")
    b = BatchDesc(layer_begin, layer_end, len(qs), num_q_heads,
                  qs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), kl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                  hc.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), sink, window,
                  None if qg is None else qg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return b, (qs, kl, hc, qg)


def rk_seg_tables_workspace_bytes(pool: Pool, layer_begin, layer_end, num_q_heads, q_start, kv_len, head_class,
                                  sink, window, q_start_global=None) -> int:
    b, keep = _batch(pool, layer_begin, layer_end, num_q_heads, q_start, kv_len, head_class, sink, window,
                     q_start_global)
    n = ctypes.c_size_t()
    _check(load().rk_seg_tables_workspace_bytes(pool.handle, ctypes.byref(b), ctypes.byref(n)))
    return n.value


def rk_seg_build_tables(pool: Pool, layer_begin: int, layer_end: int, num_q_heads: int, q_start, kv_len,
                        head_class, sink: int, window: int, device=True, workspace=None, stream=None,
                        q_start_global=None) -> Tables:
    """Build the tables; with device=True a uint8 workspace tensor is allocated on the current device
    (or `workspace` is used) and the tables are uploaded into it on the stream.  q_start_global
    (optional, per sequence, <= q_start): the GLOBAL heads' first query position."""
    b, keep = _batch(pool, layer_begin, layer_end, num_q_heads, q_start, kv_len, head_class, sink, window,
                     q_start_global)
    L = load()
    ws_ptr, ws_bytes, st = None, 0, None
    if device:
        import torch
        n = ctypes.c_size_t()
        _check(L.rk_seg_tables_workspace_bytes(pool.handle, ctypes.byref(b), ctypes.byref(n)))
        if workspace is None:
            workspace = torch.empty(max(256, n.value), dtype=torch.uint8, device="cuda")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        st = _stream(stream)
    h = ctypes.c_void_p()
    _check(L.rk_seg_build_tables(pool.handle, ctypes.byref(b), ws_ptr, ws_bytes, st, ctypes.byref(h)))
    return Tables(h.value, pool, keep, workspace)


def rk_seg_tables_export(tables: Tables, layer: int, kv_head: int, seq: int):
    """([(tok_begin, n_pages, page_off)], [physical page ids]) of one (layer, kv head, seq)."""
    L = load()
    ns, npg = ctypes.c_int32(), ctypes.c_int32()
    _check(L.rk_seg_tables_export(tables.handle, layer, kv_head, seq, None, None, 0, ctypes.byref(ns), None, 0,
                                  ctypes.byref(npg)))
    tb = np.zeros(max(1, ns.value), np.int32)
    sn = np.zeros(max(1, ns.value), np.int32)
    ids = np.zeros(max(1, npg.value), np.int32)
    P32 = ctypes.POINTER(ctypes.c_int32)
    _check(L.rk_seg_tables_export(tables.handle, layer, kv_head, seq, tb.ctypes.data_as(P32), sn.ctypes.data_as(P32),
                                  ns.value, ctypes.byref(ns), ids.ctypes.data_as(P32), npg.value, ctypes.byref(npg)))
    segs, off = [], 0
    for i in range(ns.value):
        segs.append((int(tb[i]), int(sn[i]), off))
        off += int(sn[i])
    return segs, ids[:npg.value].tolist()


def rk_seg_tables_schedule(tables: Tables, layer: int):
    """(items [n][4] = (seq, kv head, first query index, key tiles), tokens per item, key tile)."""
    L = load()
    n, T, BN = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
    _check(L.rk_seg_tables_schedule(tables.handle, layer, None, 0, ctypes.byref(n), ctypes.byref(T), ctypes.byref(BN)))
    out = np.zeros((max(1, n.value), 4), np.int32)
    _check(L.rk_seg_tables_schedule(tables.handle, layer, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value,
                                    ctypes.byref(n), ctypes.byref(T), ctypes.byref(BN)))
    return out[:n.value], T.value, BN.value


def rk_seg_tables_mass_schedule(tables: Tables, layer: int):
    """(units [n][4] = (seq, kv head, key block, query chunk), keys per unit, tokens per step, steps per
    query chunk)."""
    L = load()
    n, K, T, S = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(L.rk_seg_tables_mass_schedule(tables.handle, layer, None, 0, ctypes.byref(n), ctypes.byref(K),
                                         ctypes.byref(T), ctypes.byref(S)))
    out = np.zeros((max(1, n.value), 4), np.int32)
    _check(L.rk_seg_tables_mass_schedule(tables.handle, layer, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         n.value, ctypes.byref(n), ctypes.byref(K), ctypes.byref(T), ctypes.byref(S)))
    return out[:n.value], K.value, T.value, S.value


def rk_seg_tables_stats(tables: Tables) -> dict:
    s = TablesStats()
    _check(load().rk_seg_tables_stats(tables.handle, ctypes.byref(s)))
    return {f: int(getattr(s, f)) for f, _ in TablesStats._fields_}


def rk_seg_tables_trim(tables: Tables) -> None:
    _check(load().rk_seg_tables_trim(tables.pool.handle, tables.handle))


def rk_seg_tables_destroy(tables: Tables) -> None:
    _check(load().rk_seg_tables_destroy(tables.pool.handle, tables.handle))
    tables.handle = None


# ------------------------------------------------------------------------------------------------
# device calls
# ------------------------------------------------------------------------------------------------

def rk_seg_reuse_rerotate(tables: Tables, layer: int, seq: int, tok_begin: int, src_k, src_v, delta: int,
                          rope_base: float, rope_style: int = RK_ROPE_ROTATE_HALF, stream=None) -> None:
    """Import a reused document: src_k / src_v are [num_kv_heads][n_tok][head_dim] device tensors."""
    n_tok, D = int(src_k.shape[1]), int(src_k.shape[2])

    def head_stride(t):  # a size-1 head dimension may carry any stride
        return int(t.stride(0)) if t.shape[0] > 1 else n_tok * D
    stride = head_stride(src_k)
    rows_ok = all(t.stride(2) == 1 and (t.shape[1] <= 1 or t.stride(1) == D) for t in (src_k, src_v))
    if head_stride(src_v) != stride or not rows_ok or tuple(src_v.shape) != tuple(src_k.shape):
        raise ValueError("src_k / src_v need equal shapes and head strides and contiguous token rows")
    _check(load().rk_seg_reuse_rerotate(tables.pool.handle, tables.handle, layer, seq, tok_begin, n_tok,
                                        _ptr(src_k), _ptr(src_v), stride, int(delta), float(rope_base),
                                        int(rope_style), _stream(stream)))


def rk_seg_append_kv(tables: Tables, layer: int, k_new, v_new, stream=None) -> None:
    _check(load().rk_seg_append_kv(tables.pool.handle, tables.handle, layer, _ptr(k_new), _ptr(v_new),
                                   _stream(stream)))


def rk_seg_attn_prefill(tables: Tables, layer: int, q, k_new, v_new, o, lse=None, softmax_scale: float = 0.0,
                        stream=None) -> None:
    """Append (unless k_new and v_new are None) and attend.  q, o: [total_q][H][D]; lse: [H][total_q] fp32."""
    _check(load().rk_seg_attn_prefill(tables.pool.handle, tables.handle, layer, _ptr(q), _ptr(k_new), _ptr(v_new),
                                      _ptr(o), _ptr(lse), float(softmax_scale), _stream(stream)))


def rk_seg_key_mass(tables: Tables, layer: int, q, lse, mass, softmax_scale: float = 0.0, stream=None) -> None:
    """Per-key attention mass.  q: [total_q][H][D] as given to rk_seg_attn_prefill; lse: the [H][total_q]
    fp32 it returned; mass: [H][sum kv_len] fp32, written for every key."""
    _check(load().rk_seg_key_mass(tables.pool.handle, tables.handle, layer, _ptr(q), _ptr(lse), _ptr(mass),
                                  float(softmax_scale), _stream(stream)))


def rk_seg_tables_advance_workspace_bytes(tables: Tables, n_new) -> int:
    nn = _i32(n_new)
    n = ctypes.c_size_t()
    _check(load().rk_seg_tables_advance_workspace_bytes(tables.pool.handle, tables.handle,
                                                        nn.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                                        ctypes.byref(n)))
    return n.value


def rk_seg_tables_advance(tables: Tables, n_new, device=True, workspace=None, stream=None) -> Tables:
    """The next call on the same sequences: sequence b gains n_new[b] tokens (its query rows).  With
    device=True the device view goes into `workspace` (a uint8 tensor, reused when large enough) or
    into a new one.  Returns `tables` (the same handle)."""
    L = load()
    nn = _i32(n_new)
    pn = nn.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    ws_ptr, ws_bytes, st = None, 0, None
    if device:
        import torch
        need = rk_seg_tables_advance_workspace_bytes(tables, nn)
        if workspace is None:
            workspace = tables.workspace
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(max(256, need), dtype=torch.uint8, device="cuda")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        st = _stream(stream)
    _check(L.rk_seg_tables_advance(tables.pool.handle, tables.handle, pn, ws_ptr, ws_bytes, st))
    tables.workspace = workspace if device else None
    tables._keep = tables._keep + (nn,)
    return tables


def rk_seg_tables_decode_schedule(tables: Tables, layer: int):
    """(items [n][4] = (seq, kv head, k0, k1), comb_off [num_seqs * Hkv + 1] or None when not decode-shaped)."""
    L = load()
    n = ctypes.c_int64()
    _check(L.rk_seg_tables_decode_schedule(tables.handle, layer, None, 0, ctypes.byref(n), None, 0))
    if n.value == 0:
        return np.zeros((0, 4), np.int32), None
    nb = int(tables.pool.desc.num_kv_heads) * len(tables._keep[0]) + 1
    out = np.zeros((n.value, 4), np.int32)
    comb = np.zeros(nb, np.int32)
    _check(L.rk_seg_tables_decode_schedule(tables.handle, layer, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                           n.value, ctypes.byref(n), comb.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                           nb))
    return out, comb


def rk_seg_attn_decode(tables: Tables, layer: int, q, k_new, v_new, o, lse=None, softmax_scale: float = 0.0,
                       stream=None) -> None:
    """Decode: append (unless k_new and v_new are None), split-KV attention and combine.  q, o:
    [total_q][H][D] bf16 (one row per sequence with a query); lse: [H][total_q] fp32."""
    _check(load().rk_seg_attn_decode(tables.pool.handle, tables.handle, layer, _ptr(q), _ptr(k_new), _ptr(v_new),
                                     _ptr(o), _ptr(lse), float(softmax_scale), _stream(stream)))


RK_DECODE_SCRATCH_BYTES = 32 << 20  # the static partials array of rk_seg_attn_decode_noalloc, per GPU


def rk_seg_attn_decode_noalloc(tables: Tables, layer: int, q, k_new, v_new, o, lse=None, softmax_scale: float = 0.0,
                               stream=None) -> None:
    """rk_seg_attn_decode with its partials in the library's static per-GPU array: allocates nothing.
    Calls on one GPU that overlap in time race on that array."""
    _check(load().rk_seg_attn_decode_noalloc(tables.pool.handle, tables.handle, layer, _ptr(q), _ptr(k_new),
                                             _ptr(v_new), _ptr(o), _ptr(lse), float(softmax_scale), _stream(stream)))


def rk_seg_pack_ledger(tables: Tables, seq: int = -1) -> dict:
    """Byte ledger of sequence `seq` (-1: all) of the tables' current state."""
    out = PackLedger()
    _check(load().rk_seg_pack_ledger(tables.handle, seq, ctypes.byref(out)))
    return {f: int(getattr(out, f)) for f, _ in PackLedger._fields_}


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def rk_seg_pack_pages(tables: Tables, seq: int, dst, stream=None) -> None:
    """Copy the held pages of `seq` (-1: all) into the device tensor dst (>= the ledger's packed_bytes)."""
    _check(load().rk_seg_pack_pages(tables.pool.handle, tables.handle, seq, _ptr(dst), _nbytes(dst), _stream(stream)))


def rk_seg_unpack_pages(tables: Tables, seq: int, src, stream=None) -> None:
    """Write the packed pages in the device tensor src (exactly the ledger's packed_bytes) into the
    held pages of `seq` (-1: all) of these tables."""
    _check(load().rk_seg_unpack_pages(tables.pool.handle, tables.handle, seq, _ptr(src), _nbytes(src), _stream(stream)))


def rk_status_string(status: int) -> str:
    """The status code's name, as the library spells it."""
    return _status_name(status)


def rk_last_error() -> str:
    """The calling thread's message for its last failed call (empty if none failed)."""
    return load().rk_last_error().decode()


def rk_seg_version() -> str:
    return load().rk_seg_version().decode()
