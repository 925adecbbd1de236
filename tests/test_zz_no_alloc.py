"""rk_seg_attn_decode_noalloc (the decode variant whose split-KV partials live in the library's static
per-GPU array, for callers that cannot allocate) against rk_seg_attn_decode, through the C ABI.

Both run the same kernels over the same items, so their outputs must agree bit for bit.  Two calls in
a row, the second smaller than the first, show that a call does not depend on what an earlier call
left in the shared array.  A call whose partials exceed the array is rejected before it appends."""
import numpy as np
import pytest
import torch

import workloads
from head_aware_paged_prefill_amd import rk_seg
from head_aware_paged_prefill_amd.runner import PrefillRunner

from test_gpu_parity import say, to_dev

pytestmark = pytest.mark.gpu


def _partial_bytes(tables, layer, G, D):
    items, _ = rk_seg.rk_seg_tables_decode_schedule(tables, layer)
    slots = len(items) // 4
    return (slots * G * D * 4 + 255) // 256 * 256 + slots * G * 4


def _noalloc_matches_decode(wl, what):
    B, H, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    inp = workloads.make_inputs(wl, num_pages=workloads.pool_pages_needed_hint(wl) + wl.pool_slack
                                + 4 * B * wl.num_kv_heads)
    dinp = to_dev(inp)
    r = PrefillRunner(wl, free_order=inp.free_order, poison=True)
    try:
        r.build()
        r.import_docs(dinp.docs)
        r.attend(dinp.q, dinp.k_new, dinp.v_new)
        r.trim()
        r.advance([1] * B)
        need = _partial_bytes(r.tables, wl.layer, wl.group, D)
        say("%s: B=%d H=%d Hkv=%d D=%d partials %d bytes" % (what, B, H, wl.num_kv_heads, D, need))
        assert need <= rk_seg.RK_DECODE_SCRATCH_BYTES
        q, k, v = (t.cuda() for t in workloads.decode_inputs(wl, 0, B))
        o1 = torch.full((B, H, D), float("nan"), dtype=wl.dtype, device="cuda")
        l1 = torch.full((H, B), float("nan"), dtype=torch.float32, device="cuda")
        o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
        # the variant appends the new token itself; the existing entry point then reads the same state
        rk_seg.rk_seg_attn_decode_noalloc(r.tables, wl.layer, q, k, v, o1, l1)
        rk_seg.rk_seg_attn_decode(r.tables, wl.layer, q, None, None, o2, l2)
        torch.cuda.synchronize()
        assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all(), what
        assert torch.equal(o1, o2), "%s: outputs differ" % what
        assert torch.equal(l1, l2), "%s: lse differs" % what
        return need
    finally:
        r.close()


def test_noalloc_decode_matches_decode_on_two_calls_the_second_smaller():
    big = workloads.Workload(name="noalloc 2 x ~6K 32q/4kv D=128", config_id=411, num_layers=1, layer=0,
                             kv_lens=[6000, 4111], q_starts=[0, 3000], num_q_heads=32, num_kv_heads=4,
                             head_dim=128, page_size=16, sink=4, window=700, dtype=torch.bfloat16,
                             head_class=np.array([[1, 0, 0, 1]], np.uint8), pool_slack=7, doc_len=1000,
                             rope_base=1.0e4)
    n1 = _noalloc_matches_decode(big, big.name)
    small = workloads.random_small(5, torch.bfloat16)
    n2 = _noalloc_matches_decode(small, "noalloc " + small.name)
    assert n2 < n1


def test_noalloc_decode_rejects_partials_beyond_the_static_array():
    # 1024 sequences x 8 KV heads x 16 q heads per KV head: one workgroup of partials per (seq, kv head),
    # 8192 x (16 x 128 + 16) x 4 bytes > 32 MiB
    B, Hkv, G, D, P = 1024, 8, 16, 128, 16
    num_pages = B * Hkv
    say("noalloc oversize: B=%d Hkv=%d G=%d D=%d" % (B, Hkv, G, D))
    k_pages = torch.zeros((num_pages, P, D), dtype=torch.bfloat16, device="cuda")
    v_pages = torch.zeros((num_pages, D, P), dtype=torch.bfloat16, device="cuda")
    pool = rk_seg.rk_seg_pool_create(1, Hkv, D, P, num_pages, rk_seg.RK_BF16, k_pages, v_pages)
    tables = None
    try:
        tables = rk_seg.rk_seg_build_tables(pool, 0, 1, G * Hkv, [P - 1] * B, [P] * B, np.ones((1, Hkv), np.uint8),
                                            4, 64)
        assert _partial_bytes(tables, 0, G, D) > rk_seg.RK_DECODE_SCRATCH_BYTES
        q = torch.ones((B, G * Hkv, D), dtype=torch.bfloat16, device="cuda")
        k = torch.ones((B, Hkv, D), dtype=torch.bfloat16, device="cuda")
        o = torch.empty_like(q)
        with pytest.raises(rk_seg.RkError) as ei:
            rk_seg.rk_seg_attn_decode_noalloc(tables, 0, q, k, k, o)
        assert ei.value.status == rk_seg.RK_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert not k_pages.any() and not v_pages.any(), "a rejected call appended"
    finally:
        if tables is not None:
            rk_seg.rk_seg_tables_destroy(tables)
        rk_seg.rk_seg_pool_destroy(pool)
