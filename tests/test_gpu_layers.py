"""One tables object over several layers (rk_seg_build_tables over [layer_begin, layer_end)), each layer with
its own head classes and its own q/k/v: the prefill call and the per-key mass of every layer against the fp64
oracle, then trim, one token per sequence (rk_seg_tables_advance, all layers at once) and a decode step of every
layer against the oracle's decode row.  A layer that reads another layer's pages or classes fails (page "小红书
把 KV Cache 按「头」拆了…" (zhichai.net), section 事件内容: the cache is paged per (layer, head)).  Bars: the
attention parity bars; the mass within 2e-3 * max(1, mass) (the GPU's own lse)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from head_aware_paged_prefill_amd.runner import PrefillRunner
from oracle import decode, reference

from test_gpu_parity import check, say, to_dev

pytestmark = pytest.mark.gpu

NL = 3


def _layer_inputs(base, pages):
    # each layer its own draw (config id per layer) and its own row of the class map
    return [workloads.make_inputs(dataclasses.replace(base, layer=l, config_id=base.config_id + l), num_pages=pages)
            for l in range(NL)]


def test_three_layers_one_tables_prefill_then_decode():
    base = workloads.Workload(name="3 layers", config_id=450, num_layers=NL, layer=0, kv_lens=[420, 130],
                              q_starts=[0, 60], num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16, sink=4,
                              window=96, dtype=torch.bfloat16,
                              head_class=np.array([[1, 0], [0, 0], [1, 1]], np.uint8), pool_slack=7, doc_len=50,
                              rope_base=1.0e4)
    B, H, Hkv, D = base.num_seqs, base.num_q_heads, base.num_kv_heads, base.head_dim
    pages = NL * (workloads.pool_pages_needed_hint(base) + 2 * B * Hkv) + base.pool_slack
    inps = _layer_inputs(base, pages)
    say("3 layers: kv_lens=%s q_starts=%s classes=%s" % (base.kv_lens, base.q_starts, base.head_class.tolist()))
    r = PrefillRunner(base, free_order=inps[0].free_order, poison=True)
    try:
        r.build(0, NL)
        outs = []
        for l in range(NL):
            d = to_dev(inps[l])
            r.import_docs(d.docs, layer=l)
            outs.append(r.attend(d.q, d.k_new, d.v_new, layer=l))
        # the per-key mass of every layer, over that layer's call (its q and the GPU's lse)
        masses = [r.key_mass(to_dev(inps[l]).q, outs[l][1], layer=l) for l in range(NL)]
        torch.cuda.synchronize()
        for l in range(NL):
            o_ref, lse_ref = reference.prefill(inps[l])
            check(outs[l][0], outs[l][1], o_ref, lse_ref, base.dtype, "layer %d prefill" % l)
            want = reference.key_mass(inps[l])
            got = masses[l].double().cpu().numpy()
            err = np.abs(got - want) / np.maximum(1.0, np.abs(want))
            assert err.max() <= 2e-3, "layer %d mass: err %.3g (relative, absolute below 1)" % (l, err.max())
        r.trim()
        r.advance([1] * B)
        for l in range(NL):
            wl_l = inps[l].wl
            q, k, v = workloads.decode_inputs(wl_l, l, B)
            o, lse = r.decode(q.cuda(), k.cuda(), v.cuda(), layer=l)
            torch.cuda.synchronize()
            o_ref = np.zeros((B, H, D))
            lse_ref = np.zeros((H, B))
            for b in range(B):
                ks, vs = [], []
                for g in range(Hkv):
                    kh, vh = reference.head_kv(inps[l], b, g)
                    ks.append(np.vstack([kh, k[b, g].double().numpy()[None]]))
                    vs.append(np.vstack([vh, v[b, g].double().numpy()[None]]))
                o_ref[b], lse_ref[:, b] = decode.decode_step(q[b].double().numpy(), ks, vs, base.head_class[l],
                                                             base.sink, base.window)
            check(o, lse, o_ref, lse_ref, base.dtype, "layer %d decode" % l)
    finally:
        r.close()


def test_the_call_on_a_side_stream():
    # every step of the call enqueued on a non-default stream (torch's current stream inside the block):
    # the tables upload, the reuse import, the append and attention, the mass pass; only that stream is
    # synchronised before the outputs are read
    wl = workloads.random_small(3, torch.bfloat16)
    inp = workloads.make_inputs(wl)
    say("side stream: kv_lens=%s q_starts=%s" % (wl.kv_lens, wl.q_starts))
    o_ref, lse_ref = reference.prefill(inp)
    want = reference.key_mass(inp)
    dinp = to_dev(inp)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        r = PrefillRunner(wl, free_order=inp.free_order, poison=True)
        try:
            r.build()
            r.import_docs(dinp.docs)
            o, lse = r.attend(dinp.q, dinp.k_new, dinp.v_new)
            mass = r.key_mass(dinp.q, lse)
            s.synchronize()
            check(o, lse, o_ref, lse_ref, wl.dtype, "side stream")
            got = mass.double().cpu().numpy()
            err = np.abs(got - want) / np.maximum(1.0, np.abs(want))
            assert err.max() <= 2e-3, "side stream mass: err %.3g (relative, absolute below 1)" % err.max()
        finally:
            s.synchronize()
            r.close()
