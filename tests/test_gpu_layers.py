"""A model's layers with their own rules (from the per-layer rules file) on the GPU.

Each layer gets its own plan, rings and work lists; every layer's prefill,
prompt handoff and decode steps must match the oracle run with that layer's
spans, sequence by sequence.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f64, log, max_err

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_layers_from_rules_file(moa):
    import heterogeneous_sliding_windows_amd.rules as rules
    full = rules.load(os.path.join(GOLDEN, "model_rules.json"))
    # the first 3 layers, first 8 KV heads of each (GQA, 2 query heads per KV head)
    rs = rules.RuleSet([(a[:8], b[:8]) for a, b in full.layers[:3]])
    lens = [1200, 700]
    bsz, hq, hkv, d, n, t_steps = 2, 16, 8, 64, max(lens), 2
    plans = rs.plans(bsz, hq, d, n, seq_len=lens)
    # the layers' spans differ
    assert len({tuple(oracle.spans(a, b, lens[0])) for a, b in rs.layers}) == 3
    worst = 0.0
    try:
        for layer, plan in enumerate(plans):
            log(f"layer {layer}: lens {lens}, decode chunk {plan.decode_chunk}")
            q, k, v = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 9500 + layer)
            qs, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, t_steps, d, "bf16",
                                                      9600 + layer)
            qd = q.cuda()
            o = torch.empty_like(qd)
            kc, vc = plan.new_cache()
            ws = plan.new_workspace()
            plan.prefill_handoff(qd, k.cuda(), v.cuda(), o, kc, vc)
            outs = []
            for t in range(t_steps):
                od = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
                plan.append_decode(qs[t].cuda(), kc, vc, ks[t].cuda(), vs[t].cuda(), n + t, od, ws)
                outs.append(od.cpu())
            torch.cuda.synchronize()
            got_d = np.stack([f64(x) for x in outs])
            for b, nb in enumerate(lens):
                pad = n - nb
                # the oracle's own spans for this layer's rules at the sequence's length
                spans = oracle.spans(*rs.layers[layer], nb)
                want = oracle.prefill(f64(q[b:b + 1, :, pad:]), f64(k[b:b + 1, :, pad:]),
                                      f64(v[b:b + 1, :, pad:]), spans)
                err_p = max_err(f64(o[b:b + 1, :, pad:]), want)
                want = oracle.decode(f64(qs[:, b:b + 1]),
                                     [f64(k[b:b + 1, h, pad:]) for h in range(hkv)],
                                     [f64(v[b:b + 1, h, pad:]) for h in range(hkv)],
                                     f64(ks[:, b:b + 1]), f64(vs[:, b:b + 1]), spans, nb)
                err_d = max_err(got_d[:, b:b + 1], want)
                worst = max(worst, err_p, err_d)
                assert err_p <= 2e-2 and err_d <= 2e-2, (layer, b, err_p, err_d)
    finally:
        for p in plans:
            p.close()
    log(f"layers: worst err {worst:.3e}")


def test_decode_step_across_layers_in_one_graph(moa):
    """Three layers' rings in one K and one V allocation (RuleSet.caches), and a decode step
    of all three layers captured as one HIP graph.  Each of three replays (the rings restored
    by eager copies in between) equals the eager calls bit for bit."""
    import heterogeneous_sliding_windows_amd.rules as rules
    full = rules.load(os.path.join(GOLDEN, "model_rules.json"))
    rs = rules.RuleSet([(a[:8], b[:8]) for a, b in full.layers[:3]])
    bsz, hq, hkv, d, n = 2, 16, 8, 64, 1200
    plans = rs.plans(bsz, hq, d, n)
    caches = rules.RuleSet.caches(plans)
    pool_elems = sum(int(p.cache_elems) for p in plans)
    assert all(kc.data_ptr() - caches[0][0].data_ptr() ==
               2 * sum(int(p.cache_elems) for p in plans[:i]) for i, (kc, _) in enumerate(caches))
    try:
        for layer, (plan, (kc, vc)) in enumerate(zip(plans, caches)):
            q, k, v = (x.cuda() for x in workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16",
                                                                  9700 + layer))
            plan.prefill_handoff(q, k, v, torch.empty_like(q), kc, vc)
        steps = [tuple(x.cuda() for x in workloads.decode_step_inputs(bsz, hq, hkv, 1, d, "bf16",
                                                                      9800 + layer))
                 for layer in range(len(plans))]
        ws = [p.new_workspace() for p in plans]
        torch.cuda.synchronize()
        k_pre = [kc.clone() for kc, _ in caches]
        v_pre = [vc.clone() for _, vc in caches]

        def step(outs):
            for plan, (kc, vc), (qs, ks, vs), w, o in zip(plans, caches, steps, ws, outs):
                plan.append_decode(qs[0], kc, vc, ks[0], vs[0], n, o, w)

        def restore():
            for (kc, vc), k0, v0 in zip(caches, k_pre, v_pre):
                kc.copy_(k0)
                vc.copy_(v0)

        ref = [torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda") for _ in plans]
        step(ref)
        torch.cuda.synchronize()
        k_ref = [kc.clone() for kc, _ in caches]
        v_ref = [vc.clone() for _, vc in caches]
        restore()
        outs = [torch.empty_like(r) for r in ref]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(outs)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(outs)
        for rep in range(3):
            restore()
            for o in outs:
                o.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for layer in range(len(plans)):
                assert torch.equal(outs[layer], ref[layer]), (rep, layer)
                assert torch.equal(caches[layer][0], k_ref[layer]), (rep, layer)
                assert torch.equal(caches[layer][1], v_ref[layer]), (rep, layer)
        log(f"layers in one graph: {len(plans)} layers, rings in one pool of "
            f"{2 * pool_elems * 2 / 1e6:.1f} MB, three replays bit-identical")
    finally:
        for p in plans:
            p.close()
