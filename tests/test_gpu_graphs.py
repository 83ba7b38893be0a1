"""The hot calls inside HIP graphs: every replay must reproduce the eager calls bit for bit.

The entry points only enqueue kernels on the caller's stream (no allocation, copy or
memset), so they can be captured.  A captured decode step is fixed to its position (pos is
passed by value), so each replay here restores the rings and repeats the same step; a serving
loop re-captures per position or updates the kernel nodes' arguments.  A fused prefill + ring
handoff and a fused append + decode step are each captured once and replayed three times, with
eager work (the outputs and rings cleared by fill kernels) and synchronisations between the
replays; every replay's outputs and ring contents are checked.
"""

import pytest
import torch

import workloads
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 4, 64)])
def test_prefill_handoff_and_append_decode_in_graphs(moa, hq, hkv, d):
    bsz, n = 2, 1500
    alpha, beta = [0, 300, 64, 0][:hkv], [0.5, 0.0, 0.0, 1.0][:hkv]
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta)
    log(f"graphs: B{bsz} Hq{hq} Hkv{hkv} D{d} N{n} decode chunk {plan.decode_chunk}")
    q, k, v = (x.cuda() for x in workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 7300))
    qs, ks, vs = (x.cuda() for x in workloads.decode_step_inputs(bsz, hq, hkv, 1, d, "bf16", 7301))

    # eager reference: prefill + handoff, the rings after it, then one fused decode step
    o_ref = torch.empty_like(q)
    kc_ref, vc_ref = plan.new_cache()
    plan.prefill_handoff(q, k, v, o_ref, kc_ref, vc_ref)
    kc_pre, vc_pre = kc_ref.clone(), vc_ref.clone()
    od_ref = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
    plan.append_decode(qs[0], kc_ref, vc_ref, ks[0], vs[0], n, od_ref, plan.new_workspace())
    torch.cuda.synchronize()

    # static buffers of the graphs; one eager warm-up on a side stream, then capture
    o = torch.empty_like(q)
    od = torch.empty_like(od_ref)
    kc, vc = plan.new_cache()
    ws = plan.new_workspace()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.prefill_handoff(q, k, v, o, kc, vc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_pre, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pre):
        plan.prefill_handoff(q, k, v, o, kc, vc)
    with torch.cuda.graph(g_dec):
        plan.append_decode(qs[0], kc, vc, ks[0], vs[0], n, od, ws)
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (o, od, kc, vc):
            t.zero_()
        torch.cuda.synchronize()
        g_pre.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), rep
        assert torch.equal(kc, kc_pre) and torch.equal(vc, vc_pre), rep
        g_dec.replay()
        torch.cuda.synchronize()
        assert torch.equal(od, od_ref), rep
        assert torch.equal(kc, kc_ref) and torch.equal(vc, vc_ref), rep
    log("graphs: three replays bit-identical to the eager calls")
    plan.close()
