"""One plan used from two streams at once (the plan is read-only after creation).

Each stream gets its own inputs, outputs, rings and workspace; the results must be bit
for bit those of the same calls made one after another on one stream.
"""

import pytest
import torch

import workloads
from gpu_util import log

pytestmark = pytest.mark.gpu


def test_plan_shared_by_two_streams(moa):
    bsz, hq, hkv, d, n, steps = 3, 8, 4, 128, 1500, 4
    alpha, beta = [0, 64, 512, 0], [0.25, 0.0, 0.0, 1.0]
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta)
    log(f"two streams: decode chunk {plan.decode_chunk}")
    inputs = [workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 7100 + i) for i in range(2)]
    steps_in = [workloads.decode_step_inputs(bsz, hq, hkv, steps, d, "bf16", 7200 + i)
                for i in range(2)]

    def run(streams):
        outs = []
        state = []
        for i in range(2):
            q, k, v = (x.cuda() for x in inputs[i])
            kc, vc = plan.new_cache()
            state.append((q, k, v, torch.empty_like(q), kc, vc, plan.new_workspace()))
        torch.cuda.synchronize()
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                q, k, v, o, kc, vc, ws = state[i]
                plan.prefill_handoff(q, k, v, o, kc, vc, stream=s)
                qs, ks, vs = (x.cuda() for x in steps_in[i])
                od = []
                for t in range(steps):
                    o_t = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
                    plan.append_decode(qs[t], kc, vc, ks[t], vs[t], n + t, o_t, ws, stream=s)
                    od.append(o_t)
                outs.append((o, torch.stack(od), kc, vc))
        torch.cuda.synchronize()
        return [[x.cpu() for x in o] for o in outs]

    s0 = torch.cuda.current_stream()
    serial = run([s0, s0])
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    parallel = run([sa, sb])
    for i in range(2):
        for a, b, what in zip(serial[i], parallel[i], ("prefill o", "decode o", "k rings", "v rings")):
            assert torch.equal(a, b), (i, what)
    log("two streams: bit-identical to the serial calls")
    plan.close()
