"""Dense baseline: every span = N on the same kernels is full causal attention.

Prefill is compared with torch's float64 causal scaled-dot-product attention
(a library routine) and with the oracle; decode with the oracle.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from gpu_util import f64, log, max_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
def test_dense_prefill_is_causal_attention(moa, d):
    bsz, hq, hkv, n = 2, 8, 2, 700
    log(f"dense prefill D{d}")
    plan = moa.Plan(bsz, hq, hkv, d, n, [n] * hkv, [0.0] * hkv)
    assert list(plan.spans) == [n] * hkv
    q, k, v = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 91)
    o = torch.empty_like(q.cuda())
    plan.prefill(q.cuda(), k.cuda(), v.cuda(), o)
    torch.cuda.synchronize()
    g = hq // hkv
    ref = F.scaled_dot_product_attention(q.double(), k.double().repeat_interleave(g, dim=1),
                                         v.double().repeat_interleave(g, dim=1),
                                         is_causal=True).numpy()
    assert max_err(f64(o), ref) <= 2e-2
    want = oracle.prefill(f64(q), f64(k), f64(v), oracle.spans([n] * hkv, [0.0] * hkv, n))
    assert max_err(f64(o), want) <= 2e-2


def test_dense_decode_matches_oracle(moa):
    bsz, hq, hkv, d, n, t_steps = 2, 8, 2, 128, 1500, 3
    log("dense decode")
    plan = moa.Plan(bsz, hq, hkv, d, n, [n] * hkv, [0.0] * hkv)
    _, kp, vp = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 92)
    qs, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, t_steps, d, "bf16", 93)
    kc, vc = plan.new_cache()
    ws = plan.new_workspace()
    plan.kv_append(kc, vc, kp.cuda(), vp.cuda(), 0)
    outs = []
    for t in range(t_steps):
        plan.kv_append(kc, vc, ks[t].unsqueeze(2).cuda(), vs[t].unsqueeze(2).cuda(), n + t)
        o = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
        plan.decode(qs[t].cuda(), kc, vc, n + t, o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    want = oracle.decode(f64(qs), [f64(kp[:, h]) for h in range(hkv)],
                         [f64(vp[:, h]) for h in range(hkv)], f64(ks), f64(vs),
                         oracle.spans([n] * hkv, [0.0] * hkv, n), n)
    assert max_err(np.stack([f64(o) for o in outs]), want) <= 2e-2
