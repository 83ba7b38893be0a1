"""Large score magnitudes: q and k scaled so that softmax rows are nearly one-hot and the
running max jumps by far more than the kernels' lazy-rescale threshold, tile after tile.
Prefill and fused decode must still match the oracle (and stay finite)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f64, log, max_err

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _scaled(x, s):
    return (x.float() * s).to(torch.bfloat16)


@pytest.mark.parametrize("scale", [6.0, 20.0])
def test_prefill_large_scores(moa, scale):
    bsz, hq, hkv, d, n = 2, 8, 4, 128, 900
    alpha, beta = [0, 64, 512, 0], [0.25, 0.0, 0.0, 1.0]
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta)
    q, k, v = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 9100)
    # scores grow along the keys, so later tiles keep raising the row max
    ramp = torch.linspace(0.2, 1.0, n).view(1, 1, n, 1)
    q, k = _scaled(q, scale), _scaled(k * ramp, scale)
    log(f"prefill large scores x{scale}: spans {[int(x) for x in plan.spans]}")
    o = torch.empty(bsz, hq, n, d, dtype=torch.bfloat16, device="cuda")
    plan.prefill(q.cuda(), k.cuda(), v.cuda(), o)
    torch.cuda.synchronize()
    got = f64(o)
    assert np.isfinite(got).all()
    want = oracle.prefill(f64(q), f64(k), f64(v), plan.spans)
    err = max_err(got, want)
    log(f"prefill x{scale}: max abs err {err:.3e}")
    assert err <= TOL
    plan.close()


@pytest.mark.parametrize("scale", [6.0, 20.0])
def test_append_decode_large_scores(moa, scale):
    bsz, hq, hkv, d, n, t_steps = 2, 8, 2, 128, 2500, 3
    alpha, beta = [0, 1024], [0.5, 0.0]
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta)
    _, kp, vp = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 9200)
    qs, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, t_steps, d, "bf16", 9201)
    kp, ks, qs = _scaled(kp, scale), _scaled(ks, scale), _scaled(qs, scale)
    log(f"append_decode large scores x{scale}: spans {[int(x) for x in plan.spans]}, "
        f"chunk {plan.decode_chunk}")
    kc, vc = plan.new_cache()
    ws = plan.new_workspace()
    plan.kv_append(kc, vc, kp.cuda(), vp.cuda(), 0)
    outs = []
    for t in range(t_steps):
        o = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
        plan.append_decode(qs[t].cuda(), kc, vc, ks[t].cuda(), vs[t].cuda(), n + t, o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    got = np.stack([f64(o) for o in outs])
    assert np.isfinite(got).all()
    want = oracle.decode(f64(qs), [f64(kp[:, h]) for h in range(hkv)],
                         [f64(vp[:, h]) for h in range(hkv)], f64(ks), f64(vs), plan.spans, n)
    err = max_err(got, want)
    log(f"append_decode x{scale}: max abs err {err:.3e}")
    assert err <= TOL
    plan.close()
