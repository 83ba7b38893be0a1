"""moa_append_decode_static (fixed library scratch, no allocation) against
moa_append_decode (caller workspace) on the same inputs.

The two entry points run the same kernels, so o and the ring contents must be
bit-identical; o is also checked against the float64 oracle at the bf16
tolerance.  Calls follow each other on one GPU with plans of different sizes:
a larger grouped-query plan with split rings, then a smaller one (head dim 64),
then the first plan again at its next position.  Each later call finds the
scratch holding the previous call's partials, so a call that read a partial it
had not written would differ from the workspace call.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f64, log, max_err

pytestmark = pytest.mark.gpu

TOL = 2e-2

CASES = {
    # B, Hq, Hkv, D, N, alpha, beta: rings of 3776 and 2112 slots, split in chunks
    "large": (3, 16, 2, 128, 5000, [0, 2100], [0.75, 0.0]),
    # rings of 1500, 64, 1152 and 384 slots
    "small": (2, 4, 4, 64, 1500, [0, 64, 1100, 0], [1.0, 0.0, 0.0, 0.25]),
}


class _Setup:
    def __init__(self, moa, name, seed):
        bsz, hq, hkv, d, n, alpha, beta = CASES[name]
        self.name, self.n, self.hkv = name, n, hkv
        self.plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta)
        # spans for the oracle come from the oracle's own rule
        self.spans = oracle.spans(alpha, beta, n)
        _, self.kp, self.vp = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", seed)
        self.qs, self.ks, self.vs = workloads.decode_step_inputs(bsz, hq, hkv, 2, d, "bf16",
                                                                 seed + 1)
        self.kc, self.vc = self.plan.new_cache()
        self.plan.kv_append(self.kc, self.vc, self.kp.cuda(), self.vp.cuda(), 0)
        # twin rings for the workspace call
        self.kc2, self.vc2 = self.kc.clone(), self.vc.clone()
        self.ws = self.plan.new_workspace()
        self.outs = []

    def step(self, t):
        plan, n = self.plan, self.n
        q, kn, vn = self.qs[t].cuda(), self.ks[t].cuda(), self.vs[t].cuda()
        o = torch.full((plan.batch, plan.n_q_heads, plan.head_dim), float("nan"),
                       dtype=torch.bfloat16, device="cuda")
        o2 = torch.empty_like(o)
        log(f"append_decode_static {self.name} step {t}: B{plan.batch} Hq{plan.n_q_heads} "
            f"Hkv{plan.n_kv_heads} D{plan.head_dim} N{n}, workspace {plan.workspace_bytes} B")
        plan.append_decode_static(q, self.kc, self.vc, kn, vn, n + t, o)
        plan.append_decode(q, self.kc2, self.vc2, kn, vn, n + t, o2, self.ws)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), (self.name, t)
        assert torch.equal(self.kc.view(torch.int16), self.kc2.view(torch.int16)), (self.name, t)
        assert torch.equal(self.vc.view(torch.int16), self.vc2.view(torch.int16)), (self.name, t)
        self.outs.append(o)

    def check_oracle(self):
        hkv, t = self.hkv, len(self.outs)
        want = oracle.decode(f64(self.qs[:t]), [f64(self.kp[:, h]) for h in range(hkv)],
                             [f64(self.vp[:, h]) for h in range(hkv)], f64(self.ks[:t]),
                             f64(self.vs[:t]), self.spans, self.n)
        err = max_err(np.stack([f64(o) for o in self.outs]), want)
        log(f"{self.name}: {t} steps, max abs err vs oracle {err:.3e}")
        assert err <= TOL


def test_static_matches_workspace_calls_in_a_row(moa):
    assert moa.static_workspace_bytes() == 16 << 20
    large = _Setup(moa, "large", 9100)
    small = _Setup(moa, "small", 9200)
    assert large.plan.workspace_bytes > small.plan.workspace_bytes
    large.step(0)       # first call on this GPU: the scratch address is looked up
    small.step(0)       # smaller input; the scratch still holds the first call's partials
    large.step(1)
    large.check_oracle()
    small.check_oracle()
