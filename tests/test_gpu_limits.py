"""The largest per-head sizes the boundary accepts, against the oracle.

The kernels address one head's K and V, and one ring, with 32-bit byte offsets, so each must
stay below 2 GiB (N * D * 2 < 2^31 for a prompt head, S_h * D * 2 < 2^31 for a ring); a call
that reaches 2 GiB is refused with MOA_EUNSUPPORTED before anything is enqueued.

* Prefill fused with the ring handoff at N = 2^23 - 64, D = 128: each head's K is 16 KB short of
  2 GiB. Two KV heads (alpha 96 and 4000, beta 0: spans 128 and 4032 by the oracle's rule), two
  query heads each. Sampled rows, among them the last rows, whose tiles sit just below byte
  2^31, are compared with the oracle. Every ring slot is compared bit for bit. A fused decode
  step follows.
* Decode over the largest ring, S = N = 2^23 - 64 slots (2 GiB - 16 KB per pool): the
  prompt's K/V go to the ring with moa_kv_append, then one fused decode step attends all
  8,388,544 positions of the window, against the oracle.
* N = 2^23 (exactly 2 GiB per head) is refused by prefill, and a ring of 2^23 slots by decode.

Inputs are drawn on the GPU from seeded generators; the oracle sees only each checked row's
window, copied back.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Layout, f64, log, max_err, ring_k, ring_positions, ring_v, sample_rows

pytestmark = pytest.mark.gpu

N_MAX = (1 << 23) - 64     # D = 128: N * D * 2 = 2^31 - 16384
D = 128
TOL = 2e-2


def _bits(t):
    return t.contiguous().view(torch.int16).numpy()


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_prefill_handoff_and_decode_at_the_size_limit(moa):
    alpha, beta = [96, 4000], [0.0, 0.0]
    hq, hkv = 4, 2
    g = hq // hkv
    lay = Layout(alpha, beta, 1, D, N_MAX)
    log(f"limit prefill: B1 Hq{hq} Hkv{hkv} D{D} N{N_MAX} spans {list(lay.spans)}")
    plan = moa.Plan(1, hq, hkv, D, N_MAX, alpha, beta)
    q = workloads.device_normal_(torch.empty(1, hq, N_MAX, D, dtype=torch.bfloat16, device="cuda"), 71)
    k = workloads.device_normal_(torch.empty(1, hkv, N_MAX, D, dtype=torch.bfloat16, device="cuda"), 72)
    v = workloads.device_normal_(torch.empty(1, hkv, N_MAX, D, dtype=torch.bfloat16, device="cuda"), 73)
    o = torch.empty_like(q)
    kc, vc = plan.new_cache()
    plan.prefill_handoff(q, k, v, o, kc, vc)
    torch.cuda.synchronize()

    worst = 0.0
    for h in range(hq):
        s = int(lay.spans[h // g])
        rows = sample_rows(N_MAX, s, 24, 700 + h)
        for i in rows:
            lo = max(0, i - s + 1)
            want = oracle.prefill_rows(f64(q[0, h, i:i + 1]), f64(k[0, h // g, lo:i + 1]),
                                       f64(v[0, h // g, lo:i + 1]), s, [i - lo])
            worst = max(worst, max_err(f64(o[0, h, i:i + 1]), want))
    log(f"  prefill rows max abs err {worst:.3e}")
    assert worst <= TOL

    # the rings: positions N - S .. N - 1 at slot p mod S, bit for bit
    kc_h, vc_h = kc.cpu(), vc.cpu()
    for h in range(hkv):
        s = int(lay.spans[h])
        pos = np.arange(N_MAX - s, N_MAX)
        exp_k, held = oracle.ring_expected(_bits(k[0, h, N_MAX - s:].cpu()), pos, s, N_MAX - 1)
        exp_v, _ = oracle.ring_expected(_bits(v[0, h, N_MAX - s:].cpu()), pos, s, N_MAX - 1)
        assert (held == ring_positions(s, N_MAX - 1)).all()
        assert np.array_equal(_bits(ring_k(kc_h, lay, 0, h)), exp_k), h
        assert np.array_equal(_bits(ring_v(vc_h, lay, 0, h)), exp_v), h
    log("  rings match the oracle")

    # one fused decode step at position N
    qs, ks, vs = workloads.decode_step_inputs(1, hq, hkv, 1, D, "bf16", 74)
    od = torch.empty(1, hq, D, dtype=torch.bfloat16, device="cuda")
    plan.append_decode(qs[0].cuda(), kc, vc, ks[0].cuda(), vs[0].cuda(), N_MAX, od, plan.new_workspace())
    torch.cuda.synchronize()
    worst = 0.0
    for h in range(hkv):
        s = int(lay.spans[h])
        hk = torch.cat([k[0, h, N_MAX - s + 1:].cpu(), ks[0, 0, h:h + 1]])
        hv = torch.cat([v[0, h, N_MAX - s + 1:].cpu(), vs[0, 0, h:h + 1]])
        want = oracle.decode_step(f64(qs[0, 0, h * g:(h + 1) * g]), f64(hk), f64(hv),
                                  np.arange(N_MAX - s + 1, N_MAX + 1), N_MAX, s)
        worst = max(worst, max_err(f64(od[0, h * g:(h + 1) * g]), want))
    log(f"  decode max abs err {worst:.3e}")
    assert worst <= TOL
    del q, k, v, o, kc, vc, kc_h, vc_h
    _free()


def test_decode_over_the_largest_ring(moa):
    log(f"limit decode: ring of {N_MAX} slots, D{D}")
    plan = moa.Plan(1, 1, 1, D, N_MAX, [N_MAX], [0.0])
    assert Layout([N_MAX], [0.0], 1, D, N_MAX).spans[0] == N_MAX
    k = workloads.device_normal_(torch.empty(1, 1, N_MAX, D, dtype=torch.bfloat16, device="cuda"), 81)
    v = workloads.device_normal_(torch.empty(1, 1, N_MAX, D, dtype=torch.bfloat16, device="cuda"), 82)
    kc, vc = plan.new_cache()
    plan.kv_append(kc, vc, k, v, 0)
    qs, ks, vs = workloads.decode_step_inputs(1, 1, 1, 1, D, "bf16", 83)
    od = torch.empty(1, 1, D, dtype=torch.bfloat16, device="cuda")
    plan.append_decode(qs[0].cuda(), kc, vc, ks[0].cuda(), vs[0].cuda(), N_MAX, od, plan.new_workspace())
    torch.cuda.synchronize()
    # slot N mod S = 0 now holds the new token; the window is positions 1 .. N
    assert torch.equal(kc[:D].cpu(), ks[0, 0, 0])
    hk = torch.cat([k[0, 0, 1:].cpu(), ks[0, 0]]).float().numpy()
    hv = torch.cat([v[0, 0, 1:].cpu(), vs[0, 0]]).float().numpy()
    del kc, vc, k, v
    _free()
    want = oracle.decode_step(f64(qs[0, 0]), hk, hv, np.arange(1, N_MAX + 1), N_MAX, N_MAX)
    err = max_err(f64(od[0]), want)
    log(f"  decode over {N_MAX} keys: max abs err {err:.3e}")
    assert err <= TOL


def test_two_gib_heads_are_refused(moa):
    n = 1 << 23
    log(f"limit refusal: N {n}, D{D}")
    plan = moa.Plan(1, 1, 1, D, n, [64], [0.0])
    x = torch.empty(1, 1, n, D, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(x)
    with pytest.raises(moa.MoaError) as e:
        plan.prefill(x, x, x, o)
    assert e.value.status == moa.MOA_EUNSUPPORTED
    del x, o
    _free()
    ring = moa.Plan(1, 1, 1, D, n, [n], [0.0])
    kc, vc = ring.new_cache()
    q = torch.zeros(1, 1, D, dtype=torch.bfloat16, device="cuda")
    od = torch.empty_like(q)
    with pytest.raises(moa.MoaError) as e:
        ring.decode(q, kc, vc, n, od, ring.new_workspace())
    assert e.value.status == moa.MOA_EUNSUPPORTED
    del kc, vc
    _free()
