"""Properties checked without the oracle.

The window mean (full sizes):

With q = 0 every kept score is 0, so every kept key has the same weight and each output row is
the plain mean of V over its window: query i of a head with span S averages value rows
max(0, i - S + 1) .. i in prefill, and a decode step averages the S slots of its ring after
the new token's append.  The means are computed here in float64 from cumulative sums (prefill)
or from the ring contents (decode), so they share nothing with the oracle's softmax.  The
kernels' weights are then exactly 1 (exp2(0)); what separates them from the mean is float32
accumulation and the final bf16 rounding, so each output must lie within one bf16 ulp of the
exact mean (|mean| * 2^-7) plus 1e-4 for the float32 sums.

Grouped-query heads: a grouped plan equals an ungrouped one on repeated K/V.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Layout, f64, log, ring_v

pytestmark = pytest.mark.gpu


def _ulp_excess(got, want):
    """Largest amount by which |got - want| exceeds one bf16 ulp of want plus 1e-4 (<= 0: ok),
    and the largest |got - want|."""
    diff = np.abs(np.asarray(got, dtype=np.float64) - want)
    return float(np.max(diff - (np.abs(want) * 2.0 ** -7 + 1e-4))), float(np.max(diff))


def _window_means(v, s):
    """[N, D] float64 -> row i: mean of v[max(0, i - s + 1) .. i]."""
    n = v.shape[0]
    c = np.concatenate([np.zeros((1, v.shape[1])), np.cumsum(v, axis=0)])
    i = np.arange(n)
    lo = np.maximum(0, i - s + 1)
    return (c[i + 1] - c[lo]) / (i + 1 - lo)[:, None]


@pytest.mark.parametrize("name", ["c1_prefill", "c4_prefill"])
def test_prefill_zero_query_is_window_mean(moa, name):
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    n, g = w.n_prompt, w.n_q_heads // w.n_kv_heads
    q = torch.zeros(w.batch, w.n_q_heads, n, w.head_dim, dtype=torch.bfloat16, device="cuda")
    shp_kv = (w.batch, w.n_kv_heads, n, w.head_dim)
    k = workloads.device_normal_(torch.empty(shp_kv, dtype=torch.bfloat16, device="cuda"), 61)
    v = workloads.device_normal_(torch.empty(shp_kv, dtype=torch.bfloat16, device="cuda"), 62)
    o = torch.empty_like(q)
    log(f"{name}: q = 0, every row of every head against the window mean of v")
    plan.prefill(q, k, v, o)
    torch.cuda.synchronize()
    spans = oracle.spans(alpha, beta, n)   # the span rule only; no oracle attention
    worst = 0.0
    for hk in range(w.n_kv_heads):
        want = _window_means(f64(v[0, hk]), int(spans[hk]))
        for hq in range(hk * g, (hk + 1) * g):
            excess, err = _ulp_excess(f64(o[0, hq]), want)
            worst = max(worst, err)
            assert excess <= 0, (name, hq, int(spans[hk]), err)
    log(f"{name}: worst abs err {worst:.3e}, every element within one bf16 ulp")


@pytest.mark.parametrize("name", ["c2_decode", "c3_decode", "c4_decode"])
def test_append_decode_zero_query_is_ring_mean(moa, name):
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    # ring spans and locations from the span rule and the layout's statement, not the plan
    lay = Layout(alpha, beta, w.batch, w.head_dim, w.n_prompt)
    assert plan.cache_elems == lay.total_slots * w.head_dim
    g = w.n_q_heads // w.n_kv_heads
    kc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16,
                                              device="cuda"), 63)
    vc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16,
                                              device="cuda"), 64)
    ws = plan.new_workspace()
    q = torch.zeros(w.batch, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
    kn = workloads.device_normal_(torch.empty(w.batch, w.n_kv_heads, w.head_dim,
                                              dtype=torch.bfloat16, device="cuda"), 65)
    vn = workloads.device_normal_(torch.empty(w.batch, w.n_kv_heads, w.head_dim,
                                              dtype=torch.bfloat16, device="cuda"), 66)
    o = torch.empty_like(q)
    log(f"{name}: q = 0, every (b, h) against the mean of its ring after the append")
    plan.append_decode(q, kc, vc, kn, vn, w.n_prompt, o, ws)
    torch.cuda.synchronize()
    vc_h, o_h = vc.cpu(), f64(o)
    worst = 0.0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            want = f64(ring_v(vc_h, lay, b, h)).mean(axis=0)
            excess, err = _ulp_excess(o_h[b, h * g:(h + 1) * g], want[None, :])
            worst = max(worst, err)
            assert excess <= 0, (name, b, h, int(lay.spans[h]), err)
    log(f"{name}: worst abs err {worst:.3e}, every element within one bf16 ulp")


def test_gqa_equals_repeated_kv(moa):
    """Query head h of a grouped plan reads KV head h // G: the same as an ungrouped plan on
    K/V repeated G times with the spans repeated.  Prefill does the same arithmetic per unit
    either way (bit-identical); decode splits the rings into different chunks (within 2e-3)."""
    bsz, hq, hkv, d, n = 2, 16, 2, 128, 2100
    alpha, beta = [0, 700], [0.5, 0.0]
    g = hq // hkv
    grouped = moa.Plan(bsz, hq, hkv, d, n, alpha, beta)
    flat = moa.Plan(bsz, hq, hq, d, n, [a for a in alpha for _ in range(g)],
                    [b for b in beta for _ in range(g)])
    assert [int(s) for s in flat.spans] == [int(s) for s in grouped.spans for _ in range(g)]
    q, k, v = (x.cuda() for x in workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 6700))
    krep, vrep = k.repeat_interleave(g, dim=1).contiguous(), v.repeat_interleave(g, dim=1).contiguous()
    o_g, o_f = torch.empty_like(q), torch.empty_like(q)
    kc_g, vc_g = grouped.new_cache()
    kc_f, vc_f = flat.new_cache()
    grouped.prefill_handoff(q, k, v, o_g, kc_g, vc_g)
    flat.prefill_handoff(q, krep, vrep, o_f, kc_f, vc_f)
    qs, ks, vs = (x.cuda() for x in workloads.decode_step_inputs(bsz, hq, hkv, 1, d, "bf16", 6701))
    od_g = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
    od_f = torch.empty_like(od_g)
    grouped.append_decode(qs[0], kc_g, vc_g, ks[0], vs[0], n, od_g, grouped.new_workspace())
    flat.append_decode(qs[0], kc_f, vc_f, ks[0].repeat_interleave(g, dim=1).contiguous(),
                       vs[0].repeat_interleave(g, dim=1).contiguous(), n, od_f,
                       flat.new_workspace())
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_f)
    err = float((od_g.float() - od_f.float()).abs().max())
    log(f"gqa vs repeated kv: prefill bit-identical, decode max diff {err:.3e} "
        f"(chunks {grouped.decode_chunk} vs {flat.decode_chunk})")
    assert err <= 2e-3
    grouped.close()
    flat.close()
