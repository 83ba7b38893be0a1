"""Fused entry points against the oracle: prefill + ring handoff, append + decode.

moa_prefill_handoff: o within the prefill tolerance of the float64 oracle and
the ring bits equal to the oracle's expected slot contents.  moa_append_decode:
o within 2e-2 of the oracle's decode and the ring bits after every step as the
oracle expects.  The fused prefill must also reproduce, bit for bit, the
output of the plain prefill (same arithmetic, same order); the fused decode
adds the new key as one extra online-softmax step instead of inside a matrix
product, so its output matches the separate calls within the tolerance.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import oracle
import workloads
from gpu_util import Layout, f64, log, max_err, ring_k, ring_positions, ring_v

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
_BITS = {torch.bfloat16: torch.int16, torch.float32: torch.int32}


def _bits(t):
    return t.contiguous().view(_BITS[t.dtype]).numpy()


def _check_rings(lay, kc, vc, kp, vp, ks, vs, n, t_done):
    """Every slot holds the bits the oracle says it must after position n - 1 + t_done
    (spans and ring locations from the oracle's layout)."""
    p_last = n - 1 + t_done
    kc_h, vc_h = kc.cpu(), vc.cpu()
    for b in range(lay.batch):
        for h in range(lay.n_kv_heads):
            s = int(lay.spans[h])
            hist_k = torch.cat([kp[b, h], ks[:t_done, b, h]]) if t_done else kp[b, h]
            hist_v = torch.cat([vp[b, h], vs[:t_done, b, h]]) if t_done else vp[b, h]
            pos = np.arange(n + t_done)
            exp_k, held = oracle.ring_expected(_bits(hist_k), pos, s, p_last)
            exp_v, _ = oracle.ring_expected(_bits(hist_v), pos, s, p_last)
            assert (held == ring_positions(s, p_last)).all()
            assert np.array_equal(_bits(ring_k(kc_h, lay, b, h)), exp_k), (b, h)
            assert np.array_equal(_bits(ring_v(vc_h, lay, b, h)), exp_v), (b, h)


HANDOFF_CASES = [
    # B, Hq, Hkv, D, N, alpha, beta, dtype
    (1, 4, 4, 128, 1000, [0, 64, 100, 0], [0.0, 0.0, 0.0, 1.0], "bf16"),
    (2, 8, 2, 128, 777, [0, 300], [0.25, 0.0], "bf16"),
    (1, 4, 4, 64, 1000, [1, 64, 700, 0], [0.0, 0.0, 0.0, 0.6], "bf16"),
    (2, 16, 2, 128, 300, [0, 0], [0.0, 1.0], "bf16"),
    (1, 2, 1, 128, 1, [0], [1.0], "bf16"),
    (3, 6, 3, 128, 2049, [0, 64, 2000], [1.0, 0.0, 0.0], "bf16"),
    (2, 4, 2, 64, 333, [0, 200], [0.5, 0.0], "f32"),
    (1, 2, 2, 128, 257, [0, 64], [1.0, 0.0], "f32"),
    # the largest group the boundary takes (G = 16): one handoff per KV group
    (1, 16, 1, 128, 700, [0], [0.5], "bf16"),
    (1, 32, 2, 64, 300, [0, 100], [0.4, 0.0], "f32"),
]


@pytest.mark.parametrize("case", range(len(HANDOFF_CASES)))
def test_prefill_handoff_small(moa, case):
    bsz, hq, hkv, d, n, alpha, beta, dt = HANDOFF_CASES[case]
    log(f"prefill_handoff case {case}: B{bsz} Hq{hq} Hkv{hkv} D{d} N{n} {dt}")
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta, dtype=dt)
    lay = Layout(alpha, beta, bsz, d, n)
    q, k, v = workloads.prefill_inputs(bsz, hq, hkv, n, d, dt, 7000 + case)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o_plain = torch.empty_like(qd)
    plan.prefill(qd, kd, vd, o_plain)
    o = torch.empty_like(qd)
    kc, vc = plan.new_cache()
    plan.prefill_handoff(qd, kd, vd, o, kc, vc)
    torch.cuda.synchronize()
    want = oracle.prefill(f64(q), f64(k), f64(v), lay.spans)
    err = max_err(f64(o), want)
    log(f"case {case} spans {list(lay.spans)} max abs err {err:.3e}")
    assert err <= TOL[dt]
    assert torch.equal(o, o_plain)
    _check_rings(lay, kc, vc, k, v, None, None, n, 0)


APPEND_CASES = [
    # B, Hq, Hkv, D, N, alpha, beta, T
    (3, 4, 2, 128, 300, [0, 100], [0.0, 0.0], 5),
    (2, 4, 4, 128, 300, [0, 64, 0, 0], [0.0, 0.0, 1.0, 0.5], 4),
    (2, 16, 2, 128, 2500, [0, 1500], [1.0, 0.0], 4),
    (2, 8, 1, 64, 1100, [0], [0.97], 3),
    (1, 1, 1, 128, 5, [0], [0.5], 6),
    # new slot in the last (ragged, 64-slot) chunk, then wrapping to slot 0
    (2, 4, 2, 128, 2175, [1088, 1024], [0.0, 0.0], 3),
    # new slot in a later chunk of a multi-chunk ring
    (1, 8, 2, 64, 3100, [2048, 0], [0.0, 0.4], 3),
    # more steps than either span (64 and 100): every slot rewritten by decode tokens
    (2, 4, 2, 128, 100, [64, 0], [0.0, 1.0], 150),
    # the largest group the boundary takes (G = 16)
    (1, 16, 1, 128, 2200, [0], [0.9], 3),
]


@pytest.mark.parametrize("case", range(len(APPEND_CASES)))
def test_append_decode_small(moa, case):
    bsz, hq, hkv, d, n, alpha, beta, t_steps = APPEND_CASES[case]
    log(f"append_decode case {case}: B{bsz} Hq{hq} Hkv{hkv} D{d} N{n} T{t_steps}")
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta)
    lay = Layout(alpha, beta, bsz, d, n)
    _, kp, vp = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 8000 + 10 * case)
    qs, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, t_steps, d, "bf16", 8001 + 10 * case)
    kc, vc = plan.new_cache()
    plan.kv_append(kc, vc, kp.cuda(), vp.cuda(), 0)
    kc2, vc2 = kc.clone(), vc.clone()
    ws, ws2 = plan.new_workspace(), plan.new_workspace()
    outs = []
    for t in range(t_steps):
        q, kn, vn = qs[t].cuda(), ks[t].cuda(), vs[t].cuda()
        o = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
        plan.append_decode(q, kc, vc, kn, vn, n + t, o, ws)
        # the two calls it fuses, on a copy of the rings
        o2 = torch.empty_like(o)
        plan.kv_append(kc2, vc2, kn.unsqueeze(2), vn.unsqueeze(2), n + t)
        plan.decode(q, kc2, vc2, n + t, o2, ws2)
        torch.cuda.synchronize()
        assert max_err(f64(o), f64(o2)) <= TOL["bf16"], t
        _check_rings(lay, kc, vc, kp, vp, ks, vs, n, t + 1)
        outs.append(o)
    want = oracle.decode(f64(qs), [f64(kp[:, h]) for h in range(hkv)],
                         [f64(vp[:, h]) for h in range(hkv)], f64(ks), f64(vs), lay.spans, n)
    got = np.stack([f64(o) for o in outs])
    err = max_err(got, want)
    log(f"case {case} spans {list(lay.spans)} max abs err {err:.3e}")
    assert err <= TOL["bf16"]


def test_append_decode_span_one_returns_new_value_exactly(moa):
    log("append_decode span-1")
    bsz, hq, hkv, d, n = 2, 4, 2, 128, 70
    plan = moa.Plan(bsz, hq, hkv, d, n, [0, 0], [0.0, 0.0])
    _, kp, vp = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 91)
    qs, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, 2, d, "bf16", 92)
    kc, vc = plan.new_cache()
    ws = plan.new_workspace()
    plan.kv_append(kc, vc, kp.cuda(), vp.cuda(), 0)
    for t in range(2):
        o = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
        plan.append_decode(qs[t].cuda(), kc, vc, ks[t].cuda(), vs[t].cuda(), n + t, o, ws)
        assert torch.equal(o.cpu(), vs[t].repeat_interleave(2, dim=1))


def test_fused_argument_errors(moa):
    log("fused argument errors")
    plan = moa.Plan(1, 2, 2, 128, 64, [0, 0], [1.0, 1.0])
    kc, vc = plan.new_cache()
    q = torch.zeros(1, 2, 128, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(1, 2, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(moa.MoaError) as e:
        plan.append_decode(q, kc, vc, kn, kn, 63, o, plan.new_workspace())
    assert e.value.status == moa.MOA_EINVAL
    with pytest.raises(moa.MoaError) as e:
        plan.append_decode(q, kc, vc, kn, kn, 64, o, torch.empty(8, dtype=torch.uint8,
                                                               device="cuda"))
    assert e.value.status == moa.MOA_EWORKSPACE
    with pytest.raises(ValueError):
        plan.append_decode(q, kc, vc, kn[:, :1], kn, 64, o, plan.new_workspace())
    f32 = moa.Plan(1, 2, 2, 128, 64, [0, 0], [1.0, 1.0], dtype="f32")
    kf, vf = f32.new_cache()
    with pytest.raises(moa.MoaError) as e:
        f32.append_decode(q.float(), kf, vf, kn.float(), kn.float(), 64, o.float(),
                          f32.new_workspace())
    assert e.value.status == moa.MOA_EUNSUPPORTED


@pytest.mark.parametrize("name", ["c1_prefill", "c4_prefill"])
def test_prefill_handoff_full_size(moa, name):
    """Full-size prompt: o equals the plain prefill's bit for bit, every ring slot holds
    the prompt row of the position it should (oracle slot rule)."""
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    lay = Layout(alpha, beta, w.batch, w.head_dim, w.n_prompt)
    assert plan.cache_elems == lay.total_slots * w.head_dim
    n, d = w.n_prompt, w.head_dim
    log(f"{name}: prefill_handoff at full size")
    shape_q = (w.batch, w.n_q_heads, n, d)
    shape_kv = (w.batch, w.n_kv_heads, n, d)
    q = workloads.device_normal_(torch.empty(shape_q, dtype=torch.bfloat16, device="cuda"), 71)
    k = workloads.device_normal_(torch.empty(shape_kv, dtype=torch.bfloat16, device="cuda"), 72)
    v = workloads.device_normal_(torch.empty(shape_kv, dtype=torch.bfloat16, device="cuda"), 73)
    o_plain = torch.empty_like(q)
    plan.prefill(q, k, v, o_plain)
    o = torch.empty_like(q)
    kc, vc = plan.new_cache()
    plan.prefill_handoff(q, k, v, o, kc, vc)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)
    kc_h, vc_h, k_h, v_h = kc.cpu(), vc.cpu(), k.cpu(), v.cpu()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            s = int(lay.spans[h])
            pos = [oracle.ring_slot(p, s) for p in range(n - s, n)]
            want_slot_of = np.array(pos)
            held = np.empty(s, dtype=np.int64)
            held[want_slot_of] = np.arange(n - s, n)
            assert np.array_equal(_bits(ring_k(kc_h, lay, b, h)), _bits(k_h[b, h][held])), (b, h)
            assert np.array_equal(_bits(ring_v(vc_h, lay, b, h)), _bits(v_h[b, h][held])), (b, h)
    log(f"{name}: o identical, {w.batch * w.n_kv_heads} rings exact")


@pytest.mark.parametrize("name", ["c2_decode", "c3_decode", "c4_decode"])
def test_append_decode_full_size_every_head(moa, name):
    """Full-size rings, three fused steps, every (b, h) of every step against the oracle; the
    new positions' slots of every ring hold the new bits."""
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    lay = Layout(alpha, beta, w.batch, w.head_dim, w.n_prompt)
    assert plan.cache_elems == lay.total_slots * w.head_dim
    log(f"{name}: filling {2 * plan.cache_elems * 2 / 1e9:.2f} GB of rings")
    kc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16,
                                              device="cuda"), 83)
    vc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16,
                                              device="cuda"), 84)
    ws = plan.new_workspace()
    t_steps = 3
    n = w.n_prompt
    g = w.n_q_heads // w.n_kv_heads
    qs, ks, vs = workloads.decode_step_inputs(w.batch, w.n_q_heads, w.n_kv_heads, t_steps,
                                              w.head_dim, "bf16", w.data_seed + 50)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    kc0, vc0 = kc.cpu(), vc.cpu()   # the prompt rings, on the host
    outs = []
    for t in range(t_steps):
        log(f"{name}: fused step {t}")
        o = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
        plan.append_decode(qs[t].cuda(), kc, vc, ks[t].cuda(), vs[t].cuda(), n + t, o, ws)
        outs.append(o.cpu())
    torch.cuda.synchronize()
    kc_h, vc_h = kc.cpu(), vc.cpu()
    ks64, vs64, qs64 = f64(ks), f64(vs), f64(qs)
    outs64 = [f64(o) for o in outs]

    def check(pair):
        """Worst error of one (b, h) over the steps and the step it occurs at; ring bits."""
        b, h = pair
        s = int(lay.spans[h])
        order = np.argsort(ring_positions(s, n - 1))
        hist_k = np.empty((s + t_steps, w.head_dim))
        hist_v = np.empty((s + t_steps, w.head_dim))
        hist_k[:s] = f64(ring_k(kc0, lay, b, h))[order]
        hist_v[:s] = f64(ring_v(vc0, lay, b, h))[order]
        res = (0.0, -1)
        for t in range(t_steps):
            hist_k[s + t], hist_v[s + t] = ks64[t, b, h], vs64[t, b, h]
            want = oracle.decode_step(qs64[t, b, h * g:(h + 1) * g], hist_k[:s + t + 1],
                                      hist_v[:s + t + 1], np.arange(n - s, n + t + 1), n + t, s)
            res = max(res, (max_err(outs64[t][b, h * g:(h + 1) * g], want), t))
        # the last min(s, T) new positions sit in their slots
        slots_ok = all(
            torch.equal(ring_k(kc_h, lay, b, h)[oracle.ring_slot(n + t, s)], ks[t, b, h]) and
            torch.equal(ring_v(vc_h, lay, b, h)[oracle.ring_slot(n + t, s)], vs[t, b, h])
            for t in range(max(0, t_steps - s), t_steps))
        return res, slots_ok

    with threadpool_limits(1), ThreadPoolExecutor(8) as ex:
        res = list(ex.map(check, pairs))
    worst = max(e for (e, _), _ in res)
    bad = [(b, h, t, e) for (b, h), ((e, t), _) in zip(pairs, res) if e > TOL["bf16"]]
    assert not bad, (name, bad[:8])
    assert all(ok for _, ok in res), [p for p, (_, ok) in zip(pairs, res) if not ok][:8]
    log(f"{name}: every (b, h) of {t_steps} steps, worst err {worst:.3e}")
