"""Ring append and split-K decode parity: HIP kernels against the oracle.

Ring contents are compared bit for bit (bf16 bits) with the oracle's
expected slot contents read through the layout include/moa.h documents;
decode outputs within max-abs 2e-2 of the float64 oracle on the same bits.
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

TOL = 2e-2


def _prompt_and_steps(bsz, hq, hkv, n, d, t_steps, seed):
    _, kp, vp = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", seed)
    qs, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, t_steps, d, "bf16", seed + 1)
    return kp, vp, qs, ks, vs


def _check_rings(lay, kc, vc, kp, vp, ks, vs, n, t_done):
    """Every slot of every ring holds the bits of the position it should (spans and ring
    locations from the oracle's layout)."""
    p_last = n - 1 + t_done
    kc_h, vc_h = kc.cpu(), vc.cpu()
    for b in range(lay.batch):
        for h in range(lay.n_kv_heads):
            s = int(lay.spans[h])
            hist_k = torch.cat([kp[b, h], ks[:t_done, b, h]]) if t_done else kp[b, h]
            hist_v = torch.cat([vp[b, h], vs[:t_done, b, h]]) if t_done else vp[b, h]
            pos = np.arange(n + t_done)
            exp_k, held = oracle.ring_expected(hist_k.view(torch.int16).numpy(), pos, s, p_last)
            exp_v, _ = oracle.ring_expected(hist_v.view(torch.int16).numpy(), pos, s, p_last)
            assert (held == ring_positions(s, p_last)).all()
            assert np.array_equal(ring_k(kc_h, lay, b, h).view(torch.int16).numpy(), exp_k), (b, h)
            assert np.array_equal(ring_v(vc_h, lay, b, h).contiguous().view(torch.int16).numpy(),
                                  exp_v), (b, h)


CASES = [
    # B, Hq, Hkv, D, N, alpha, beta, T
    (3, 4, 2, 128, 300, [0, 100], [0.0, 0.0], 5),
    (2, 4, 4, 128, 300, [0, 64, 0, 0], [0.0, 0.0, 1.0, 0.5], 4),
    (2, 16, 2, 128, 2500, [0, 1500], [1.0, 0.0], 4),
    (2, 8, 1, 64, 1100, [0], [0.97], 3),
    (1, 1, 1, 128, 5, [0], [0.5], 6),
    (2, 6, 3, 64, 2049, [0, 64, 2000], [1.0, 0.0, 0.0], 3),
    # rings of exactly one and two 1024-slot chunks
    (1, 4, 2, 128, 1024, [1024, 0], [0.0, 0.5], 3),
    (1, 2, 2, 128, 2048, [0, 0], [1.0, 0.5], 3),
    # the largest group the boundary takes (G = 16), multi-chunk rings, D 128 and 64
    (2, 16, 1, 128, 1500, [0], [0.6], 3),
    (1, 32, 2, 64, 2100, [0, 1100], [0.5, 0.0], 3),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_handoff_append_decode(moa, case):
    bsz, hq, hkv, d, n, alpha, beta, t_steps = CASES[case]
    log(f"decode case {case}: B{bsz} Hq{hq} Hkv{hkv} D{d} N{n} T{t_steps}")
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta)
    lay = Layout(alpha, beta, bsz, d, n)
    kp, vp, qs, ks, vs = _prompt_and_steps(bsz, hq, hkv, n, d, t_steps, 5000 + 10 * case)
    kc, vc = plan.new_cache()
    ws = plan.new_workspace()
    plan.kv_append(kc, vc, kp.cuda(), vp.cuda(), 0)
    torch.cuda.synchronize()
    _check_rings(lay, kc, vc, kp, vp, ks, vs, n, 0)
    outs = []
    for t in range(t_steps):
        plan.kv_append(kc, vc, ks[t].unsqueeze(2).cuda(), vs[t].unsqueeze(2).cuda(), n + t)
        o = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
        plan.decode(qs[t].cuda(), kc, vc, n + t, o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    _check_rings(lay, kc, vc, kp, vp, ks, vs, n, t_steps)
    want = oracle.decode(f64(qs), [f64(kp[:, h]) for h in range(hkv)],
                         [f64(vp[:, h]) for h in range(hkv)], f64(ks), f64(vs), lay.spans, n)
    got = np.stack([f64(o) for o in outs])
    err = max_err(got, want)
    log(f"case {case} spans {list(lay.spans)} max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL


def test_decode_span_one_returns_new_value_exactly(moa):
    log("decode span-1")
    bsz, hq, hkv, d, n = 2, 4, 2, 128, 70
    plan = moa.Plan(bsz, hq, hkv, d, n, [0, 0], [0.0, 0.0])
    kp, vp, qs, ks, vs = _prompt_and_steps(bsz, hq, hkv, n, d, 2, 61)
    kc, vc = plan.new_cache()
    ws = plan.new_workspace()
    plan.kv_append(kc, vc, kp.cuda(), vp.cuda(), 0)
    for t in range(2):
        plan.kv_append(kc, vc, ks[t].unsqueeze(2).cuda(), vs[t].unsqueeze(2).cuda(), n + t)
        o = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
        plan.decode(qs[t].cuda(), kc, vc, n + t, o, ws)
        assert torch.equal(o.cpu(), vs[t].repeat_interleave(2, dim=1))


def test_decode_repeat_is_deterministic(moa):
    """Same inputs twice give the same bits (no ordering-dependent reduction)."""
    log("decode determinism")
    bsz, hq, hkv, d, n = 2, 8, 2, 128, 3000
    plan = moa.Plan(bsz, hq, hkv, d, n, [0, 0], [1.0, 0.6])
    kp, vp, qs, ks, vs = _prompt_and_steps(bsz, hq, hkv, n, d, 1, 63)
    kc, vc = plan.new_cache()
    ws = plan.new_workspace()
    plan.kv_append(kc, vc, kp.cuda(), vp.cuda(), 0)
    plan.kv_append(kc, vc, ks[0].unsqueeze(2).cuda(), vs[0].unsqueeze(2).cuda(), n)
    o1 = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    plan.decode(qs[0].cuda(), kc, vc, n, o1, ws)
    plan.decode(qs[0].cuda(), kc, vc, n, o2, ws)
    assert torch.equal(o1, o2)


def test_decode_argument_errors(moa):
    log("decode argument errors")
    plan = moa.Plan(1, 2, 2, 128, 64, [0, 0], [1.0, 1.0])
    kc, vc = plan.new_cache()
    q = torch.zeros(1, 2, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(moa.MoaError) as e:
        plan.decode(q, kc, vc, 64, o, small)
    assert e.value.status == moa.MOA_EWORKSPACE
    with pytest.raises(moa.MoaError) as e:
        plan.decode(q, kc, vc, 63, o, plan.new_workspace())
    assert e.value.status == moa.MOA_EINVAL
    f32 = moa.Plan(1, 2, 2, 128, 64, [0, 0], [1.0, 1.0], dtype="f32")
    kf, vf = f32.new_cache()
    with pytest.raises(moa.MoaError) as e:
        f32.decode(q.float(), kf, vf, 64, o.float(), f32.new_workspace())
    assert e.value.status == moa.MOA_EUNSUPPORTED
    with pytest.raises(ValueError):
        plan.decode(q[:, :1], kc, vc, 64, o, plan.new_workspace())


# Grouped heads at a size where the plan takes the fixed cut at 3072 slots (the rule of
# moa_plan_decode_chunks: more rings than one round of resident workgroups, and at least
# eight rounds of chunks): B128 Hq64 Hkv8 D128 N24576 with the 64-head 64k rules.
GQA_3072 = workloads.Workload("gqa_chunk3072", "decode", 128, 64, 8, 128, 24576, "bf16", 3, "c4",
                              2005, "B128 Hq64 Hkv8 D128 N24576 bf16, 3072-slot decode chunks")


# Grouped heads at sizes where the plan takes the balanced cut, launched longest first (the
# rule of moa_plan_decode_chunks), with the 64-head 64k rules: group size 4 at head dim 128,
# and group size 8 at head dim 64 (two rounds of 1280 resident workgroups).
GQA_BAL4 = workloads.Workload("gqa_balanced_g4", "decode", 16, 32, 8, 128, 24576, "bf16", 3, "c4",
                              2006, "B16 Hq32 Hkv8 D128 N24576 bf16, balanced decode cut")
GQA_BAL_D64 = workloads.Workload("gqa_balanced_d64", "decode", 32, 64, 8, 64, 32768, "bf16", 3,
                                 "c4", 2007, "B32 Hq64 Hkv8 D64 N32768 bf16, balanced decode cut")
EXTRA = {w.name: w for w in (GQA_3072, GQA_BAL4, GQA_BAL_D64)}


@pytest.mark.parametrize("name", ["c2_decode", "c3_decode", "c4_decode", "gqa_chunk3072",
                                  "gqa_balanced_g4", "gqa_balanced_d64"])
def test_decode_full_size_every_head(moa, name):
    """Full-size rings (device-filled with seeded N(0,1)), three steps, every (b, h) of every
    step checked against the oracle's explicit-window decode."""
    w = EXTRA.get(name) or workloads.WORKLOADS[name]
    alpha, beta = workloads.rules("c4_decode" if name in EXTRA else name)
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    lay = Layout(alpha, beta, w.batch, w.head_dim, w.n_prompt)
    assert plan.cache_elems == lay.total_slots * w.head_dim
    ch = plan.decode_chunks()
    uneven = bool(np.any((ch[:, 3] != plan.decode_chunk) & (ch[:, 2] + ch[:, 3] < lay.spans[ch[:, 1]])))
    ring_order = bool((np.diff(ch[:, 0] * w.n_kv_heads + ch[:, 1]) >= 0).all())
    log(f"{name}: decode chunk {plan.decode_chunk} slots, {len(ch)} chunks"
        f"{', launched longest first' if not ring_order else ''}")
    if name == "gqa_chunk3072":         # the fixed cut
        assert plan.decode_chunk == 3072 and not uneven and ring_order
    if name in ("c4_decode", "gqa_balanced_g4", "gqa_balanced_d64"):   # balanced, longest first
        assert not ring_order and (np.diff(ch[:, 3]) <= 0).all()
        assert len(ch) <= 2 * 256 * (2 if w.head_dim == 128 else 5)
    log(f"{name}: filling {2 * plan.cache_elems * 2 / 1e9:.2f} GB of rings")
    kc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16,
                                              device="cuda"), 81)
    vc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16,
                                              device="cuda"), 82)
    ws = plan.new_workspace()
    t_steps = 3
    n = w.n_prompt
    g = w.n_q_heads // w.n_kv_heads
    qs, ks, vs = workloads.decode_step_inputs(w.batch, w.n_q_heads, w.n_kv_heads, t_steps,
                                              w.head_dim, "bf16", w.data_seed)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    # the prompt rings as the steps find them, on the host (bf16)
    kc_h, vc_h = kc.cpu(), vc.cpu()
    outs = []
    for t in range(t_steps):
        log(f"{name}: step {t}")
        plan.kv_append(kc, vc, ks[t].unsqueeze(2).cuda(), vs[t].unsqueeze(2).cuda(), n + t)
        o = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
        plan.decode(qs[t].cuda(), kc, vc, n + t, o, ws)
        outs.append(o.cpu())
    torch.cuda.synchronize()
    ks64, vs64, qs64 = f64(ks), f64(vs), f64(qs)
    outs64 = [f64(o) for o in outs]

    def check(pair):
        """Worst error of one (b, h) over the steps, and the step it occurs at."""
        b, h = pair
        s = int(lay.spans[h])
        order = np.argsort(ring_positions(s, n - 1))   # the prompt tail, by position
        hist_k = np.empty((s + t_steps, w.head_dim))
        hist_v = np.empty((s + t_steps, w.head_dim))
        hist_k[:s] = f64(ring_k(kc_h, lay, b, h))[order]
        hist_v[:s] = f64(ring_v(vc_h, lay, b, h))[order]
        res = (0.0, -1)
        for t in range(t_steps):
            hist_k[s + t], hist_v[s + t] = ks64[t, b, h], vs64[t, b, h]
            want = oracle.decode_step(qs64[t, b, h * g:(h + 1) * g], hist_k[:s + t + 1],
                                      hist_v[:s + t + 1], np.arange(n - s, n + t + 1), n + t, s)
            res = max(res, (max_err(outs64[t][b, h * g:(h + 1) * g], want), t))
        return res

    # eight heads at a time, one BLAS thread each (long rings would oversubscribe the cores)
    with threadpool_limits(1), ThreadPoolExecutor(8) as ex:
        errs = list(ex.map(check, pairs))
    worst = max(e for e, _ in errs)
    bad = [(b, h, t, e) for (b, h), (e, t) in zip(pairs, errs) if e > TOL]
    assert not bad, (name, bad[:8])
    log(f"{name}: every (b, h) of {t_steps} steps, worst err {worst:.3e}")


@pytest.mark.parametrize("name", ["c2_decode", "c3_decode", "c4_decode"])
def test_decode_full_size_long_run(moa, name):
    """All T steps of a decode workload through the fused call (the bench's step) on
    full-size rings: every (b, h) checked against the oracle at steps 0, 1, 2, T/2 and T-1,
    the first and last sequence at every step, and their rings bit for bit after the last
    step (by then the steps have overwritten the oldest T slots of every ring)."""
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    lay = Layout(alpha, beta, w.batch, w.head_dim, w.n_prompt)
    t_steps, n, g, bsz = w.steps, w.n_prompt, w.n_q_heads // w.n_kv_heads, w.batch
    log(f"{name} long run: {t_steps} fused steps, filling {2 * plan.cache_elems * 2 / 1e9:.2f} GB")
    kc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16,
                                              device="cuda"), 83)
    vc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16,
                                              device="cuda"), 84)
    kc_h, vc_h = kc.cpu(), vc.cpu()       # the prompt rings, for the oracle's history
    ws = plan.new_workspace()
    qs, ks, vs = workloads.decode_step_inputs(bsz, w.n_q_heads, w.n_kv_heads, t_steps,
                                              w.head_dim, "bf16", w.data_seed + 7)
    all_b = {0, 1, 2, t_steps // 2, t_steps - 1}
    edge_b = sorted({0, bsz - 1})
    outs = {}
    o = torch.empty(bsz, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
    for t in range(t_steps):
        plan.append_decode(qs[t].cuda(), kc, vc, ks[t].cuda(), vs[t].cuda(), n + t, o, ws)
        outs[t] = f64(o) if t in all_b else f64(o[edge_b])
        if t % 64 == 0:
            log(f"{name}: step {t}")
    torch.cuda.synchronize()
    ks64, vs64, qs64 = f64(ks), f64(vs), f64(qs)

    def check(pair):
        b, h = pair
        s = int(lay.spans[h])
        order = np.argsort(ring_positions(s, n - 1))   # the prompt tail, by position
        hist_k = np.concatenate([f64(ring_k(kc_h, lay, b, h))[order], ks64[:, b, h]])
        hist_v = np.concatenate([f64(ring_v(vc_h, lay, b, h))[order], vs64[:, b, h]])
        steps = range(t_steps) if b in edge_b else sorted(all_b)
        res = (0.0, -1)
        for t in steps:
            got = outs[t][b] if t in all_b else outs[t][edge_b.index(b)]
            want = oracle.decode_step(qs64[t, b, h * g:(h + 1) * g], hist_k[:s + t + 1],
                                      hist_v[:s + t + 1], np.arange(n - s, n + t + 1), n + t, s)
            res = max(res, (max_err(got[h * g:(h + 1) * g], want), t))
        return res

    pairs = [(b, h) for b in range(bsz) for h in range(w.n_kv_heads)]
    with threadpool_limits(1), ThreadPoolExecutor(8) as ex:
        errs = []
        for i in range(0, len(pairs), 256):
            errs += list(ex.map(check, pairs[i:i + 256]))
            log(f"{name}: checked {min(i + 256, len(pairs))} of {len(pairs)} (b, h)")
    worst = max(e for e, _ in errs)
    bad = [(b, h, t, e) for (b, h), (e, t) in zip(pairs, errs) if e > TOL]
    assert not bad, (name, bad[:8])
    log(f"{name}: {t_steps} steps, worst err {worst:.3e}")

    # rings of the first and last sequence after the last step, bit for bit
    kc_e, vc_e = kc.cpu(), vc.cpu()
    p_last = n - 1 + t_steps
    for b in edge_b:
        for h in range(w.n_kv_heads):
            s = int(lay.spans[h])
            order = np.argsort(ring_positions(s, n - 1))
            hk = torch.cat([ring_k(kc_h, lay, b, h)[order], ks[:, b, h]])
            hv = torch.cat([ring_v(vc_h, lay, b, h)[order], vs[:, b, h]])
            pos = np.arange(n - s, n + t_steps)
            exp_k, held = oracle.ring_expected(hk.view(torch.int16).numpy(), pos, s, p_last)
            exp_v, _ = oracle.ring_expected(hv.contiguous().view(torch.int16).numpy(), pos, s,
                                            p_last)
            assert (held == ring_positions(s, p_last)).all()
            assert np.array_equal(ring_k(kc_e, lay, b, h).view(torch.int16).numpy(), exp_k), (b, h)
            assert np.array_equal(ring_v(vc_e, lay, b, h).contiguous().view(torch.int16).numpy(),
                                  exp_v), (b, h)
    log(f"{name}: rings of sequences {edge_b} match the oracle after {t_steps} steps")
