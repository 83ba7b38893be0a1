"""Seeded random configurations through the whole path, against the oracle.

Each case draws its own shape from a seeded PCG64 stream:
- batch 1-4, 1-4 KV heads of group size 1, 2 or 4, head dim 64 or 128, and a prompt of
  1-700 tokens; or, in the wide-group cases, batch 1-2, 1-2 KV heads of group size 8 or 16
  and a prompt of 700-1500 tokens;
- a uniform or a left-padded ragged batch (NaN in the padding rows);
- rules with non-dyadic beta, and alpha up to past N;
- bf16 for most cases, fp32 for every fourth.

Checks on every case:
- the plain prefill against the oracle;
- the fused prefill + handoff bit for bit against it;
- every ring slot after the handoff against the oracle's layout.

bf16 cases also run three decode steps (fused, separate, fused) and check their outputs
and the rings again. Spans and ring locations come from the oracle alone.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Layout, f64, log, max_err, ring_k, ring_positions, ring_v

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
_BITS = {torch.bfloat16: torch.int16, torch.float32: torch.int32}
N_CASES = int(os.environ.get("MOA_RANDOM_CASES", "24"))   # more for an extended run
N_WIDE = int(os.environ.get("MOA_RANDOM_WIDE_CASES", "8"))


def _bits(t):
    return t.contiguous().view(_BITS[t.dtype]).numpy()


def _case(i, wide=False):
    rng = np.random.Generator(np.random.PCG64((7373 if wide else 4242) + i))
    if wide:    # wide groups, longer prompts
        hkv = int(rng.integers(1, 3))
        g = int(rng.choice([8, 16]))
        d = int(rng.choice([64, 128]))
        bsz = int(rng.integers(1, 3))
        n = int(rng.integers(700, 1501))
    else:
        hkv = int(rng.integers(1, 5))
        g = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        bsz = int(rng.integers(1, 5))
        n = int(rng.integers(1, 701))
    dt = "f32" if i % 4 == 3 else "bf16"
    lens = None
    if bsz > 1 and rng.integers(0, 2):
        lens = [int(x) for x in rng.integers(1, n + 1, bsz)]
        lens[int(rng.integers(0, bsz))] = n
    alpha = [int(rng.integers(1, n + 200)) if rng.integers(0, 2) else 0 for _ in range(hkv)]
    beta = [float(rng.random()) if rng.integers(0, 3) else 0.0 for _ in range(hkv)]
    return bsz, hkv * g, hkv, d, n, lens, alpha, beta, dt


def _check_rings(lay, kc, vc, hist_k, hist_v, done):
    kc_h, vc_h = kc.cpu(), vc.cpu()
    for b, nb in enumerate(lay.seq_len):
        p_last = nb - 1 + done
        for h in range(lay.n_kv_heads):
            s = int(lay.seq_spans[b, h])
            pos = np.arange(nb + done)
            exp_k, held = oracle.ring_expected(_bits(hist_k[b][h]), pos, s, p_last)
            exp_v, _ = oracle.ring_expected(_bits(hist_v[b][h]), pos, s, p_last)
            assert (held == ring_positions(s, p_last)).all()
            assert np.array_equal(_bits(ring_k(kc_h, lay, b, h)), exp_k), (b, h, done)
            assert np.array_equal(_bits(ring_v(vc_h, lay, b, h)), exp_v), (b, h, done)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_configuration(moa, case):
    _run_case(moa, case, *_case(case))


@pytest.mark.parametrize("case", range(N_WIDE))
def test_random_configuration_wide_groups(moa, case):
    _run_case(moa, case, *_case(case, wide=True))


def _run_case(moa, case, bsz, hq, hkv, d, n, lens, alpha, beta, dt):
    log(f"random case {case}: B{bsz} Hq{hq} Hkv{hkv} D{d} N{n} lens {lens} {dt} "
        f"alpha {alpha} beta {[round(x, 4) for x in beta]}")
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta, dtype=dt, seq_len=lens)
    lay = Layout(alpha, beta, bsz, d, n, seq_len=lens)
    g = hq // hkv
    q, k, v = workloads.prefill_inputs(bsz, hq, hkv, n, d, dt, 9500 + case)
    for b, nb in enumerate(lay.seq_len):
        for t in (q, k, v):
            t[b, :, :n - nb] = float("nan")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o_plain = torch.empty_like(qd)
    o = torch.empty_like(qd)
    kc, vc = plan.new_cache()
    plan.prefill(qd, kd, vd, o_plain)
    plan.prefill_handoff(qd, kd, vd, o, kc, vc)
    torch.cuda.synchronize()
    o_h, o_plain_h = o.cpu(), o_plain.cpu()
    worst = 0.0
    for b, nb in enumerate(lay.seq_len):
        pad = n - nb
        want = oracle.prefill(f64(q[b:b + 1, :, pad:]), f64(k[b:b + 1, :, pad:]),
                              f64(v[b:b + 1, :, pad:]), lay.seq_spans[b])
        worst = max(worst, max_err(f64(o_h[b:b + 1, :, pad:]), want))
        assert torch.equal(o_h[b, :, pad:], o_plain_h[b, :, pad:]), b
    log(f"  prefill max abs err {worst:.3e} (spans {lay.seq_spans.tolist()})")
    assert worst <= TOL[dt]
    hist_k = [[k[b, h, n - nb:] for h in range(hkv)] for b, nb in enumerate(lay.seq_len)]
    hist_v = [[v[b, h, n - nb:] for h in range(hkv)] for b, nb in enumerate(lay.seq_len)]
    _check_rings(lay, kc, vc, hist_k, hist_v, 0)
    if dt != "bf16":
        return

    t_steps = 3
    qs, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, t_steps, d, dt, 9600 + case)
    ws = plan.new_workspace()
    worst = 0.0
    for t in range(t_steps):
        od = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
        if t % 2 == 0:
            plan.append_decode(qs[t].cuda(), kc, vc, ks[t].cuda(), vs[t].cuda(), n + t, od, ws)
        else:
            plan.kv_append(kc, vc, ks[t].unsqueeze(2).cuda(), vs[t].unsqueeze(2).cuda(), n + t)
            plan.decode(qs[t].cuda(), kc, vc, n + t, od, ws)
        torch.cuda.synchronize()
        got = f64(od)
        for b, nb in enumerate(lay.seq_len):
            for h in range(hkv):
                hist_k[b][h] = torch.cat([hist_k[b][h], ks[t, b, h:h + 1]])
                hist_v[b][h] = torch.cat([hist_v[b][h], vs[t, b, h:h + 1]])
                want = oracle.decode_step(f64(qs[t, b, h * g:(h + 1) * g]), f64(hist_k[b][h]),
                                          f64(hist_v[b][h]), np.arange(nb + t + 1), nb + t,
                                          int(lay.seq_spans[b, h]))
                worst = max(worst, max_err(got[b, h * g:(h + 1) * g], want))
        _check_rings(lay, kc, vc, hist_k, hist_v, t + 1)
    log(f"  decode ({t_steps} steps) max abs err {worst:.3e}")
    assert worst <= TOL[dt]
