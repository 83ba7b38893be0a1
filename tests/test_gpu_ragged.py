"""Per-sequence prompt lengths (left-padded ragged batch) against the oracle.

Sequence b of a ragged plan must behave exactly like a batch of one with
N = N_b: its spans are the rule at N_b, its prefill rows, ring contents and
decode outputs are those the oracle computes for that sequence alone.  The
padding rows of q, k and v hold NaN, so any read of them would poison the
outputs; o is pre-filled with a sentinel that padding rows must keep.
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
SENTINEL = 7.0
_BITS = {torch.bfloat16: torch.int16, torch.float32: torch.int32}


def _bits(t):
    return t.contiguous().view(_BITS[t.dtype]).numpy()


def _poison(t, lens):
    """NaN in the left-padding rows of a [B, H, N, D] tensor."""
    n = t.shape[2]
    for b, nb in enumerate(lens):
        t[b, :, :n - nb] = float("nan")
    return t


def _check_rings(lay, kc, vc, kp, vp, ks, vs, t_done):
    """Ring (b, h) holds the oracle's slots for sequence b's own history (spans and ring
    locations from the oracle's layout)."""
    kc_h, vc_h = kc.cpu(), vc.cpu()
    n = max(lay.seq_len)
    for b, nb in enumerate(lay.seq_len):
        pad = n - nb
        for h in range(lay.n_kv_heads):
            s = int(lay.seq_spans[b, h])
            hist_k, hist_v = kp[b, h, pad:], vp[b, h, pad:]
            if t_done:
                hist_k = torch.cat([hist_k, ks[:t_done, b, h]])
                hist_v = torch.cat([hist_v, vs[:t_done, b, h]])
            pos = np.arange(nb + t_done)
            exp_k, held = oracle.ring_expected(_bits(hist_k), pos, s, nb - 1 + t_done)
            exp_v, _ = oracle.ring_expected(_bits(hist_v), pos, s, nb - 1 + t_done)
            assert (held == ring_positions(s, nb - 1 + t_done)).all()
            assert np.array_equal(_bits(ring_k(kc_h, lay, b, h)), exp_k), (b, h)
            assert np.array_equal(_bits(ring_v(vc_h, lay, b, h)), exp_v), (b, h)


CASES = [
    # Hq, Hkv, D, seq_len, alpha, beta, dtype
    (4, 2, 128, [300, 1, 64, 299], [0, 100], [0.5, 0.0], "bf16"),
    (8, 4, 64, [1000, 513, 777], [0, 64, 300, 0], [0.25, 0.0, 0.0, 1.0], "bf16"),
    (16, 2, 128, [2500, 2499, 1024, 1025, 31], [0, 1500], [1.0, 0.0], "bf16"),
    (4, 2, 64, [333, 100, 200], [0, 200], [0.5, 0.0], "f32"),
    (2, 2, 128, [257, 130], [0, 64], [1.0, 0.0], "f32"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_ragged_prefill_and_handoff(moa, case):
    hq, hkv, d, lens, alpha, beta, dt = CASES[case]
    bsz, n = len(lens), max(lens)
    log(f"ragged prefill case {case}: B{bsz} Hq{hq} Hkv{hkv} D{d} lens {lens} {dt}")
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta, dtype=dt, seq_len=lens)
    lay = Layout(alpha, beta, bsz, d, n, seq_len=lens)
    q, k, v = workloads.prefill_inputs(bsz, hq, hkv, n, d, dt, 9000 + case)
    q, k, v = _poison(q, lens), _poison(k, lens), _poison(v, lens)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, SENTINEL)
    plan.prefill(qd, kd, vd, o)
    o2 = torch.full_like(qd, SENTINEL)
    kc, vc = plan.new_cache()
    plan.prefill_handoff(qd, kd, vd, o2, kc, vc)
    kc2, vc2 = plan.new_cache()
    plan.kv_append(kc2, vc2, kd, vd, 0)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    o_h = o.cpu()
    worst = 0.0
    for b, nb in enumerate(lens):
        pad = n - nb
        want = oracle.prefill(f64(q[b:b + 1, :, pad:]), f64(k[b:b + 1, :, pad:]),
                              f64(v[b:b + 1, :, pad:]), lay.seq_spans[b])
        err = max_err(f64(o_h[b:b + 1, :, pad:]), want)
        worst = max(worst, err)
        assert err <= TOL[dt], (b, nb, err)
        assert (o_h[b, :, :pad] == SENTINEL).all(), b
    log(f"case {case} worst err {worst:.3e}")
    _check_rings(lay, kc, vc, k, v, None, None, 0)
    _check_rings(lay, kc2, vc2, k, v, None, None, 0)


DECODE_CASES = [c for c in CASES if c[6] == "bf16"]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_ragged_decode(moa, case, fused):
    hq, hkv, d, lens, alpha, beta, _ = DECODE_CASES[case]
    bsz, n, t_steps = len(lens), max(lens), 3
    log(f"ragged decode case {case} fused={fused}: B{bsz} lens {lens}")
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta, seq_len=lens)
    lay = Layout(alpha, beta, bsz, d, n, seq_len=lens)
    _, kp, vp = workloads.prefill_inputs(bsz, hq, hkv, n, d, "bf16", 9100 + case)
    kp, vp = _poison(kp, lens), _poison(vp, lens)
    qs, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, t_steps, d, "bf16", 9101 + case)
    kc, vc = plan.new_cache()
    ws = plan.new_workspace()
    plan.kv_append(kc, vc, kp.cuda(), vp.cuda(), 0)
    outs = []
    for t in range(t_steps):
        o = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
        if fused:
            plan.append_decode(qs[t].cuda(), kc, vc, ks[t].cuda(), vs[t].cuda(), n + t, o, ws)
        else:
            plan.kv_append(kc, vc, ks[t].unsqueeze(2).cuda(), vs[t].unsqueeze(2).cuda(), n + t)
            plan.decode(qs[t].cuda(), kc, vc, n + t, o, ws)
        outs.append(o.cpu())
    torch.cuda.synchronize()
    _check_rings(lay, kc, vc, kp, vp, ks, vs, t_steps)
    got = np.stack([f64(o) for o in outs])
    worst = 0.0
    for b, nb in enumerate(lens):
        pad = n - nb
        want = oracle.decode(f64(qs[:, b:b + 1]), [f64(kp[b:b + 1, h, pad:]) for h in range(hkv)],
                             [f64(vp[b:b + 1, h, pad:]) for h in range(hkv)],
                             f64(ks[:, b:b + 1]), f64(vs[:, b:b + 1]), lay.seq_spans[b], nb)
        err = max_err(got[:, b:b + 1], want)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (b, nb, err)
    log(f"case {case} worst err {worst:.3e}")


def test_ragged_full_size_every_head(moa):
    """Vicuna-7B-shaped rules (32 heads, N up to 16384), 16 sequences of seeded lengths,
    device-filled prompt K/V handed over by the fused prefill, then fused decode steps;
    every (sequence, head) against the oracle: three 64-row prefill blocks per query head
    and both decode steps."""
    name = "c2_decode"
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    rng = np.random.Generator(np.random.PCG64(4242))
    lens = [int(x) for x in rng.integers(1, w.n_prompt + 1, 15)] + [w.n_prompt]
    bsz, n, d, hq, hkv = len(lens), w.n_prompt, w.head_dim, w.n_q_heads, w.n_kv_heads
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta, seq_len=lens)
    log(f"ragged full size: B{bsz} lens {lens}")
    shape_q, shape_kv = (bsz, hq, n, d), (bsz, hkv, n, d)
    q = workloads.device_normal_(torch.empty(shape_q, dtype=torch.bfloat16, device="cuda"), 91)
    k = workloads.device_normal_(torch.empty(shape_kv, dtype=torch.bfloat16, device="cuda"), 92)
    v = workloads.device_normal_(torch.empty(shape_kv, dtype=torch.bfloat16, device="cuda"), 93)
    o = torch.empty_like(q)
    kc, vc = plan.new_cache()
    ws = plan.new_workspace()
    plan.prefill_handoff(q, k, v, o, kc, vc)
    t_steps = 2
    qs, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, t_steps, d, "bf16", 94)
    outs = []
    for t in range(t_steps):
        od = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
        plan.append_decode(qs[t].cuda(), kc, vc, ks[t].cuda(), vs[t].cuda(), n + t, od, ws)
        outs.append(od.cpu())
    torch.cuda.synchronize()
    g = hq // hkv
    k64, v64, ks64, vs64, qs64 = f64(k), f64(v), f64(ks), f64(vs), f64(qs)
    outs64 = [f64(od) for od in outs]
    o_h, q_h = o.cpu(), q.cpu()
    blk = 64

    def check(pair):
        """Worst prefill and decode errors of one (sequence, KV head)."""
        b, h = pair
        nb, pad = lens[b], n - lens[b]
        s = int(oracle.spans(alpha, beta, nb)[h])
        kb, vb = k64[b, h, pad:], v64[b, h, pad:]
        # prefill: 64-row blocks at the sequence's first rows, around S_h and its last rows
        e_pre = 0.0
        starts = sorted({0, min(max(0, s - blk // 2), max(0, nb - blk)), max(0, nb - blk)})
        for hh in range(h * g, (h + 1) * g):
            for i0 in starts:
                r = min(blk, nb - i0)
                want = oracle.prefill_row_block(f64(q_h[b, hh, pad + i0:pad + i0 + r]), kb, vb,
                                                s, i0)
                e_pre = max(e_pre, max_err(f64(o_h[b, hh, pad + i0:pad + i0 + r]), want))
        e_dec = 0.0
        hist_k = np.concatenate([kb[nb - s:], ks64[:t_steps, b, h]])
        hist_v = np.concatenate([vb[nb - s:], vs64[:t_steps, b, h]])
        for t in range(t_steps):
            want = oracle.decode_step(qs64[t, b, h * g:(h + 1) * g], hist_k[:s + t + 1],
                                      hist_v[:s + t + 1], np.arange(nb - s, nb + t + 1), nb + t, s)
            e_dec = max(e_dec, max_err(outs64[t][b, h * g:(h + 1) * g], want))
        return e_pre, e_dec

    pairs = [(b, h) for b in range(bsz) for h in range(hkv)]
    with threadpool_limits(1), ThreadPoolExecutor(8) as ex:
        errs = list(ex.map(check, pairs))
    bad = [(p, e) for p, e in zip(pairs, errs) if max(e) > TOL["bf16"]]
    assert not bad, bad[:8]
    log(f"ragged full size, every (b, h): worst prefill err {max(e[0] for e in errs):.3e}, "
        f"decode err {max(e[1] for e in errs):.3e}")
