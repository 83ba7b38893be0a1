"""Appends of several tokens at once after the prompt (moa_kv_append with n_new > 1 at
pos0 > 0) against the oracle.

The chunks are shorter than a ring, longer than a ring (only the last S rows of such a
chunk survive, each at slot p mod S), a single token, and longer than every ring. Both
uniform and left-padded ragged batches are covered. After every chunk, every slot of
every ring must hold the bits of the position the oracle's ring layout puts there. A
decode of the last position then attends exactly the window of the whole history. fp32
plans have no decode, so only their rings are checked.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Layout, f64, log, max_err, ring_k, ring_positions, ring_v

pytestmark = pytest.mark.gpu

_BITS = {torch.bfloat16: torch.int16, torch.float32: torch.int32}


def _bits(t):
    return t.contiguous().view(_BITS[t.dtype]).numpy()


CASES = [
    # Hq, Hkv, D, N, seq_len, alpha, beta, dtype, chunk sizes
    (4, 2, 64, 300, None, [64, 0], [0.0, 0.5], "bf16", [5, 70, 1, 200, 33]),
    (8, 4, 128, 513, [513, 200, 64], [0, 64, 300, 0], [0.25, 0.0, 0.0, 1.0], "bf16",
     [64, 3, 129, 1, 600]),
    (4, 2, 128, 257, [257, 130], [0, 64], [1.0, 0.0], "f32", [3, 64, 65, 1, 300]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_append_chunks_mid_stream(moa, case):
    hq, hkv, d, n, lens, alpha, beta, dt, chunks = CASES[case]
    bsz = 2 if lens is None else len(lens)
    log(f"append chunks case {case}: B{bsz} Hq{hq} Hkv{hkv} D{d} N{n} lens {lens} {dt} "
        f"chunks {chunks}")
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta, dtype=dt, seq_len=lens)
    lay = Layout(alpha, beta, bsz, d, n, seq_len=lens)
    _, kp, vp = workloads.prefill_inputs(bsz, hq, hkv, n, d, dt, 9300 + case)
    for b, nb in enumerate(lay.seq_len):      # padding rows hold NaN: never read
        kp[b, :, :n - nb] = float("nan")
        vp[b, :, :n - nb] = float("nan")
    kc, vc = plan.new_cache()
    plan.kv_append(kc, vc, kp.cuda(), vp.cuda(), 0)
    hist_k = [[kp[b, h, n - nb:] for h in range(hkv)] for b, nb in enumerate(lay.seq_len)]
    hist_v = [[vp[b, h, n - nb:] for h in range(hkv)] for b, nb in enumerate(lay.seq_len)]
    done = 0
    for i, c in enumerate(chunks):
        _, ks, vs = workloads.decode_step_inputs(bsz, hq, hkv, c, d, dt, 9310 + 10 * case + i)
        kn = ks.permute(1, 2, 0, 3).contiguous()          # [B, Hkv, c, D]
        vn = vs.permute(1, 2, 0, 3).contiguous()
        plan.kv_append(kc, vc, kn.cuda(), vn.cuda(), n + done)
        done += c
        torch.cuda.synchronize()
        kc_h, vc_h = kc.cpu(), vc.cpu()
        for b, nb in enumerate(lay.seq_len):
            p_last = nb - 1 + done
            for h in range(hkv):
                hist_k[b][h] = torch.cat([hist_k[b][h], kn[b, h]])
                hist_v[b][h] = torch.cat([hist_v[b][h], vn[b, h]])
                s = int(lay.seq_spans[b, h])
                pos = np.arange(nb + done)
                exp_k, held = oracle.ring_expected(_bits(hist_k[b][h]), pos, s, p_last)
                exp_v, _ = oracle.ring_expected(_bits(hist_v[b][h]), pos, s, p_last)
                assert (held == ring_positions(s, p_last)).all()
                assert np.array_equal(_bits(ring_k(kc_h, lay, b, h)), exp_k), (i, c, b, h)
                assert np.array_equal(_bits(ring_v(vc_h, lay, b, h)), exp_v), (i, c, b, h)
        log(f"  chunk {i} ({c} tokens): rings match the oracle")
    if dt != "bf16":
        return
    # one decode of the last position over the rings the chunks left
    g = hq // hkv
    qs, _, _ = workloads.decode_step_inputs(bsz, hq, hkv, 1, d, dt, 9399 + case)
    o = torch.empty(bsz, hq, d, dtype=torch.bfloat16, device="cuda")
    plan.decode(qs[0].cuda(), kc, vc, n + done - 1, o, plan.new_workspace())
    torch.cuda.synchronize()
    got = f64(o)
    worst = 0.0
    for b, nb in enumerate(lay.seq_len):
        p = nb - 1 + done
        for h in range(hkv):
            want = oracle.decode_step(f64(qs[0, b, h * g:(h + 1) * g]), f64(hist_k[b][h]),
                                      f64(hist_v[b][h]), np.arange(nb + done), p,
                                      int(lay.seq_spans[b, h]))
            worst = max(worst, max_err(got[b, h * g:(h + 1) * g], want))
    log(f"  decode after the chunks: max abs err {worst:.3e}")
    assert worst <= 2e-2
