"""Prefill parity: HIP kernels (through the C ABI) against the float64 oracle.

Tolerances: max-abs 1e-4 for float32, 2e-2 for bfloat16 inputs with float32
accumulation; the oracle sees the same bf16 bits, up-cast to float64.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f64, log, max_err, sample_rows

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _run_prefill(moa, plan, q, k, v):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(qd)
    plan.prefill(qd, kd, vd, o)
    torch.cuda.synchronize()
    return o


def test_c0_tiny_prefill_fp32(moa):
    w = workloads.WORKLOADS["c0_prefill"]
    alpha, beta = workloads.rules("c0_prefill")
    log("prefill c0 fp32 B1 H4 D64 N512")
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta,
                    dtype="f32")
    spans = oracle.spans(alpha, beta, w.n_prompt)
    assert list(spans) == [64, 128, 256, 512]
    q, k, v = workloads.prefill_inputs(w.batch, w.n_q_heads, w.n_kv_heads, w.n_prompt,
                                       w.head_dim, "f32", w.data_seed)
    o = _run_prefill(moa, plan, q, k, v)
    want = oracle.prefill(f64(q), f64(k), f64(v), spans)
    err = max_err(f64(o), want)
    log(f"c0 max abs err {err:.3e}")
    assert err <= TOL["f32"]


CASES = [
    # B, Hq, Hkv, D, N, alpha, beta, dtype
    (1, 4, 4, 128, 1000, [0, 64, 100, 0], [0.0, 0.0, 0.0, 1.0], "bf16"),
    (2, 8, 2, 128, 777, [0, 300], [0.25, 0.0], "bf16"),
    (1, 4, 4, 64, 1000, [1, 64, 700, 0], [0.0, 0.0, 0.0, 0.6], "bf16"),
    (2, 16, 2, 128, 300, [0, 0], [0.0, 1.0], "bf16"),
    (1, 2, 1, 128, 1, [0], [1.0], "bf16"),
    (1, 2, 2, 128, 130, [64, 0], [0.0, 0.0], "bf16"),
    (5, 4, 2, 128, 700, [0, 300], [0.5, 0.0], "bf16"),
    # prompt lengths at and just past tile boundaries (64-key tiles, 128-row units)
    (1, 4, 2, 128, 128, [0, 64], [1.0, 0.0], "bf16"),
    (1, 2, 2, 64, 64, [0, 1], [1.0, 0.0], "bf16"),
    (2, 4, 4, 128, 65, [0, 64, 1, 0], [0.5, 0.0, 0.0, 1.0], "bf16"),
    (1, 4, 2, 128, 256, [128, 0], [0.0, 0.5], "bf16"),
    (2, 4, 2, 64, 333, [0, 200], [0.5, 0.0], "f32"),
    # the largest group the boundary takes (G = 16), both dtypes
    (1, 16, 1, 128, 700, [0], [0.5], "bf16"),
    (1, 32, 2, 64, 300, [0, 100], [0.4, 0.0], "f32"),
    (1, 2, 2, 128, 257, [0, 64], [1.0, 0.0], "f32"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_small(moa, case):
    bsz, hq, hkv, d, n, alpha, beta, dt = CASES[case]
    log(f"prefill small case {case}: B{bsz} Hq{hq} Hkv{hkv} D{d} N{n} {dt}")
    plan = moa.Plan(bsz, hq, hkv, d, n, alpha, beta, dtype=dt)
    q, k, v = workloads.prefill_inputs(bsz, hq, hkv, n, d, dt, 3000 + case)
    o = _run_prefill(moa, plan, q, k, v)
    spans = oracle.spans(alpha, beta, n)
    want = oracle.prefill(f64(q), f64(k), f64(v), spans)
    err = max_err(f64(o), want)
    log(f"case {case} spans {list(spans)} max abs err {err:.3e}")
    assert np.isfinite(f64(o)).all()
    assert err <= TOL[dt]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_span_one_returns_v_exactly(moa, dt):
    log(f"prefill span-1 {dt}")
    plan = moa.Plan(2, 4, 2, 128, 200, [0, 0], [0.0, 0.0], dtype=dt)
    assert list(oracle.spans([0, 0], [0.0, 0.0], 200)) == [1, 1]
    q, k, v = workloads.prefill_inputs(2, 4, 2, 200, 128, dt, 41)
    o = _run_prefill(moa, plan, q, k, v).cpu()
    vrep = v.repeat_interleave(2, dim=1)
    assert torch.equal(o, vrep)


def test_prefill_constant_v(moa):
    log("prefill constant V")
    plan = moa.Plan(1, 4, 4, 128, 500, [0, 64, 0, 200], [1.0, 0.0, 0.3, 0.0])
    q, k, _ = workloads.prefill_inputs(1, 4, 4, 500, 128, "bf16", 43)
    v = torch.full((1, 4, 500, 128), 0.375, dtype=torch.bfloat16)
    o = _run_prefill(moa, plan, q, k, v)
    assert max_err(f64(o), 0.375) <= 0.375 * 2 ** -8


def test_c1_prefill_full_size_sampled_rows(moa):
    """Vicuna-7B-shaped prefill at full size; every head checked on sampled rows."""
    w = workloads.WORKLOADS["c1_prefill"]
    alpha, beta = workloads.rules("c1_prefill")
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    q, k, v = workloads.prefill_inputs(w.batch, w.n_q_heads, w.n_kv_heads, w.n_prompt,
                                       w.head_dim, "bf16", w.data_seed)
    log("prefill c1 full size")
    o = _run_prefill(moa, plan, q, k, v).cpu()
    spans = oracle.spans(alpha, beta, w.n_prompt)
    worst = 0.0
    for h in range(w.n_q_heads):
        s = int(spans[h])
        rows = sample_rows(w.n_prompt, s, 24, 100 + h)
        want = oracle.prefill_rows(f64(q[0, h, rows]), f64(k[0, h]), f64(v[0, h]), s, rows)
        err = max_err(f64(o[0, h, rows]), want)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (h, s, err)
    log(f"c1 worst sampled err {worst:.3e}")


def test_c1_prefill_full_size_every_row(moa):
    """Vicuna-7B-shaped prefill checked in full: every row of every head against the
    oracle's explicit-mask prefill, one head at a time (an 8192 x 8192 float64 score matrix
    per head)."""
    w = workloads.WORKLOADS["c1_prefill"]
    alpha, beta = workloads.rules("c1_prefill")
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    q, k, v = workloads.prefill_inputs(w.batch, w.n_q_heads, w.n_kv_heads, w.n_prompt,
                                       w.head_dim, "bf16", w.data_seed)
    log("prefill c1 full size, every row")
    o = _run_prefill(moa, plan, q, k, v).cpu()
    spans = oracle.spans(alpha, beta, w.n_prompt)
    worst = 0.0
    for h in range(w.n_q_heads):
        s = int(spans[h])
        want = oracle.prefill(f64(q[:, h:h + 1]), f64(k[:, h:h + 1]), f64(v[:, h:h + 1]), [s])
        err = max_err(f64(o[:, h:h + 1]), want)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (h, s, err)
    log(f"c1 every row: worst err {worst:.3e}")


def test_c4_prefill_full_size_row_blocks(moa):
    """Llama3-70B-shaped GQA prefill (N=65536) on device-generated inputs.  Every query head
    is checked on 512 rows: four blocks of 128 consecutive rows (the first rows, the rows
    around S_h, a seeded random block and the last rows) against the oracle's
    explicit-mask row block."""
    w = workloads.WORKLOADS["c4_prefill"]
    alpha, beta = workloads.rules("c4_prefill")
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    shp_q = (w.batch, w.n_q_heads, w.n_prompt, w.head_dim)
    shp_kv = (w.batch, w.n_kv_heads, w.n_prompt, w.head_dim)
    q = workloads.device_normal_(torch.empty(shp_q, dtype=torch.bfloat16, device="cuda"), 71)
    k = workloads.device_normal_(torch.empty(shp_kv, dtype=torch.bfloat16, device="cuda"), 72)
    v = workloads.device_normal_(torch.empty(shp_kv, dtype=torch.bfloat16, device="cuda"), 73)
    o = torch.empty_like(q)
    log("prefill c4 full size")
    plan.prefill(q, k, v, o)
    torch.cuda.synchronize()
    n, g, blk = w.n_prompt, w.n_q_heads // w.n_kv_heads, 128
    rng = np.random.Generator(np.random.PCG64(204))
    spans = oracle.spans(alpha, beta, n)
    worst = 0.0
    for hk in range(w.n_kv_heads):
        s = int(spans[hk])
        kh, vh = f64(k[0, hk]), f64(v[0, hk])
        for hq in range(hk * g, hk * g + g):
            starts = [0, min(max(0, s - blk // 2), n - blk), int(rng.integers(0, n - blk)), n - blk]
            for i0 in starts:
                want = oracle.prefill_row_block(f64(q[0, hq, i0:i0 + blk]), kh, vh, s, i0)
                err = max_err(f64(o[0, hq, i0:i0 + blk]), want)
                worst = max(worst, err)
                assert err <= TOL["bf16"], (hq, s, i0, err)
    log(f"c4 prefill worst err over 512 rows of every head {worst:.3e}")
