"""Benchmark of the heterogeneous sliding-window attention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c2_decode]
                    [--prefill-workload c1_prefill] [--no-cpu-baseline]

A step is one decode step of the whole batch: the new token's K/V appended
to every head's ring, then split-K decode attention over the rings, both in
moa_append_decode (a split-K partial kernel that also writes the new rows,
and a small combine kernel).  The same rings are also stepped with the two
separate calls (moa_kv_append, then moa_decode), reported beside it.  The
default workload is
the Vicuna-7B-shaped decode (B64, H32, D128, prompt 16384, 50 % mean
density); `value` is decode tokens/s of that batch (B tokens per step) with
every input resident in HBM.  The same run times the Vicuna-7B-shaped
prefill (B1, H32, D128, N8192) and reports its TFLOP/s over the kept
(query, key) pairs only.

Rooflines: the decode kernel against 8 TB/s HBM (algorithmic bytes: K and V
ring reads, q read, o write), the prefill kernel against 2.5 PFLOP/s dense
bf16 MFMA (4*D flops per kept pair).  Kernel durations come from HIP events
recorded on the launch stream around every launch in the timed region.

The CPU baseline times the oracle (oracle/, float64 numpy) on a bounded
sample of the same workload on this host; it is a reported baseline only.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("decode attn tokens/s + HBM GB/s % peak; prefill TFLOP/s % MFMA peak")
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix cores
DECODE_COUNTERS = os.path.join(ROOT, "profiles", "decode_c2_counters.json")
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_c1_counters.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kept_pairs(s, n):
    """Kept (query, key) pairs of one head with span s over n rows."""
    s = min(int(s), int(n))
    return n * s - s * (s - 1) // 2


def prefill_flops(plan):
    g = plan.n_q_heads // plan.n_kv_heads
    pairs = sum(kept_pairs(plan.spans[h // g], plan.n_prompt) for h in range(plan.n_q_heads))
    return 4.0 * plan.head_dim * plan.batch * pairs


def decode_kernel_bytes(plan):
    """K and V ring reads (S_h slots per head, padding excluded) plus q read and o write, bf16."""
    d, b = plan.head_dim, plan.batch
    return 2 * 2 * d * b * int(np.sum(plan.spans, dtype=np.int64)) + 2 * 2 * d * b * plan.n_q_heads


def append_bytes(plan):
    """New K and V rows read and written once, bf16."""
    return 2 * 2 * 2 * plan.head_dim * plan.batch * plan.n_kv_heads


def src_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "heterogeneous_sliding_windows_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(path, *sources):
    """Per-launch HBM bytes of a kernel from committed counter runs, or None when its
    sources changed since the counters were taken."""
    try:
        with open(path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("src_sha") != src_sha(*sources):
        return None
    return c.get("traffic_bytes_per_launch")


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count()


# ---------------------------------------------------------------------------
# GPU legs
# ---------------------------------------------------------------------------

def run_decode(moa, workloads, torch, name, steps, warmup, dense=False):
    """Times the decode step both ways on the same rings: "fused" (moa_append_decode, one
    launch + combine) and "separate" (moa_kv_append, then moa_decode).  Positions run on
    from one mode to the next, so each step is a real append-then-attend."""
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    if dense:   # every head keeps the whole prompt: the dense-cache baseline
        alpha, beta = [w.n_prompt] * w.n_kv_heads, [0.0] * w.n_kv_heads
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta)
    log(f"{name}: rings {2 * plan.cache_elems * 2 / 1e9:.2f} GB, {plan.decode_chunks().shape[0]}"
        f" decode chunks, workspace {plan.workspace_bytes / 1e6:.1f} MB")
    dev = torch.device("cuda")
    kc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16, device=dev), 11)
    vc = workloads.device_normal_(torch.empty(plan.cache_elems, dtype=torch.bfloat16, device=dev), 12)
    ws = plan.new_workspace()
    modes = ("fused", "separate")
    total = len(modes) * (warmup + steps)
    qs = workloads.device_normal_(torch.empty(total, w.batch, w.n_q_heads, w.head_dim,
                                              dtype=torch.bfloat16, device=dev), 13)
    ks = workloads.device_normal_(torch.empty(total, w.batch, w.n_kv_heads, 1, w.head_dim,
                                              dtype=torch.bfloat16, device=dev), 14)
    vs = workloads.device_normal_(torch.empty(total, w.batch, w.n_kv_heads, 1, w.head_dim,
                                              dtype=torch.bfloat16, device=dev), 15)
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device=dev)
    n = w.n_prompt
    stream = torch.cuda.current_stream()
    res = dict(plan=plan, w=w)
    t = 0
    for mode in modes:
        def attend(t, mode=mode):
            if mode == "fused":
                plan.append_decode(qs[t], kc, vc, ks[t, :, :, 0], vs[t, :, :, 0], n + t, out, ws,
                                   stream=stream)
            else:
                plan.decode(qs[t], kc, vc, n + t, out, ws, stream=stream)

        def append(t, mode=mode):
            if mode == "separate":
                plan.kv_append(kc, vc, ks[t], vs[t], n + t, stream=stream)

        for _ in range(warmup):
            append(t)
            attend(t)
            t += 1
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(steps):
            append(t)
            ev[i][0].record(stream)
            attend(t)
            ev[i][1].record(stream)
            t += 1
        t_end.record(stream)
        torch.cuda.synchronize()
        res[mode] = dict(elapsed_ms=t_start.elapsed_time(t_end),
                         decode_ms=float(np.mean([a.elapsed_time(b) for a, b in ev])))
        assert torch.isfinite(out.float()).all(), "non-finite decode output"
    del kc, vc, ws, qs, ks, vs
    torch.cuda.empty_cache()
    return res


def run_prefill(moa, workloads, torch, name, iters, warmup, dense=False, warmup_ms=0.0):
    """Mean prefill time per call, and the prompt's handoff to the rings both ways: a separate
    moa_kv_append(pos0 = 0, n_new = N) and the fused moa_prefill_handoff.

    Before each of the two timed runs (plain, fused), the same call runs `warmup` times and
    then until warmup_ms have passed: under a sustained matrix load the shader clock dips
    and takes 30-45 ms to settle, and again after a switch to another kernel, and the timed
    calls are meant to see the settled clock."""
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    if dense:   # every head keeps the whole prompt: full causal attention
        alpha, beta = [w.n_prompt] * w.n_kv_heads, [0.0] * w.n_kv_heads
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta,
                    dtype=w.dtype)
    dev = torch.device("cuda")
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    shp_q = (w.batch, w.n_q_heads, w.n_prompt, w.head_dim)
    shp_kv = (w.batch, w.n_kv_heads, w.n_prompt, w.head_dim)
    q = workloads.device_normal_(torch.empty(shp_q, dtype=tdt, device=dev), 21)
    k = workloads.device_normal_(torch.empty(shp_kv, dtype=tdt, device=dev), 22)
    v = workloads.device_normal_(torch.empty(shp_kv, dtype=tdt, device=dev), 23)
    o = torch.empty_like(q)
    kc, vc = plan.new_cache()
    stream = torch.cuda.current_stream()

    def timed(fn, count):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(count)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    def warm(fn):
        t0 = time.perf_counter()
        done = 0
        while done < warmup or (time.perf_counter() - t0) * 1e3 < warmup_ms:
            fn()
            done += 1
            if done >= warmup:
                torch.cuda.synchronize()   # so that the wall clock follows the GPU
        torch.cuda.synchronize()

    plain = lambda: plan.prefill(q, k, v, o, stream=stream)
    fused = lambda: plan.prefill_handoff(q, k, v, o, kc, vc, stream=stream)
    warm(plain)
    ms = timed(plain, iters)
    handoff_ms = timed(lambda: plan.kv_append(kc, vc, k, v, 0, stream=stream), 5)
    warm(fused)
    fused_ms = timed(fused, iters)
    assert torch.isfinite(o.float()).all(), "non-finite prefill output"
    res = dict(plan=plan, ms=ms, handoff_ms=handoff_ms, fused_ms=fused_ms, w=w)
    del q, k, v, o, kc, vc
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# CPU baseline legs (the oracle as it stands)
# ---------------------------------------------------------------------------

def cpu_baseline_decode(plan, budget_s):
    import oracle
    rng = np.random.Generator(np.random.PCG64(31))
    d, g, n = plan.head_dim, plan.n_q_heads // plan.n_kv_heads, plan.n_prompt
    hist = []
    for h in range(plan.n_kv_heads):
        s = int(plan.spans[h])
        pos = np.arange(n - s + 1, n + 1)
        hist.append((rng.standard_normal((s, d), dtype=np.float32),
                     rng.standard_normal((s, d), dtype=np.float32), pos, s))
    q = rng.standard_normal((plan.n_q_heads, d), dtype=np.float32)
    tokens = 0
    t0 = time.perf_counter()
    while True:
        for h, (hk, hv, pos, s) in enumerate(hist):
            oracle.decode_step(q[h * g:(h + 1) * g], hk, hv, pos, n, s)
        tokens += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": tokens / el, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "cpu": cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": f"{tokens} decode tokens (one sequence each, all {plan.n_kv_heads} KV heads, "
                      f"full rings) in {el:.1f} s, float64 numpy"}


def cpu_baseline_prefill(plan, budget_s):
    import oracle
    rng = np.random.Generator(np.random.PCG64(32))
    d, n, g = plan.head_dim, plan.n_prompt, plan.n_q_heads // plan.n_kv_heads
    k = rng.standard_normal((n, d), dtype=np.float32)
    v = rng.standard_normal((n, d), dtype=np.float32)
    flops, rows_done = 0.0, 0
    t0 = time.perf_counter()
    h = 0
    while True:
        s = int(plan.spans[(h % plan.n_q_heads) // g])
        rows = [int(x) for x in rng.integers(0, n, 16)]
        oracle.prefill_rows(rng.standard_normal((16, d), dtype=np.float32), k, v, s, rows)
        flops += sum(4.0 * d * min(r + 1, s) for r in rows)
        rows_done += 16
        h += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle", "cpu": cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": f"{rows_done} random query rows over the heads' spans in {el:.1f} s, "
                      f"float64 numpy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="c2_decode")
    ap.add_argument("--prefill-workload", default="c1_prefill")
    ap.add_argument("--prefill-iters", type=int, default=20)
    ap.add_argument("--prefill-warmup-ms", type=float, default=60.0,
                    help="least warmup of each prefill call before it is timed")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads' legs (C3 and C4 decode, C4 prefill)")
    ap.add_argument("--extra-steps", type=int, default=64,
                    help="timed decode steps of each extra decode leg")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-cache baseline (every span = N) on the same kernels")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times (the "
                         "known-size kernel that scales the HBM byte counters)")
    ap.add_argument("--prealloc-gb", type=float, default=0.0, metavar="GB",
                    help="allocate, fill and free GB of device memory before the legs, so the "
                         "rings land where a process that allocates late would put them")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): heads and sequences "
              "never interact in attention, so a multi-GPU run would shard KV-head groups or "
              "sequences with no exchange inside the path, and none is built here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 5}))
        return
    import heterogeneous_sliding_windows_amd as moa
    import workloads

    if args.prealloc_gb > 0:
        log(f"allocating, filling and freeing {args.prealloc_gb:g} GB before the legs")
        big = torch.empty(int(args.prealloc_gb * 2**30), dtype=torch.uint8, device="cuda")
        big.fill_(1)
        torch.cuda.synchronize()
        del big
        torch.cuda.empty_cache()
    log(f"decode workload {args.workload}: warmup {args.warmup}, steps {args.steps}")
    dres = run_decode(moa, workloads, torch, args.workload, args.steps, args.warmup)
    plan, w = dres["plan"], dres["w"]
    fused, sep = dres["fused"], dres["separate"]
    ms_step = fused["elapsed_ms"] / args.steps
    tokens_s = w.batch * args.steps / (fused["elapsed_ms"] / 1e3)
    # the fused launch reads the rings, q and the new rows, and writes o and the new rows
    kbytes = decode_kernel_bytes(plan) + append_bytes(plan)
    step_bytes = kbytes
    achieved = kbytes / (fused["decode_ms"] / 1e3) / 1e9
    sep_ms = sep["elapsed_ms"] / args.steps
    sep_achieved = decode_kernel_bytes(plan) / (sep["decode_ms"] / 1e3) / 1e9
    log(f"decode (fused append+decode): {ms_step:.3f} ms/step, kernel {fused['decode_ms']:.3f} ms,"
        f" {achieved:.0f} GB/s, {tokens_s:.0f} tokens/s")
    log(f"decode (kv_append, then decode): {sep_ms:.3f} ms/step, decode kernel "
        f"{sep['decode_ms']:.3f} ms, {sep_achieved:.0f} GB/s")

    line = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 q/k/v and rings, seeded per-head rules "
                "(tests/golden/rules.json)",
        "config": {"workload": f"{w.name}: {w.title}", "batch": w.batch,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "n_prompt": w.n_prompt,
                   "mean_density": round(float(np.mean(plan.spans)) / w.n_prompt, 4),
                   "step": "moa_append_decode: append of 1 token/seq fused into decode, "
                           "one layer",
                   **({"prealloc_gb": args.prealloc_gb} if args.prealloc_gb > 0 else {})},
        "hbm": {"step_GBps": round(step_bytes / (ms_step / 1e3) / 1e9, 1),
                "step_frac": round(step_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": counter_traffic(DECODE_COUNTERS, "decode.hip", "moa_device.h"),
                     "kernel": f"moa_append_decode = decode_kernel<{w.head_dim}, true> + "
                               f"decode_combine_kernel<{w.head_dim}, true>",
                     "algorithmic_bytes_per_launch": kbytes,
                     "avg_launch_ms": round(fused["decode_ms"], 4)},
        "separate_calls": {
            "step": "moa_kv_append(1 token/seq), then moa_decode",
            "ms_per_step": round(sep_ms, 4),
            "tokens_per_s": round(w.batch * args.steps / (sep["elapsed_ms"] / 1e3), 1),
            "decode_ms": round(sep["decode_ms"], 4),
            "decode_GBps": round(sep_achieved, 1)},
    }

    if not args.no_dense:
        log("dense-cache baseline: same workload, every span = N")
        dres2 = run_decode(moa, workloads, torch, args.workload, args.steps, args.warmup,
                           dense=True)
        dms = dres2["fused"]["elapsed_ms"] / args.steps
        alpha, beta = workloads.rules(args.workload)
        budget = 288 * 10**9
        b_moa = moa.max_batch(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta,
                              "bf16", budget)
        b_dense = moa.max_batch(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt,
                                [w.n_prompt] * w.n_kv_heads, [0.0] * w.n_kv_heads, "bf16", budget)
        line["dense_baseline"] = {
            "ms_per_step": round(dms, 4),
            "tokens_per_s": round(w.batch * args.steps / (dres2["fused"]["elapsed_ms"] / 1e3), 1),
            "moa_speedup_equal_batch": round(dms / ms_step, 3),
            "hbm_GBps": round((decode_kernel_bytes(dres2["plan"]) + append_bytes(dres2["plan"]))
                              / (dres2["fused"]["decode_ms"] / 1e3) / 1e9, 1),
            "max_batch_288GB": {"moa": b_moa, "dense": b_dense},
        }
        log(f"dense: {dms:.3f} ms/step, MoA speedup {dms / ms_step:.2f}x at equal batch; "
            f"max batch in 288 GB: MoA {b_moa}, dense {b_dense}")

    if not args.no_prefill:
        log(f"prefill workload {args.prefill_workload}")
        pres = run_prefill(moa, workloads, torch, args.prefill_workload, args.prefill_iters, 3,
                           warmup_ms=args.prefill_warmup_ms)
        pplan, pw = pres["plan"], pres["w"]
        fl = prefill_flops(pplan)
        tf = fl / (pres["ms"] / 1e3) / 1e12
        f32 = pw.dtype == "f32"
        peak = MFMA_F32_PEAK_TFLOPS if f32 else MFMA_BF16_PEAK_TFLOPS
        log(f"prefill: {pres['ms']:.3f} ms, {tf:.1f} TFLOP/s, handoff {pres['handoff_ms']:.3f} ms;"
            f" fused prefill+handoff {pres['fused_ms']:.3f} ms")
        line["prefill"] = {
            "workload": f"{pw.name}: {pw.title}", "ms": round(pres["ms"], 4),
            "tflops": round(tf, 2), "handoff_ms": round(pres["handoff_ms"], 4),
            "fused_prefill_handoff_ms": round(pres["fused_ms"], 4),
            "flops": fl, "warmup_ms": args.prefill_warmup_ms,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                         "traffic": (counter_traffic(PREFILL_COUNTERS, "prefill.hip", "moa_device.h",
                                                     "moa_internal.h", "moa_abi.cpp")
                                     if pw.name == "c1_prefill" else None),
                         "kernel": f"prefill_{'f32' if f32 else 'bf16'}_kernel<{pw.head_dim}>"},
        }
        if not args.no_dense:
            pd = run_prefill(moa, workloads, torch, args.prefill_workload, args.prefill_iters, 3,
                             dense=True, warmup_ms=args.prefill_warmup_ms)
            line["prefill"]["dense_baseline"] = {
                "ms": round(pd["ms"], 4),
                "tflops": round(prefill_flops(pd["plan"]) / (pd["ms"] / 1e3) / 1e12, 2),
                "moa_speedup": round(pd["ms"] / pres["ms"], 3)}
            log(f"dense prefill: {pd['ms']:.3f} ms, MoA speedup {pd['ms'] / pres['ms']:.2f}x")

    if not args.no_extra:
        # the other workloads, measured the same way (not the headline): fused decode steps,
        # and the 64-head 64k GQA prompt
        other = {}
        for name in ("c3_decode", "c4_decode"):
            r = run_decode(moa, workloads, torch, name, args.extra_steps, 8)
            p, wx = r["plan"], r["w"]
            ms = r["fused"]["elapsed_ms"] / args.extra_steps
            gbps = (decode_kernel_bytes(p) + append_bytes(p)) / (r["fused"]["decode_ms"] / 1e3) / 1e9
            other[name] = {"workload": f"{wx.name}: {wx.title}", "steps": args.extra_steps,
                           "ms_per_step": round(ms, 4),
                           "tokens_per_s": round(wx.batch / (ms / 1e3), 1),
                           "kernel_GBps": round(gbps, 1),
                           "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                           "decode_chunk": p.decode_chunk}
            log(f"{name}: {ms:.4f} ms/step, {gbps:.0f} GB/s ({gbps / HBM_PEAK_GBPS:.1%} of peak)")
        r = run_prefill(moa, workloads, torch, "c4_prefill", 10, 2,
                        warmup_ms=args.prefill_warmup_ms)
        tf4 = prefill_flops(r["plan"]) / (r["ms"] / 1e3) / 1e12
        other["c4_prefill"] = {"workload": f"{r['w'].name}: {r['w'].title}",
                               "ms": round(r["ms"], 3), "tflops": round(tf4, 1),
                               "mfma_frac": round(tf4 / MFMA_BF16_PEAK_TFLOPS, 4),
                               "fused_prefill_handoff_ms": round(r["fused_ms"], 3)}
        log(f"c4_prefill: {r['ms']:.2f} ms, {tf4:.0f} TFLOP/s ({tf4 / MFMA_BF16_PEAK_TFLOPS:.1%})")
        line["other_workloads"] = other

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline_decode(plan, args.cpu_budget)
        if not args.no_prefill:
            line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(pplan, args.cpu_budget / 2)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
