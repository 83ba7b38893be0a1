"""Host-side tests of libmoa through its C ABI (no GPU needed).

The library must load and export every symbol include/moa.h declares; its
span and offset tables must equal the oracle's bit for bit; its work lists
must match a brute force over the oracle's explicit mask; invalid arguments
must be rejected with the documented status before any device work.
"""

import ctypes
import heapq
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol(moa):
    with open(os.path.join(ROOT, "include", "moa.h")) as f:
        header = f.read()
    # function declarations: a return type at the start of a line, then the name
    declared = sorted(set(re.findall(
        r"^(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moa_[a-z_0-9]+)\s*\(", header, re.M)))
    assert declared, "no declarations found"
    assert sorted(moa.EXPORTS) == declared
    lib = ctypes.CDLL(moa.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert "gfx950" in moa.version()


def test_binding_fails_loudly_without_the_library(moa, tmp_path):
    """The package has no fallback: without libmoa.so next to it, importing it raises."""
    import importlib.util
    import shutil
    import sys
    pkg = tmp_path / "moa_copy"
    pkg.mkdir()
    for f in ("__init__.py", "rules.py"):
        shutil.copy(os.path.join(os.path.dirname(moa.__file__), f), pkg / f)
    spec = importlib.util.spec_from_file_location("moa_copy", pkg / "__init__.py",
                                                  submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules["moa_copy"] = mod
    try:
        with pytest.raises(ImportError, match="is not built"):
            spec.loader.exec_module(mod)
    finally:
        sys.modules.pop("moa_copy", None)


def _rule_cases():
    rng = np.random.Generator(np.random.PCG64(5))
    cases = []
    for n in (1, 2, 63, 64, 65, 100, 512, 777, 1000, 8192, 16384, 32768, 65536, 2**31 - 1):
        alpha = [0, 1, 63, 64, 65, 512, 1600, 4096, 5600, 10**9] + list(rng.integers(0, 70000, 6))
        beta = [0.0, 0.25, 0.5, 0.75, 1.0, 0.9, 1e-3, 0.3, 2.0, 0.1] + list(rng.random(6))
        cases.append((alpha, beta, n))
    return cases


@pytest.mark.parametrize("case", range(14))
def test_spans_bit_exact(moa, case):
    alpha, beta, n = _rule_cases()[case]
    assert list(moa.spans(alpha, beta, n)) == list(oracle.spans(alpha, beta, n))


def test_spans_random_doubles(moa):
    rng = np.random.Generator(np.random.PCG64(11))
    for n in (100, 4097, 8192, 65536, 1_000_003):
        alpha = rng.integers(0, 2 * n, 500)
        beta = rng.random(500) * 1.5
        assert list(moa.spans(alpha, beta, n)) == list(oracle.spans(alpha, beta, n))


def test_ring_offsets_bit_exact(moa):
    span = np.array([1, 64, 7, 8192, 3, 65536, 33], dtype=np.int32)
    off, tot = moa.ring_offsets(span)
    o_off, o_tot = oracle.ring_offsets(span, pitch=32)
    assert list(off) == list(o_off) and tot == o_tot


def test_ring_view_helpers_follow_the_oracle_layout():
    """The GPU tests read rings through gpu_util's tensor views; on a pool whose every element
    holds its own index, those views give exactly the oracle's K and V element indices."""
    import torch

    from gpu_util import ring_k, ring_v

    class _Plan:
        head_dim = 64
        seq_spans = np.array([[1, 33], [100, 64]])
        ring_offsets = np.zeros((2, 2), dtype=np.int64)

    spans = _Plan.seq_spans.ravel()
    off, total = oracle.ring_offsets(spans, pitch=32)
    _Plan.ring_offsets = off.reshape(2, 2)
    pool = torch.arange(total * _Plan.head_dim, dtype=torch.int64)
    for b in range(2):
        for h in range(2):
            start, sp = int(_Plan.ring_offsets[b, h]), int(_Plan.seq_spans[b, h])
            want_k = [[oracle.pool_index_k(start, sl, e, 64) for e in range(64)] for sl in range(sp)]
            want_v = [[oracle.pool_index_v(start, sl, e, 64) for e in range(64)] for sl in range(sp)]
            assert ring_k(pool, _Plan, b, h).tolist() == want_k
            assert ring_v(pool, _Plan, b, h).tolist() == want_v


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_workload_plan_tables(moa, name):
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta,
                    dtype=w.dtype, host_only=True)
    s = oracle.spans(alpha, beta, w.n_prompt)
    assert list(plan.spans) == list(s)
    off, tot = oracle.ring_offsets(s, pitch=32)
    assert list(plan.offsets) == list(off) and plan.slots_per_seq == tot
    assert plan.cache_elems == w.batch * tot * w.head_dim
    if name == "c0_prefill":
        assert list(plan.spans) == [64, 128, 256, 512]
    plan.close()


def _check_prefill_items(items, n, n_q_heads, span_of_q):
    """Items {b, h_q, q_tile, kt_lo, kt_hi, wg} of one sequence with n tokens: each (h_q, q_tile)
    once; [kt_lo, kt_hi] = exactly the live 64-key tiles of the oracle's mask rows."""
    n_qt = (n + 127) // 128
    assert len(items) == n_q_heads * n_qt
    seen = set()
    for _, hq, qt, lo, hi, _ in items:
        assert (hq, qt) not in seen
        seen.add((hq, qt))
        s = span_of_q(hq)
        rows = np.arange(qt * 128, min(qt * 128 + 128, n))
        # brute force: live tiles from the explicit mask rows
        m = oracle.band_mask(s, n)[rows]
        live = [kt for kt in range((n + 63) // 64) if m[:, kt * 64:(kt + 1) * 64].any()]
        assert live == list(range(lo, hi + 1)), (hq, qt, lo, hi, live[:3], live[-3:])


def _schedule_of(items):
    """Workgroup order rebuilt from the stated rule: runs of up to 16 consecutive query tiles
    of one (b, h_q) from the last tile down; runs longest first (tiles + 3 per unit; ties in
    (b, h_q, run) order); groups of 8 runs, one per XCD in snake order; XCD x's k-th unit in
    workgroup 8k + x, a group as deep as its longest run; the last 256 units of each XCD's
    queue then take its last 256 unit workgroups in descending tile count (stable).  Returns
    ({unit: wg}, table length, XCD loads, the costliest run)."""
    key = {tuple(r[:3]): r for r in items}
    tiles = {}
    for b, hq, qt in key:
        tiles.setdefault((b, hq), []).append(qt)
    runs = []
    for b, hq in sorted(tiles):
        qts = sorted(tiles[(b, hq)], reverse=True)
        assert qts == list(range(len(qts) - 1, -1, -1))
        for i in range(0, len(qts), 16):
            run = [(b, hq, t) for t in qts[i:i + 16]]
            runs.append((sum(key[u][4] - key[u][3] + 1 + 3 for u in run), len(runs), run))
    runs.sort(key=lambda r: (-r[0], r[1]))
    wg, k0, load = {}, 0, [0] * 8
    for g in range(0, len(runs), 8):
        group = runs[g:g + 8]
        for j, (cost, _, run) in enumerate(group):
            x = j if (g // 8) % 2 == 0 else 7 - j
            wg.update({u: 8 * (k0 + i) + x for i, u in enumerate(run)})
            load[x] += cost
        k0 += max(len(r[2]) for r in group)
    for x in range(8):
        queue = sorted((w, u) for u, w in wg.items() if w % 8 == x)[-256:]
        by_tiles = sorted((u for _, u in queue), key=lambda u: -(key[u][4] - key[u][3] + 1))
        wg.update({u: w for (w, _), u in zip(queue, by_tiles)})
    return wg, 8 * k0, load, max(r[0] for r in runs)


def _check_schedule(items, per_sequence_lengths):
    """The launch table follows its stated rule: over all sequences' units for a plan with
    per-sequence lengths; otherwise sequence 0's table, run once per sequence."""
    assert list(items[:, 5]) == sorted(items[:, 5]) and len(set(items[:, 5])) == len(items)
    if per_sequence_lengths:
        wg, _, load, top = _schedule_of(items)
    else:
        wg0, t, load, top = _schedule_of(items[items[:, 0] == 0])
        wg = {(b, hq, qt): b * t + wg0[(0, hq, qt)] for b, hq, qt in (tuple(r[:3]) for r in items)}
    assert [wg[tuple(r[:3])] for r in items] == list(items[:, 5])
    # snake dealing keeps the XCDs' totals within the costliest run of each other
    assert max(load) - min(load) <= top


@pytest.mark.parametrize("n,alpha,beta,hq,hkv", [
    (1, [0], [0.0], 1, 1),
    (200, [0, 64, 100, 0], [0.0, 0.0, 0.0, 1.0], 8, 4),
    (1000, [0, 1, 512, 5000], [0.0, 0.1, 0.25, 0.0], 4, 4),
    (777, [64, 0], [0.0, 0.5], 16, 2),
])
def test_prefill_items_bruteforce(moa, n, alpha, beta, hq, hkv):
    plan = moa.Plan(2, hq, hkv, 128, n, alpha, beta, host_only=True)
    s = oracle.spans(alpha, beta, n)
    g = hq // hkv
    items = plan.prefill_items()
    for b in range(2):                        # both sequences' units, each once
        _check_prefill_items(items[items[:, 0] == b], n, hq, lambda h: int(s[h // g]))
    _check_schedule(items, False)


def test_prefill_items_full_size_tables(moa):
    """Tile ranges at the full prefill sizes, via the union-of-windows rule checked against mask rows."""
    for name in ("c1_prefill", "c4_prefill"):
        w = workloads.WORKLOADS[name]
        alpha, beta = workloads.rules(name)
        plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta,
                        host_only=True)
        s = oracle.spans(alpha, beta, w.n_prompt)
        items = plan.prefill_items()
        g = w.n_q_heads // w.n_kv_heads
        n = w.n_prompt
        j = np.arange(n)
        rng = np.random.Generator(np.random.PCG64(3))
        for idx in rng.integers(0, len(items), 200):
            _, hq, qt, lo, hi, _ = items[idx]
            sp = int(s[hq // g])
            r0, r1 = qt * 128, min(qt * 128 + 128, n) - 1
            kept = np.zeros(n, dtype=bool)
            for i in (r0, r1):                   # the band's extreme rows bound the union
                kept |= (j <= i) & (j >= i - sp + 1)
            kept[max(0, r0 - sp + 1):r1 + 1] = True
            tiles = np.nonzero(kept.reshape(-1, 64).any(axis=1))[0]
            assert (tiles.min(), tiles.max()) == (lo, hi)
        _check_schedule(items, False)
        plan.close()


def _cut_step(s, cut):
    """Chunk length of a ring of s slots under a cut: ("fixed", c) -> c; ("even", t) -> the
    ring's ceil(s / t) chunks share ceil(s / count) slots, rounded up to a multiple of 32;
    ("balanced", k, total) -> the same with max(1, floor((s k + floor(total / 2)) / total))
    chunks."""
    if cut[0] == "fixed":
        return cut[1]
    if cut[0] == "even":
        n = -(-s // cut[1])
    else:
        _, k, total = cut
        n = max(1, (s * k + total // 2) // total)
    return -(-(-(-s // n)) // 32) * 32


def _decode_cut(spans, g, d):
    """The decode cut include/moa.h states, restated, for a plan whose rings have these spans
    in (b, h) order, g query heads per KV head, head dimension d."""
    spans = [int(x) for x in spans]

    def count(cut):
        return sum(-(-s // _cut_step(s, cut)) for s in spans)

    def makespan(cut, slots):
        free = [0] * slots           # when each resident workgroup slot frees
        end = 0
        for s in spans:
            st = _cut_step(s, cut)
            for first in range(0, s, st):
                t = heapq.heappop(free) + min(st, s - first) + 32
                heapq.heappush(free, t)
                end = max(end, t)
        return end

    c = 1024
    if g > 1:
        c = next((x for x in (3072, 2048, 1536) if count(("fixed", x)) >= 2048), 1024)
    slots = 256 * (2 if d == 128 else 5)
    cut = ("fixed", c)
    if count(cut) < 8 * slots:
        t_fixed = makespan(cut, slots)
        best = min((makespan(("even", t), slots), t) for t in
                   (1024, 1536, 2048, 2560, 3072, 3584, 4096, 4608, 5120, 6144, 8192) if t >= c)
        if best[0] * 100 <= t_fixed * 92:
            cut = ("even", best[1])
    if g >= 4 and count(cut) > slots and len(spans) <= slots:
        total = sum(spans)
        for k in range(2 * slots, len(spans) - 1, -1):
            if count(("balanced", k, total)) <= 2 * slots:
                return ("balanced", k, total)
    return cut


def _cut_table(spans, hkv, cut):
    """{b, h, first, n} of every chunk in launch order: rings in (b, h) order, each ring's
    chunks from its first slot; a balanced cut launches them longest first (stable)."""
    rows = []
    for i, s in enumerate(int(x) for x in spans):
        st = _cut_step(s, cut)
        rows += [(i // hkv, i % hkv, f, min(st, s - f)) for f in range(0, s, st)]
    if cut[0] == "balanced":
        rows = sorted(rows, key=lambda r: -r[3])
    return np.array(rows, dtype=np.int32).reshape(-1, 4)


@pytest.mark.parametrize("batch,hq,hkv,d,n,kind", [
    (64, 32, 32, 128, 16384, "fixed"), (16, 64, 8, 128, 65536, "balanced"),
    (8, 64, 8, 128, 65536, "even"), (4, 64, 8, 128, 65536, "even"),
    (32, 64, 8, 128, 65536, "balanced"), (72, 64, 8, 128, 65536, "fixed"),
    (128, 64, 8, 128, 24576, "fixed"), (64, 256, 32, 128, 16384, None),
    (1, 8, 2, 128, 1000, None), (2000, 8, 1, 128, 4096, "even"),
    (3, 8, 2, 64, 20000, None), (40, 16, 2, 64, 30000, None), (2, 40, 40, 128, 32768, None),
    (6, 32, 4, 64, 60000, None)])
def test_decode_chunk_rule(moa, batch, hq, hkv, d, n, kind):
    """The fixed cut (1024 slots for ungrouped heads; with G > 1 the largest of 3072, 2048,
    1536 that leaves at least 2048 chunks, else 1024); an even cut where the dispatch model
    include/moa.h states finishes at least 8 % sooner; for groups of 4 or more heads that still
    need more than one round of resident workgroups, the balanced cut launched longest first.  The
    chunk table is rebuilt from the rule.  `kind` pins the outcome where it is known."""
    alpha, beta = workloads.rules("c4_decode")
    alpha, beta = (list(alpha) * 8)[:hkv], (list(beta) * 8)[:hkv]
    plan = moa.Plan(batch, hq, hkv, d, n, alpha, beta, host_only=True)
    s = np.tile(oracle.spans(alpha, beta, n), batch)
    cut = _decode_cut(s, hq // hkv, d)
    if kind is not None:
        assert cut[0] == kind, cut
    ch = plan.decode_chunks()
    want = _cut_table(s, hkv, cut)
    assert np.array_equal(ch, want)
    assert plan.decode_chunk == (int(want[:, 3].max()) if cut[0] == "balanced" else cut[1])
    _check_chunks(plan, ch)
    plan.close()


@pytest.mark.parametrize("name", ["c2_decode", "c3_decode", "c4_decode"])
def test_decode_chunks_cover_rings(moa, name):
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)
    plan = moa.Plan(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta,
                    host_only=True)
    ch = plan.decode_chunks()
    _check_chunks(plan, ch)
    assert plan.workspace_bytes >= len(ch) * (w.n_q_heads // w.n_kv_heads) * \
        (w.head_dim + 2) * 4
    plan.close()


def _check_chunks(plan, ch):
    """Every slot of every ring (b, h) in exactly one chunk of at most decode_chunk slots,
    starting on a 32-slot block; the launch order either keeps rings in (b, h) order or runs
    the chunks longest first."""
    c = plan.decode_chunk
    ring_order = bool((np.diff(ch[:, 0] * plan.n_kv_heads + ch[:, 1]) >= 0).all())
    assert ring_order or bool((np.diff(ch[:, 3]) <= 0).all())
    for b in range(plan.batch):
        for h in range(plan.n_kv_heads):
            s = int(plan.seq_spans[b, h])
            mine = ch[(ch[:, 0] == b) & (ch[:, 1] == h)]
            covered = np.zeros(s, dtype=int)
            for _, _, first, cnt in mine:
                assert 1 <= cnt <= c and first % 32 == 0
                covered[first:first + cnt] += 1
            assert (covered == 1).all()


@pytest.mark.parametrize("name", ["c2_decode", "c3_decode", "c4_decode"])
def test_max_batch_budget(moa, name):
    """Largest batch whose pools + decode workspace fit: bytes(B) <= budget < bytes(B+1);
    a dense cache (every span N) fits about density-times fewer sequences."""
    w = workloads.WORKLOADS[name]
    alpha, beta = workloads.rules(name)

    def bytes_for(batch, a, b):
        plan = moa.Plan(batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, a, b,
                        host_only=True)
        n = 2 * plan.cache_elems * 2 + plan.workspace_bytes
        plan.close()
        return n

    for budget in (10**9, 96 * 10**9, 288 * 10**9):
        bmax = moa.max_batch(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta,
                             "bf16", budget)
        if bmax > 0:
            assert bytes_for(bmax, alpha, beta) <= budget
        assert bytes_for(bmax + 1, alpha, beta) > budget
    dense = [w.n_prompt] * w.n_kv_heads, [0.0] * w.n_kv_heads
    b_moa = moa.max_batch(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta, "bf16",
                          288 * 10**9)
    b_dense = moa.max_batch(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, *dense, "bf16",
                            288 * 10**9)
    density = float(np.mean(oracle.spans(alpha, beta, w.n_prompt))) / w.n_prompt
    assert abs(b_dense / b_moa - density) < 0.02


def test_max_batch_huge_budgets(moa):
    """Budgets near 2^64 return at once, capped at the largest batch a plan accepts (int32);
    the byte counts never wrap."""
    import time
    alpha, beta = workloads.rules("c2_decode")
    w = workloads.WORKLOADS["c2_decode"]
    t0 = time.perf_counter()
    for budget in (2**64 - 1, 2**63, 2**62):
        b = moa.max_batch(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta, "bf16",
                          budget)
        assert 0 < b <= 2**31 - 1
    assert moa.max_batch(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta, "bf16",
                         2**64 - 1) == 2**31 - 1
    # a tiny model under a huge budget: the cap, not a wrapped product
    assert moa.max_batch(1, 1, 64, 1, [0], [0.0], "bf16", 2**64 - 1) == 2**31 - 1
    # 2^62 bytes / ~136 MB per C2 sequence is about 3.4e10 sequences: capped
    assert moa.max_batch(w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_prompt, alpha, beta, "bf16",
                         2**62) == 2**31 - 1
    assert time.perf_counter() - t0 < 5.0


def test_misaligned_pointers_are_rejected(moa):
    """Every compute entry point refuses device pointers that are not 16-byte aligned before any
    device work (the check precedes the plan's device checks, so a host-only plan shows it)."""
    plan = moa.Plan(1, 2, 2, 64, 50, [0, 0], [1.0, 1.0], host_only=True)
    lib = moa._lib
    ok, bad = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8)
    calls = {
        "moa_prefill": lambda x: lib.moa_prefill(plan._h, ok, ok, x, ok, None),
        "moa_prefill_handoff": lambda x: lib.moa_prefill_handoff(plan._h, ok, ok, ok, ok, ok, x,
                                                                 None),
        "moa_kv_append": lambda x: lib.moa_kv_append(plan._h, ok, ok, x, ok, 0, 1, None),
        "moa_decode": lambda x: lib.moa_decode(plan._h, ok, ok, ok, 50, ok, x, 1 << 30, None),
        "moa_append_decode": lambda x: lib.moa_append_decode(plan._h, ok, ok, ok, x, ok, 50, ok, ok,
                                                             1 << 30, None),
        "moa_append_decode_static": lambda x: lib.moa_append_decode_static(
            plan._h, x, ok, ok, ok, ok, 50, ok, None),
    }
    for name, call in calls.items():
        assert call(bad) == moa.MOA_EINVAL, name
        assert "16-byte aligned" in moa.last_error() and name in moa.last_error(), name
        # aligned pointers get past the check, to the host-only refusal
        assert call(ok) == moa.MOA_EINVAL, name
        assert "HOST_ONLY" in moa.last_error(), name
    plan.close()


# ---------------------------------------------------------------------------
# error paths (checked before any device work, so they run without a GPU)
# ---------------------------------------------------------------------------

def _plan_err(moa, **kw):
    args = dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, n_prompt=100,
                alpha=[0, 0], beta=[0.5, 0.5], dtype="bf16", host_only=True)
    args.update(kw)
    with pytest.raises(moa.MoaError) as e:
        moa.Plan(**args)
    return e.value.status


def test_plan_errors(moa):
    assert _plan_err(moa, n_q_heads=3) == moa.MOA_EINVAL
    assert _plan_err(moa, head_dim=96) == moa.MOA_EUNSUPPORTED
    assert _plan_err(moa, n_q_heads=64, n_kv_heads=2) == moa.MOA_EUNSUPPORTED
    assert _plan_err(moa, alpha=[-1, 0]) == moa.MOA_EINVAL
    assert _plan_err(moa, beta=[float("nan"), 0.0]) == moa.MOA_EINVAL
    assert _plan_err(moa, beta=[float("inf"), 0.0]) == moa.MOA_EINVAL
    assert _plan_err(moa, beta=[-0.5, 0.0]) == moa.MOA_EINVAL
    assert _plan_err(moa, batch=0) == moa.MOA_EINVAL
    assert _plan_err(moa, n_prompt=0) == moa.MOA_EINVAL
    assert _plan_err(moa, n_prompt=2**31) == moa.MOA_EINVAL
    assert "multiple" in moa.last_error() or "n_prompt" in moa.last_error()


def test_raw_abi_errors(moa):
    lib = moa._lib
    out = moa._P()
    assert lib.moa_plan_create(None, 0, ctypes.byref(out)) == moa.MOA_EINVAL
    assert "NULL" in moa.last_error()
    assert lib.moa_plan_create(None, 0, None) == moa.MOA_EINVAL
    assert lib.moa_spans(None, None, 1, 10, None) == moa.MOA_EINVAL
    assert lib.moa_plan_destroy(None) == moa.MOA_OK
    assert lib.moa_prefill(None, None, None, None, None, None) == moa.MOA_EINVAL
    assert lib.moa_prefill_handoff(None, None, None, None, None, None, None,
                                   None) == moa.MOA_EINVAL
    assert lib.moa_append_decode(None, None, None, None, None, None, 0, None, None, 0,
                                 None) == moa.MOA_EINVAL
    assert lib.moa_cache_elems(None) == 0
    assert lib.moa_decode_workspace_bytes(None) == 0
    # unknown flag bits
    a, ap = moa._i64([0])
    b, bp = moa._f64([1.0])
    pr = moa._Problem(1, 1, 1, 128, 10, ap, bp, moa.MOA_BF16)
    assert lib.moa_plan_create(ctypes.byref(pr), 0x10, ctypes.byref(out)) == moa.MOA_EINVAL
    pr.dtype = 7
    assert lib.moa_plan_create(ctypes.byref(pr), moa.MOA_PLAN_HOST_ONLY,
                               ctypes.byref(out)) == moa.MOA_EUNSUPPORTED


def test_host_only_plan_refuses_compute(moa):
    plan = moa.Plan(1, 2, 2, 64, 50, [0, 0], [1.0, 1.0], host_only=True)
    lib = moa._lib
    dummy = ctypes.c_void_p(16)   # never dereferenced: the plan check fails first
    assert lib.moa_prefill(plan._h, dummy, dummy, dummy, dummy, None) == moa.MOA_EINVAL
    assert "HOST_ONLY" in moa.last_error()
    assert lib.moa_kv_append(plan._h, dummy, dummy, dummy, dummy, 0, 1, None) == moa.MOA_EINVAL
    assert lib.moa_decode(plan._h, dummy, dummy, dummy, 50, dummy, dummy, 1 << 30,
                          None) == moa.MOA_EINVAL
    assert lib.moa_prefill_handoff(plan._h, dummy, dummy, dummy, dummy, dummy, dummy,
                                   None) == moa.MOA_EINVAL
    assert "HOST_ONLY" in moa.last_error()
    assert lib.moa_append_decode(plan._h, dummy, dummy, dummy, dummy, dummy, 50, dummy, dummy,
                                 1 << 30, None) == moa.MOA_EINVAL
    assert "HOST_ONLY" in moa.last_error()
    plan.close()


def test_static_decode_rejects_plan_beyond_scratch(moa):
    """moa_append_decode_static refuses a plan whose partials exceed the fixed scratch, before
    any device work and whatever the pointers (the size check needs no device)."""
    lib = moa._lib
    assert moa.static_workspace_bytes() == 16 << 20
    # 2 KV heads of 65536 slots in 1024-slot chunks at batch 256: 32768 chunks of 520 bytes
    big = moa.Plan(256, 2, 2, 128, 65536, [0, 0], [1.0, 1.0], host_only=True)
    assert big.workspace_bytes > moa.static_workspace_bytes()
    dummy = ctypes.c_void_p(16)   # never dereferenced
    assert lib.moa_append_decode_static(big._h, dummy, dummy, dummy, dummy, dummy, 65536, dummy,
                                        None) == moa.MOA_EWORKSPACE
    assert "16777216" in moa.last_error() and "moa_append_decode_static" in moa.last_error()
    # a plan that fits goes on to the ordinary checks (here: host-only plan)
    small = moa.Plan(2, 2, 2, 128, 4096, [0, 0], [1.0, 1.0], host_only=True)
    assert small.workspace_bytes <= moa.static_workspace_bytes()
    assert lib.moa_append_decode_static(small._h, dummy, dummy, dummy, dummy, dummy, 4096, dummy,
                                        None) == moa.MOA_EINVAL
    assert "HOST_ONLY" in moa.last_error()
    assert lib.moa_append_decode_static(None, dummy, dummy, dummy, dummy, dummy, 0, dummy,
                                        None) == moa.MOA_EINVAL
    big.close()
    small.close()


def test_error_message_is_thread_local(moa):
    import threading
    moa._lib.moa_spans(None, None, 1, 10, None)
    msgs = []

    def other():
        msgs.append(moa.last_error())
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert msgs == [""]
    assert moa.last_error() != ""


def test_concurrent_plans_are_independent(moa):
    """Plans created and destroyed on 8 threads at once (the binding's foreign calls release
    the GIL) give exactly the tables of the same plans made on one thread."""
    import threading
    shapes = [(2, 8, 4, 128, 1000, [0, 64, 300, 0], [0.25, 0.0, 0.0, 1.0], None),
              (3, 4, 2, 64, 777, [0, 100], [0.5, 0.0], [777, 1, 300]),
              (16, 64, 8, 128, 65536, *workloads.rules("c4_decode"), None)]

    def tables(shape):
        b, hq, hkv, d, n, a, be, lens = shape
        p = moa.Plan(b, hq, hkv, d, n, a, be, seq_len=lens, host_only=True)
        try:
            return (p.seq_spans.tolist(), p.ring_offsets.tolist(), p.prefill_items().tolist(),
                    p.decode_chunks().tolist(), p.decode_chunk, p.workspace_bytes, p.cache_elems)
        finally:
            p.close()

    want = [tables(sh) for sh in shapes]
    errors = []

    def worker(k):
        try:
            for i in range(6):
                j = (k + i) % len(shapes)
                assert tables(shapes[j]) == want[j], (k, i, j)
        except Exception as e:   # collected and re-raised on the main thread
            errors.append(e)
    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[0]


# ---------------------------------------------------------------------------
# per-sequence prompt lengths (left-padded ragged batch)
# ---------------------------------------------------------------------------

RAGGED = [
    # Hq, Hkv, D, seq_len, alpha, beta
    (4, 2, 128, [300, 1, 64, 299], [0, 100], [0.5, 0.0]),
    (8, 4, 64, [1000, 513, 777], [0, 64, 300, 0], [0.25, 0.0, 0.0, 1.0]),
    (16, 2, 128, [2500, 2499, 1024, 1025, 31], [0, 1500], [1.0, 0.0]),
]


@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_ragged_plan_tables(moa, case):
    hq, hkv, d, lens, alpha, beta = RAGGED[case]
    n = max(lens)
    plan = moa.Plan(len(lens), hq, hkv, d, n, alpha, beta, seq_len=lens, host_only=True)
    assert plan.ragged and plan.spans is None
    assert list(plan.seq_len) == lens
    all_spans = []
    for b, nb in enumerate(lens):
        s = oracle.spans(alpha, beta, nb)
        assert list(plan.seq_spans[b]) == list(s), b
        all_spans += list(s)
    # rings of sequence 0, then sequence 1, ...: one block of 32-slot-pitch rings
    off, tot = oracle.ring_offsets(all_spans, pitch=32)
    assert list(plan.ring_offsets.reshape(-1)) == list(off)
    assert plan.cache_elems == tot * d
    with pytest.raises(moa.MoaError) as e:
        moa._check(moa._lib.moa_plan_tables(plan._h, None, None, None))
    assert e.value.status == moa.MOA_EUNSUPPORTED
    plan.close()


def test_uniform_plan_seq_tables(moa):
    """Without per-sequence lengths, the per-sequence tables repeat sequence 0's."""
    plan = moa.Plan(3, 8, 4, 128, 1000, [0, 64, 300, 0], [0.25, 0.0, 0.0, 1.0], host_only=True)
    for b in range(3):
        assert list(plan.seq_spans[b]) == list(plan.spans)
        assert list(plan.ring_offsets[b]) == list(b * plan.slots_per_seq + plan.offsets)
    assert list(plan.seq_len) == [1000] * 3
    plan.close()


@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_ragged_prefill_items_bruteforce(moa, case):
    hq, hkv, d, lens, alpha, beta = RAGGED[case]
    plan = moa.Plan(len(lens), hq, hkv, d, max(lens), alpha, beta, seq_len=lens, host_only=True)
    items = plan.prefill_items()
    g = hq // hkv
    for b, nb in enumerate(lens):
        s = oracle.spans(alpha, beta, nb)
        _check_prefill_items(items[items[:, 0] == b], nb, hq, lambda h: int(s[h // g]))
    assert set(items[:, 0]) == set(range(len(lens)))
    _check_schedule(items, True)
    plan.close()


@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_ragged_decode_chunks(moa, case):
    hq, hkv, d, lens, alpha, beta = RAGGED[case]
    plan = moa.Plan(len(lens), hq, hkv, d, max(lens), alpha, beta, seq_len=lens, host_only=True)
    _check_chunks(plan, plan.decode_chunks())
    plan.close()


def test_ragged_plan_errors(moa):
    args = dict(batch=3, n_q_heads=4, n_kv_heads=2, head_dim=128, n_prompt=100,
                alpha=[0, 0], beta=[0.5, 0.5], dtype="bf16", host_only=True)
    for lens in ([100, 0, 5], [100, 101, 5], [99, 50, 5], [-1, 100, 3]):
        with pytest.raises(moa.MoaError) as e:
            moa.Plan(**args, seq_len=lens)
        assert e.value.status == moa.MOA_EINVAL, lens
    with pytest.raises(ValueError):
        moa.Plan(**args, seq_len=[100, 50])
    out = moa._P()
    a, ap = moa._i64([0, 0])
    b, bp = moa._f64([0.5, 0.5])
    pr = moa._Problem(3, 4, 2, 128, 100, ap, bp, moa.MOA_BF16)
    assert moa._lib.moa_plan_create_ragged(ctypes.byref(pr), None, moa.MOA_PLAN_HOST_ONLY,
                                           ctypes.byref(out)) == moa.MOA_EINVAL
