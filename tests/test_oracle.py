"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin uses a different route than the oracle's own code: the pages'
worked example (tests/golden/worked_example.json), exact rational arithmetic,
a brute-force scan, torch's float64 scaled-dot-product attention (causal, and
with a mask built from tril/triu), a pure-Python loop implementation, closed
forms (span 1 returns v, constant V returns the constant, rows sum to one),
and planted mutations that each of these must catch.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import moa_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ---------------------------------------------------------------------------
# Span table
# ---------------------------------------------------------------------------

def check_worked_example():
    """Project page, Finding 2: heads A/B/C at 4k (40 %, 100 %, 90 %) and 16k."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    for kilo in (1000, 1024):
        n4 = 4 * 1024                      # a "4k" input in tokens
        a = ex["heads"]["A"]
        b = ex["heads"]["B"]
        c = ex["heads"]["C"]
        s_a = oracle.span_of(a["span_k"] * kilo, a["beta"], n4)
        s_b = oracle.span_of(b["span_k"] * kilo, b["beta"], n4)
        s_c = oracle.span_of(c["alpha"], c["beta"], n4)
        for s, head in ((s_a, a), (s_b, b), (s_c, c)):
            assert abs(100.0 * s / n4 - head["percent_of_input"]) <= 2.5, (kilo, s, head)
        # at 4k, B and C both cover nearly everything
        assert s_b / n4 >= 0.9 and s_c / n4 >= 0.9
        # at 16k, B's window is the same size as its rule, C keeps growing
        n16 = 16 * 1024
        s_b16 = oracle.span_of(b["span_k"] * kilo, b["beta"], n16)
        s_c16 = oracle.span_of(c["alpha"], c["beta"], n16)
        assert s_b16 >= b["span_k"] * kilo and s_b16 - b["span_k"] * kilo < 64
        assert s_b16 < n16
        assert s_c16 > s_c and abs(s_c16 / n16 - c["beta"]) < 0.01
        # A and B are fixed windows: the same at every figure length once N exceeds them
        for nk in ex["input_lengths_k"]:
            n = nk * 1024
            if n >= a["span_k"] * kilo + 64:
                assert oracle.span_of(a["span_k"] * kilo, 0.0, n) == s_a


def test_worked_example():
    check_worked_example()


def _smallest_block_multiple_at_least(x):
    """Brute-force scan for the smallest non-negative multiple of 64 >= x."""
    m = 0
    while m < x:
        m += 64
    return m


GRID_ALPHA = [512 * i for i in range(9)]
GRID_BETA = [0.0, 0.25, 0.5, 0.75, 1.0]


def check_spans_bruteforce():
    """span == clamp(smallest multiple of 64 >= exact alpha+beta*N, 1, N), by scan and by Fraction."""
    lengths = [1, 63, 64, 65, 100, 511, 512, 777, 1000, 4097, 8192, 16384, 32768, 65536]
    alphas = GRID_ALPHA + [1, 63, 64, 65, 1600, 5600, 100000]
    betas = GRID_BETA + [0.9, 0.3, 1e-3, 2.0]
    for n in lengths:
        for a in alphas:
            for b in betas:
                exact = Fraction(a) + Fraction(b) * n
                # the rule is evaluated in IEEE double, one rounding per operation
                x = Fraction(float(a) + float(b) * float(n))
                if b in GRID_BETA:
                    assert x == exact          # the candidate grids are exact in double
                if x >= n:
                    want = n
                else:
                    want = min(max(_smallest_block_multiple_at_least(x), 1), n)
                assert oracle.span_of(a, b, n) == want, (a, b, n)


def test_spans_bruteforce():
    check_spans_bruteforce()


def test_spans_tiny_workload():
    """The tiny workload's rules (64,0),(128,0),(0,.5),(0,1) at N=512 give spans 64/128/256/512."""
    assert list(oracle.spans([64, 128, 0, 0], [0.0, 0.0, 0.5, 1.0], 512)) == [64, 128, 256, 512]


def test_span_edges():
    assert oracle.span_of(0, 0.0, 100) == 1           # nothing but the query itself
    assert oracle.span_of(1, 0.0, 100) == 64
    assert oracle.span_of(1, 0.0, 10) == 10            # clamp below a block
    assert oracle.span_of(10**12, 0.0, 5) == 5
    assert oracle.span_of(0, float("inf"), 5) == 5
    with pytest.raises(ValueError):
        oracle.span_of(0, float("nan"), 5)


def test_rules_fixture_is_reproducible_and_meets_density():
    import subprocess, sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(GOLDEN, "make_rules.py"), "--check"],
                       cwd=root, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    with open(os.path.join(GOLDEN, "rules.json")) as f:
        rules = json.load(f)
    for name, r in rules.items():
        s = oracle.spans(r["alpha"], r["beta"], r["n_prompt"])
        assert abs(s.mean() / r["n_prompt"] - r["target_density"]) <= r["tol"]


# ---------------------------------------------------------------------------
# Offsets and ring slots
# ---------------------------------------------------------------------------

def test_ring_offsets_prefix_sum():
    span = [5, 1, 64, 7]
    off, total = oracle.ring_offsets(span)
    assert total == sum(span)
    for h in range(len(span)):
        assert off[h] == sum(span[:h])
    # the heads' slot ranges tile [0, total) without overlap
    covered = np.zeros(total, dtype=int)
    for h, s in enumerate(span):
        covered[off[h]:off[h] + s] += 1
    assert (covered == 1).all()


def check_ring_layout():
    """Ring pitch, offsets and pool indices against values worked by hand from the layout's
    statement and against the properties the layout must have: rings of whole pitch blocks
    that tile the sequence's block without overlap, and K/V element maps that are bijections
    onto the ring's region with the adjacency each layout promises."""
    # by hand: spans 1, 64, 7, 33 at a 32-slot pitch take 32, 64, 32, 64 slots
    off, total = oracle.ring_offsets([1, 64, 7, 33], pitch=32)
    assert list(off) == [0, 32, 96, 128] and total == 192
    off, total = oracle.ring_offsets([5, 1, 64, 7])      # unpadded: prefix sums of the spans
    assert list(off) == [0, 5, 6, 70] and total == 77
    rng = np.random.Generator(np.random.PCG64(17))
    for pitch in (1, 32, 64):
        span = [int(x) for x in rng.integers(1, 300, 12)] + [1, pitch, pitch + 1]
        off, total = oracle.ring_offsets(span, pitch=pitch)
        covered = np.zeros(total, dtype=int)
        for h, sp in enumerate(span):
            r = oracle.ring_pitch(sp, pitch)
            assert r % pitch == 0 and 0 <= r - sp < pitch
            assert off[h] % pitch == 0
            covered[off[h]:off[h] + r] += 1
        assert (covered == 1).all()
    # element maps: each ring's slots x dims fill [start*D, (start+R)*D) exactly once
    for d in (64, 128):
        for start, sp in ((0, 1), (32, 33), (96, 100), (64, 64)):
            r = oracle.ring_pitch(sp, 32)
            for fn in (oracle.pool_index_k, oracle.pool_index_v):
                idx = sorted(fn(start, sl, e, d) for sl in range(r) for e in range(d))
                assert idx == list(range(start * d, (start + r) * d)), (fn.__name__, d, sp)
            for sl in range(r):
                # K: a slot's dims are one contiguous row
                assert oracle.pool_index_k(start, sl, d - 1, d) - oracle.pool_index_k(start, sl, 0, d) == d - 1
                # V: within a 32-slot block, consecutive slots of one dim are adjacent
                if sl % 32 != 31 and sl + 1 < r:
                    assert (oracle.pool_index_v(start, sl + 1, 5, d)
                            == oracle.pool_index_v(start, sl, 5, d) + 1)


def test_ring_layout():
    check_ring_layout()


@pytest.mark.parametrize("s", [1, 2, 5, 64, 100])
def test_ring_holds_last_s_positions(s):
    """After positions 0..p are written in order, the ring holds exactly (p-s, p], each once."""
    ring = {}
    d = 3
    rows = _rand(7, 300, d)
    for p in range(300):
        ring[oracle.ring_slot(p, s)] = p            # sequential overwrite
        if p + 1 >= s:
            held = sorted(ring.values())
            assert held == list(range(p - s + 1, p + 1))
            exp, pos = oracle.ring_expected(rows[:p + 1], np.arange(p + 1), s, p)
            for sl, q in ring.items():
                assert pos[sl] == q
                assert np.array_equal(exp[sl], rows[q])
    # a slot is reused exactly s positions later
    for p in range(s, 200):
        assert oracle.ring_slot(p, s) == oracle.ring_slot(p - s, s)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def check_full_span_is_causal_sdpa():
    """S >= N is full causal attention (torch float64 SDPA, is_causal)."""
    bsz, h, n, d = 2, 3, 37, 16
    q, k, v = _rand(1, bsz, h, n, d), _rand(2, bsz, h, n, d), _rand(3, bsz, h, n, d)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                         torch.from_numpy(v), is_causal=True).numpy()
    for span in ([n] * h, [n, n, n]):
        out = oracle.prefill(q, k, v, span)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # a rule that saturates gives the same
    span = oracle.spans([0, 10**6, 0], [1.0, 0.0, 5.0], n)
    np.testing.assert_allclose(oracle.prefill(q, k, v, span), ref, rtol=0, atol=1e-12)


def test_full_span_is_causal_sdpa():
    check_full_span_is_causal_sdpa()


def check_band_vs_tril_triu_mask():
    """Any span equals SDPA with a mask built as tril().triu(-(S-1))."""
    bsz, h, n, d = 1, 4, 45, 8
    q, k, v = _rand(4, bsz, h, n, d), _rand(5, bsz, h, n, d), _rand(6, bsz, h, n, d)
    span = [1, 3, 16, 44]
    out = oracle.prefill(q, k, v, span)
    for hh, s in enumerate(span):
        m = torch.ones(n, n, dtype=torch.bool).tril().triu(-(s - 1))
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[:, hh:hh + 1]),
                                             torch.from_numpy(k[:, hh:hh + 1]),
                                             torch.from_numpy(v[:, hh:hh + 1]),
                                             attn_mask=m).numpy()
        np.testing.assert_allclose(out[:, hh:hh + 1], ref, rtol=0, atol=1e-12)


def test_band_vs_tril_triu_mask():
    check_band_vs_tril_triu_mask()


def check_span_one_returns_v():
    """S = 1: every query attends only itself, so O = V exactly."""
    n, d = 50, 8
    q, k, v = _rand(7, 1, 2, n, d), _rand(8, 1, 2, n, d), _rand(9, 1, 2, n, d)
    out = oracle.prefill(q, k, v, [1, 1])
    assert np.array_equal(out, v)


def test_span_one_returns_v():
    check_span_one_returns_v()


def check_rows_are_stochastic():
    """Every row of the masked softmax sums to one, is zero off the band, has min(i+1, S) entries."""
    n, d = 70, 8
    q, k = _rand(10, n, d), _rand(11, n, d)
    for s in (1, 2, 9, 64, 70, 200):
        p = oracle.attention_probs(q, k, s)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        for i in range(n):
            nz = np.nonzero(p[i])[0]
            assert len(nz) == min(i + 1, s)
            assert nz.min() == max(0, i - s + 1) and nz.max() == i


def test_rows_are_stochastic():
    check_rows_are_stochastic()


def test_constant_v_returns_constant():
    n, d = 40, 4
    q, k = _rand(12, 1, 1, n, d), _rand(13, 1, 1, n, d)
    v = np.full((1, 1, n, d), 0.375)
    out = oracle.prefill(q, k, v, [11])
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-14)


def _brute_force(q, k, v, s):
    """Pure-Python loops: for each query, the keys at most s-1 positions back."""
    n, d = len(q), len(q[0])
    out = []
    for i in range(n):
        js = [j for j in range(n) if i - s < j <= i]
        sc = [sum(q[i][t] * k[j][t] for t in range(d)) / math.sqrt(d) for j in js]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        z = sum(w)
        out.append([sum(w[a] * v[js[a]][t] for a in range(len(js))) / z for t in range(d)])
    return np.array(out)


def check_bruteforce_tiny():
    n, d = 13, 4
    q, k, v = _rand(14, 1, 1, n, d), _rand(15, 1, 1, n, d), _rand(16, 1, 1, n, d)
    for s in (1, 2, 5, 13):
        want = _brute_force(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), s)
        got = oracle.prefill(q, k, v, [s])[0, 0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
        rows = [0, 3, 12]
        got_rows = oracle.prefill_rows(q[0, 0, rows], k[0, 0], v[0, 0], s, rows)
        np.testing.assert_allclose(got_rows, want[rows], rtol=0, atol=1e-12)
        for i0, r in ((0, 4), (3, 5), (7, 6), (12, 1), (0, 13)):
            got_blk = oracle.prefill_row_block(q[0, 0, i0:i0 + r], k[0, 0], v[0, 0], s, i0)
            np.testing.assert_allclose(got_blk, want[i0:i0 + r], rtol=0, atol=1e-12)


def test_bruteforce_tiny():
    check_bruteforce_tiny()


def check_gqa_equals_repeated_kv():
    """Query head h reads KV head h // G: same as MHA with K/V repeated G times."""
    bsz, hkv, g, n, d = 2, 3, 4, 29, 8
    q = _rand(17, bsz, hkv * g, n, d)
    k, v = _rand(18, bsz, hkv, n, d), _rand(19, bsz, hkv, n, d)
    span = [3, 29, 11]
    out = oracle.prefill(q, k, v, span)
    krep, vrep = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    for h in range(hkv * g):
        s = span[h // g]
        m = torch.ones(n, n, dtype=torch.bool).tril().triu(-(s - 1))
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[:, h:h + 1]),
                                             torch.from_numpy(krep[:, h:h + 1]),
                                             torch.from_numpy(vrep[:, h:h + 1]),
                                             attn_mask=m).numpy()
        np.testing.assert_allclose(out[:, h:h + 1], ref, rtol=0, atol=1e-12)


def test_gqa_equals_repeated_kv():
    check_gqa_equals_repeated_kv()


def check_decode_equals_prefill_row():
    """Decode of position N+t equals row N+t of a prefill over prompt + new tokens (spans fixed)."""
    bsz, hkv, g, n, t_steps, d = 2, 3, 2, 20, 6, 8
    span = [1, 7, 20]
    hq = hkv * g
    kp, vp = _rand(20, bsz, hkv, n, d), _rand(21, bsz, hkv, n, d)
    qs = _rand(22, t_steps, bsz, hq, d)
    ks, vs = _rand(23, t_steps, bsz, hkv, d), _rand(24, t_steps, bsz, hkv, d)
    out = oracle.decode(qs, [kp[:, h] for h in range(hkv)], [vp[:, h] for h in range(hkv)],
                        ks, vs, span, n)
    # concatenated sequence; query rows of the prompt are arbitrary
    kc = np.concatenate([kp, ks.transpose(1, 2, 0, 3)], axis=2)
    vc = np.concatenate([vp, vs.transpose(1, 2, 0, 3)], axis=2)
    qc = np.concatenate([_rand(25, bsz, hq, n, d), qs.transpose(1, 2, 0, 3)], axis=2)
    full = oracle.prefill(qc, kc, vc, span)
    for t in range(t_steps):
        np.testing.assert_allclose(out[t], full[:, :, n + t], rtol=0, atol=1e-12)
    # only the last S_h prompt rows matter
    tails_k = [kp[:, h, n - s:] for h, s in enumerate(span)]
    tails_v = [vp[:, h, n - s:] for h, s in enumerate(span)]
    out2 = oracle.decode(qs, tails_k, tails_v, ks, vs, span, n)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12)
    # S = 1 heads return the new value exactly
    for t in range(t_steps):
        for hh in range(g):
            assert np.array_equal(out[t, :, hh], vs[t, :, 0])


def test_decode_equals_prefill_row():
    check_decode_equals_prefill_row()


# ---------------------------------------------------------------------------
# Planted mistakes: every one must trip at least one pin above
# ---------------------------------------------------------------------------

PINS = [check_worked_example, check_spans_bruteforce, check_full_span_is_causal_sdpa,
        check_band_vs_tril_triu_mask, check_span_one_returns_v, check_rows_are_stochastic,
        check_bruteforce_tiny, check_gqa_equals_repeated_kv, check_decode_equals_prefill_row,
        check_ring_layout]


def _mut_window_wide(s, n):
    i = np.arange(n)[:, None]; j = np.arange(n)[None, :]
    return (j <= i) & (j >= i - s)


def _mut_window_narrow(s, n):
    i = np.arange(n)[:, None]; j = np.arange(n)[None, :]
    return (j <= i) & (j >= i - s + 2)


def _mut_not_causal(s, n):
    i = np.arange(n)[:, None]; j = np.arange(n)[None, :]
    return (j >= i - s + 1) & (j <= i + 1)


def _mut_span_floor(alpha, beta, n):
    x = float(alpha) + float(beta) * float(n)
    if x >= n:
        return int(n)
    return int(min(max(64 * math.floor(x / 64), 1), n))


def _mut_span_no_clamp(alpha, beta, n):
    x = float(alpha) + float(beta) * float(n)
    return int(max(64 * math.ceil(x / 64), 1))


def _mut_kv_head(h_q, n_q_heads, n_kv_heads):
    return h_q % n_kv_heads


def _mut_decode_step_wide(q, hist_k, hist_v, hist_pos, p, s, scale=None):
    return _orig_decode_step(q, hist_k, hist_v, hist_pos, p, s + 1, scale)


_orig_decode_step = moa_oracle.decode_step
_orig_attention_probs = moa_oracle.attention_probs


def _mut_no_scale(q, k, s, scale=None):
    return _orig_attention_probs(q, k, s, 1.0)


def _mut_swap_kv_prefill(q, k, v, span, scale=None):
    return _orig_prefill(q, v, k, span, scale)


_orig_prefill = moa_oracle.prefill


def _mut_block_keys_late(q_rows, k, v, s, i0, scale=None):
    """Keys taken from i0 - s + 2 on: the oldest kept key of the block's first row dropped."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    r, d = q_rows.shape
    j0 = max(0, i0 - s + 2)
    out = np.empty((r, d))
    for a in range(r):
        i = i0 + a
        lo = max(j0, i - s + 1)
        kk, vv = np.asarray(k[lo:i + 1], dtype=np.float64), np.asarray(v[lo:i + 1], dtype=np.float64)
        z = kk @ q_rows[a] / math.sqrt(d)
        e = np.exp(z - z.max())
        out[a] = (e / e.sum()) @ vv
    return out

def _mut_ring_pitch_floor(s, pitch):
    return max(1, int(s) // int(pitch)) * int(pitch)


def _mut_pool_index_v_dim_stride(ring_start, slot, d, head_dim, block=32):
    """Dimension stride of a whole row instead of one block's width."""
    return (int(ring_start) * int(head_dim) + (int(slot) // block) * block * int(head_dim)
            + int(d) * int(head_dim) + int(slot) % block)


MUTATIONS = {
    "window_wide": ("band_mask", _mut_window_wide),
    "window_narrow": ("band_mask", _mut_window_narrow),
    "not_causal": ("band_mask", _mut_not_causal),
    "span_floor": ("span_of", _mut_span_floor),
    "span_no_clamp": ("span_of", _mut_span_no_clamp),
    "kv_head_mod": ("kv_head_of", _mut_kv_head),
    "decode_window_wide": ("decode_step", _mut_decode_step_wide),
    "no_scale": ("attention_probs", _mut_no_scale),
    "swap_kv": ("prefill", _mut_swap_kv_prefill),
    "block_keys_late": ("prefill_row_block", _mut_block_keys_late),
    "ring_pitch_floor": ("ring_pitch", _mut_ring_pitch_floor),
    "pool_v_dim_stride": ("pool_index_v", _mut_pool_index_v_dim_stride),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(moa_oracle, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutation {name} passed every pin"
