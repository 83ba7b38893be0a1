"""Plain float64 definition of heterogeneous sliding-window attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import this module.

Conventions.  B batch, Hq query heads, Hkv KV heads (Hq a multiple of Hkv),
N prompt length, D head dimension.  Prefill tensors: q [B, Hq, N, D],
k and v [B, Hkv, N, D].  Spans are per KV head.  All arithmetic is float64
numpy; inputs of any float dtype are up-cast first.
"""

import math

import numpy as np

# Compute-block size a span is rounded up to.  The project page's section
# "Elastic search space" only says that candidate rules respect the hardware's
# compute-block size; 64 is the value this implementation adopts.
BLOCK = 64


# ---------------------------------------------------------------------------
# Span table
# ---------------------------------------------------------------------------

def span_of(alpha, beta, n):
    """Span of one head at input length n.

    Mixture of Attention project page, "Finding 2": a head's span is the
    linear rule S = alpha + beta * N.  Section "Elastic search space": spans
    respect the compute-block size, read here as rounding UP to a multiple of
    BLOCK.  Finding 2's head B (a fixed 5.6k window shown as 100 % of a 4k
    input) fixes that a span saturates at N.  The lower clamp to 1 keeps at
    least the query itself (alpha = beta = 0).

    alpha + beta * n is evaluated in IEEE double with each operation rounded
    (Python floats never fuse a multiply-add); the ceiling and the clamps are
    exact integer operations.
    """
    if n < 1:
        raise ValueError("input length must be >= 1")
    x = float(alpha) + float(beta) * float(n)
    if math.isnan(x):
        raise ValueError("span rule evaluates to NaN")
    if x >= n:                      # saturated; also covers +inf
        return int(n)
    r = BLOCK * math.ceil(x / BLOCK)
    return int(min(max(r, 1), n))


def spans(alpha, beta, n):
    """Span table, one entry per KV head (Finding 2 rule applied head by head)."""
    alpha = list(alpha)
    beta = list(beta)
    if len(alpha) != len(beta):
        raise ValueError("alpha and beta must have one entry per KV head")
    return np.array([span_of(a, b, n) for a, b in zip(alpha, beta)], dtype=np.int64)


# ---------------------------------------------------------------------------
# Fixed-size, head-specific KV cache (ring of S_h slots per head)
# ---------------------------------------------------------------------------

def ring_pitch(s, pitch):
    """Slots a ring of s slots occupies in the pool when every ring starts on a
    multiple of `pitch` slots: s rounded up to a multiple of pitch.

    The pages fix only that head h's cache holds S_h slots (project page,
    "Demo" step 03).  Padding each ring to a whole number of pitch-slot blocks
    is a layout choice; the slots s .. pitch - 1 past the ring are never
    attended.  pitch = 1 is the unpadded layout.
    """
    s, pitch = int(s), int(pitch)
    if s < 1 or pitch < 1:
        raise ValueError("span and pitch must be >= 1")
    return -(-s // pitch) * pitch


def ring_offsets(span, pitch=1):
    """Start of each head's ring inside one sequence's cache block.

    Project page, "Demo" step 03 and "Inference speed and memory efficiency":
    deployment keeps a fixed-size KV cache per head, so head h owns S_h slots.
    Heads are laid end to end, each ring taking ring_pitch(S_h, pitch) slots:
    offset[h] is the exclusive prefix sum of those sizes and a sequence's block
    holds their sum.  With pitch = 1 that is the prefix sum of the spans.
    """
    offset = []
    total = 0
    for s in span:
        offset.append(total)
        total += ring_pitch(s, pitch)
    return np.array(offset, dtype=np.int64), total


def pool_index_k(ring_start, slot, d, head_dim):
    """Element index of K (slot, d) of a ring that starts at pool slot
    ring_start: slots are rows of head_dim elements (slot-major)."""
    return (int(ring_start) + int(slot)) * int(head_dim) + int(d)


def pool_index_v(ring_start, slot, d, head_dim, block=32):
    """Element index of V (slot, d) of a ring that starts at pool slot
    ring_start: the ring is cut into blocks of `block` consecutive slots, and
    each block is stored dimension-major ([head_dim][block]), so the slots of
    one dimension within a block are adjacent.  A layout choice, like the
    pitch: the pages only fix the ring's size."""
    slot, d, hd, blk = int(slot), int(d), int(head_dim), int(block)
    return int(ring_start) * hd + (slot // blk) * blk * hd + d * blk + slot % blk


def ring_slot(p, s):
    """Slot that absolute position p occupies in a ring of s slots.

    The pages do not say how positions map to slots; any bijection gives the
    same attention output (softmax does not depend on key order).  The
    reading adopted is slot = p mod s, a function of the position alone.
    """
    return int(p) % int(s)


def ring_expected(hist_k, hist_pos, s, p_last):
    """Contents a ring of s slots must hold after positions up to p_last.

    hist_k [T, D] holds rows for the absolute positions hist_pos [T] (any
    superset of the last s positions).  Slot ring_slot(p, s) holds the row of
    the unique position p in (p_last - s, p_last] congruent to it.
    Returns [s, D] and the position held by each slot.
    """
    hist_pos = np.asarray(hist_pos)
    out = np.zeros((s, hist_k.shape[1]), dtype=hist_k.dtype)
    held = np.full(s, -1, dtype=np.int64)
    for p in range(p_last - s + 1, p_last + 1):
        idx = np.nonzero(hist_pos == p)[0]
        if len(idx) != 1:
            raise ValueError(f"position {p} missing from the history")
        sl = ring_slot(p, s)
        out[sl] = hist_k[idx[0]]
        held[sl] = p
    return out, held


# ---------------------------------------------------------------------------
# Masked softmax attention
# ---------------------------------------------------------------------------

def kv_head_of(h_q, n_q_heads, n_kv_heads):
    """KV head read by query head h_q under grouped-query sharing.

    Not on the pages; the reading is the usual contiguous grouping
    h_kv = h_q // (Hq / Hkv), with one span per KV head.
    """
    if n_q_heads % n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return h_q // (n_q_heads // n_kv_heads)


def band_mask(s, n):
    """Explicit [n, n] boolean mask of one head with span s.

    Blog digest section 2.1: a sliding-window mask is the base pattern; the
    project page's Finding 2 figure keeps a band of the N x N causal matrix.
    Query i keeps keys j with i - s + 1 <= j <= i (at most s keys, itself
    included).
    """
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i) & (j >= i - s + 1)


def attention_probs(q, k, s, scale=None):
    """Row-stochastic attention matrix of one head: masked softmax of q k^T.

    q, k: [n, d].  Masked entries are exactly zero.  scale defaults to
    1/sqrt(d) (a reading: the pages do not state the scale).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    z = (q @ k.T) * scale
    z = np.where(band_mask(s, n), z, -np.inf)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def prefill(q, k, v, span, scale=None):
    """Prefill output O[b, h] = P(b, h) @ V[b, h_kv(h)] for every head.

    q [B, Hq, N, D]; k, v [B, Hkv, N, D]; span [Hkv].  Returns float64
    [B, Hq, N, D].  P is attention_probs with the span of the query head's
    KV head.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, hq, n, d = q.shape
    hkv = k.shape[1]
    out = np.empty_like(q)
    for b in range(bsz):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            p = attention_probs(q[b, h], k[b, g], int(span[g]), scale)
            out[b, h] = p @ v[b, g]
    return out


def prefill_rows(q_rows, k, v, s, rows, scale=None):
    """Selected output rows of one head, each computed on its own.

    q_rows [R, D] are the queries of rows `rows`; k, v [N, D] the head's keys
    and values.  For each row i the explicit mask row (the band of
    band_mask, built over all N keys) selects the kept keys, then a softmax
    over them weights V.  Returns float64 [R, D].
    """
    k = np.asarray(k)
    v = np.asarray(v)
    n, d = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    j = np.arange(n)
    out = np.empty((len(rows), d), dtype=np.float64)
    for r, i in enumerate(rows):
        keep = np.nonzero((j <= i) & (j >= i - s + 1))[0]
        kk = np.asarray(k[keep], dtype=np.float64)
        vv = np.asarray(v[keep], dtype=np.float64)
        z = (kk @ np.asarray(q_rows[r], dtype=np.float64)) * scale
        e = np.exp(z - z.max())
        out[r] = (e / e.sum()) @ vv
    return out


def prefill_row_block(q_rows, k, v, s, i0, scale=None):
    """Output rows i0 .. i0 + R - 1 of one head (R = len(q_rows)), as a block.

    The same definition as attention_probs, restricted to the keys any of these
    rows can keep: keys max(0, i0 - s + 1) .. i0 + R - 1, with the explicit
    band mask of each row over them (blog digest section 2.1; project page
    "Finding 2" figure).  k, v [N, D].  Returns float64 [R, D].
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    r, d = q_rows.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    j0 = max(0, i0 - s + 1)
    j1 = i0 + r
    kk = np.asarray(k[j0:j1], dtype=np.float64)
    vv = np.asarray(v[j0:j1], dtype=np.float64)
    i = np.arange(i0, j1)[:, None]
    j = np.arange(j0, j1)[None, :]
    z = (q_rows @ kk.T) * scale
    z = np.where((j <= i) & (j >= i - s + 1), z, -np.inf)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)) @ vv


# ---------------------------------------------------------------------------
# Decode over a fixed-size window
# ---------------------------------------------------------------------------

def decode_step(q, hist_k, hist_v, hist_pos, p, s, scale=None):
    """Attention output of the token at absolute position p, for one KV head.

    q [G, D] are the queries of the G query heads that share this KV head;
    hist_k, hist_v [T, D] a plain history (not a ring) of rows at absolute
    positions hist_pos [T], which must already include position p
    (append-before-attend, a reading: the window is inclusive of the query,
    as in prefill).  The span s is the one fixed from the prompt length
    (project page, "Demo" step 03: the deployed KV cache has a fixed size), so
    the kept keys are exactly positions p - s + 1 .. p.
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    hist_pos = np.asarray(hist_pos)
    keep = np.nonzero((hist_pos <= p) & (hist_pos >= p - s + 1))[0]
    kk = np.asarray(hist_k[keep], dtype=np.float64)
    vv = np.asarray(hist_v[keep], dtype=np.float64)
    z = (q @ kk.T) * scale
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)) @ vv


def decode(q_steps, k_prompt, v_prompt, k_steps, v_steps, span, n_prompt, scale=None):
    """T decode steps after a prompt of length n_prompt.

    q_steps [T, B, Hq, D]; k_steps, v_steps [T, B, Hkv, D] (the new token's
    key and value at each step); k_prompt, v_prompt: one array per KV head h,
    shaped [B, L_h, D], holding the prompt positions n_prompt - L_h ..
    n_prompt - 1 (any L_h >= span[h] suffices; the whole prompt works).
    Step t decodes absolute position n_prompt + t.  Returns float64
    [T, B, Hq, D].
    """
    q_steps = np.asarray(q_steps)
    t_steps, bsz, hq, d = q_steps.shape
    hkv = len(k_prompt)
    g = hq // hkv
    out = np.empty(q_steps.shape, dtype=np.float64)
    for b in range(bsz):
        for h in range(hkv):
            lp = k_prompt[h].shape[1]
            pos = list(range(n_prompt - lp, n_prompt))
            hk = [np.asarray(k_prompt[h][b], dtype=np.float64)]
            hv = [np.asarray(v_prompt[h][b], dtype=np.float64)]
            for t in range(t_steps):
                p = n_prompt + t
                pos.append(p)
                hk.append(np.asarray(k_steps[t, b, h], dtype=np.float64)[None])
                hv.append(np.asarray(v_steps[t, b, h], dtype=np.float64)[None])
                ck = np.concatenate(hk)
                cv = np.concatenate(hv)
                hk, hv = [ck], [cv]
                out[t, b, h * g:(h + 1) * g] = decode_step(
                    q_steps[t, b, h * g:(h + 1) * g], ck, cv, pos, p, int(span[h]), scale)
    return out
