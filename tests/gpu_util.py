"""Helpers shared by the GPU parity tests (test code, not product code)."""

import sys

import numpy as np
import torch

import oracle


def log(msg):
    """Name the case before each GPU step, so a failing run says which it was."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def f64(t):
    """Torch tensor (any device / float dtype) -> float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()


class Layout:
    """Spans and ring locations of a problem, from the oracle alone (never from a plan).

    seq_spans [B, Hkv]: oracle.spans at each sequence's own length; ring_offsets [B, Hkv]:
    first slot of each ring, the rings of all sequences laid end to end in (b, h) order at
    a 32-slot pitch (oracle.ring_offsets); spans [Hkv] when every sequence has length n,
    else None; total_slots: slots of the whole pool.
    """

    def __init__(self, alpha, beta, batch, head_dim, n, seq_len=None):
        lens = [int(n)] * batch if seq_len is None else [int(x) for x in seq_len]
        self.head_dim, self.batch, self.n_kv_heads = int(head_dim), int(batch), len(alpha)
        self.seq_len = lens
        self.seq_spans = np.stack([oracle.spans(alpha, beta, nb) for nb in lens])
        off, self.total_slots = oracle.ring_offsets(self.seq_spans.ravel(), pitch=32)
        self.ring_offsets = off.reshape(self.seq_spans.shape)
        self.spans = self.seq_spans[0].copy() if seq_len is None else None


def ring_k(pool, plan, b, h):
    """[S, D] view of K ring (b, h): slot-major rows (oracle.pool_index_k)."""
    s, d = int(plan.seq_spans[b, h]), plan.head_dim
    base = int(plan.ring_offsets[b, h]) * d
    return pool[base:base + s * d].view(s, d)


def ring_v(pool, plan, b, h):
    """[S, D] copy of V ring (b, h): stored in 32-slot blocks, each [D][32]
    (oracle.pool_index_v; tests/test_host.py pins this view to it)."""
    s, d = int(plan.seq_spans[b, h]), plan.head_dim
    r = oracle.ring_pitch(s, 32)
    base = int(plan.ring_offsets[b, h]) * d
    blocks = pool[base:base + r * d].view(r // 32, d, 32)     # [block][dim][slot]
    return blocks.permute(0, 2, 1).reshape(r, d)[:s]


def ring_positions(s, p_last):
    """Absolute position held by each slot of a ring of s slots after p_last (slot = p mod s)."""
    pos = np.empty(s, dtype=np.int64)
    for p in range(p_last - s + 1, p_last + 1):
        pos[p % s] = p
    return pos


def sample_rows(n, s, count, seed):
    """Edge rows of a head with span s plus seeded random rows, sorted and unique."""
    edges = [0, 1, 63, 64, 127, 128, s - 2, s - 1, s, s + 1, n - 129, n - 128, n - 65, n - 64,
             n - 2, n - 1]
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = set(r for r in edges if 0 <= r < n)
    rows.update(int(x) for x in rng.integers(0, n, count))
    return sorted(rows)


def max_err(got, want):
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - want))) if np.size(want) else 0.0
