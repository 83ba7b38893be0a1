"""Per-layer, per-head span rules from a JSON file.

The rule search exports one (alpha, beta) rule per head and layer as JSON,
and those rules then drive the attention kernel (blog digest "MoA: Mixture
of Sparse Attention for Automatic Large Language Model Compression",
section 5; the paper's abstract gives different heads and layers distinct
configurations).  The pages show no file format, so the schema is this
library's own:

    {"format": "moa-rules", "version": 1, "n_kv_heads": H,
     "layers": [{"alpha": [a_0, ..., a_{H-1}], "beta": [b_0, ..., b_{H-1}]},
                ...]}

alpha entries are non-negative integers and beta entries non-negative finite
numbers; layer l's rule for KV head h gives that head the span
clamp(64 * ceil((alpha + beta * N) / 64), 1, N) at input length N.  This
module only parses and validates the file and creates one Plan per layer;
spans, rings and work lists all come from libmoa.
"""

import json
import math

import numpy as np

from . import Plan, spans as _spans

FORMAT = "moa-rules"
VERSION = 1


class RuleSet:
    """(alpha, beta) per KV head for every layer of a model."""

    def __init__(self, layers):
        if not layers:
            raise ValueError("a rule set needs at least one layer")
        self.layers = []
        for i, (alpha, beta) in enumerate(layers):
            a = np.asarray(alpha, dtype=np.int64)
            b = np.asarray(beta, dtype=np.float64)
            if a.ndim != 1 or a.shape != b.shape or len(a) == 0:
                raise ValueError(f"layer {i}: alpha and beta need one entry per KV head")
            if self.layers and len(a) != len(self.layers[0][0]):
                raise ValueError(f"layer {i}: {len(a)} KV heads, layer 0 has "
                                 f"{len(self.layers[0][0])}")
            if (a < 0).any() or not np.isfinite(b).all() or (b < 0).any():
                raise ValueError(f"layer {i}: alpha must be >= 0, beta finite and >= 0")
            self.layers.append((a, b))

    @property
    def n_layers(self):
        return len(self.layers)

    @property
    def n_kv_heads(self):
        return len(self.layers[0][0])

    def spans(self, n_prompt):
        """[n_layers, n_kv_heads] spans at input length n_prompt (computed by libmoa)."""
        return np.stack([_spans(a, b, n_prompt) for a, b in self.layers])

    def plans(self, batch, n_q_heads, head_dim, n_prompt, dtype="bf16", seq_len=None,
              host_only=False):
        """One Plan per layer (each with its own rings and work lists)."""
        out = []
        try:
            for a, b in self.layers:
                out.append(Plan(batch, n_q_heads, self.n_kv_heads, head_dim, n_prompt, a, b,
                                dtype=dtype, host_only=host_only, seq_len=seq_len))
        except Exception:
            for p in out:
                p.close()
            raise
        return out

    @staticmethod
    def caches(plans):
        """Rings of every layer in one K and one V allocation: [(k_cache, v_cache)] per layer.

        A plan's ring pool is one contiguous range, so layer l's rings are a slice of the
        shared pool.  Each pool is a whole number of 32-slot blocks of D elements, so every
        slice starts at least 4 KB into the allocation and keeps the rings' alignment.
        Zero-filled, on the current GPU."""
        import torch
        if not plans:
            return []
        dt = plans[0]._torch_dtype()
        if any(p._torch_dtype() != dt for p in plans):
            raise ValueError("all layers need the same dtype")
        total = sum(int(p.cache_elems) for p in plans)
        k = torch.zeros(total, dtype=dt, device="cuda")
        v = torch.zeros(total, dtype=dt, device="cuda")
        out, off = [], 0
        for p in plans:
            n = int(p.cache_elems)
            out.append((k[off:off + n], v[off:off + n]))
            off += n
        return out

    def to_dict(self):
        return {"format": FORMAT, "version": VERSION, "n_kv_heads": self.n_kv_heads,
                "layers": [{"alpha": [int(x) for x in a], "beta": [float(x) for x in b]}
                           for a, b in self.layers]}

    def __eq__(self, other):
        return (isinstance(other, RuleSet) and self.n_layers == other.n_layers and
                all((a1 == a2).all() and (b1 == b2).all()
                    for (a1, b1), (a2, b2) in zip(self.layers, other.layers)))


def _int_entry(x, where):
    if isinstance(x, bool) or not isinstance(x, (int, float)) or \
            (isinstance(x, float) and (not math.isfinite(x) or x != int(x))):
        raise ValueError(f"{where}: alpha entries must be integers, got {x!r}")
    return int(x)


def _float_entry(x, where):
    if isinstance(x, bool) or not isinstance(x, (int, float)):
        raise ValueError(f"{where}: beta entries must be numbers, got {x!r}")
    return float(x)


def from_dict(d):
    """Validate a parsed rules document and return its RuleSet."""
    if not isinstance(d, dict):
        raise ValueError("a rules document is a JSON object")
    if d.get("format") != FORMAT:
        raise ValueError(f"format must be {FORMAT!r}, got {d.get('format')!r}")
    if d.get("version") != VERSION:
        raise ValueError(f"unsupported version {d.get('version')!r} (this reader knows {VERSION})")
    layers = d.get("layers")
    if not isinstance(layers, list) or not layers:
        raise ValueError("layers must be a non-empty list")
    h = d.get("n_kv_heads")
    parsed = []
    for i, layer in enumerate(layers):
        if not isinstance(layer, dict) or "alpha" not in layer or "beta" not in layer:
            raise ValueError(f"layer {i}: needs 'alpha' and 'beta' lists")
        alpha = [_int_entry(x, f"layer {i}") for x in layer["alpha"]]
        beta = [_float_entry(x, f"layer {i}") for x in layer["beta"]]
        if len(alpha) != h or len(beta) != h:
            raise ValueError(f"layer {i}: n_kv_heads is {h!r}, got {len(alpha)} alpha and "
                             f"{len(beta)} beta entries")
        parsed.append((alpha, beta))
    return RuleSet(parsed)


def load(path):
    """Read and validate a rules file."""
    with open(path) as f:
        return from_dict(json.load(f))


def save(rules, path):
    with open(path, "w") as f:
        json.dump(rules.to_dict(), f, indent=1)
        f.write("\n")
