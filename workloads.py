"""Seeded synthetic workloads for the heterogeneous sliding-window attention path.

Shapes, per-head rule sets and random numbers only: this module holds none of
the method's arithmetic (no span, mask, softmax or layout computation), so the
oracle and the HIP path can both take their inputs from it.

Every workload stands in for a model layer the MoA pages measure (Vicuna-7B,
Vicuna-13B, Llama3-70B shaped attention layers); no dataset or weights are
used.  Rule sets are read from tests/golden/rules.json (seeded draws from the
candidate grids, rejection-sampled to a mean-density target by
tests/golden/make_rules.py).  Data values are iid N(0, 1) float32, cast to
bfloat16 with round-to-nearest-even for the bf16 workloads.

Host generation uses numpy PCG64 streams keyed by
SeedSequence([seed, tensor_id, b, h]) so that any (tensor, batch, head) slice
can be regenerated on its own; device generation (for the large decode rings
and for timing runs) uses torch's seeded device generator.
"""

import json
import os
from dataclasses import dataclass

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
RULES_PATH = os.path.join(ROOT, "tests", "golden", "rules.json")

# tensor ids of the per-slice random streams
T_Q, T_K, T_V, T_QSTEP, T_KSTEP, T_VSTEP, T_KRING, T_VRING = range(8)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_prompt: int
    dtype: str           # "f32" or "bf16"
    steps: int           # decode steps (0 for prefill)
    rules: str           # key into rules.json, or "c0"
    data_seed: int
    title: str


WORKLOADS = {
    "c0_prefill": Workload("c0_prefill", "prefill", 1, 4, 4, 64, 512, "f32", 0, "c0", 2000,
                           "tiny prefill: B1 H4 D64 N512 fp32, spans 64/128/256/512"),
    "c1_prefill": Workload("c1_prefill", "prefill", 1, 32, 32, 128, 8192, "bf16", 0, "c1", 2001,
                           "Vicuna-7B-shaped prefill: B1 H32 D128 N8192 bf16, 50% density"),
    "c2_decode": Workload("c2_decode", "decode", 64, 32, 32, 128, 16384, "bf16", 256, "c2", 2002,
                          "Vicuna-7B-shaped decode: B64 H32 D128 N16384 bf16, 50% density, 256 steps"),
    "c3_decode": Workload("c3_decode", "decode", 32, 40, 40, 128, 32768, "bf16", 256, "c3", 2003,
                          "Vicuna-13B-shaped decode: B32 H40 D128 N32768 bf16, 25% density, 256 steps"),
    "c4_prefill": Workload("c4_prefill", "prefill", 1, 64, 8, 128, 65536, "bf16", 0, "c4", 2004,
                           "Llama3-70B-shaped GQA prefill: B1 Hq64 Hkv8 D128 N65536 bf16, 50% density"),
    "c4_decode": Workload("c4_decode", "decode", 16, 64, 8, 128, 65536, "bf16", 128, "c4", 2004,
                          "Llama3-70B-shaped GQA decode: B16 Hq64 Hkv8 D128 N65536 bf16, 50% density, 128 steps"),
}

# The tiny workload's rules are given explicitly: (alpha, beta) per head.
C0_RULES = ([64, 128, 0, 0], [0.0, 0.0, 0.5, 1.0])


def rules(name):
    """(alpha list, beta list) of a workload or of a rules.json key."""
    key = WORKLOADS[name].rules if name in WORKLOADS else name
    if key == "c0":
        return list(C0_RULES[0]), list(C0_RULES[1])
    with open(RULES_PATH) as f:
        r = json.load(f)[key]
    return [int(a) for a in r["alpha"]], [float(b) for b in r["beta"]]


def torch_dtype(dtype):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


# ---------------------------------------------------------------------------
# Host (numpy) generation, slice by slice
# ---------------------------------------------------------------------------

def normal_slice(seed, tensor_id, b, h, shape):
    """iid N(0,1) float32 block for one (tensor, batch row, head)."""
    ss = np.random.SeedSequence([int(seed), int(tensor_id), int(b), int(h)])
    return np.random.Generator(np.random.PCG64(ss)).standard_normal(shape, dtype=np.float32)


def to_dtype(x, dtype):
    """float32 array -> torch CPU tensor in the workload dtype (RNE for bf16)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype))


def random_tensor(seed, tensor_id, batch, heads, rows, dim, dtype):
    """[batch, heads, rows, dim] tensor whose (b, h) slices are normal_slice."""
    out = np.empty((batch, heads, rows, dim), dtype=np.float32)
    for b in range(batch):
        for h in range(heads):
            out[b, h] = normal_slice(seed, tensor_id, b, h, (rows, dim))
    return to_dtype(out, dtype)


def prefill_inputs(batch, n_q_heads, n_kv_heads, n, dim, dtype, seed):
    """Q [B,Hq,N,D], K and V [B,Hkv,N,D] as CPU tensors."""
    q = random_tensor(seed, T_Q, batch, n_q_heads, n, dim, dtype)
    k = random_tensor(seed, T_K, batch, n_kv_heads, n, dim, dtype)
    v = random_tensor(seed, T_V, batch, n_kv_heads, n, dim, dtype)
    return q, k, v


def decode_step_inputs(batch, n_q_heads, n_kv_heads, steps, dim, dtype, seed):
    """Per-step q [T,B,Hq,D], k_new and v_new [T,B,Hkv,D] as CPU tensors.

    Slice (b, h) holds that head's values for all T steps, so one head's
    inputs can be regenerated alone.
    """
    def gen(tid, heads):
        out = np.empty((steps, batch, heads, dim), dtype=np.float32)
        for b in range(batch):
            for h in range(heads):
                out[:, b, h] = normal_slice(seed, tid, b, h, (steps, dim))
        return to_dtype(out, dtype)
    return gen(T_QSTEP, n_q_heads), gen(T_KSTEP, n_kv_heads), gen(T_VSTEP, n_kv_heads)


def prompt_tail(seed, tensor_id, b, h, rows, dim, dtype):
    """The last `rows` prompt keys (or values) of one (b, h), as [rows, D]."""
    return to_dtype(normal_slice(seed, tensor_id, b, h, (rows, dim)), dtype)


# ---------------------------------------------------------------------------
# Device generation (large rings, timing runs)
# ---------------------------------------------------------------------------

def device_normal_(t, seed):
    """Fill a device tensor in place with N(0,1) draws from a seeded generator."""
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    if t.dtype == torch.float32:
        t.normal_(generator=g)
    else:
        # draw in float32 and round once, like the host path
        chunk = 1 << 26
        flat = t.view(-1)
        for s in range(0, flat.numel(), chunk):
            e = min(s + chunk, flat.numel())
            flat[s:e].copy_(torch.randn(e - s, generator=g, device=t.device, dtype=torch.float32))
    return t
