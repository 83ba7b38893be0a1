"""CPU oracle for heterogeneous sliding-window attention (MoA's deployment path).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import, call or link this package; only the test suite,
the smoke check and the benchmark's CPU-baseline leg use it.

The oracle is the plain definition of what the method computes, written out in
float64 numpy with an explicit per-head mask.  It shares no code, table or
constant generator with the HIP path.  Every function names the passage of the
MoA pages it follows:

* "Mixture of Attention" project page (fuvty.github.io, MoA), section
  "Finding 2" (发现二): the linear span rule S = alpha + beta * N, and the worked
  example of heads A/B/C whose spans saturate at the input length; section
  "Elastic search space" (弹性搜索空间): candidate spans respect the hardware's
  compute-block size; section "Inference speed and memory efficiency"
  (推理速度与显存效率) and "Demo" step 03 (演示): deployment uses a fixed-size,
  head-specific KV cache.
* "MoA: Mixture of Sparse Attention for Automatic Large Language Model
  Compression" blog digest (zijie-tian.site), section 2.1 "Elastic sparse
  rules": a sliding-window mask is the base pattern; section 5: the
  deployment kernel keeps a static KV cache.

Readings of points the pages leave open (block size 64, rounding up before
clamping, window inclusive of the query, span fixed at the prompt length during
decode, append-before-attend, slot = position mod span, scale 1/sqrt(D), query
head h uses KV head h // (H_q / H_kv)) are stated where they are used.

Parity status: every function here is pinned by tests that do not re-use its
own formula (closed forms, the pages' worked example, torch's causal SDPA in
float64, a pure-Python brute force, a differently built mask, and planted
mutations).  No function is parity-unpinned.
"""

from .moa_oracle import (  # noqa: F401
    BLOCK,
    span_of,
    spans,
    ring_pitch,
    ring_offsets,
    pool_index_k,
    pool_index_v,
    ring_slot,
    kv_head_of,
    band_mask,
    attention_probs,
    prefill,
    prefill_row_block,
    prefill_rows,
    decode_step,
    decode,
    ring_expected,
)
