/*
 * moa.h -- C ABI of libmoa, heterogeneous sliding-window attention on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Every KV head h has its own causal window of S_h keys:
 * a query at position i attends keys max(0, i - S_h + 1) .. i.  The span
 * follows the linear rule S = alpha + beta * N of the "Mixture of Attention"
 * project page (section "Finding 2"), rounded up to the 64-wide compute block
 * (section "Elastic search space" asks candidate spans to respect the
 * hardware block size) and clamped to [1, N] (Finding 2's head B saturates at
 * the input length).  Decode reads a fixed-size, head-specific KV cache of S_h
 * slots per head (project page, "Demo" step 03 and "Inference speed and
 * memory efficiency"; the blog digest "MoA: Mixture of Sparse Attention for
 * Automatic Large Language Model Compression", section 5, describes the
 * kernel's static KV cache).
 *
 * Conventions used by every entry point.
 *  - B batch, Hq query heads, Hkv KV heads (Hq % Hkv == 0, G = Hq / Hkv),
 *    D head dimension (64 or 128), N prompt length.  Query head h reads KV
 *    head h / G.
 *  - Element type: the plan's dtype (MOA_F32 = IEEE float32, MOA_BF16 =
 *    bfloat16).  Accumulation is float32 for both.  Softmax scale 1/sqrt(D).
 *  - Device pointers are hipMalloc'ed (or torch CUDA/HIP) memory on the
 *    current device, owned by the caller, contiguous, 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    device work is enqueued asynchronously on it; no call synchronises.
 *  - Return value: MOA_OK (0) or a negative moa_status.  On failure no device
 *    work has been enqueued and moa_last_error() describes the problem (a
 *    thread-local string, valid until the next failing call on the thread).
 *    Faults inside kernels surface at the caller's next synchronisation, as
 *    with any HIP launch.
 *  - Threads: a plan is read-only after creation; distinct threads and
 *    streams may use one plan concurrently.  Calls that write the same cache
 *    or workspace must be ordered by the caller.
 *  - HIP graphs: the compute calls only enqueue kernels (no allocation, copy
 *    or memset), so they can be captured.  Positions (pos0, pos) reach the
 *    kernels by value: a captured decode step appends and attends the same
 *    position on every replay.  To advance, capture again or update the
 *    captured kernel nodes' arguments (hipGraphExecKernelNodeSetParams).
 *  - Per-sequence prompt lengths (moa_plan_create_ragged): sequence b has a
 *    prompt of N_b <= N tokens, N = the longest.  Every [.., N, D] tensor
 *    keeps its shape; sequence b's prompt fills its last N_b rows (left
 *    padding), so padded row r holds the sequence's own position
 *    r - (N - N_b).  Spans are per sequence, S_{b,h} = the span rule at N_b,
 *    and so are the rings.  Positions passed to the calls below are padded
 *    positions: position P of the call is position P - (N - N_b) of sequence
 *    b.  A plan without per-sequence lengths is the case N_b = N.
 *
 * KV cache ("ring pool") layout.  One pool for K and one for V, each of
 * moa_cache_elems() elements.  Ring (b, h) has S_{b,h} slots, stored with a
 * pitch of R = 32 * ceil(S / 32) slots (slots S .. R - 1 are padding, never
 * read as keys), starting at slot ring[b][h] of the pool: the rings of
 * sequence b follow each other in head order, and the sequences' blocks
 * follow each other (with one prompt length: ring[b][h] = b*slots_per_seq +
 * offset[h], see moa_ring_offsets).  The sequence's own position p lives in
 * slot p mod S_{b,h}.
 *    K element (b, h, slot, d) at  (ring[b][h] + slot)*D + d
 *    V element (b, h, slot, d) at  ring[b][h]*D + (slot / 32)*32*D + d*32
 *                                  + slot % 32
 * (V rings are stored in blocks of 32 slots, each block dimension-major, so
 * decode's P.V product reads 8 consecutive slots of one dimension as a
 * matrix-core operand and streams each block as 8 KB of contiguous memory.)
 */
#ifndef MOA_H
#define MOA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOA_OK = 0,
  MOA_EINVAL = -1,        /* bad argument: null pointer, bad size, bad rule */
  MOA_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. head_dim 96)  */
  MOA_ENOMEM = -3,        /* host or device allocation of plan tables failed */
  MOA_EHIP = -4,          /* a HIP runtime call failed (message has the code) */
  MOA_EWORKSPACE = -5     /* decode workspace smaller than required          */
} moa_status;

typedef enum { MOA_F32 = 0, MOA_BF16 = 1 } moa_dtype;

/* The problem a plan is built for: shapes plus one (alpha, beta) rule per KV
 * head (project page, "Finding 2").  alpha and beta are host arrays of
 * n_kv_heads entries, read during moa_plan_create only.  alpha >= 0 and beta
 * >= 0 finite are required. */
typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t n_q_heads;    /* Hq >= 1 */
  int32_t n_kv_heads;   /* Hkv >= 1, divides Hq, G = Hq/Hkv <= 16 */
  int32_t head_dim;     /* D: 64 or 128 */
  int64_t n_prompt;     /* N >= 1, < 2^31 */
  const int64_t* alpha; /* [n_kv_heads] */
  const double* beta;   /* [n_kv_heads] */
  int32_t dtype;        /* moa_dtype */
} moa_problem;

typedef struct moa_plan* moa_plan_t;

/* moa_plan_create flags */
#define MOA_PLAN_HOST_ONLY 1u  /* build host tables only: no device memory is
                                  touched, compute entry points then fail with
                                  MOA_EINVAL.  For inspecting tables on a
                                  machine without a GPU. */

/* ---- host-only table builders (no GPU needed) ---------------------------- */

/* Span table.  span[h] = clamp(64 * ceil(x / 64), 1, N) with
 * x = (double)alpha[h] + beta[h] * (double)N evaluated in IEEE double with one
 * rounding per operation (no fused multiply-add); x >= N gives N.  Project
 * page, "Finding 2" (linear rule, saturation at N) and "Elastic search space"
 * (block-size alignment).  span: host array of n_kv_heads int32, written by
 * the call.  Errors: MOA_EINVAL for null arrays, n_kv_heads < 1, N < 1 or
 * N >= 2^31, alpha < 0, beta < 0 or beta not finite. */
int moa_spans(const int64_t* alpha, const double* beta, int32_t n_kv_heads,
              int64_t n_prompt, int32_t* span);

/* Ring offsets: offset[h] = sum of the ring pitches R of heads 0..h-1 (host
 * int64 array of n_kv_heads), *slots_per_seq = sum of all pitches, with
 * R = 32 * ceil(span / 32).  Project page, "Demo" step 03: a fixed-size
 * cache per head.  Errors: MOA_EINVAL for null pointers, n_kv_heads < 1 or
 * any span < 1. */
int moa_ring_offsets(const int32_t* span, int32_t n_kv_heads, int64_t* offset,
                     int64_t* slots_per_seq);

/* ---- plans ---------------------------------------------------------------- */

/* Validate `problem`, build the span, offset and work tables, and (unless
 * MOA_PLAN_HOST_ONLY) copy them to the current HIP device.  *out receives a
 * plan owned by the caller, released with moa_plan_destroy.  Errors:
 * MOA_EINVAL (bad shapes or rules), MOA_EUNSUPPORTED (head_dim not 64/128,
 * G > 16, unknown dtype), MOA_ENOMEM, MOA_EHIP. */
int moa_plan_create(const moa_problem* problem, uint32_t flags, moa_plan_t* out);

/* Same, for a batch whose sequences have their own prompt lengths: seq_len
 * is a host array of `batch` int64 entries in [1, n_prompt], read during the
 * call, and problem->n_prompt must equal its largest entry (the padded
 * length N).  Spans, rings and work lists are per sequence (see "Per-sequence
 * prompt lengths" above): each input's own length sets its spans, as the
 * rules scale with the input length (blog digest, section 2.1; the newx.sg
 * paper page's "AI Summary" calls the sparsity sequence-length adaptive).
 * Errors: those of moa_plan_create, and MOA_EINVAL for a null seq_len or a
 * bad entry. */
int moa_plan_create_ragged(const moa_problem* problem, const int64_t* seq_len,
                           uint32_t flags, moa_plan_t* out);

/* Free the plan's host and device tables.  NULL is accepted.  The caller must
 * ensure no enqueued work still reads the plan (synchronise first). */
int moa_plan_destroy(moa_plan_t plan);

/* Host copies of a plan's tables when every sequence shares them; any
 * output pointer may be NULL.  span: int32[n_kv_heads]; offset:
 * int64[n_kv_heads].  MOA_EUNSUPPORTED for a plan with per-sequence lengths
 * (use moa_plan_seq_tables). */
int moa_plan_tables(moa_plan_t plan, int32_t* span, int64_t* offset,
                    int64_t* slots_per_seq);

/* Host copies of the per-sequence tables of any plan; any output pointer may
 * be NULL.  span: int32[B * n_kv_heads], S of ring (b, h) at b*Hkv + h;
 * ring_offset: int64[B * n_kv_heads], first slot of ring (b, h) in the
 * pools; seq_len: int64[B]. */
int moa_plan_seq_tables(moa_plan_t plan, int32_t* span, int64_t* ring_offset,
                        int64_t* seq_len);

/* Elements in ONE cache pool (K or V): D times the slots of all rings.  0 on
 * error. */
int64_t moa_cache_elems(moa_plan_t plan);

/* Bytes of device workspace moa_decode needs (>= 256).  0 on error. */
size_t moa_decode_workspace_bytes(moa_plan_t plan);

/* KV-memory budget: the largest batch whose two ring pools (K and V) plus the
 * decode workspace fit in budget_bytes, for `problem` with its batch field
 * ignored.  Per sequence that is 2 * slots_per_seq * D * element size plus
 * the decode partials.  A bounded cache lets a larger batch fit (project
 * page, "Inference speed and memory efficiency"); the same problem with
 * every span equal to N gives the dense cache's figure.  Returns the batch
 * (>= 0, at most INT32_MAX: a plan's batch is int32) or a negative
 * moa_status (the problem is validated as by moa_plan_create).  Any budget
 * up to UINT64_MAX is accepted; byte counts that would overflow 64 bits count
 * as not fitting.  The workspace follows the decode cut (moa_plan_decode_
 * chunks), which can shrink it as the batch grows, so bytes(B) is not
 * strictly monotone; the batch returned satisfies bytes(B) <= budget <
 * bytes(B + 1), searched from budget / (bytes of one sequence). */
int64_t moa_max_batch(const moa_problem* problem, uint64_t budget_bytes);

/* Work-list inspection, for tests.  Prefill items are int32 sextuples
 * {b, h_q, q_tile, kt_lo, kt_hi, wg}: query rows q_tile*128 .. +127 of
 * sequence b (its own positions) read key tiles kt_lo .. kt_hi (64 keys
 * each), i.e. every tile holding at least one kept (query, key) pair and no
 * other, in workgroup wg of the launch; items are listed in wg order.  The
 * schedule: each (b, h_q)'s query tiles form runs of up to 16 consecutive
 * tiles, from its last tile down; runs are sorted by cost (the units' tile
 * counts plus 3 per unit), longest first, equal costs in (b, h_q, run)
 * order; groups of 8 consecutive runs go one run per XCD, XCD j for the j-th
 * run of an even group and 7 - j of an odd one; XCD x's k-th unit runs in
 * workgroup 8k + x, and a group spans as many rounds of 8 workgroups as its
 * longest run; then the last 256 units of each XCD's queue are reordered by
 * tile count, most first (a stable sort, so equal counts keep their order),
 * into the same workgroups.  Workgroup numbers missing from the list are
 * padding.  A plan
 * without per-sequence lengths schedules sequence 0's units this way (T
 * entries, padding included, a multiple of 8) and runs that table once per
 * sequence: sequence b's unit at entry e runs in workgroup b*T + e.
 * Decode chunks are int32 quadruples {b, h_kv, first_slot, n_slots} of all
 * sequences, in launch order; every chunk starts at a multiple of 32 slots and
 * holds at most moa_plan_decode_chunk() slots.  Let R be the decode
 * workgroups resident at once (512 for D = 128, 1280 for D = 64).  The fixed
 * cut takes c = 1024 when G = 1, else the largest of 3072, 2048, 1536 that
 * still gives the plan at least 2048 chunks (1024 if none does), and cuts
 * each ring into chunks of c slots, the last one shorter.  A plan whose fixed
 * cut has fewer than 8 * R chunks may take an even cut instead: a ring of s
 * slots gets ceil(s / c) chunks of ceil(s / ceil(s / c)) slots rounded up to
 * a multiple of 32, the last one shorter.  The planner models a launch as
 * chunks taken in order, each by the first of R slots to free, which it holds
 * for n_slots + 32; of the even cuts at c in {1024, 1536, 2048, 2560, 3072,
 * 3584, 4096, 4608, 5120, 6144, 8192}, c no smaller than the fixed cut's, it
 * takes the one whose modeled end is earliest (the smaller c on a tie) if
 * that end is at most 92% of the fixed cut's, else the fixed cut.  Then, when
 * G >= 4, the cut so far has more than R chunks and the plan has at most R
 * rings, it takes the balanced cut: with total the slots of all rings, a
 * ring of s slots gets n = max(1, floor((s * k + floor(total / 2)) / total))
 * chunks of ceil(s / n) slots rounded up to a multiple of 32, the last one
 * shorter, for the largest k <= 2 * R whose chunk count is at most 2 * R.  A
 * fixed or even cut launches rings in (b, h_kv) order, each ring's chunks
 * from its first slot, and moa_plan_decode_chunk() is c; a balanced cut
 * launches the same chunks longest first (a stable sort of that order) and
 * reports its longest chunk.  The even and balanced cuts never have more
 * chunks than the fixed cut or 2 * R, whichever is larger.  Pass out = NULL
 * to get the count; the
 * return value is the item count (>= 0) or a negative moa_status. */
int64_t moa_plan_prefill_items(moa_plan_t plan, int32_t* out);
int64_t moa_plan_decode_chunks(moa_plan_t plan, int32_t* out);
int32_t moa_plan_decode_chunk(moa_plan_t plan);

/* ---- the hot path --------------------------------------------------------- */

/* Prefill attention, every head at once.
 *   q [B, Hq, N, D], k and v [B, Hkv, N, D] (inputs), o [B, Hq, N, D]
 *   (output), all in the plan's dtype.
 *   o[b,h,i,:] = sum_{j=max(0,i-S+1)}^{i} softmax_j(q_i . k_j / sqrt(D)) v_j,
 *   S = span of KV head h / G (of sequence b), i and j the sequence's own
 *   positions; with per-sequence lengths the padding rows of q, k and v are
 *   not read and those of o are not written.
 * Blog digest section 2.1 (sliding-window base mask) and project page
 * "Finding 2" (per-head span; the figure keeps a band of the causal matrix).
 * Key tiles outside a head's window are never read.  Errors: MOA_EINVAL for
 * null pointers or a host-only plan; MOA_EUNSUPPORTED when one head's K or V
 * (N * D elements) reaches 2 GiB; MOA_EHIP if the launch fails. */
int moa_prefill(moa_plan_t plan, const void* q, const void* k, const void* v,
                void* o, void* stream);

/* Prefill (as moa_prefill) fused with the handoff of the prompt to the KV
 * rings (as moa_kv_append(pos0 = 0, n_new = N)) in one launch: positions
 * N_b - S .. N_b - 1 of every (b, h) go to slot p mod S of k_cache/v_cache
 * (the layout above), read once from k and v while the attention streams
 * them.  Project page, "Demo" step 03 (the exported rules feed a kernel
 * with a fixed-size, head-specific cache).  o and the ring contents equal
 * those of the two separate calls.  k and v must not overlap the caches.
 * Errors: those of moa_prefill, and MOA_EINVAL for null caches. */
int moa_prefill_handoff(moa_plan_t plan, const void* q, const void* k, const void* v,
                        void* o, void* k_cache, void* v_cache, void* stream);

/* Write positions pos0 .. pos0 + n_new - 1 of every (b, h) into the ring
 * pools.  k_new, v_new: [B, Hkv, n_new, D] in the plan's dtype; row t holds
 * padded position pos0 + t, i.e. position p = pos0 + t - (N - N_b) of
 * sequence b (rows with p < 0 are padding and are skipped).  Only the last
 * S of the rows with p >= 0 are written for ring (b, h) (the earlier ones
 * would be overwritten in the same call), each into slot p mod S.
 * pos0 = 0, n_new = N hands the prompts' K/V (the prefill layout) over to
 * the cache after prefill; n_new = 1, pos0 = P appends one decode token.
 * Errors: MOA_EINVAL for null pointers, pos0 < 0, n_new < 1 or a host-only
 * plan. */
int moa_kv_append(moa_plan_t plan, void* k_cache, void* v_cache,
                  const void* k_new, const void* v_new, int64_t pos0,
                  int64_t n_new, void* stream);

/* Decode attention for the token at padded position pos >= N (position
 * p = pos - (N - N_b) of sequence b), whose key and value moa_kv_append must
 * already have written (append, then attend).  The span stays the one
 * computed from the prompt length (the deployed cache has a fixed size), so
 * ring (b, h) attends positions p - S + 1 .. p, which are exactly its S
 * slots.
 *   q [B, Hq, D] (input), o [B, Hq, D] (output), plan dtype MOA_BF16.
 * Split-K: each head's ring is cut into chunks of at most
 * moa_plan_decode_chunk() slots; a head with one chunk writes o directly,
 * otherwise each chunk writes its partial (max, sum, P.V) to `workspace` and
 * a second kernel merges the partials of every (sequence, KV head) in chunk
 * order.  workspace: device memory of at least moa_decode_workspace_bytes
 * bytes; its contents need not be initialised and are scratch afterwards
 * (calls that overlap on one workspace race).  Errors: MOA_EINVAL (null
 * pointers, pos < N, host-only plan), MOA_EUNSUPPORTED (dtype MOA_F32, or
 * a head whose ring reaches 2 GiB: S_h * D * 2 >= 2^31), MOA_EWORKSPACE. */
int moa_decode(moa_plan_t plan, const void* q, const void* k_cache,
               const void* v_cache, int64_t pos, void* o, void* workspace,
               size_t ws_bytes, void* stream);

/* One decode step without the separate append launch: moa_kv_append(pos,
 * n_new = 1) of k_new, v_new [B, Hkv, D] fused into moa_decode(pos).  The
 * decode chunk holding slot p mod S of a ring ignores that slot and adds the
 * new key and value from k_new/v_new instead; the merge kernel, which runs
 * after every chunk has read its slots, writes them into the ring (it runs
 * even when no ring is split).  Project page, "Demo" step 03 and "Inference
 * speed and memory efficiency" (fixed-size per-head cache, append then
 * attend).  The ring contents afterwards equal those of the two separate
 * calls; o equals theirs up to rounding (the new key's weight is not rounded
 * to bfloat16 for a matrix-core product).  Same arguments, workspace and
 * errors as moa_decode, plus MOA_EINVAL for null k_new/v_new or
 * pos >= 2^62. */
int moa_append_decode(moa_plan_t plan, const void* q, void* k_cache, void* v_cache,
                      const void* k_new, const void* v_new, int64_t pos, void* o,
                      void* workspace, size_t ws_bytes, void* stream);

/* moa_append_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, with the split-K partials kept in a fixed
 * scratch array inside the library instead of a caller workspace.  The caller
 * still passes inputs, caches and o.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); its first call on a device looks up
 * that device's copy of the scratch once.
 *  - Limit: plans whose moa_decode_workspace_bytes exceeds
 *    moa_static_workspace_bytes() (16 MiB) are rejected with MOA_EWORKSPACE
 *    before anything is enqueued.
 *  - Each GPU holds one scratch array until the process ends, shared by every
 *    call on that GPU, whatever the plan or stream: calls that overlap on one
 *    GPU race (order them on one stream or synchronise).  The scratch needs no
 *    initial contents; each call writes every partial it reads.
 * Other arguments and errors: those of moa_append_decode. */
int moa_append_decode_static(moa_plan_t plan, const void* q, void* k_cache, void* v_cache,
                             const void* k_new, const void* v_new, int64_t pos, void* o,
                             void* stream);

/* Bytes of the fixed scratch behind moa_append_decode_static (16 MiB). */
size_t moa_static_workspace_bytes(void);

/* Message of the last failing call on this thread ("" if none). */
const char* moa_last_error(void);

/* Library version string. */
const char* moa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOA_H */
