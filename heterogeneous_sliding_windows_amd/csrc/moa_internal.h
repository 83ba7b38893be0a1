// Internal declarations shared by the C ABI (moa_abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "../../include/moa.h"

namespace moa {

// Prefill tiling: a work item is 128 query rows of one (b, h_q); keys are
// streamed in tiles of 64.  Both are fixed by the kernels.
constexpr int kPrefillBM = 128;
constexpr int kPrefillBN = 64;
// Prefill schedule: runs of up to kPrefillRun consecutive query tiles of one
// (b, h_q) stay on one XCD (16 measured best on the 32-head 8k and the
// 64-head 64k prompts); a unit's cost for balancing the XCDs is its key
// tiles plus kPrefillUnitOverhead (its start and end, measured at about
// three tiles' time).
constexpr int kPrefillRun = 16;
constexpr int kPrefillUnitOverhead = 3;
// The last kPrefillTailUnits units of each XCD's queue (about three rounds of
// the 96 workgroup slots an XCD holds; 384 measured the same) run in
// descending tile count, so that the launch ends on its shortest units
// instead of on the long first units of the last runs.
constexpr size_t kPrefillTailUnits = 256;
// Decode chunk (slots of one head's ring per workgroup) for ungrouped heads.
constexpr int kDecodeChunk = 1024;
// A chunk of a KV group publishes G partial rows, and those writes, mixed
// into a read stream near the HBM limit, cost far more than their bytes; so a
// plan with G > 1 takes the largest of these sizes that still leaves
// kDecodeMinChunks chunks (four rounds of the 512 workgroups MI355X holds).
constexpr int kDecodeGroupChunks[4] = {3072, 2048, 1536, 1024};
constexpr int64_t kDecodeMinChunks = 2048;
// The chunk size of a plan; chunks_at(c) = chunks of all its rings at size c.
template <class F>
int decode_chunk_for(int G, F chunks_at) {
  if (G > 1)
    for (int c : kDecodeGroupChunks)
      if (chunks_at(c) >= kDecodeMinChunks) return c;
  return kDecodeChunk;
}

// How the rings are cut into decode chunks.  Fixed: chunks of `size` slots
// from each ring's start, the last one shorter.  Even: a ring of s slots gets
// ceil(s / size) chunks of one length, ceil(s / count) rounded up to a
// multiple of 32 (the V pool's block), the last one shorter.  Balanced: a
// ring gets n = max(1, floor((s * k + total / 2) / total)) chunks of one
// length, ceil(s / n) rounded up to 32, where total is the slots of all the
// plan's rings: every chunk of the plan about total / k slots long.
enum class CutKind { kFixed, kEven, kBalanced };
struct DecodeCut {
  CutKind kind;
  int32_t size;       // fixed: chunk slots; even: target slots; balanced: 0
  int64_t k = 0;      // balanced: the chunk count the split aims at
  int64_t total = 0;  // balanced: slots of all rings
};
// A plan whose fixed cut gives fewer than kDecodeModelRounds rounds of
// resident workgroups ends on a partly filled last round, and there the cut
// decides the launch time.  For such plans the planner models the launch:
// workgroups start in chunk order, each on the first free slot of the
// resident set, and hold it for their slot count plus kDecodeModelOverhead;
// the launch ends with its last chunk.  Of the even cuts at the targets of
// kDecodeEvenTargets no smaller than the fixed cut's size (so the even cut
// never has more chunks, nor a larger workspace), it takes the one the model
// finishes first (the smaller target on a tie), if that is no later than
// kDecodeModelGainPct percent of the fixed cut's time; else the fixed cut.
// (The model overstates a ragged last round about two to three times: the
// workgroups still running there get more bandwidth each than the model gives
// them, hence the margin.)
constexpr int kDecodeEvenTargets[11] = {1024, 1536, 2048, 2560, 3072, 3584,
                                        4096, 4608, 5120, 6144, 8192};
constexpr int64_t kDecodeModelRounds = 8;
constexpr int64_t kDecodeModelOverhead = 32;
constexpr int64_t kDecodeModelGainPct = 92;
// Groups of at least kDecodeBalancedMinG query heads whose cut so far still
// takes more than one round of resident workgroups, in plans of at most one
// round of rings, take the balanced cut instead, at the largest k <=
// kDecodeBalancedRounds rounds of resident workgroups whose chunk count fits
// that many rounds, and launch its chunks longest first.  Measured on the
// 64-head 64k GQA rings (G = 8) at batch 12 to 64: 2 to 6 % faster than the
// cuts above; at batch 4 and 8, where those cuts fit one round, it was
// slower, hence the round condition.  Groups of 4 gained up to 3 %; groups of
// 2, whose chunks publish few partial rows, moved by -1.6 to +2.2 %.
constexpr int64_t kDecodeBalancedRounds = 2;
constexpr int kDecodeBalancedMinG = 4;
// Decode workgroups resident per CU (256 threads each, one wave per SIMD):
// the occupancy the compiled kernels reach, set by their register and LDS use.
constexpr int kDecodeResidentD64 = 5;
constexpr int kDecodeResidentD128 = 2;
constexpr int kCUs = 256;
inline int decode_resident(int D) {
  return kCUs * (D == 128 ? kDecodeResidentD128 : kDecodeResidentD64);
}
// Chunk length of a ring of s slots under cut c (every chunk but the last).
inline int32_t cut_step(int32_t s, const DecodeCut& c) {
  if (c.kind == CutKind::kFixed || s <= 0) return c.size;
  int64_t n;
  if (c.kind == CutKind::kEven) {
    n = (s + c.size - 1) / c.size;
  } else {
    n = ((int64_t)s * c.k + c.total / 2) / c.total;
    if (n < 1) n = 1;
  }
  const int64_t len = (s + n - 1) / n;
  return (int32_t)((len + 31) / 32 * 32);
}
inline int32_t cut_count(int32_t s, const DecodeCut& c) {
  if (s <= 0) return 0;
  const int32_t step = cut_step(s, c);
  return (s + step - 1) / step;
}
// The cut of `copies` sequences, each with the rings `span` (one sequence's,
// or all of a plan's with copies = 1), for G query heads per KV head of
// dimension D; *n_chunks receives its chunk count (INT64_MAX on overflow).
DecodeCut decode_cut(const std::vector<int32_t>& span, int64_t copies, int G, int D,
                     int64_t* n_chunks);

struct PlanDevice {
  int32_t* span = nullptr;          // [B*Hkv] span of ring (b, h)
  int64_t* ring = nullptr;          // [B*Hkv] first slot of ring (b, h) in the pools
  int32_t* seq_len = nullptr;       // [B] prompt length of each sequence
  int4* prefill_items = nullptr;    // launch table {b*Hq + h_q, q_tile, kt_lo, kt_hi}, bq < 0: padding
  int4* decode_chunks = nullptr;    // [n_chunks] {b*Hkv + h, first_slot, n_slots, chunks_of_ring}
  int2* head_chunks = nullptr;      // [B*Hkv] {first chunk index, chunk count}
  int32_t* decode_order = nullptr;  // [n_chunks] chunk of each decode workgroup; null: the identity
};

}  // namespace moa

// A problem and its tables.  Sequence b's prompt has seq_len[b] <= N tokens;
// in the [B, H, N, D] tensors it occupies the last seq_len[b] rows (left
// padding), and its absolute position p sits at padded row p + N - seq_len[b].
// A plan made without per-sequence lengths has seq_len[b] = N for every b.
struct moa_plan {
  int32_t B = 0, Hq = 0, Hkv = 0, D = 0, G = 0, dtype = 0;
  int64_t N = 0;                          // padded prompt length = max seq_len
  bool ragged = false;                    // made by moa_plan_create_ragged
  bool host_only = false;
  int device = -1;
  std::vector<int64_t> seq_len;           // [B]
  std::vector<int32_t> span;              // [B*Hkv]
  std::vector<int64_t> ring;              // [B*Hkv] first slot of each ring
  int64_t total_slots = 0;                // slots of all sequences' rings
  // Prefill launch table, 4 per entry {b*Hq + h_q, q_tile, kt_lo, kt_hi}
  // (bq = -1: padding), entry 8k + x running XCD x's k-th unit.  Without
  // per-sequence lengths the table holds one sequence's units (b = 0) and the
  // launch runs it for every sequence in turn: workgroup b * prefill_seq_grid
  // + e runs entry e for sequence b.  Otherwise it lists every sequence's
  // units and prefill_seq_grid is 0.
  std::vector<int32_t> prefill_items;
  int64_t prefill_seq_grid = 0;
  int64_t n_prefill_units = 0;            // units of all sequences
  std::vector<int32_t> decode_chunks;     // 4 per chunk, all sequences: {b*Hkv + h, first, n, chunks_of_ring}
  std::vector<int32_t> head_chunks;       // 2 per (b, h): {first chunk, count}
  std::vector<int32_t> decode_order;      // launch order of the chunks (balanced cut), else empty
  moa::DecodeCut decode_cut{moa::CutKind::kFixed, moa::kDecodeChunk};
  int32_t decode_chunk = moa::kDecodeChunk;   // longest chunk of the cut
  int64_t n_chunks = 0;                   // decode chunks of all sequences
  bool any_split = false;                 // some ring has more than one chunk
  moa::PlanDevice dev;
};

namespace moa {

// Kernel launchers (one per source file).  They assume validated arguments.
// Prefill of the plan's dtype; with kc, vc non-null it also writes the
// prompt's last S_h positions into the rings (the fused handoff).
hipError_t launch_prefill(const moa_plan& p, const void* q, const void* k, const void* v,
                          void* o, void* kc, void* vc, hipStream_t s);
hipError_t launch_kv_append(const moa_plan& p, void* kc, void* vc, const void* kn,
                            const void* vn, int64_t pos0, int64_t n_new,
                            hipStream_t s);
hipError_t launch_decode_bf16(const moa_plan& p, const void* q, const void* kc,
                              const void* vc, void* o, void* ws, hipStream_t s);
// Append of one position (pos) fused into the decode launch.
hipError_t launch_append_decode_bf16(const moa_plan& p, const void* q, void* kc, void* vc,
                                     const void* kn, const void* vn, int64_t pos, void* o,
                                     void* ws, hipStream_t s);

// Size of the fixed device scratch behind moa_append_decode_static (one copy
// per GPU, held until the process ends), and its address on the current
// device (looked up once per device).
constexpr size_t kStaticWsBytes = (size_t)16 << 20;
hipError_t static_workspace(void** ptr);

// Workspace layout of the split-K decode: float o[n_chunks][G][D], then
// float2 ml[n_chunks][G] (running max, sum), chunks of all sequences.
struct DecodeWs {
  float* o;
  float2* ml;
};

inline size_t decode_ws_bytes(const moa_plan& p) {
  size_t bytes = (size_t)p.n_chunks * (size_t)p.G * ((size_t)p.D + 2) * sizeof(float);
  bytes = (bytes + 255) & ~(size_t)255;
  return bytes < 256 ? 256 : bytes;
}

inline DecodeWs decode_ws_layout(const moa_plan& p, void* ws) {
  DecodeWs w;
  w.o = static_cast<float*>(ws);
  w.ml = reinterpret_cast<float2*>(w.o + (size_t)p.n_chunks * (size_t)p.G * (size_t)p.D);
  return w;
}

}  // namespace moa
