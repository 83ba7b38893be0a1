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
// Default decode chunk (slots of one head's ring per workgroup).
constexpr int kDecodeChunk = 1024;

struct PlanDevice {
  int32_t* span = nullptr;          // [Hkv]
  int64_t* offset = nullptr;        // [Hkv]
  int4* prefill_items = nullptr;    // [n_prefill_items] {bh, q_tile, kt_lo, kt_hi}
  int4* decode_chunks = nullptr;    // [n_chunks] {h_kv, first_slot, n_slots, chunks_of_head}
  int2* head_chunks = nullptr;      // [Hkv] {first chunk index, chunk count}
};

}  // namespace moa

struct moa_plan {
  int32_t B = 0, Hq = 0, Hkv = 0, D = 0, G = 0, dtype = 0;
  int64_t N = 0;
  bool host_only = false;
  int device = -1;
  std::vector<int32_t> span;
  std::vector<int64_t> offset;
  int64_t slots = 0;                      // slots per sequence = sum of spans
  std::vector<int32_t> prefill_items;     // 4 per item
  std::vector<int32_t> decode_chunks;     // 4 per chunk (h, first, n, chunks_of_head)
  std::vector<int32_t> head_chunks;       // 2 per KV head (first, count)
  int32_t decode_chunk = moa::kDecodeChunk;
  int64_t n_chunks = 0;                   // chunks per sequence
  bool any_split = false;                 // some head has more than one chunk
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

// Workspace layout of the split-K decode: float o[n_parts][G][D], then
// float2 ml[n_parts][G] (running max, sum), n_parts = B * n_chunks.
struct DecodeWs {
  float* o;
  float2* ml;
};

inline size_t decode_ws_bytes(const moa_plan& p) {
  const size_t parts = (size_t)p.B * (size_t)p.n_chunks;
  size_t bytes = parts * (size_t)p.G * ((size_t)p.D + 2) * sizeof(float);
  bytes = (bytes + 255) & ~(size_t)255;
  return bytes < 256 ? 256 : bytes;
}

inline DecodeWs decode_ws_layout(const moa_plan& p, void* ws) {
  const size_t parts = (size_t)p.B * (size_t)p.n_chunks;
  DecodeWs w;
  w.o = static_cast<float*>(ws);
  w.ml = reinterpret_cast<float2*>(w.o + parts * (size_t)p.G * (size_t)p.D);
  return w;
}

}  // namespace moa
