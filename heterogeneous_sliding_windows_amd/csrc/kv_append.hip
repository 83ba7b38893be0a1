// Append rows to the fixed-size per-head KV rings (gfx950).
//
// Position p of KV head h lives in slot p mod S_h of that head's ring; an
// append of positions pos0 .. pos0 + n_new - 1 writes only the last
// min(n_new, S_h) of them (the others would be overwritten within the same
// call), so no two threads ever write one slot.  Positions are padded ones:
// a sequence with a shorter prompt (left padding) subtracts its padding.
// K rings are slot-major rows of D elements; V rings are stored in blocks of
// 32 slots, each block dimension-major ([D][32]), the layout decode's P.V
// product reads.  "Mixture of Attention" project page, "Demo" step 03: the
// deployed KV cache has a fixed size per head.

#include "moa_device.h"
#include "moa_internal.h"

namespace moa {
namespace {

// Rows: (b, h) pairs times the last keep_max rows of each.  Row t of (b, h)
// holds padded position pos0 + t, i.e. the sequence's own position
// p = pos0 + t - (Npad - N_b); rows with p < 0 are left padding.  Of the
// rows with p >= 0 only the last min(S, count) are written (earlier ones
// would be overwritten in the same call).  Returns the slot, or -1 for a row
// that is not written.
__device__ __forceinline__ int64_t append_slot(const int32_t* __restrict__ span,
                                               const int32_t* __restrict__ seq_len, int Hkv,
                                               int Npad, int64_t pos0, int64_t n_new, int64_t bh,
                                               int64_t tb, int64_t* t_out) {
  const int64_t S = span[bh];
  const int64_t pad = Npad - seq_len[bh / Hkv];
  const int64_t first_valid = pad > pos0 ? pad - pos0 : 0;   // first row with p >= 0
  const int64_t count = n_new - first_valid;
  const int64_t keep = S < count ? S : count;
  if (tb >= keep) return -1;
  const int64_t t = n_new - 1 - tb;
  *t_out = t;
  return (pos0 + t - pad) % S;
}

// One thread moves 16 bytes (VEC elements) of one row.
template <typename T, int D>
__device__ __forceinline__ void append_k(
    T* __restrict__ kc, const T* __restrict__ kn, const int32_t* __restrict__ span,
    const int64_t* __restrict__ ring, const int32_t* __restrict__ seq_len, int Hkv, int Npad,
    int64_t pos0, int64_t n_new, int64_t keep_max, int64_t total) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPR = D / VEC;  // 16-byte chunks per row
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int c = (int)(idx % CPR);
    const int64_t row = idx / CPR;
    const int64_t tb = row % keep_max;        // 0 = newest position
    const int64_t bh = row / keep_max;
    int64_t t = 0;
    const int64_t slot = append_slot(span, seq_len, Hkv, Npad, pos0, n_new, bh, tb, &t);
    if (slot < 0) continue;
    const uint4* src = reinterpret_cast<const uint4*>(kn + (bh * n_new + t) * D) + c;
    uint4* dst = reinterpret_cast<uint4*>(kc + (ring[bh] + slot) * D) + c;
    *dst = *src;
  }
}

// Positions vary fastest across threads so that the transposed stores of
// neighbouring threads land on neighbouring slots of one V^T block row.
template <typename T, int D>
__device__ __forceinline__ void append_v(
    T* __restrict__ vc, const T* __restrict__ vn, const int32_t* __restrict__ span,
    const int64_t* __restrict__ ring, const int32_t* __restrict__ seq_len, int Hkv, int Npad,
    int64_t pos0, int64_t n_new, int64_t keep_max, int64_t total) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPR = D / VEC;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t tb = idx % keep_max;
    const int64_t rest = idx / keep_max;
    const int c = (int)(rest % CPR);
    const int64_t bh = rest / CPR;
    int64_t t = 0;
    const int64_t slot = append_slot(span, seq_len, Hkv, Npad, pos0, n_new, bh, tb, &t);
    if (slot < 0) continue;
    const uint4 x = *(reinterpret_cast<const uint4*>(vn + (bh * n_new + t) * D) + c);
    T vals[VEC];
    __builtin_memcpy(vals, &x, 16);
    T* dst = vc + ring[bh] * D + (slot >> 5) * (32 * D) + (c * VEC) * 32 + (slot & 31);
#pragma unroll
    for (int e = 0; e < VEC; ++e) dst[e * 32] = vals[e];
  }
}

// blockIdx.y selects the K ring (0) or the V ring (1): one launch per append.
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kernel(
    T* __restrict__ kc, T* __restrict__ vc, const T* __restrict__ kn, const T* __restrict__ vn,
    const int32_t* __restrict__ span, const int64_t* __restrict__ ring,
    const int32_t* __restrict__ seq_len, int Hkv, int Npad, int64_t pos0, int64_t n_new,
    int64_t keep_max, int64_t total) {
  if (blockIdx.y == 0)
    append_k<T, D>(kc, kn, span, ring, seq_len, Hkv, Npad, pos0, n_new, keep_max, total);
  else
    append_v<T, D>(vc, vn, span, ring, seq_len, Hkv, Npad, pos0, n_new, keep_max, total);
}

template <typename T, int D>
hipError_t launch(const moa_plan& p, void* kc, void* vc, const void* kn, const void* vn,
                  int64_t pos0, int64_t n_new, hipStream_t s) {
  constexpr int CPR = D / (16 / sizeof(T));
  int64_t smax = 0;
  for (int32_t x : p.span) smax = x > smax ? x : smax;
  const int64_t keep_max = n_new < smax ? n_new : smax;
  const int64_t total = (int64_t)p.B * p.Hkv * keep_max * CPR;
  int64_t blocks = (total + 255) / 256;
  if (blocks > (1 << 30)) blocks = 1 << 30;
  hipLaunchKernelGGL((append_kernel<T, D>), dim3((unsigned)blocks, 2), dim3(256), 0, s,
                     static_cast<T*>(kc), static_cast<T*>(vc), static_cast<const T*>(kn),
                     static_cast<const T*>(vn), p.dev.span, p.dev.ring, p.dev.seq_len, p.Hkv,
                     (int)p.N, pos0, n_new, keep_max, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const moa_plan& p, void* kc, void* vc, const void* kn, const void* vn,
                            int64_t pos0, int64_t n_new, hipStream_t s) {
  if (p.dtype == MOA_BF16)
    return p.D == 64 ? launch<bf16, 64>(p, kc, vc, kn, vn, pos0, n_new, s)
                     : launch<bf16, 128>(p, kc, vc, kn, vn, pos0, n_new, s);
  return p.D == 64 ? launch<float, 64>(p, kc, vc, kn, vn, pos0, n_new, s)
                   : launch<float, 128>(p, kc, vc, kn, vn, pos0, n_new, s);
}

}  // namespace moa
