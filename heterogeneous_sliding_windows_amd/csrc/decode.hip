// Split-K decode over the fixed-size per-head KV rings (gfx950).
//
// One token per sequence attends all S_h slots of its heads' rings: the span
// is fixed from the prompt length, so after append-then-attend the ring holds
// exactly positions pos - S_h + 1 .. pos ("Mixture of Attention" project page,
// "Demo" step 03 and "Inference speed and memory efficiency": a fixed-size,
// head-specific KV cache; blog digest section 5: static KV cache).
//
// The step is bound by HBM bandwidth: every K and V element of every ring is
// read once.  Design:
//  * one workgroup (4 waves) per chunk of up to kDecodeChunk slots of one
//    (sequence, KV head); the waves stream interleaved blocks of 32 slots;
//  * S^T = K Q^T and O^T += V^T P^T run on the 16x16x32 bf16 matrix cores
//    with the G <= 16 query heads of the KV group on the N dimension, so the
//    dot products need no cross-lane reduction;
//  * within a 32-slot block, MFMA row m of key tile t is slot
//    8*(m/4) + 4*t + m%4; the S^T output then sits in exactly the layout the
//    P^T operand of the P.V product needs (lane l: head l%16, slots
//    8*(l/16) .. +7), so scores never move between lanes;
//  * V rings are stored in blocks of 32 slots, each block dimension-major
//    ([D][32]): a P.V operand is one 16-byte load of 8 consecutive slots of one
//    dimension, and each wave iteration streams one contiguous 8 KB block
//    (every load instruction covers 1 KB of whole lines, so the V stream is
//    read with the nontemporal hint; K rows are read as half lines, which the
//    hint would evict before their second half is used);
//  * online softmax per head (running max and sum, exp2 with the scale
//    folded in); the four waves merge in LDS;
//  * a head with one chunk writes its output directly; otherwise each chunk
//    writes (max, sum, o[D]) to the workspace and a second, small kernel
//    merges the partials of every (sequence, query head) in a fixed order
//    (deterministic).  The kernel boundary publishes the partials to every
//    XCD; a per-workgroup device-scope fence instead would write back the
//    whole L2 of the XCD once per chunk, which costs far more than the
//    second launch.
//
// Fused append (APPEND = true): the new token's key and value go to slot
// pos mod S_h.  The partial kernel never reads them from the ring: inside
// the streaming loop that slot is dropped (score -inf, value zero), and after
// the loop wave 0 of the chunk holding it adds the new key and value from
// k_new/v_new as one more step of its online softmax.  The ring write itself
// is left to the combine kernel, which runs after the streaming has ended:
// writes interleaved with the saturated read stream (even whole-line ones)
// measured several times dearer than the same writes in a phase of their own.

#include <cfloat>
#include <mutex>

#include "moa_device.h"
#include "moa_internal.h"

namespace moa {

// Fixed decode scratch for callers that cannot allocate (moa_append_decode_static).
// Each GPU the library runs on holds its own copy, at its own address, until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kStaticWsBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_workspace(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

constexpr int kWaves = 4;

template <int D, bool APPEND>
__global__ __launch_bounds__(256) void decode_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int4* __restrict__ chunks, const int32_t* __restrict__ span,
    const int64_t* __restrict__ ring_off, const int32_t* __restrict__ seq_len, int Npad, int Hq,
    int G, float scale_log2, bf16* __restrict__ o, float* __restrict__ ws_o,
    float2* __restrict__ ws_ml, const bf16* __restrict__ kn, const bf16* __restrict__ vn,
    int64_t pos, const int32_t* __restrict__ order) {
  constexpr int KS = D / 32;  // k-steps of the Q.K product
  constexpr int VT = D / 16;  // 16-dim tiles of the output
  __shared__ float sh_o[kWaves][D][17];
  __shared__ float sh_m[kWaves][16];
  __shared__ float sh_l[kWaves][16];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;   // query head within the group
  const int quad = lane >> 4;

  // chunk of all sequences' rings; a plan may launch them in another order
  const int part = order != nullptr ? order[blockIdx.x] : (int)blockIdx.x;
  const int4 ch = chunks[part];
  const int bh = ch.x, first = ch.y, len = ch.z, n_head_chunks = ch.w;
  const int Hkv = Hq / G;
  const int b = bh / Hkv;
  const int h = bh - b * Hkv;
  const int S = span[bh];
  const int64_t ring = ring_off[bh];
  // K rows of this chunk and the whole V^T ring of this head; loads past the
  // chunk's K rows return zero.
  const __amdgpu_buffer_rsrc_t krs =
      buffer_rsrc(kc + (ring + first) * D, (uint32_t)len * D * 2);
  const int R = (S + 31) & ~31;                   // ring pitch (slots)
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(vc + ring * D, (uint32_t)(D * R * 2));

  // Fused append: chunk-relative block (sub_k0) and slot in it (sub_r) of the
  // new position; sub_k0 = -1 when the slot lies in another chunk.
  int sub_k0 = -1, sub_r = 0;
  const bf16* knew = nullptr;
  const bf16* vnew = nullptr;
  if constexpr (APPEND) {
    // the sequence's own position (left padding), mod S in 32-bit arithmetic
    // whenever it is below 2^31
    const uint64_t up = (uint64_t)(pos - (Npad - seq_len[b]));
    const int ns = (up >> 31) == 0 ? (int)((uint32_t)up % (uint32_t)S) : (int)(up % (uint64_t)S);
    const int rel = ns - first;
    if (rel >= 0 && rel < len) {
      sub_k0 = rel & ~31;
      sub_r = rel & 31;
    }
    knew = kn + (int64_t)bh * D;
    vnew = vn + (int64_t)bh * D;
  }
  // Q^T operand: head col of the group (zero rows beyond G).
  bf16x8 qop[KS];
  const bool head_ok = col < G;
  const bf16* qrow = q + ((int64_t)b * Hq + (int64_t)h * G + (head_ok ? col : 0)) * D;
#pragma unroll
  for (int s = 0; s < KS; ++s) qop[s] = head_ok ? ld16(qrow + 32 * s + 8 * quad) : zero_bf16x8();

  floatx4 acc[VT];
#pragma unroll
  for (int t = 0; t < VT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // The four waves take interleaved 32-slot blocks, so at any time they read
  // neighbouring slots: both 64-byte halves of each 128-byte line of a V^T
  // row are requested together and the line is fetched from HBM once.
  const uint32_t krow_off = (8 * (col >> 2) + (col & 3)) * D * 2 + 16 * quad;
  // V^T ring: blocks of 32 slots, each block [D][32] contiguous (8 KB at
  // D = 128); lane (col, quad) of dim tile t reads row 16t + col, slots
  // 8*quad .. +7 of the block: one load instruction covers 1 KB contiguous.
  const uint32_t vlane = ((uint32_t)col * 32 + 8 * quad) * 2;
  const uint32_t vblk = 32u * D * 2;                // bytes per block
  const int w1 = len;
  for (int k0 = 32 * wave; k0 < w1; k0 += 32 * kWaves) {
    // ---- loads: K rows of both key tiles, V^T rows of every dim tile
    bf16x8 kop[2][KS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kop[t][s] = buffer_ld16(krs, krow_off + (uint32_t)(k0 + 4 * t) * D * 2 + 64 * s, 0);
    bf16x8 vop[VT];
    const uint32_t vbase = (uint32_t)((first + k0) >> 5) * vblk + vlane;
#pragma unroll
    for (int t = 0; t < VT; ++t) vop[t] = buffer_ld16_nt(vrs, vbase, t * 16 * 32 * 2);
    if (k0 + 32 > w1) {
      // ragged end of the segment: slots past it belong to other chunks or to
      // the ring's padding; clear them so they cannot reach P.V
#pragma unroll
      for (int t = 0; t < VT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + 8 * quad + e >= w1) vop[t][e] = (bf16)0.f;
    }
    // ---- scores S^T: lane holds head col, slots k0 + 8*quad + 4*t + r
    floatx4 sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sc[t] = mfma16(kop[t][s], qop[s], sc[t]);
    }
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = sc[e >> 2][e & 3];
      sv[e] = (k0 + 8 * quad + e < w1) ? x : -INFINITY;
    }
    if constexpr (APPEND) {
      if (k0 == sub_k0 && quad == (sub_r >> 3)) {
        // the new position's slot still holds the position it replaces:
        // drop it here; the new key and value are added after the loop
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e == (sub_r & 7)) {
            sv[e] = -INFINITY;
#pragma unroll
            for (int t = 0; t < VT; ++t) vop[t][e] = (bf16)0.f;
          }
      }
    }
    float bm = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sv[e]);
    bm = half_swap_max(row_swap_max(bm));
    // slot k0 is always valid, so bm is finite, unless it is the dropped
    // slot of a fused append: then keep the reference finite (p and alpha
    // are 0 for a block with no kept slot)
    float m_new = fmaxf(m_run, bm);
    if constexpr (APPEND) m_new = fmaxf(m_new, -FLT_MAX);
    const float alpha = fast_exp2((m_run - m_new) * scale_log2);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < VT; ++t) acc[t] *= alpha;
    const float mb = m_new * scale_log2;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(__builtin_fmaf(sv[e], scale_log2, -mb));
      l_run += p[e];
    }
    const bf16x8 pop = to_bf16x8(p);
#pragma unroll
    for (int t = 0; t < VT; ++t) acc[t] = mfma16(vop[t], pop, acc[t]);
  }
  // sum over the four lane quarters (each summed its own slots)
  l_run = half_swap_sum(row_swap_sum(l_run));

  if constexpr (APPEND) {
    if (sub_k0 >= 0 && wave == 0) {
      // the new key and value, one more online-softmax step of wave 0 (its
      // reference max is finite: it always streams the chunk's first block)
      float sc_new = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kx = ld16(knew + 32 * s + 8 * quad);
#pragma unroll
        for (int e = 0; e < 8; ++e) sc_new = __builtin_fmaf((float)qop[s][e], (float)kx[e], sc_new);
      }
      sc_new += __shfl_xor(sc_new, 16, 64);
      sc_new += __shfl_xor(sc_new, 32, 64);
      const float m_new = fmaxf(m_run, sc_new);
      const float alpha = fast_exp2((m_run - m_new) * scale_log2);
      const float p = fast_exp2(__builtin_fmaf(sc_new, scale_log2, -m_new * scale_log2));
      m_run = m_new;
      l_run = l_run * alpha + p;
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        // acc[t][r] holds dim 16t + 4quad + r of head col
        const bf16x4 vx = *reinterpret_cast<const bf16x4*>(vnew + 16 * t + 4 * quad);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = acc[t][r] * alpha + p * (float)vx[r];
      }
    }
  }

  // ---- merge the waves of the workgroup
  if (quad == 0) {
    sh_m[wave][col] = m_run;   // -inf for a wave without slots
    sh_l[wave][col] = l_run;
  }
#pragma unroll
  for (int t = 0; t < VT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) sh_o[wave][16 * t + 4 * quad + r][col] = acc[t][r];
  __syncthreads();

  // thread -> (head g, dims): 16 heads x 16 threads, D/16 dims each
  constexpr int DPT = D / 16;
  const int g = tid >> 4;
  const int dgrp = tid & 15;
  const bool g_ok = g < G;
  float m_tot = -INFINITY, l_tot = 0.f;
  float out[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) out[i] = 0.f;
  if (g_ok) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m_tot = fmaxf(m_tot, sh_m[w][g]);
    float wgt[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wgt[w] = sh_m[w][g] == -INFINITY ? 0.f : fast_exp2((sh_m[w][g] - m_tot) * scale_log2);
      l_tot += wgt[w] * sh_l[w][g];
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const int d = dgrp * DPT + i;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += wgt[w] * sh_o[w][d][g];
      out[i] = s;
    }
  }
  bf16* orow = o + ((int64_t)b * Hq + (int64_t)h * G + (g_ok ? g : 0)) * D + dgrp * DPT;
  if (n_head_chunks == 1) {
    if (g_ok) {
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int i = 0; i < DPT; ++i) orow[i] = (bf16)(out[i] * inv);
    }
    return;
  }

  // ---- split-K: publish this chunk's partial for the combine kernel
  if (g_ok) {
    float* wrow = ws_o + ((int64_t)part * G + g) * D + dgrp * DPT;
#pragma unroll
    for (int i = 0; i < DPT; i += 4)
      *reinterpret_cast<float4*>(wrow + i) = make_float4(out[i], out[i + 1], out[i + 2], out[i + 3]);
    if (dgrp == 0) ws_ml[(int64_t)part * G + g] = make_float2(m_tot, l_tot);
  }
}

// Merge the chunk partials of each (sequence, query head) whose KV head has
// more than one chunk: M = max m_c, L = sum l_c 2^{(m_c - M) c},
// O = sum o_c 2^{(m_c - M) c} / L.  One workgroup per (sequence, query head);
// thread (cg, dg) merges chunks cg, cg + 8, ... for dims 4dg .. 4dg+3 (all
// loads independent), then the 8 chunk groups merge in LDS in a fixed order.
// With APPEND, the workgroup of the first query head of each KV group also
// writes the new key and value of (sequence, KV head) into slot pos mod S_h
// of the rings (the partial kernel has finished reading them).
template <int D, bool APPEND>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const int2* __restrict__ head_chunks, int Hq, int G, float scale_log2,
    const float* __restrict__ ws_o, const float2* __restrict__ ws_ml, bf16* __restrict__ o,
    const bf16* __restrict__ kn, const bf16* __restrict__ vn, bf16* __restrict__ kc,
    bf16* __restrict__ vc, const int32_t* __restrict__ span, const int64_t* __restrict__ ring_off,
    const int32_t* __restrict__ seq_len, int Npad, int64_t pos) {
  constexpr int DG = D / 4;          // float4 groups of a row
  constexpr int CG = 256 / DG;       // chunk groups
  __shared__ float sh_m[CG], sh_l[CG];
  __shared__ float4 sh_o[CG][DG];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / Hq;
  const int hq = blockIdx.x - b * Hq;
  const int h = hq / G;
  const int g = hq - h * G;
  const int bh = b * (Hq / G) + h;   // (sequence, KV head)
  if constexpr (APPEND) {
    if (g == 0) {
      const int S = span[bh];
      const uint64_t up = (uint64_t)(pos - (Npad - seq_len[b]));
      const int slot = (up >> 31) == 0 ? (int)((uint32_t)up % (uint32_t)S) : (int)(up % (uint64_t)S);
      const int64_t ring = ring_off[bh];
      const int64_t row = (int64_t)bh * D;
      if (tid < D / 8) st16(kc + (ring + slot) * D + 8 * tid, ld16(kn + row + 8 * tid));
      if (tid < D)
        vc[(ring + (slot & ~31)) * D + tid * 32 + (slot & 31)] = vn[row + tid];
    }
  }
  const int2 hc = head_chunks[bh];
  if (hc.y <= 1) return;
  const int dg = tid % DG;
  const int cg = tid / DG;
  const int64_t part0 = hc.x;
  float M = -INFINITY, L = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int c = cg; c < hc.y; c += CG) {
    const int64_t pc = (part0 + c) * G + g;
    const float2 ml = ws_ml[pc];
    const float4 x = *reinterpret_cast<const float4*>(ws_o + pc * D + 4 * dg);
    const float mn = fmaxf(M, ml.x);
    const float sa = fast_exp2((M - mn) * scale_log2);
    const float sb = fast_exp2((ml.x - mn) * scale_log2);
    M = mn;
    L = L * sa + ml.y * sb;
    a.x = a.x * sa + x.x * sb;
    a.y = a.y * sa + x.y * sb;
    a.z = a.z * sa + x.z * sb;
    a.w = a.w * sa + x.w * sb;
  }
  if (dg == 0) {
    sh_m[cg] = M;   // -inf for a group without chunks
    sh_l[cg] = L;
  }
  sh_o[cg][dg] = a;
  __syncthreads();
  if (cg != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < CG; ++i) Mt = fmaxf(Mt, sh_m[i]);
  float Lt = 0.f;
  float4 ot = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < CG; ++i) {
    const float w = sh_m[i] == -INFINITY ? 0.f : fast_exp2((sh_m[i] - Mt) * scale_log2);
    const float4 x = sh_o[i][dg];
    Lt += w * sh_l[i];
    ot.x += w * x.x;
    ot.y += w * x.y;
    ot.z += w * x.z;
    ot.w += w * x.w;
  }
  const float inv = 1.f / Lt;
  bf16x4 r;
  r[0] = (bf16)(ot.x * inv);
  r[1] = (bf16)(ot.y * inv);
  r[2] = (bf16)(ot.z * inv);
  r[3] = (bf16)(ot.w * inv);
  *reinterpret_cast<bf16x4*>(o + ((int64_t)b * Hq + hq) * D + 4 * dg) = r;
}

template <int D, bool APPEND>
hipError_t launch(const moa_plan& p, const void* q, const void* kc, const void* vc, void* o,
                  void* ws, const void* kn, const void* vn, int64_t pos, hipStream_t s) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  DecodeWs w = decode_ws_layout(p, ws);
  hipLaunchKernelGGL((decode_kernel<D, APPEND>), dim3((unsigned)p.n_chunks), dim3(256), 0, s,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(kc),
                     static_cast<const bf16*>(vc), p.dev.decode_chunks, p.dev.span, p.dev.ring,
                     p.dev.seq_len, (int)p.N, p.Hq, p.G, scale_log2, static_cast<bf16*>(o), w.o,
                     w.ml, static_cast<const bf16*>(kn), static_cast<const bf16*>(vn), pos,
                     p.dev.decode_order);
  hipError_t e = hipGetLastError();
  // the combine runs when some head is split, and always for a fused append
  // (it writes the new rows)
  if (e != hipSuccess || (!p.any_split && !APPEND)) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D, APPEND>), dim3((unsigned)(p.B * p.Hq)), dim3(256),
                     0, s, p.dev.head_chunks, p.Hq, p.G, scale_log2, w.o, w.ml,
                     static_cast<bf16*>(o), static_cast<const bf16*>(kn),
                     static_cast<const bf16*>(vn), const_cast<bf16*>(static_cast<const bf16*>(kc)),
                     const_cast<bf16*>(static_cast<const bf16*>(vc)), p.dev.span, p.dev.ring,
                     p.dev.seq_len, (int)p.N, pos);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const moa_plan& p, const void* q, const void* kc, const void* vc,
                              void* o, void* ws, hipStream_t s) {
  return p.D == 64 ? launch<64, false>(p, q, kc, vc, o, ws, nullptr, nullptr, 0, s)
                   : launch<128, false>(p, q, kc, vc, o, ws, nullptr, nullptr, 0, s);
}

hipError_t launch_append_decode_bf16(const moa_plan& p, const void* q, void* kc, void* vc,
                                     const void* kn, const void* vn, int64_t pos, void* o,
                                     void* ws, hipStream_t s) {
  return p.D == 64 ? launch<64, true>(p, q, kc, vc, o, ws, kn, vn, pos, s)
                   : launch<128, true>(p, q, kc, vc, o, ws, kn, vn, pos, s);
}

}  // namespace moa
