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
//  * V rings are dimension-major, so each P.V operand is one 16-byte load of
//    8 consecutive slots of one dimension;
//  * online softmax per head (running max and sum, exp2 with the scale
//    folded in); the four waves merge in LDS;
//  * a head with one chunk writes its output directly; otherwise each chunk
//    writes (max, sum, o[D]) to the workspace and a second, small kernel
//    merges the partials of every (sequence, KV head) in chunk order
//    (deterministic).  The kernel boundary publishes the partials to every
//    XCD; a per-workgroup device-scope fence instead would write back the
//    whole L2 of the XCD once per chunk, which costs far more than the
//    second launch.

#include "moa_device.h"
#include "moa_internal.h"

namespace moa {
namespace {

constexpr int kWaves = 4;

template <int D>
__global__ __launch_bounds__(256) void decode_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int4* __restrict__ chunks, const int2* __restrict__ head_chunks,
    const int32_t* __restrict__ span, const int64_t* __restrict__ offset, int64_t slots,
    int n_chunks, int Hq, int G, float scale_log2, bf16* __restrict__ o,
    float* __restrict__ ws_o, float2* __restrict__ ws_ml) {
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

  const int part = blockIdx.x;
  const int b = part / n_chunks;
  const int ci = part - b * n_chunks;
  const int4 ch = chunks[ci];
  const int h = ch.x, first = ch.y, len = ch.z, n_head_chunks = ch.w;
  const int S = span[h];
  const int64_t ring = (int64_t)b * slots + offset[h];
  // K rows of this chunk and the whole V^T ring of this head; loads past the
  // chunk's K rows return zero.
  const __amdgpu_buffer_rsrc_t krs =
      buffer_rsrc(kc + (ring + first) * D, (uint32_t)len * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(vc + ring * D, (uint32_t)(D * S * 2));

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
  const uint32_t vrow_off = ((uint32_t)col * S + first + 8 * quad) * 2;
  const uint32_t vtile = 16u * (uint32_t)S * 2;   // bytes between 16-dim tiles
  const int w1 = len;
  const bool v_aligned = (S & 7) == 0;   // V^T rows start on 16-byte boundaries
  for (int k0 = 32 * wave; k0 < w1; k0 += 32 * kWaves) {
    // ---- loads: K rows of both key tiles, V^T rows of every dim tile
    bf16x8 kop[2][KS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kop[t][s] = buffer_ld16(krs, krow_off + (uint32_t)(k0 + 4 * t) * D * 2 + 64 * s, 0);
    bf16x8 vop[VT];
    if (v_aligned) {
#pragma unroll
      for (int t = 0; t < VT; ++t) vop[t] = buffer_ld16(vrs, vrow_off + 2u * k0, t * vtile);
      if (k0 + 32 > w1) {
        // ragged end of the chunk: slots past it belong to other chunks (or lie
        // past the ring and read as zero); clear them so they cannot reach P.V
#pragma unroll
        for (int t = 0; t < VT; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k0 + 8 * quad + e >= w1) vop[t][e] = (bf16)0.f;
      }
    } else {
      // S_h not a multiple of 8 (S_h = 1, or S_h = N for such N): V^T rows
      // are not 16-byte aligned, so read element by element
      const bf16* vrow = vc + ring * D + (int64_t)col * S + first + k0 + 8 * quad;
#pragma unroll
      for (int t = 0; t < VT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          vop[t][e] = k0 + 8 * quad + e < w1 ? vrow[(int64_t)16 * t * S + e] : (bf16)0.f;
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
    float bm = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sv[e]);
    bm = wave_max_xor(bm, 16);
    bm = wave_max_xor(bm, 32);
    // slot k0 is always valid, so bm is finite
    const float m_new = fmaxf(m_run, bm);
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
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

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

// Merge the chunk partials of each (sequence, KV head) with more than one
// chunk, in chunk order: M = max m_c, L = sum l_c 2^{(m_c - M) c},
// O = sum o_c 2^{(m_c - M) c} / L.  One workgroup per (sequence, KV head).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const int2* __restrict__ head_chunks, int n_chunks, int Hq, int Hkv, int G,
    float scale_log2, const float* __restrict__ ws_o, const float2* __restrict__ ws_ml,
    bf16* __restrict__ o) {
  constexpr int DPT = D / 16;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / Hkv;
  const int h = blockIdx.x - b * Hkv;
  const int2 hc = head_chunks[h];
  const int g = tid >> 4;
  const int dgrp = tid & 15;
  if (hc.y <= 1 || g >= G) return;
  const int64_t part0 = (int64_t)b * n_chunks + hc.x;
  float M = -INFINITY, L = 0.f;
  float a[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) a[i] = 0.f;
#pragma unroll 4
  for (int c = 0; c < hc.y; ++c) {
    const int64_t pc = (part0 + c) * G + g;
    const float2 ml = ws_ml[pc];
    float x[DPT];
#pragma unroll
    for (int i = 0; i < DPT; i += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(ws_o + pc * D + dgrp * DPT + i);
      x[i] = v4.x; x[i + 1] = v4.y; x[i + 2] = v4.z; x[i + 3] = v4.w;
    }
    const float mn = fmaxf(M, ml.x);
    const float sa = fast_exp2((M - mn) * scale_log2);
    const float sb = fast_exp2((ml.x - mn) * scale_log2);
    M = mn;
    L = L * sa + ml.y * sb;
#pragma unroll
    for (int i = 0; i < DPT; ++i) a[i] = a[i] * sa + x[i] * sb;
  }
  const float inv = 1.f / L;
  bf16* orow = o + ((int64_t)b * Hq + (int64_t)h * G + g) * D + dgrp * DPT;
#pragma unroll
  for (int i = 0; i < DPT; ++i) orow[i] = (bf16)(a[i] * inv);
}

template <int D>
hipError_t launch(const moa_plan& p, const void* q, const void* kc, const void* vc, void* o,
                  void* ws, hipStream_t s) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  const int64_t parts = (int64_t)p.B * p.n_chunks;
  DecodeWs w = decode_ws_layout(p, ws);
  hipLaunchKernelGGL(decode_kernel<D>, dim3((unsigned)parts), dim3(256), 0, s,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(kc),
                     static_cast<const bf16*>(vc), p.dev.decode_chunks, p.dev.head_chunks,
                     p.dev.span, p.dev.offset, p.slots, (int)p.n_chunks, p.Hq, p.G,
                     scale_log2, static_cast<bf16*>(o), w.o, w.ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.any_split) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)(p.B * p.Hkv)), dim3(256), 0, s,
                     p.dev.head_chunks, (int)p.n_chunks, p.Hq, p.Hkv, p.G, scale_log2, w.o, w.ml,
                     static_cast<bf16*>(o));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const moa_plan& p, const void* q, const void* kc, const void* vc,
                              void* o, void* ws, hipStream_t s) {
  return p.D == 64 ? launch<64>(p, q, kc, vc, o, ws, s) : launch<128>(p, q, kc, vc, o, ws, s);
}

}  // namespace moa
