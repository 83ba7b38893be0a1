// Prefill attention with a per-head sliding window (gfx950).
//
// o[b,h,i] = sum over j in [max(0, i - S + 1), i] of softmax_j(q_i.k_j/sqrt(D)) v_j,
// S the span of KV head h / G.  Blog digest "MoA: Mixture of Sparse Attention
// for Automatic Large Language Model Compression", section 2.1: a
// sliding-window mask is the base pattern; "Mixture of Attention" project
// page, "Finding 2": each head has its own span, and the figure keeps a band
// of the causal matrix.
//
// Work units come from the plan's launch table: 128 query rows of one
// (b, h_q) and the range of 64-key tiles that hold at least one kept pair;
// tiles outside the window are never loaded.  The table is XCD-aware:
// workgroups are dealt to the 8 XCDs round-robin, and the host lays the units
// out so that each XCD runs runs of up to 16 consecutive query tiles of one
// head (whose key windows overlap, so they meet in that XCD's L2), longest
// runs first, with about the same work on every XCD.  Padding entries exit at
// once.  A sequence of N_b tokens occupies the last N_b of the Npad rows of
// its [H, Npad, D] slices (left padding): the kernels shift its base pointers
// by Npad - N_b rows and work in its own positions 0 .. N_b - 1; padding rows
// are neither read nor written.
//
// bf16 kernel (4 waves, 32 query rows each):
//  * S^T = K Q^T on 32x32x16 bf16 MFMA, so each lane owns one query row and
//    the row max needs one exchange with the partner lane (l ^ 32);
//  * key rows of a 32-key MFMA tile are permuted (row m = 16a + 8b + 4h + c
//    reads key 16a + 8h + 4b + c), which puts the scores of lane half h on
//    keys 16j + 8h .. +7 of P.V step j: the P^T operand is the lane's own
//    scores, converted to bf16, with no data movement;
//  * K and V tiles go from memory straight into LDS (16-byte LDS-direct
//    buffer loads, no staging registers), in a chunk-swizzled layout that
//    both fragment reads meet without bank conflicts; the V^T operand of the
//    P.V product (8 consecutive keys of one dimension per lane) comes from
//    two transposed LDS reads (ds_read_b64_tr_b16);
//  * LDS tiles are double-buffered: tile t+1's loads are issued before tile
//    t is computed (one wait and one barrier a tile);
//  * O goes through LDS: each wave writes its normalised rows to LDS and
//    stores them as whole 16-byte chunks, four complete rows per store
//    instruction;
//  * masks are evaluated only on tiles a wave's rows do not fully keep, and a
//    wave skips tiles none of its rows keep;
//  * online softmax in fp32 with exp2: the scores leave the matrix cores raw
//    (fp32) and 1/sqrt(D)*log2(e) is applied in fp32 before each
//    exponential; O and the row sum are rescaled only when a row's max grows
//    by more than 8 in the exp2 domain (a factor of 2^8), which most tiles
//    after the first never trigger.
//
// f32 kernel (the float32 dtype): 2 threads per query row, each owning half
// of the head dimension; K/V tiles in LDS; plain FMA arithmetic.
//
// Fused handoff (RING = true): besides o, the launch writes positions
// N - S_h .. N - 1 of every (b, h_kv) into the KV rings, as an append of the
// whole prompt would.  Key tile kt is the diagonal tile of query tile
// kt*BN/BM, whose item always streams it; the workgroup of the first query
// head of each KV group (g = 0) stores the rows of its diagonal tiles that the
// ring keeps, reading them from LDS.  Every ring row is therefore written
// once, and K/V are read from HBM once.  The diagonal tiles are the unit's
// last one or two, still in their buffers when the loop ends, so the stores
// follow the loop and the loop itself is the plain kernel's.

#include "moa_device.h"
#include "moa_internal.h"

namespace moa {
namespace {

constexpr int BM = kPrefillBM;
constexpr int BN = kPrefillBN;

// LDS layout of a 64-row K or V tile (row = key): 16-byte chunks (8 dims)
// in groups of four; group cg holds its 64-byte slice of all 64 rows, and
// the chunk's place inside the slice is XOR-swizzled by row bits 2-3.  Byte
// offset of chunk c of row r:
__device__ __forceinline__ constexpr int tile_off(int r, int c) {
  return (c >> 2) * 4096 + r * 64 + (((c & 3) ^ ((r >> 2) & 3)) << 4);
}
// (One wave's 16-byte LDS-direct load fills 1 KB: 16 rows of one group.
// The 16 lanes of an LDS read phase meet 16 different rows of one chunk
// column in different banks, for the K reads and the transposed V reads.)

template <int D, bool RING>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, const int4* __restrict__ items, const int32_t* __restrict__ span,
    const int32_t* __restrict__ seq_len, int seq_grid, int Hq, int Hkv, int G, int Npad,
    float scale_log2, bf16* __restrict__ kc, bf16* __restrict__ vc,
    const int64_t* __restrict__ ring) {
  constexpr int KS = D / 16;       // k-steps of the Q.K product
  constexpr int OT = D / 32;       // 32-dim tiles of the output
  constexpr int ROWB = D * 2;      // bytes of a K/V row
  constexpr int TILEB = BN * ROWB; // bytes of a K or V tile
  constexpr int NDMA = D / 32;     // LDS-direct rounds per tile (chunk groups)
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // the table runs once per sequence (seq_grid > 0) or names the sequence
  const unsigned copy = seq_grid > 0 ? blockIdx.x / (unsigned)seq_grid : 0u;
  const int4 it = items[blockIdx.x - copy * (unsigned)seq_grid];
  if (it.x < 0) return;   // padding entry of the launch table
  const int b = it.x / Hq + (int)copy;
  const int hq = it.x % Hq, qt = it.y, kt_lo = it.z, kt_hi = it.w;
  const int bh = b * Hq + hq;
  const int hkv = hq / G;
  const int S = span[b * Hkv + hkv];
  // the sequence's own rows: the last N of the Npad padded rows
  const int N = seq_len[b];
  const int64_t pad = Npad - N;
  const bf16* qb = q + ((int64_t)bh * Npad + pad) * D;
  const bf16* kb = k + (((int64_t)b * Hkv + hkv) * Npad + pad) * D;
  const bf16* vb = v + (((int64_t)b * Hkv + hkv) * Npad + pad) * D;
  bf16* ob = o + ((int64_t)bh * Npad + pad) * D;
  // fused handoff: this workgroup's K/V rings (only g = 0 writes them)
  bf16* kring = nullptr;
  bf16* vring = nullptr;
  if constexpr (RING) {
    if (hq == hkv * G) {
      const int64_t r0 = ring[b * Hkv + hkv] * D;
      kring = kc + r0;
      vring = vc + r0;
    }
  }

  // LDS-direct staging: round i of wave w fills bytes i*4096 + w*1024 +
  // 16*lane of a tile, i.e. chunk group i, rows 16w + lane/4, slice place
  // lane % 4, which holds chunk 4i + ((lane % 4) ^ (lane / 16 % 4)) of that
  // row.  Rows at or past N read as zero (buffer bounds).
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(kb, (uint32_t)N * ROWB);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(vb, (uint32_t)N * ROWB);
  const uint32_t dma_off =
      (uint32_t)(16 * wave + (lane >> 2)) * ROWB + (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  // The loads are issued from inline assembly so that the compiler, which
  // cannot tell that they fill the other buffer, does not wait for them
  // before every LDS read of the current one; the explicit vmcnt(0) before
  // each barrier is their only wait.  They write no registers.
  auto dma_tile = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const uint32_t soff = (uint32_t)kt * TILEB + i * 64;
      const int dst = i * 4096 + wave * 1024;
      lds_direct_ld16(krs, dma_off, soff, (char*)&Ks[buf][0] + dst);
      lds_direct_ld16(vrs, dma_off, soff, (char*)&Vs[buf][0] + dst);
    }
  };

  // the first tile's loads go out before Q's, so their latencies overlap
  dma_tile(kt_lo, 0);

  const int iw0 = qt * BM + wave * 32;  // first query row of this wave
  const int my_q = iw0 + l32;

  // Q goes to the matrix cores as stored: the scores come out raw (fp32), and
  // log2(e)/sqrt(D) is applied in fp32 before each exponential.  Scaling Q in
  // bf16 first would round every score by up to 2^-9 of its size, which at
  // large logits moves the weights by far more than bf16 output rounding.
  bf16x8 qop[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qop[s] = my_q < N ? ld16(qb + (int64_t)my_q * D + 16 * s + 8 * half) : zero_bf16x8();
  // the lazy-rescale threshold, 8 in the exp2 domain, in raw score units
  const float thr = 8.f / scale_log2;

  floatx16 acc[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  // m_run: the row's running max (raw score), -inf before its first kept
  // key.  m_ref: the reference the scores are taken against (m_run once set,
  // 0 before); -m_ref seeds the Q.K accumulators, so the matrix cores return
  // score - m_ref, which times scale_log2 is the exp2 argument.
  float m_run = -INFINITY, m_ref = 0.f;
  float l_a = 0.f, l_b = 0.f;   // row sum, two partial chains
  floatx16 minit;
#pragma unroll
  for (int r = 0; r < 16; ++r) minit[r] = 0.f;

  // K fragment (Q.K, tile t, k-step s): row 32t + kperm, chunk 2s + half.
  // With kperm's row bits 2-3 fixed per lane, the byte offset is a per-lane
  // base (one for even s, one for odd s) plus (s / 2) * 4096 + t * 2048.
  const int kperm = 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
  const int kx = (kperm >> 2) & 3;
  const int k_even = kperm * 64 + ((half ^ kx) << 4);
  const int k_odd = kperm * 64 + (((2 + half) ^ kx) << 4);
  // V^T fragment (P.V step j, dim tile t): two transposed 8-byte reads, rd =
  // 0, 1 (keys 16j + 8*(g/2) + 4rd + 0..3 of dims 32t + 16*(g%2) + i, lane =
  // 16g + i).  Lane i of each 16-lane group points at row +i/4, dims +4(i%4).
  const int vg = lane >> 4, vi = lane & 15;
  const int v_lane = (8 * (vg >> 1) + (vi >> 2)) * 64 + 8 * (vi & 1);
  const int v_c = 2 * (vg & 1) + ((vi >> 1) & 1);
  const int v_rd0 = v_lane + ((v_c ^ ((2 * (vg >> 1)) & 3)) << 4);
  const int v_rd1 = v_lane + ((v_c ^ ((2 * (vg >> 1) + 1) & 3)) << 4);

  // Fused handoff: the tile's rows that the ring keeps (positions N - S ..
  // N - 1, slot p mod S) go from LDS to the rings.  K: 16-byte chunks.  V:
  // transposed reads give 4 consecutive keys of one dimension, stored as one
  // 8-byte run when the 4 slots are consecutive (S a multiple of 4, or S = N:
  // slot = p), else element by element.
  auto ring_tile = [&](int kt, int buf) {
    if constexpr (RING) {
      if (kring == nullptr || kt * BN / BM != qt || (kt + 1) * BN <= N - S) return;
      const char* kl = (const char*)&Ks[buf][0];
      const char* vl = (const char*)&Vs[buf][0];
      constexpr int CPR = D / 8;
#pragma unroll
      for (int u = 0; u < CPR / 4; ++u) {
        const int id = u * 256 + tid;
        const int r = id / CPR, c = id % CPR;
        const int p = kt * BN + r;
        if (p >= N - S && p < N)
          st16(kring + (int64_t)(p % S) * D + 8 * c, *reinterpret_cast<const bf16x8*>(kl + tile_off(r, c)));
      }
      // 16 key groups x D/16 dim blocks, one per 16-lane group and round
      const int grp = tid >> 4;
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
        const int unit = u * 16 + grp;
        const int kg = unit & 15, m = unit >> 4;
        const int r = 4 * kg + (vi >> 2);
        const int dim0 = 16 * m + 4 * (vi & 3);
        const int off = tile_off(r, dim0 >> 3) + 2 * (dim0 & 7);
        const bf16x4 x = lds_read_tr16(vl + off);
        const int p0 = kt * BN + 4 * kg;
        const int d = 16 * m + vi;
        if (p0 >= N - S && p0 + 3 < N && (S % 4 == 0 || S == N)) {
          const int slot0 = p0 % S;
          *reinterpret_cast<bf16x4*>(vring + (int64_t)(slot0 >> 5) * (32 * D) + d * 32 + (slot0 & 31)) = x;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int p = p0 + e;
            if (p >= N - S && p < N) {
              const int slot = p % S;
              vring[(int64_t)(slot >> 5) * (32 * D) + d * 32 + (slot & 31)] = x[e];
            }
          }
        }
      }
    }
  };

  // Double-buffered LDS-direct tiles: tile kt+1's loads are issued before
  // tile kt is computed; one wait and one barrier a tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int buf = (kt - kt_lo) & 1;
    if (kt < kt_hi) dma_tile(kt + 1, buf ^ 1);

    const int j0 = kt * BN;
    const bool active = iw0 < N && j0 <= iw0 + 31 && j0 + BN - 1 >= iw0 - S + 1;
    if (active) {
      const bool full = j0 + BN - 1 <= iw0 && j0 >= iw0 + 31 - S + 1 && j0 + BN <= N;
      const char* kl = (const char*)&Ks[buf][0];
      const char* vl = (const char*)&Vs[buf][0];
      floatx16 st[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st[t] = minit;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int off = ((s & 1) ? k_odd : k_even) + (s >> 1) * 4096 + t * 2048;
          st[t] = mfma32(*reinterpret_cast<const bf16x8*>(kl + off), qop[s], st[t]);
        }
      }
      // keep four K-fragment reads in flight ahead of the matrix cores
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * KS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // st[t][r] is raw score - m_ref of query my_q and key
      // j0 + 32t + 16(r>>3) + 8half + (r&7)
      if (!full) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * t + 16 * (r >> 3) + 8 * half + (r & 7);
            const bool ok = key <= my_q && key >= my_q - S + 1 && key < N;
            st[t][r] = ok ? st[t][r] : -INFINITY;
          }
      }
      float mx = st[0][0];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[t][r]);
      mx = half_swap_max(mx);
      // Lazy rescale: the reference moves (and O, l are rescaled) only when
      // some row's tile max exceeds it by more than 8 in the exp2 domain, or
      // sets it at the row's first kept key; otherwise p <= 256, harmless in
      // fp32 and bf16.  The final O / l is unchanged.
      if (__ballot(mx > thr || (m_run == -INFINITY && mx != -INFINITY))) {
        const float m_new = fmaxf(m_run, mx == -INFINITY ? -INFINITY : m_ref + mx);
        const bool set = m_new != -INFINITY;   // else: no kept key yet, nothing moves
        const float alpha = set ? fast_exp2((m_run - m_new) * scale_log2) : 1.f;   // 0 at the first key
        const float delta = set ? m_new - m_ref : 0.f;
        if (set) {
          m_run = m_new;
          m_ref = m_new;
        }
        l_a *= alpha;
        l_b *= alpha;
#pragma unroll
        for (int t = 0; t < OT; ++t) acc[t] *= alpha;
#pragma unroll
        for (int t = 0; t < 2; ++t) st[t] -= delta;
#pragma unroll
        for (int r = 0; r < 16; ++r) minit[r] = -m_ref;
      }
      float p[2][16];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[t][r] = fast_exp2(st[t][r] * scale_log2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 pop = to_bf16x8(&p[j >> 1][8 * (j & 1)]);
        // the row sum of the bf16 weights the P.V product uses, two per step
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2 pair = {pop[2 * i], pop[2 * i + 1]};
          if (i & 1) l_b = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, l_b, false);
          else       l_a = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, l_a, false);
        }
#pragma unroll
        for (int t = 0; t < OT; ++t) {
          const int base = t * 4096 + 16 * j * 64;
          const bf16x4 a0 = lds_read_tr16(vl + base + v_rd0);
          const bf16x4 a1 = lds_read_tr16(vl + base + 4 * 64 + v_rd1);
          const bf16x8 vop = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[t] = mfma32(vop, pop, acc[t]);
        }
      }
      // same for the V^T fragments of the P.V product
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
      for (int i = 0; i < 4 * OT - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): tile kt+1 is in LDS
    __syncthreads();
  }

  if constexpr (RING) {
    // The ring keeps rows of the unit's diagonal key tiles (2 qt and 2 qt + 1),
    // the loop's last one or two tiles, which are still in their buffers.
    if (kt_hi - 1 >= kt_lo) ring_tile(kt_hi - 1, (kt_hi - 1 - kt_lo) & 1);
    ring_tile(kt_hi, (kt_hi - kt_lo) & 1);
    __syncthreads();   // before O is staged in the K buffers
  }

  // O through LDS: each wave writes its 32 normalised rows into its own part
  // of the (now idle) K buffers, chunk c of row r at byte
  // 16 * (c ^ (r mod chunks per row)), and reads them back as whole 16-byte
  // chunks, so that each store instruction writes four complete output rows.
  // Rows at or past N are not stored.
  const float l_run = half_swap_sum(l_a + l_b);
  const float inv = 1.f / l_run;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  char* ow = (char*)&Ks[0][0] + wave * (32 * D * 2);
#pragma unroll
  for (int t = 0; t < OT; ++t)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 x;
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = (bf16)(acc[t][4 * a + c] * inv);
      const int ch = 4 * t + a;              // chunk 32t + 8a .. +7 of the row
      *reinterpret_cast<bf16x4*>(ow + l32 * (2 * D) + ((ch ^ (l32 % CPR)) << 4) + 8 * half) = x;
    }
  // Each lane reads back chunks that other lanes wrote.  Lanes sharing data
  // through LDS need a barrier between the writes and the reads; without one
  // the compiler may move a lane's reads above its writes, which do not alias.
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int r = (i * 64 + lane) / CPR, ch = lane % CPR;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(ow + r * (2 * D) + ((ch ^ (r % CPR)) << 4));
    if (iw0 + r < N) st16(ob + (int64_t)(iw0 + r) * D + 8 * ch, x);
  }
}

template <int D, bool RING>
__global__ __launch_bounds__(256) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, const int4* __restrict__ items, const int32_t* __restrict__ span,
    const int32_t* __restrict__ seq_len, int seq_grid, int Hq, int Hkv, int G, int Npad,
    float scale_log2, float* __restrict__ kc, float* __restrict__ vc,
    const int64_t* __restrict__ ring) {
  constexpr int DH = D / 2;
  __shared__ __attribute__((aligned(16))) float Ks[BN * D];
  __shared__ __attribute__((aligned(16))) float Vs[BN * D];
  const int tid = threadIdx.x;
  const int half = tid & 1;
  // the table runs once per sequence (seq_grid > 0) or names the sequence
  const unsigned copy = seq_grid > 0 ? blockIdx.x / (unsigned)seq_grid : 0u;
  const int4 it = items[blockIdx.x - copy * (unsigned)seq_grid];
  if (it.x < 0) return;   // padding entry of the launch table
  const int b = it.x / Hq + (int)copy;
  const int hq = it.x % Hq, qt = it.y, kt_lo = it.z, kt_hi = it.w;
  const int bh = b * Hq + hq;
  const int hkv = hq / G;
  const int S = span[b * Hkv + hkv];
  const int N = seq_len[b];
  const int64_t pad = Npad - N;
  const float* kb = k + (((int64_t)b * Hkv + hkv) * Npad + pad) * D;
  const float* vb = v + (((int64_t)b * Hkv + hkv) * Npad + pad) * D;
  const int my_q = qt * BM + (tid >> 1);
  // fused handoff (see the file comment): only g = 0 writes the rings
  float* kring = nullptr;
  float* vring = nullptr;
  if constexpr (RING) {
    if (hq == hkv * G) {
      const int64_t r0 = ring[b * Hkv + hkv] * D;
      kring = kc + r0;
      vring = vc + r0;
    }
  }

  float qr[DH];
  const float* qrow = q + ((int64_t)bh * Npad + pad + (my_q < N ? my_q : 0)) * D + half * DH;
#pragma unroll
  for (int e = 0; e < DH; e += 4) {
    const float4 x = *reinterpret_cast<const float4*>(qrow + e);
    qr[e] = x.x; qr[e + 1] = x.y; qr[e + 2] = x.z; qr[e + 3] = x.w;
  }
  float acc[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) acc[e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int j0 = kt * BN;
    __syncthreads();
    for (int i = tid; i < BN * D / 4; i += 256) {
      const int key = j0 + (i * 4) / D;
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (key < N) {
        kx = *reinterpret_cast<const float4*>(kb + (int64_t)j0 * D + 4 * i);
        vx = *reinterpret_cast<const float4*>(vb + (int64_t)j0 * D + 4 * i);
      }
      *reinterpret_cast<float4*>(&Ks[4 * i]) = kx;
      *reinterpret_cast<float4*>(&Vs[4 * i]) = vx;
      if constexpr (RING) {
        if (kring != nullptr && kt * BN / BM == qt && key >= N - S && key < N) {
          const int slot = key % S;
          const int d = (4 * i) % D;
          *reinterpret_cast<float4*>(kring + (int64_t)slot * D + d) = kx;
          float* dst = vring + (int64_t)(slot >> 5) * (32 * D) + d * 32 + (slot & 31);
          dst[0] = vx.x;
          dst[32] = vx.y;
          dst[64] = vx.z;
          dst[96] = vx.w;
        }
      }
    }
    __syncthreads();
    float sc[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float* kr = &Ks[j * D + half * DH];
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < DH; ++e) s = __builtin_fmaf(qr[e], kr[e], s);
      s += __shfl_xor(s, 1, 64);
      const int key = j0 + j;
      const bool ok = key <= my_q && key >= my_q - S + 1 && key < N;
      sc[j] = ok ? s : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * scale_log2);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < DH; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      // (s - m) first: a score equal to the running max gives exactly 1
      const float p = exp2f((sc[j] - m_use) * scale_log2);
      l_run += p;
      const float* vr = &Vs[j * D + half * DH];
#pragma unroll
      for (int e = 0; e < DH; ++e) acc[e] = __builtin_fmaf(p, vr[e], acc[e]);
    }
  }
  if (my_q >= N) return;
  const float inv = 1.f / l_run;
  float* orow = o + ((int64_t)bh * Npad + pad + my_q) * D + half * DH;
#pragma unroll
  for (int e = 0; e < DH; e += 4)
    *reinterpret_cast<float4*>(orow + e) =
        make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
}

template <int D, bool RING>
void launch_bf16(const moa_plan& p, const void* q, const void* k, const void* v, void* o, void* kc,
                 void* vc, hipStream_t s) {
  const unsigned table = (unsigned)(p.prefill_items.size() / 4);
  const unsigned grid = p.prefill_seq_grid > 0 ? table * (unsigned)p.B : table;
  const float scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, RING>), dim3(grid), dim3(256), 0, s,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<bf16*>(o), p.dev.prefill_items,
                     p.dev.span, p.dev.seq_len, (int)p.prefill_seq_grid, p.Hq, p.Hkv, p.G, (int)p.N,
                     scale_log2,
                     static_cast<bf16*>(kc), static_cast<bf16*>(vc), p.dev.ring);
}

template <int D, bool RING>
void launch_f32(const moa_plan& p, const void* q, const void* k, const void* v, void* o, void* kc,
                void* vc, hipStream_t s) {
  const unsigned table = (unsigned)(p.prefill_items.size() / 4);
  const unsigned grid = p.prefill_seq_grid > 0 ? table * (unsigned)p.B : table;
  const float scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((prefill_f32_kernel<D, RING>), dim3(grid), dim3(256), 0, s,
                     static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), static_cast<float*>(o), p.dev.prefill_items,
                     p.dev.span, p.dev.seq_len, (int)p.prefill_seq_grid, p.Hq, p.Hkv, p.G, (int)p.N,
                     scale_log2,
                     static_cast<float*>(kc), static_cast<float*>(vc), p.dev.ring);
}

}  // namespace

// kc = vc = nullptr: attention only; otherwise also the ring handoff.
hipError_t launch_prefill(const moa_plan& p, const void* q, const void* k, const void* v, void* o,
                          void* kc, void* vc, hipStream_t s) {
  const bool ring = kc != nullptr;
  if (p.dtype == MOA_BF16) {
    if (p.D == 64)
      ring ? launch_bf16<64, true>(p, q, k, v, o, kc, vc, s)
           : launch_bf16<64, false>(p, q, k, v, o, kc, vc, s);
    else
      ring ? launch_bf16<128, true>(p, q, k, v, o, kc, vc, s)
           : launch_bf16<128, false>(p, q, k, v, o, kc, vc, s);
  } else {
    if (p.D == 64)
      ring ? launch_f32<64, true>(p, q, k, v, o, kc, vc, s)
           : launch_f32<64, false>(p, q, k, v, o, kc, vc, s);
    else
      ring ? launch_f32<128, true>(p, q, k, v, o, kc, vc, s)
           : launch_f32<128, false>(p, q, k, v, o, kc, vc, s);
  }
  return hipGetLastError();
}

}  // namespace moa
