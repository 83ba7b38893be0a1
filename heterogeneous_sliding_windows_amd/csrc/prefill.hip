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
// bf16 kernel (4 waves, 32 query rows each; three workgroups a CU):
//  * S^T = K Q^T on 32x32x16 bf16 MFMA, so each lane owns one query row and
//    the row max needs one exchange with the partner lane (l ^ 32);
//  * key rows of a 32-key MFMA tile are permuted (row m = 16a + 8b + 4h + c
//    reads key 16a + 8h + 4b + c), which puts the scores of lane half h on
//    keys 16j + 8h .. +7 of P.V step j: the P^T operand is the lane's own
//    scores, converted to bf16, with no data movement;
//  * each 64-key tile of the unit is streamed as two 32-key sub-tiles, which
//    go from memory straight into LDS (16-byte LDS-direct buffer loads, no
//    staging registers), in a chunk-swizzled layout that both fragment reads
//    meet without bank conflicts; the V^T operand of the P.V product (8
//    consecutive keys of one dimension per lane) comes from two transposed
//    LDS reads (ds_read_b64_tr_b16).  32 KB of LDS and 166 VGPRs a lane let
//    three workgroups share a CU;
//  * LDS sub-tiles are double-buffered: sub-tile t+1's loads are issued
//    before sub-tile t is computed (one wait and one barrier a sub-tile);
//  * O goes through LDS: each wave writes its normalised rows to LDS and
//    stores them as whole 16-byte chunks, four complete rows per store
//    instruction;
//  * masks are evaluated only on sub-tiles a wave's rows do not fully keep,
//    and a wave skips sub-tiles none of its rows keep;
//  * online softmax in fp32 with exp2: the scores leave the matrix cores raw
//    (fp32) and 1/sqrt(D)*log2(e) is applied in fp32 before each
//    exponential; O and the row sum are rescaled only when a row's max grows
//    by more than 8 in the exp2 domain (a factor of 2^8), which most
//    sub-tiles after the first never trigger.
//
// f32 kernel (the float32 dtype): the same units and softmax on fp32 matrix
// cores (v_mfma_f32_16x16x4f32), K/V tiles in LDS, an exact running max (no
// lazy rescale).
//
// Fused handoff (RING = true): besides o, the launch writes positions
// N - S_h .. N - 1 of every (b, h_kv) into the KV rings, as an append of the
// whole prompt would.  The keys of query tile qt's rows (128 qt .. 128 qt +
// 127) are its unit's last four sub-tiles; the workgroup of the first query
// head of each KV group (g = 0) stores the rows of them that the ring keeps,
// after its loop, staging each such sub-tile once more (the loop has just
// read it, so it comes from L2).  Every ring row is therefore written once.
// The loop itself is the plain kernel's, so o is bit-identical to it.  The
// f32 kernel stores the same rows from its tile loop.

#include "moa_device.h"
#include "moa_internal.h"

namespace moa {
namespace {

constexpr int BM = kPrefillBM;
constexpr int BN = kPrefillBN;

// The bf16 kernel streams each 64-key tile of the plan as two 32-key
// sub-tiles, so that a workgroup needs 32 KB of LDS and 166 VGPRs a lane, and
// three workgroups (three waves a SIMD) share a CU.
constexpr int BS = 32;

// LDS layout of a 32-row K or V sub-tile (row = key): 16-byte chunks (8
// dims) in groups of four; group cg holds its 64-byte slice of all 32 rows,
// and the chunk's place inside the slice is XOR-swizzled by row bits 2-3.
// Byte offset of chunk c of row r:
__device__ __forceinline__ constexpr int tile_off(int r, int c) {
  return (c >> 2) * 2048 + r * 64 + (((c & 3) ^ ((r >> 2) & 3)) << 4);
}
// (One wave's 16-byte LDS-direct load fills 1 KB: 16 rows of one group.
// The 16 lanes of an LDS read phase meet 16 different rows of one chunk
// column in different banks, for the K reads and the transposed V reads.)

template <int D, bool RING>
__global__ __launch_bounds__(256, 3) void prefill_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, const int4* __restrict__ items, const int32_t* __restrict__ span,
    const int32_t* __restrict__ seq_len, int seq_grid, int Hq, int Hkv, int G, int Npad,
    float scale_log2, bf16* __restrict__ kc, bf16* __restrict__ vc,
    const int64_t* __restrict__ ring) {
  constexpr int KS = D / 16;       // k-steps of the Q.K product
  constexpr int OT = D / 32;       // 32-dim tiles of the output
  constexpr int ROWB = D * 2;      // bytes of a K/V row
  constexpr int TILEB = BS * ROWB; // bytes of a K or V sub-tile
  constexpr int NDMA = D / 64;     // LDS-direct rounds per sub-tile
  constexpr int TE = BS * D;       // elements of a sub-tile
  // sub-tile buffers: K in 0 and 1, V in 2 and 3 (one array, so that the O
  // epilogue can stage all four waves' rows in it)
  __shared__ __attribute__((aligned(16))) bf16 lds[4 * TE];

  const int tid = threadIdx.x;
  // wave-uniform, so that the LDS addresses of the tile loads are scalar
  // arithmetic (no VALU write of an SGPR ahead of a load)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // LDS-direct staging: round i of wave w fills bytes g*2048 + (w%2)*1024 +
  // 16*lane of a sub-tile, g = 2i + w/2: chunk group g, rows 16(w%2) +
  // lane/4, slice place lane % 4, which holds chunk 4g + ((lane % 4) ^
  // (lane / 16 % 4)) of that row.  Rows at or past N read as zero (buffer
  // bounds).
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(kb, (uint32_t)N * ROWB);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(vb, (uint32_t)N * ROWB);
  const uint32_t dma_off = (uint32_t)(16 * (wave & 1) + (lane >> 2)) * ROWB +
                           (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  // The loads are issued from inline assembly so that the compiler, which
  // cannot tell that they fill the other buffer, does not wait for them
  // before every LDS read of the current one; the explicit vmcnt(0) before
  // each barrier is their only wait.  They write no registers.
  auto dma_tile = [&](int st, int buf) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int grp = 2 * i + (wave >> 1);
      const uint32_t soff = (uint32_t)st * TILEB + grp * 64;
      const int dst = grp * 2048 + (wave & 1) * 1024;
      lds_direct_ld16(krs, dma_off, soff, (char*)&lds[buf * TE] + dst);
      lds_direct_ld16(vrs, dma_off, soff, (char*)&lds[(2 + buf) * TE] + dst);
    }
  };

  // The unit's sub-tiles: those of its 64-key tiles, less a leading one that
  // no row of the unit keeps.
  const int lo_key = qt * BM - S + 1;
  int st_lo = 2 * kt_lo;
  if (lo_key > 0 && lo_key / BS > st_lo) st_lo = lo_key / BS;
  const int st_hi = 2 * kt_hi + 1;
  // the first sub-tile's loads go out before Q's, so their latencies overlap
  dma_tile(st_lo, 0);

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

  // K fragment (Q.K k-step s): row kperm, chunk 2s + half.  With kperm's row
  // bits 2-3 fixed per lane, the byte offset is a per-lane base (one for even
  // s, one for odd s) plus (s / 2) * 2048.
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

  // Double-buffered LDS-direct sub-tiles: sub-tile st+1's loads are issued
  // before sub-tile st is computed; one wait and one barrier a sub-tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  for (int st = st_lo; st <= st_hi; ++st) {
    const int buf = (st - st_lo) & 1;
    if (st < st_hi) dma_tile(st + 1, buf ^ 1);

    const int j0 = st * BS;
    const bool active = iw0 < N && j0 <= iw0 + 31 && j0 + BS - 1 >= iw0 - S + 1;
    if (active) {
      const bool full = j0 + BS - 1 <= iw0 && j0 >= iw0 + 31 - S + 1 && j0 + BS <= N;
      const char* kl = (const char*)&lds[buf * TE];
      const char* vl = (const char*)&lds[(2 + buf) * TE];
      floatx16 sc = minit;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int off = ((s & 1) ? k_odd : k_even) + (s >> 1) * 2048;
        sc = mfma32(*reinterpret_cast<const bf16x8*>(kl + off), qop[s], sc);
      }
      // keep four K-fragment reads in flight ahead of the matrix cores
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < KS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // sc[r] is raw score - m_ref of query my_q and key
      // j0 + 16(r>>3) + 8half + (r&7)
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 16 * (r >> 3) + 8 * half + (r & 7);
          const bool ok = key <= my_q && key >= my_q - S + 1 && key < N;
          sc[r] = ok ? sc[r] : -INFINITY;
        }
      }
      float mx = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = half_swap_max(mx);
      // Lazy rescale: the reference moves (and O, l are rescaled) only when
      // some row's sub-tile max exceeds it by more than 8 in the exp2 domain,
      // or sets it at the row's first kept key; otherwise p <= 256, harmless
      // in fp32 and bf16.  The final O / l is unchanged.
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
        sc -= delta;
#pragma unroll
        for (int r = 0; r < 16; ++r) minit[r] = -m_ref;
      }
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = fast_exp2(sc[r] * scale_log2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 pop = to_bf16x8(&p[8 * j]);
        // the row sum of the bf16 weights the P.V product uses, two per step
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2 pair = {pop[2 * i], pop[2 * i + 1]};
          if (i & 1) l_b = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, l_b, false);
          else       l_a = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, l_a, false);
        }
#pragma unroll
        for (int t = 0; t < OT; ++t) {
          const int base = t * 2048 + 16 * j * 64;
          const bf16x4 a0 = lds_read_tr16(vl + base + v_rd0);
          const bf16x4 a1 = lds_read_tr16(vl + base + 4 * 64 + v_rd1);
          const bf16x8 vop = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[t] = mfma32(vop, pop, acc[t]);
        }
      }
      // same for the V^T fragments of the P.V product
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
      for (int i = 0; i < 2 * OT - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): sub-tile st+1 is in LDS
    __syncthreads();
  }

  if constexpr (RING) {
    // Fused handoff: the ring keeps positions N - S .. N - 1 at slot p mod
    // S.  Each key sub-tile's ring rows are written by the unit of its query
    // tile (the unit's last four sub-tiles, 4 qt .. 4 qt + 3), after the
    // loop: each such sub-tile is staged again (from L2, where the loop just
    // read it) into buffers 0 and 2 and copied out.  K: 16-byte chunks.  V:
    // transposed reads give 4 consecutive keys of one dimension, stored as
    // one 8-byte run when the 4 slots are consecutive (S a multiple of 4, or
    // S = N: slot = p), else element by element.
    if (kring != nullptr) {
      constexpr int CPR = D / 8;
      const char* kl = (const char*)&lds[0];
      const char* vl = (const char*)&lds[2 * TE];
      const int grp = tid >> 4;
      for (int st = 4 * qt; st <= st_hi; ++st) {
        if ((st + 1) * BS <= N - S || st * BS >= N) continue;   // no row of it is kept
        dma_tile(st, 0);
        __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0)
        __syncthreads();
#pragma unroll
        for (int u = 0; u < CPR / 8; ++u) {
          const int id = u * 256 + tid;
          const int r = id / CPR, c = id % CPR;
          const int p = st * BS + r;
          if (p >= N - S && p < N)
            st16(kring + (int64_t)(p % S) * D + 8 * c,
                 *reinterpret_cast<const bf16x8*>(kl + tile_off(r, c)));
        }
        // 8 key groups x D/16 dim blocks, one per 16-lane group and round
#pragma unroll
        for (int u = 0; u < D / 32; ++u) {
          const int unit = u * 16 + grp;
          const int kg = unit & 7, m = unit >> 3;
          const int r = 4 * kg + (vi >> 2);
          const int dim0 = 16 * m + 4 * (vi & 3);
          const int off = tile_off(r, dim0 >> 3) + 2 * (dim0 & 7);
          const bf16x4 x = lds_read_tr16(vl + off);
          const int p0 = st * BS + 4 * kg;
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
        __syncthreads();   // before the buffers are filled again
      }
    }
  }

  // O through LDS: each wave writes its 32 normalised rows into its own
  // quarter of the (now idle) sub-tile buffers, chunk c of row r at byte
  // 16 * (c ^ (r mod chunks per row)), and reads them back as whole 16-byte
  // chunks, so that each store instruction writes four complete output rows.
  // Rows at or past N are not stored.
  const float l_run = half_swap_sum(l_a + l_b);
  const float inv = 1.f / l_run;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  char* ow = (char*)&lds[0] + wave * (32 * D * 2);
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

// f32 kernel: 4 waves of 32 query rows (two 16-row blocks qb), both products
// on v_mfma_f32_16x16x4f32 (A 16x4: lane l gives row l%16, k l/16; B 4x16:
// lane l gives k l/16, column l%16; C 16x16: lane l holds rows 4*(l/16)+r,
// column l%16).  S^T = K Q^T puts the query on the column, so lane l owns
// query 16qb + l%16 and holds keys 16kb + 4*(l/16) + r of key block kb: the
// row max and row sum are in-lane plus two exchanges across the lane groups,
// and the P^T operand of O^T = V^T P^T is the lane's own weight (step (kb,
// r) contracts keys 16kb + 4g + r, g = 0..3).  Each contraction may take its
// index in any order, so the dimensions are permuted to make every operand
// read a 16-byte one: Q.K step s pairs lane group g with dimension g*(D/4) +
// s, and output block db holds dimensions i*(D/16) + db in row i.  K and V
// tiles sit in LDS with each row's 16-byte chunks rotated by the key (chunk c
// of key r at (c + r) mod (D/4)), so the 16 rows (or 16 chunks) a read phase
// meets fall in different banks.
template <int D, bool RING>
__global__ __launch_bounds__(256) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, const int4* __restrict__ items, const int32_t* __restrict__ span,
    const int32_t* __restrict__ seq_len, int seq_grid, int Hq, int Hkv, int G, int Npad,
    float scale_log2, float* __restrict__ kc, float* __restrict__ vc,
    const int64_t* __restrict__ ring) {
  constexpr int C4 = D / 4;    // 16-byte chunks per K/V row; also the Q.K k-steps
  constexpr int DB = D / 16;   // 16-dim output blocks
  __shared__ float4 Ks[BN * C4];
  __shared__ float4 Vs[BN * C4];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 15;     // query column (S^T, O^T) / key or dim row (operands)
  const int g = lane >> 4;     // lane group
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
  const int iw0 = qt * BM + wave * 32;   // first query row of this wave
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

  // B operand of Q.K step s: Q[query 16qb + j][dim g*C4 + s], loaded once
  float qv[2][C4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = iw0 + 16 * qb + j;
    const float* qrow = q + ((int64_t)bh * Npad + pad + (row < N ? row : 0)) * D + g * C4;
#pragma unroll
    for (int c = 0; c < C4; c += 4) {
      const float4 x = row < N ? *reinterpret_cast<const float4*>(qrow + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      qv[qb][c] = x.x; qv[qb][c + 1] = x.y; qv[qb][c + 2] = x.z; qv[qb][c + 3] = x.w;
    }
  }
  floatx4 acc[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int d = 0; d < DB; ++d) acc[qb][d] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.f, 0.f};   // this lane's keys; the row sum adds the 4 lane groups

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int j0 = kt * BN;
    __syncthreads();
    for (int i = tid; i < BN * C4; i += 256) {
      const int r = i / C4, c = i % C4;
      const int key = j0 + r;
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (key < N) {
        kx = *reinterpret_cast<const float4*>(kb + (int64_t)key * D + 4 * c);
        vx = *reinterpret_cast<const float4*>(vb + (int64_t)key * D + 4 * c);
      }
      Ks[r * C4 + (c + r) % C4] = kx;
      Vs[r * C4 + (c + r) % C4] = vx;
      if constexpr (RING) {
        if (kring != nullptr && kt * BN / BM == qt && key >= N - S && key < N) {
          const int slot = key % S;
          *reinterpret_cast<float4*>(kring + (int64_t)slot * D + 4 * c) = kx;
          float* dst = vring + (int64_t)(slot >> 5) * (32 * D) + 4 * c * 32 + (slot & 31);
          dst[0] = vx.x;
          dst[32] = vx.y;
          dst[64] = vx.z;
          dst[96] = vx.w;
        }
      }
    }
    __syncthreads();

    // S^T blocks: st[qb][kb][r] = score of query iw0 + 16qb + j, key j0 + 16kb + 4g + r
    floatx4 st[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) st[qb][kb2] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) {
      const int r = 16 * kb2 + j;   // A row: key r of the tile
#pragma unroll
      for (int c = 0; c < C4 / 4; ++c) {
        const float4 kf = Ks[r * C4 + (g * (C4 / 4) + c + r) % C4];   // dims g*C4 + 4c .. +3
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          st[qb][kb2] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.x, qv[qb][4 * c + 0], st[qb][kb2], 0, 0, 0);
          st[qb][kb2] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.y, qv[qb][4 * c + 1], st[qb][kb2], 0, 0, 0);
          st[qb][kb2] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.z, qv[qb][4 * c + 2], st[qb][kb2], 0, 0, 0);
          st[qb][kb2] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.w, qv[qb][4 * c + 3], st[qb][kb2], 0, 0, 0);
        }
      }
    }
    // online softmax per row (fp32, exact running max; masked scores -> weight 0)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int my_q = iw0 + 16 * qb + j;
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = j0 + 16 * kb2 + 4 * g + r;
          const bool ok = key <= my_q && key >= my_q - S + 1 && key < N;
          st[qb][kb2][r] = ok ? st[qb][kb2][r] : -INFINITY;
          mx = fmaxf(mx, st[qb][kb2][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[qb], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2((m_run[qb] - m_use) * scale_log2);
      m_run[qb] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // (s - m) first: a score equal to the running max gives exactly 1
          const float pw = exp2f((st[qb][kb2][r] - m_use) * scale_log2);
          st[qb][kb2][r] = pw;
          ls += pw;
        }
      l_part[qb] = l_part[qb] * alpha + ls;
#pragma unroll
      for (int d = 0; d < DB; ++d) acc[qb][d] *= alpha;
    }
    // O^T += V^T P^T, step (kb, r): keys 16kb + 4g + r; A = V[key][dim j*DB + db]
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * kb2 + 4 * g + r;
        float va[DB];
#pragma unroll
        for (int u = 0; u < DB / 4; ++u) {
          const float4 x = Vs[key * C4 + (j * (DB / 4) + u + key) % C4];   // dims j*DB + 4u .. +3
          va[4 * u] = x.x; va[4 * u + 1] = x.y; va[4 * u + 2] = x.z; va[4 * u + 3] = x.w;
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int d = 0; d < DB; ++d)
            acc[qb][d] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[d], st[qb][kb2][r], acc[qb][d], 0, 0, 0);
      }
  }
  // acc[qb][db][r'] = O[query iw0 + 16qb + j][dim (4g + r')*DB + db]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = l_part[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int my_q = iw0 + 16 * qb + j;
    if (my_q >= N) continue;
    const float inv = 1.f / l;
    float* orow = o + ((int64_t)bh * Npad + pad + my_q) * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int u = 0; u < DB / 4; ++u)
        *reinterpret_cast<float4*>(orow + (4 * g + r) * DB + 4 * u) =
            make_float4(acc[qb][4 * u][r] * inv, acc[qb][4 * u + 1][r] * inv,
                        acc[qb][4 * u + 2][r] * inv, acc[qb][4 * u + 3][r] * inv);
  }
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
