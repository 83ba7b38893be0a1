// C ABI of libmoa: argument checks, the host planner (span table, ring
// offsets, prefill tile list, decode chunk list) and kernel dispatch.
//
// Built with -ffp-contract=off so that alpha + beta * N is evaluated with one
// rounding per operation, as the span table's definition requires.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <new>
#include <queue>
#include <string>
#include <vector>

#include "moa_internal.h"

namespace moa {

namespace {

// Chunks of `copies` sequences with rings `span` under cut c; INT64_MAX on overflow.
int64_t count_chunks(const std::vector<int32_t>& span, int64_t copies, const DecodeCut& c) {
  uint64_t one = 0;
  for (const int32_t s : span) one += (uint64_t)cut_count(s, c);
  uint64_t n;
  if (__builtin_mul_overflow((uint64_t)copies, one, &n) || n > (uint64_t)INT64_MAX)
    return INT64_MAX;
  return (int64_t)n;
}

// The modeled end of a decode launch under cut c (the model DecodeCut states):
// chunks in launch order, each on the resident slot that frees first.
int64_t decode_makespan(const std::vector<int32_t>& span, int64_t copies, const DecodeCut& c,
                        int slots) {
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
  for (int i = 0; i < slots; ++i) free_at.push(0);
  int64_t end = 0;
  for (int64_t r = 0; r < copies; ++r)
    for (const int32_t s : span) {
      const int32_t step = cut_step(s, c);
      for (int32_t first = 0; first < s; first += step) {
        const int64_t t = free_at.top() + std::min(step, s - first) + kDecodeModelOverhead;
        free_at.pop();
        free_at.push(t);
        end = std::max(end, t);
      }
    }
  return end;
}

}  // namespace

DecodeCut decode_cut(const std::vector<int32_t>& span, int64_t copies, int G, int D,
                     int64_t* n_chunks) {
  const int c = decode_chunk_for(G, [&](int cc) {
    return count_chunks(span, copies, {CutKind::kFixed, cc});
  });
  const DecodeCut fixed{CutKind::kFixed, c};
  DecodeCut cut = fixed;
  *n_chunks = count_chunks(span, copies, fixed);
  const int slots = decode_resident(D);
  if (*n_chunks < kDecodeModelRounds * slots) {
    const int64_t t_fixed = decode_makespan(span, copies, fixed, slots);
    DecodeCut best = fixed;
    int64_t t_best = INT64_MAX;
    for (const int target : kDecodeEvenTargets) {
      if (target < c) continue;
      const DecodeCut even{CutKind::kEven, target};
      const int64_t t = decode_makespan(span, copies, even, slots);
      if (t < t_best) {
        t_best = t;
        best = even;
      }
    }
    if (best.kind == CutKind::kEven && t_best * 100 <= t_fixed * kDecodeModelGainPct) {
      cut = best;
      *n_chunks = count_chunks(span, copies, best);
    }
  }
  uint64_t rings;
  if (G >= kDecodeBalancedMinG && *n_chunks > slots && !__builtin_mul_overflow((uint64_t)copies, (uint64_t)span.size(), &rings) &&
      rings <= (uint64_t)slots) {
    int64_t total = 0;
    for (const int32_t s : span) total += s;
    total *= copies;   // rings <= slots, so at most 2^31 * 2^11
    const int64_t cap = kDecodeBalancedRounds * slots;
    for (int64_t k = cap; k >= (int64_t)rings; --k) {
      const DecodeCut bal{CutKind::kBalanced, 0, k, total};
      const int64_t n = count_chunks(span, copies, bal);
      if (n <= cap) {
        *n_chunks = n;
        return bal;
      }
    }
  }
  return cut;
}

}  // namespace moa

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOA_EHIP, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

constexpr int64_t kMaxN = (int64_t)1 << 31;

// Span of one head (project page, "Finding 2" and "Elastic search space"):
// clamp(64 * ceil(x / 64), 1, N) with x = alpha + beta * N in IEEE double.
#pragma clang fp contract(off)
int32_t span_of(int64_t alpha, double beta, int64_t n) {
  const double x = (double)alpha + beta * (double)n;
  if (!(x > 0.0)) return 1;                    // x <= 0: the query alone
  if (x >= (double)n) return (int32_t)n;       // saturated
  const double r = 64.0 * std::ceil(x / 64.0);  // exact: x < 2^31
  int64_t s = (int64_t)r;
  if (s < 1) s = 1;
  if (s > n) s = n;
  return (int32_t)s;
}

int check_rules(const int64_t* alpha, const double* beta, int32_t hkv, int64_t n) {
  if (!alpha || !beta) return fail(MOA_EINVAL, "alpha and beta must not be NULL");
  if (hkv < 1) return fail(MOA_EINVAL, "n_kv_heads must be >= 1 (got %d)", hkv);
  if (n < 1 || n >= kMaxN) return fail(MOA_EINVAL, "n_prompt must be in [1, 2^31) (got %lld)", (long long)n);
  for (int32_t h = 0; h < hkv; ++h) {
    if (alpha[h] < 0) return fail(MOA_EINVAL, "alpha[%d] = %lld is negative", h, (long long)alpha[h]);
    if (!std::isfinite(beta[h]) || beta[h] < 0.0)
      return fail(MOA_EINVAL, "beta[%d] = %g must be finite and >= 0", h, beta[h]);
  }
  return MOA_OK;
}

template <class T>
int dev_upload(T** dst, const std::vector<T>& src) {
  *dst = nullptr;
  if (src.empty()) return MOA_OK;
  hipError_t e = hipMalloc((void**)dst, src.size() * sizeof(T));
  if (e != hipSuccess) {
    *dst = nullptr;
    return e == hipErrorOutOfMemory ? fail(MOA_ENOMEM, "hipMalloc of plan tables: out of memory")
                                    : hip_fail(e, "hipMalloc (plan tables)");
  }
  e = hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (plan tables)");
  return MOA_OK;
}

void free_device(moa_plan* p) {
  hipFree(p->dev.span);
  hipFree(p->dev.ring);
  hipFree(p->dev.seq_len);
  hipFree(p->dev.prefill_items);
  hipFree(p->dev.decode_chunks);
  hipFree(p->dev.head_chunks);
  hipFree(p->dev.decode_order);
  p->dev = moa::PlanDevice{};
}

// Span and ring tables of every (sequence, KV head): S = span_of(alpha_h,
// beta_h, N_b); sequence b's rings follow each other (pitch: span rounded up
// to 32 slots), and the sequences' blocks follow each other.
void build_ring_tables(moa_plan* p, const int64_t* alpha, const double* beta) {
  p->span.resize((size_t)p->B * p->Hkv);
  p->ring.resize((size_t)p->B * p->Hkv);
  int64_t total = 0;
  for (int32_t b = 0; b < p->B; ++b)
    for (int32_t h = 0; h < p->Hkv; ++h) {
      const size_t i = (size_t)b * p->Hkv + h;
      p->span[i] = (b > 0 && !p->ragged) ? p->span[h] : span_of(alpha[h], beta[h], p->seq_len[b]);
      p->ring[i] = total;
      total += ((int64_t)p->span[i] + 31) / 32 * 32;
    }
  p->total_slots = total;
}

// Prefill schedule.  A work unit is 128 query rows of one (b, h_q) with the
// range of 64-key tiles that hold a kept pair: the windows of rows i0..i1
// together cover the contiguous keys [max(0, i0 - S + 1), i1], so the live
// tiles form one range.  Each (b, h_q)'s units form runs of up to
// kPrefillRun consecutive query tiles, from the last tile down (neighbouring
// tiles read overlapping key windows, so a run's units share one XCD's L2).
// Runs are sorted by cost (tiles plus a per-unit overhead), longest first,
// and dealt to the 8 XCDs in groups of 8, one run per XCD, in snake order
// (XCD 0..7 for even groups, 7..0 for odd ones) so that the XCDs' totals
// even out.  Workgroups are dealt to the XCDs round-robin, so XCD x's k-th
// unit sits at 8k + x; a group takes as many rounds of 8 as its longest run
// and shorter runs are padded (bq = -1).  With one prompt length every
// sequence has the same units, so the table is built for sequence 0 and the
// launch runs it once per sequence (its length is a multiple of 8, so each
// copy keeps the XCD assignment); with per-sequence lengths the table holds
// every sequence's units.
void build_prefill_items(moa_plan* p) {
  struct Unit { int32_t bq, qt, lo, hi; };
  struct Run { int64_t cost; size_t first; int32_t n; };
  std::vector<Unit> units;
  std::vector<Run> runs;
  const int32_t nb = p->ragged ? p->B : 1;
  for (int32_t b = 0; b < nb; ++b) {
    const int64_t n = p->seq_len[b];
    const int64_t n_qt = (n + moa::kPrefillBM - 1) / moa::kPrefillBM;
    for (int32_t h = 0; h < p->Hq; ++h) {
      const int64_t s = p->span[(size_t)b * p->Hkv + h / p->G];
      for (int64_t top = n_qt - 1; top >= 0; top -= moa::kPrefillRun) {
        Run r{0, units.size(), 0};
        for (int64_t qt = top; qt >= 0 && qt > top - moa::kPrefillRun; --qt) {
          const int64_t i0 = qt * moa::kPrefillBM;
          const int64_t i1 = std::min<int64_t>(i0 + moa::kPrefillBM, n) - 1;
          const int64_t j0 = std::max<int64_t>(0, i0 - s + 1);
          const Unit u{b * p->Hq + h, (int32_t)qt, (int32_t)(j0 / moa::kPrefillBN),
                       (int32_t)(i1 / moa::kPrefillBN)};
          units.push_back(u);
          r.cost += u.hi - u.lo + 1 + moa::kPrefillUnitOverhead;
          ++r.n;
        }
        runs.push_back(r);
      }
    }
  }
  std::stable_sort(runs.begin(), runs.end(),
                   [](const Run& a, const Run& b) { return a.cost > b.cost; });
  size_t rounds = 0;
  for (size_t g = 0; g < runs.size(); g += 8) {
    int32_t depth = 0;
    for (size_t r = g; r < std::min(g + 8, runs.size()); ++r) depth = std::max(depth, runs[r].n);
    rounds += (size_t)depth;
  }
  p->prefill_items.assign(rounds * 8 * 4, 0);
  for (size_t i = 0; i < rounds * 8; ++i) {
    p->prefill_items[4 * i + 0] = -1;   // padding: the workgroup exits at once
    p->prefill_items[4 * i + 3] = -1;
  }
  size_t k0 = 0;   // first round of the current group
  for (size_t g = 0; g < runs.size(); g += 8) {
    int32_t depth = 0;
    for (size_t j = 0; j < 8 && g + j < runs.size(); ++j) {
      const Run& r = runs[g + j];
      const size_t x = (g / 8) % 2 == 0 ? j : 7 - j;
      for (int32_t i = 0; i < r.n; ++i) {
        const Unit& u = units[r.first + i];
        int32_t* e = &p->prefill_items[(8 * (k0 + i) + x) * 4];
        e[0] = u.bq;
        e[1] = u.qt;
        e[2] = u.lo;
        e[3] = u.hi;
      }
      depth = std::max(depth, r.n);
    }
    k0 += (size_t)depth;
  }
  // The tail of each XCD's queue, longest units first (stable: equal tile
  // counts keep their queue order).
  for (int x = 0; x < 8; ++x) {
    std::vector<size_t> pos;   // XCD x's entries that hold a unit, in queue order
    for (size_t k = 0; k < rounds; ++k)
      if (p->prefill_items[(8 * k + x) * 4] >= 0) pos.push_back(8 * k + x);
    const size_t t0 = pos.size() > moa::kPrefillTailUnits ? pos.size() - moa::kPrefillTailUnits : 0;
    std::vector<std::array<int32_t, 4>> tail;
    for (size_t i = t0; i < pos.size(); ++i) {
      const int32_t* e = &p->prefill_items[pos[i] * 4];
      tail.push_back({e[0], e[1], e[2], e[3]});
    }
    std::stable_sort(tail.begin(), tail.end(),
                     [](const std::array<int32_t, 4>& a, const std::array<int32_t, 4>& b) {
                       return a[3] - a[2] > b[3] - b[2];
                     });
    for (size_t i = t0; i < pos.size(); ++i)
      std::copy(tail[i - t0].begin(), tail[i - t0].end(), &p->prefill_items[pos[i] * 4]);
  }
  p->prefill_seq_grid = p->ragged ? 0 : (int64_t)rounds * 8;
  p->n_prefill_units = (int64_t)units.size() * (p->ragged ? 1 : p->B);
}

// Decode chunk list of all sequences: each ring's S slots cut into chunks of
// at most decode_chunk slots, in (b, h) order.
void build_decode_chunks(moa_plan* p) {
  const moa::DecodeCut& cut = p->decode_cut;
  p->decode_chunks.clear();
  p->head_chunks.assign((size_t)p->B * p->Hkv * 2, 0);
  p->any_split = false;
  int32_t longest = 0;
  int64_t idx = 0;
  for (int32_t bh = 0; bh < p->B * p->Hkv; ++bh) {
    const int32_t s = p->span[bh];
    const int32_t step = moa::cut_step(s, cut);
    const int32_t cnt = moa::cut_count(s, cut);
    longest = std::max(longest, std::min(step, s));
    p->any_split |= cnt > 1;
    p->head_chunks[2 * (size_t)bh + 0] = (int32_t)idx;
    p->head_chunks[2 * (size_t)bh + 1] = cnt;
    for (int32_t k = 0; k < cnt; ++k) {
      p->decode_chunks.push_back(bh);
      p->decode_chunks.push_back(k * step);
      p->decode_chunks.push_back(std::min(step, s - k * step));
      p->decode_chunks.push_back(cnt);
      ++idx;
    }
  }
  p->n_chunks = idx;
  // the size bound of the cut: fixed size or even target, else the longest chunk
  p->decode_chunk = cut.kind == moa::CutKind::kBalanced ? longest : cut.size;
  // the balanced cut launches its chunks longest first (stable: equal lengths
  // keep the (b, h) order); the chunk table itself stays ring-contiguous
  p->decode_order.clear();
  if (cut.kind == moa::CutKind::kBalanced) {
    p->decode_order.resize((size_t)idx);
    for (int64_t i = 0; i < idx; ++i) p->decode_order[(size_t)i] = (int32_t)i;
    std::stable_sort(p->decode_order.begin(), p->decode_order.end(), [&](int32_t a, int32_t b) {
      return p->decode_chunks[4 * (size_t)a + 2] > p->decode_chunks[4 * (size_t)b + 2];
    });
  }
}

// Device pointers must be 16-byte aligned (include/moa.h): the kernels move
// 16-byte vectors through them.  Null entries are skipped (checked elsewhere).
int check_aligned(const char* who, std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if (x != nullptr && (reinterpret_cast<uintptr_t>(x) & 15u) != 0)
      return fail(MOA_EINVAL, "%s: device pointer %p is not 16-byte aligned", who, x);
  return MOA_OK;
}

int check_plan(moa_plan_t p, bool need_device) {
  if (!p) return fail(MOA_EINVAL, "plan is NULL");
  if (need_device && p->host_only)
    return fail(MOA_EINVAL, "plan was created with MOA_PLAN_HOST_ONLY; no device tables");
  return MOA_OK;
}

int set_device(const moa_plan* p) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != p->device)
    return fail(MOA_EINVAL, "plan was created on device %d but device %d is current", p->device, cur);
  return MOA_OK;
}

// Checks shared by moa_prefill and moa_prefill_handoff (the plan's device
// must be current).
int check_prefill(moa_plan_t p, const void* q, const void* k, const void* v, const void* o,
                  const char* who) {
  int st = check_plan(p, false);
  if (st != MOA_OK) return st;
  if (!q || !k || !v || !o) return fail(MOA_EINVAL, "%s: q, k, v and o must not be NULL", who);
  if ((st = check_aligned(who, {q, k, v, o})) != MOA_OK) return st;
  if ((st = check_plan(p, true)) != MOA_OK) return st;
  if (p->N * p->D * (p->dtype == MOA_BF16 ? 2 : 4) >= ((int64_t)1 << 31))
    return fail(MOA_EUNSUPPORTED, "%s: one head's K/V (N x head_dim) must stay below 2 GiB", who);
  const uint64_t table = p->prefill_items.size() / 4;
  if ((p->prefill_seq_grid > 0 ? table * (uint64_t)p->B : table) > 0xFFFFFFFFull)
    return fail(MOA_EUNSUPPORTED, "%s: the prefill launch needs more than 2^32 - 1 workgroups", who);
  return set_device(p);
}

// Checks shared by moa_decode, moa_append_decode and moa_append_decode_static
// (a null ws with ws_bytes = 0 skips the workspace checks: the static variant
// brings its own).
int check_decode(moa_plan_t p, const void* q, const void* kc, const void* vc, int64_t pos,
                 const void* o, const void* ws, size_t ws_bytes, bool need_ws, const char* who) {
  int st = check_plan(p, false);
  if (st != MOA_OK) return st;
  if (!q || !kc || !vc || !o) return fail(MOA_EINVAL, "%s: q, caches and o must not be NULL", who);
  if (need_ws && !ws) return fail(MOA_EINVAL, "%s: workspace must not be NULL", who);
  if ((st = check_aligned(who, {q, kc, vc, o, need_ws ? ws : nullptr})) != MOA_OK) return st;
  if ((st = check_plan(p, true)) != MOA_OK) return st;
  if (pos < p->N)
    return fail(MOA_EINVAL, "%s: pos (%lld) must be >= the prompt length %lld", who,
                (long long)pos, (long long)p->N);
  if (p->dtype != MOA_BF16) return fail(MOA_EUNSUPPORTED, "%s supports bfloat16 plans only", who);
  {
    // the decode kernel addresses one head's ring with 32-bit byte offsets
    int32_t smax = 0;
    for (int32_t x : p->span) smax = x > smax ? x : smax;
    const int64_t pitch = ((int64_t)smax + 31) / 32 * 32;
    if (pitch * p->D * 2 >= ((int64_t)1 << 31))
      return fail(MOA_EUNSUPPORTED, "%s: span %d x head_dim %d exceeds 2 GiB per ring", who, smax,
                  p->D);
  }
  const size_t need = moa::decode_ws_bytes(*p);
  if (need_ws && ws_bytes < need)
    return fail(MOA_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, ws_bytes, need);
  return set_device(p);
}

int create_plan(const moa_problem* pr, const int64_t* seq_len, uint32_t flags, moa_plan_t* out) {
  if (!out) return fail(MOA_EINVAL, "out must not be NULL");
  *out = nullptr;
  if (!pr) return fail(MOA_EINVAL, "problem must not be NULL");
  if (flags & ~MOA_PLAN_HOST_ONLY) return fail(MOA_EINVAL, "unknown flags 0x%x", flags);
  if (pr->batch < 1) return fail(MOA_EINVAL, "batch must be >= 1 (got %d)", pr->batch);
  if (pr->n_q_heads < 1) return fail(MOA_EINVAL, "n_q_heads must be >= 1 (got %d)", pr->n_q_heads);
  int st = check_rules(pr->alpha, pr->beta, pr->n_kv_heads, pr->n_prompt);
  if (st != MOA_OK) return st;
  if (pr->n_q_heads % pr->n_kv_heads)
    return fail(MOA_EINVAL, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", pr->n_q_heads,
                pr->n_kv_heads);
  if (pr->n_q_heads / pr->n_kv_heads > 16)
    return fail(MOA_EUNSUPPORTED, "query heads per KV head must be <= 16 (got %d)",
                pr->n_q_heads / pr->n_kv_heads);
  if (pr->head_dim != 64 && pr->head_dim != 128)
    return fail(MOA_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", pr->head_dim);
  if (pr->dtype != MOA_F32 && pr->dtype != MOA_BF16)
    return fail(MOA_EUNSUPPORTED, "unknown dtype %d", pr->dtype);
  if (seq_len) {
    int64_t mx = 0;
    for (int32_t b = 0; b < pr->batch; ++b) {
      if (seq_len[b] < 1 || seq_len[b] > pr->n_prompt)
        return fail(MOA_EINVAL, "seq_len[%d] = %lld must be in [1, n_prompt = %lld]", b,
                    (long long)seq_len[b], (long long)pr->n_prompt);
      mx = std::max(mx, seq_len[b]);
    }
    if (mx != pr->n_prompt)
      return fail(MOA_EINVAL, "n_prompt (%lld) must equal the longest seq_len (%lld)",
                  (long long)pr->n_prompt, (long long)mx);
  }
  // Every element index of the largest tensor must fit int64 comfortably and
  // the per-launch item counts must fit int32 grids.
  const double elems = (double)pr->batch * pr->n_q_heads * (double)pr->n_prompt * pr->head_dim;
  if (elems > 9.0e15) return fail(MOA_EINVAL, "problem too large");
  const double items = (double)pr->batch * pr->n_q_heads *
                       ((pr->n_prompt + moa::kPrefillBM - 1) / moa::kPrefillBM);
  if (items > 2.0e9) return fail(MOA_EINVAL, "too many prefill tiles for one launch");
  if ((double)pr->batch * pr->n_kv_heads * (double)pr->n_prompt / 32.0 > 2.0e9)
    return fail(MOA_EINVAL, "too many decode chunks for one launch");

  moa_plan* p = new (std::nothrow) moa_plan;
  if (!p) return fail(MOA_ENOMEM, "host allocation of the plan failed");
  try {
    p->B = pr->batch;
    p->Hq = pr->n_q_heads;
    p->Hkv = pr->n_kv_heads;
    p->G = pr->n_q_heads / pr->n_kv_heads;
    p->D = pr->head_dim;
    p->N = pr->n_prompt;
    p->dtype = pr->dtype;
    p->ragged = seq_len != nullptr;
    p->host_only = (flags & MOA_PLAN_HOST_ONLY) != 0;
    p->seq_len.assign(p->B, p->N);
    if (seq_len) std::copy(seq_len, seq_len + p->B, p->seq_len.begin());
    build_ring_tables(p, pr->alpha, pr->beta);
    build_prefill_items(p);
    int64_t n_chunks = 0;
    p->decode_cut = moa::decode_cut(p->span, 1, p->G, p->D, &n_chunks);
    build_decode_chunks(p);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(MOA_ENOMEM, "host allocation of plan tables failed");
  }

  if (!p->host_only) {
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "hipGetDevice");
    }
    std::vector<int4> items(p->prefill_items.size() / 4), chunks(p->decode_chunks.size() / 4);
    std::vector<int2> hc(p->head_chunks.size() / 2);
    std::vector<int32_t> lens(p->seq_len.begin(), p->seq_len.end());
    std::memcpy(items.data(), p->prefill_items.data(), p->prefill_items.size() * 4);
    std::memcpy(chunks.data(), p->decode_chunks.data(), p->decode_chunks.size() * 4);
    std::memcpy(hc.data(), p->head_chunks.data(), p->head_chunks.size() * 4);
    if ((st = dev_upload(&p->dev.span, p->span)) != MOA_OK ||
        (st = dev_upload(&p->dev.ring, p->ring)) != MOA_OK ||
        (st = dev_upload(&p->dev.seq_len, lens)) != MOA_OK ||
        (st = dev_upload(&p->dev.prefill_items, items)) != MOA_OK ||
        (st = dev_upload(&p->dev.decode_chunks, chunks)) != MOA_OK ||
        (st = dev_upload(&p->dev.head_chunks, hc)) != MOA_OK ||
        (st = dev_upload(&p->dev.decode_order, p->decode_order)) != MOA_OK) {
      free_device(p);
      delete p;
      return st;
    }
  }
  *out = p;
  return MOA_OK;
}

}  // namespace

extern "C" {

int moa_spans(const int64_t* alpha, const double* beta, int32_t n_kv_heads, int64_t n_prompt,
              int32_t* span) {
  int st = check_rules(alpha, beta, n_kv_heads, n_prompt);
  if (st != MOA_OK) return st;
  if (!span) return fail(MOA_EINVAL, "span output must not be NULL");
  for (int32_t h = 0; h < n_kv_heads; ++h) span[h] = span_of(alpha[h], beta[h], n_prompt);
  return MOA_OK;
}

int moa_ring_offsets(const int32_t* span, int32_t n_kv_heads, int64_t* offset,
                     int64_t* slots_per_seq) {
  if (!span || !offset || !slots_per_seq) return fail(MOA_EINVAL, "NULL argument to moa_ring_offsets");
  if (n_kv_heads < 1) return fail(MOA_EINVAL, "n_kv_heads must be >= 1 (got %d)", n_kv_heads);
  int64_t total = 0;
  for (int32_t h = 0; h < n_kv_heads; ++h) {
    if (span[h] < 1) return fail(MOA_EINVAL, "span[%d] = %d must be >= 1", h, span[h]);
    offset[h] = total;
    total += ((int64_t)span[h] + 31) / 32 * 32;   // ring pitch: span rounded up to 32 slots
  }
  *slots_per_seq = total;
  return MOA_OK;
}

int moa_plan_create(const moa_problem* pr, uint32_t flags, moa_plan_t* out) {
  return create_plan(pr, nullptr, flags, out);
}

int moa_plan_create_ragged(const moa_problem* pr, const int64_t* seq_len, uint32_t flags,
                           moa_plan_t* out) {
  if (out) *out = nullptr;
  if (!seq_len) return fail(MOA_EINVAL, "seq_len must not be NULL");
  return create_plan(pr, seq_len, flags, out);
}

int moa_plan_destroy(moa_plan_t p) {
  if (!p) return MOA_OK;
  if (!p->host_only) free_device(p);
  delete p;
  return MOA_OK;
}

int moa_plan_tables(moa_plan_t p, int32_t* span, int64_t* offset, int64_t* slots_per_seq) {
  int st = check_plan(p, false);
  if (st != MOA_OK) return st;
  if (p->ragged)
    return fail(MOA_EUNSUPPORTED, "plan has per-sequence lengths; use moa_plan_seq_tables");
  // sequence 0's tables serve every sequence
  if (span) std::copy(p->span.begin(), p->span.begin() + p->Hkv, span);
  if (offset) std::copy(p->ring.begin(), p->ring.begin() + p->Hkv, offset);
  if (slots_per_seq) *slots_per_seq = p->total_slots / p->B;
  return MOA_OK;
}

int moa_plan_seq_tables(moa_plan_t p, int32_t* span, int64_t* ring_offset, int64_t* seq_len) {
  int st = check_plan(p, false);
  if (st != MOA_OK) return st;
  if (span) std::copy(p->span.begin(), p->span.end(), span);
  if (ring_offset) std::copy(p->ring.begin(), p->ring.end(), ring_offset);
  if (seq_len) std::copy(p->seq_len.begin(), p->seq_len.end(), seq_len);
  return MOA_OK;
}

int64_t moa_cache_elems(moa_plan_t p) {
  if (check_plan(p, false) != MOA_OK) return 0;
  return p->total_slots * p->D;
}

size_t moa_decode_workspace_bytes(moa_plan_t p) {
  if (check_plan(p, false) != MOA_OK) return 0;
  return moa::decode_ws_bytes(*p);
}

int64_t moa_max_batch(const moa_problem* pr, uint64_t budget_bytes) {
  if (!pr) return fail(MOA_EINVAL, "problem must not be NULL");
  moa_problem one = *pr;
  one.batch = 1;
  moa_plan_t p = nullptr;
  int st = moa_plan_create(&one, MOA_PLAN_HOST_ONLY, &p);
  if (st != MOA_OK) return st;
  // bytes(B) = both pools + the decode workspace moa_decode_workspace_bytes
  // reports for batch B; the largest B with bytes(B) <= budget
  const uint64_t elem = p->dtype == MOA_BF16 ? 2 : 4;
  const uint64_t cache = 2ull * (uint64_t)p->total_slots * (uint64_t)p->D * elem;
  const int G = p->G, D = p->D;
  const uint64_t row = (uint64_t)G * ((uint64_t)p->D + 2) * 4ull;   // partial bytes per chunk
  const std::vector<int32_t> span = p->span;
  moa_plan_destroy(p);
  // chunks of one sequence's rings at chunk size c
  auto per_seq = [&](int c) {
    uint64_t n = 0;
    for (const int32_t sp : span) n += (uint64_t)((sp + c - 1) / c);
    return n;
  };
  // bytes(b): both pools of b sequences plus the workspace a plan of batch b
  // would take; UINT64_MAX when that overflows (it cannot fit any budget)
  auto bytes = [&](uint64_t b) -> uint64_t {
    int64_t n_chunks = 0;
    moa::decode_cut(span, (int64_t)b, G, D, &n_chunks);
    if (n_chunks == INT64_MAX) return UINT64_MAX;
    const uint64_t chunks = (uint64_t)n_chunks;
    uint64_t pools, ws;
    if (__builtin_mul_overflow(b, cache, &pools) ||
        __builtin_mul_overflow(chunks, row, &ws) || ws > UINT64_MAX - 511)
      return UINT64_MAX;
    ws = (ws + 255) & ~(uint64_t)255;
    if (ws < 256) ws = 256;
    uint64_t total;
    if (__builtin_add_overflow(pools, ws, &total)) return UINT64_MAX;
    return total;
  };
  // a plan's batch is int32, so the answer is capped there
  const uint64_t kMaxB = (uint64_t)INT32_MAX;
  uint64_t b = budget_bytes / (cache + per_seq(moa::kDecodeChunk) * row);
  if (b > kMaxB) b = kMaxB;
  while (b > 0 && bytes(b) > budget_bytes) --b;
  while (b < kMaxB && bytes(b + 1) <= budget_bytes) ++b;
  return (int64_t)b;
}

int64_t moa_plan_prefill_items(moa_plan_t p, int32_t* out) {
  int st = check_plan(p, false);
  if (st != MOA_OK) return st;
  if (out) {
    const int64_t T = (int64_t)p->prefill_items.size() / 4;
    const int32_t copies = p->prefill_seq_grid > 0 ? p->B : 1;
    int64_t j = 0;
    for (int32_t c = 0; c < copies; ++c)
      for (int64_t i = 0; i < T; ++i) {
        const int32_t* e = &p->prefill_items[4 * i];
        if (e[0] < 0) continue;
        int32_t* r = out + 6 * j++;
        r[0] = e[0] / p->Hq + c;
        r[1] = e[0] % p->Hq;
        r[2] = e[1];
        r[3] = e[2];
        r[4] = e[3];
        r[5] = (int32_t)(c * T + i);
      }
  }
  return p->n_prefill_units;
}

int64_t moa_plan_decode_chunks(moa_plan_t p, int32_t* out) {
  int st = check_plan(p, false);
  if (st != MOA_OK) return st;
  const size_t n = p->decode_chunks.size() / 4;
  if (out)
    for (size_t i = 0; i < n; ++i) {   // in launch order
      const size_t c = p->decode_order.empty() ? i : (size_t)p->decode_order[i];
      const int32_t bh = p->decode_chunks[4 * c];
      out[4 * i + 0] = bh / p->Hkv;
      out[4 * i + 1] = bh % p->Hkv;
      out[4 * i + 2] = p->decode_chunks[4 * c + 1];
      out[4 * i + 3] = p->decode_chunks[4 * c + 2];
    }
  return (int64_t)n;
}

int32_t moa_plan_decode_chunk(moa_plan_t p) {
  int st = check_plan(p, false);
  if (st != MOA_OK) return st;
  return p->decode_chunk;
}

int moa_prefill(moa_plan_t p, const void* q, const void* k, const void* v, void* o, void* stream) {
  int st = check_prefill(p, q, k, v, o, "moa_prefill");
  if (st != MOA_OK) return st;
  hipError_t e = moa::launch_prefill(*p, q, k, v, o, nullptr, nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return MOA_OK;
}

int moa_prefill_handoff(moa_plan_t p, const void* q, const void* k, const void* v, void* o,
                        void* kc, void* vc, void* stream) {
  if (!kc || !vc) return fail(MOA_EINVAL, "moa_prefill_handoff: k_cache and v_cache must not be NULL");
  int st = check_aligned("moa_prefill_handoff", {kc, vc});
  if (st != MOA_OK) return st;
  if ((st = check_prefill(p, q, k, v, o, "moa_prefill_handoff")) != MOA_OK) return st;
  hipError_t e = moa::launch_prefill(*p, q, k, v, o, kc, vc, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill_handoff launch");
  return MOA_OK;
}

int moa_kv_append(moa_plan_t p, void* kc, void* vc, const void* kn, const void* vn, int64_t pos0,
                  int64_t n_new, void* stream) {
  int st = check_plan(p, false);
  if (st != MOA_OK) return st;
  if (!kc || !vc || !kn || !vn)
    return fail(MOA_EINVAL, "moa_kv_append: caches and new rows must not be NULL");
  if ((st = check_aligned("moa_kv_append", {kc, vc, kn, vn})) != MOA_OK) return st;
  if ((st = check_plan(p, true)) != MOA_OK) return st;
  if (pos0 < 0) return fail(MOA_EINVAL, "moa_kv_append: pos0 must be >= 0 (got %lld)", (long long)pos0);
  if (n_new < 1) return fail(MOA_EINVAL, "moa_kv_append: n_new must be >= 1 (got %lld)", (long long)n_new);
  if (n_new >= kMaxN || pos0 > ((int64_t)1 << 62) - n_new)
    return fail(MOA_EINVAL, "moa_kv_append: positions out of range");
  if ((st = set_device(p)) != MOA_OK) return st;
  hipError_t e = moa::launch_kv_append(*p, kc, vc, kn, vn, pos0, n_new, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  return MOA_OK;
}

int moa_decode(moa_plan_t p, const void* q, const void* kc, const void* vc, int64_t pos, void* o,
               void* ws, size_t ws_bytes, void* stream) {
  int st = check_decode(p, q, kc, vc, pos, o, ws, ws_bytes, true, "moa_decode");
  if (st != MOA_OK) return st;
  hipError_t e = moa::launch_decode_bf16(*p, q, kc, vc, o, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return MOA_OK;
}

int moa_append_decode(moa_plan_t p, const void* q, void* kc, void* vc, const void* kn,
                      const void* vn, int64_t pos, void* o, void* ws, size_t ws_bytes,
                      void* stream) {
  if (p != nullptr && (!kn || !vn))
    return fail(MOA_EINVAL, "moa_append_decode: k_new and v_new must not be NULL");
  int st = check_aligned("moa_append_decode", {kn, vn});
  if (st != MOA_OK) return st;
  if ((st = check_decode(p, q, kc, vc, pos, o, ws, ws_bytes, true, "moa_append_decode")) != MOA_OK)
    return st;
  if (pos >= ((int64_t)1 << 62))
    return fail(MOA_EINVAL, "moa_append_decode: pos out of range");
  hipError_t e =
      moa::launch_append_decode_bf16(*p, q, kc, vc, kn, vn, pos, o, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append_decode launch");
  return MOA_OK;
}

int moa_append_decode_static(moa_plan_t p, const void* q, void* kc, void* vc, const void* kn,
                             const void* vn, int64_t pos, void* o, void* stream) {
  // the size check comes first: it needs no device and names the limit
  if (p != nullptr && moa::decode_ws_bytes(*p) > moa::kStaticWsBytes)
    return fail(MOA_EWORKSPACE,
                "moa_append_decode_static: the plan needs %zu bytes of decode scratch, more than "
                "the fixed %zu (use moa_append_decode with a workspace)",
                moa::decode_ws_bytes(*p), moa::kStaticWsBytes);
  // the other checks are moa_append_decode's; the workspace is the fixed scratch
  if (p != nullptr && (!kn || !vn))
    return fail(MOA_EINVAL, "moa_append_decode_static: k_new and v_new must not be NULL");
  int st = check_aligned("moa_append_decode_static", {kn, vn});
  if (st != MOA_OK) return st;
  if ((st = check_decode(p, q, kc, vc, pos, o, nullptr, 0, false, "moa_append_decode_static")) !=
      MOA_OK)
    return st;
  if (pos >= ((int64_t)1 << 62))
    return fail(MOA_EINVAL, "moa_append_decode_static: pos out of range");
  void* ws = nullptr;
  hipError_t e = moa::static_workspace(&ws);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (decode scratch)");
  e = moa::launch_append_decode_bf16(*p, q, kc, vc, kn, vn, pos, o, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append_decode_static launch");
  return MOA_OK;
}

size_t moa_static_workspace_bytes(void) { return moa::kStaticWsBytes; }

const char* moa_last_error(void) { return g_last_error.c_str(); }

const char* moa_version(void) { return "libmoa 0.1 (gfx950)"; }

}  // extern "C"
