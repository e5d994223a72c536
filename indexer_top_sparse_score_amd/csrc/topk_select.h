// Exact per-row Top-K selection by one workgroup of NT threads.
//
// Method: Baidu AI Cloud, "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (keep the Top-K most
// relevant historical positions).  Readings: ties go to the lower position,
// the kept positions are written in ascending order, -1 pads to K.
//
// Scores are compared through score_key (order-preserving, NaN below every
// number).  The selection is exact.  A row takes one of these routes:
//  - at most K slots: keep every slot;
//  - at most kRegKeys slots: select on all of its keys, held in registers;
//  - a summary row (sum_row: more than 16384 and at most kSumMaxLen slots,
//    K <= kSumMaxK): select on the row's summary -- the kSumM largest keys
//    of each segment of G slots with their offsets, and the segment's next
//    key -- which the indexer's epilogue (or the standalone summary pass)
//    wrote:
//      1. T1 = the K-th largest summary key.  The summary keys sit at distinct
//         slots, so the row holds at least K keys >= T1.
//      2. A segment whose next key is >= T1 hides further keys >= T1: it is
//         saturated.  Every other segment keeps all of its keys >= T1 in the
//         summary.
//      3. Nothing saturated (the usual case): the summary's keys >= T1 are
//         exactly the row's, T = T1, and the summary itself is emitted.
//      4. Otherwise the candidates -- summary keys >= T1 of unsaturated
//         segments and the saturated segments' keys >= T1, which the waves
//         re-read from the score row, one segment per wave at a time -- are
//         exactly the row's keys >= T1.  They are staged in LDS in slot
//         order, T is their K-th largest, and they are emitted.  Too many of
//         them (or too many saturated segments) falls back to the streamed
//         route.
//  - otherwise (streamed): histogram passes over the row's keys read from
//    memory narrow the range to T, then one pass emits.
//
// The kept slots are staged in LDS (slot -> position) and written out at the
// end in one coalesced pass, with the KV row offsets when wanted.
//
// Selection of the K-th largest key (select_kth): histograms of 2048 bins
// laid over the current key range [lo, hi] narrow the range to the bin that
// holds the wanted rank, until one key value remains or the bin holds at
// most kSmall keys, which one wave then ranks directly.
//
// The code is kept small on purpose: a selection runs once per row, so its
// instructions are fetched cold, and a long unrolled body costs more in
// instruction fetch than it saves in issue.  Loops over LDS stay loops.
#pragma once

#include <type_traits>

#include "dsa_common.h"

namespace dsa {
namespace sel {

constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;   // 2048
constexpr int kSmall = 64;             // bin size ranked directly by one wave
constexpr int kRegKeys = kSumEntries;  // keys held in registers by a workgroup (both routes)
constexpr int kCandMax = 8192;         // candidates staged in LDS (saturated summary rows)
constexpr int kStageK = 2048;          // largest K whose selection is staged in LDS
constexpr int kSatMax = 512;           // saturated segments re-read by the waves

// LDS of one selection.  hist doubles as the histogram of every pass.
template <int NT>
struct Smem {
  static constexpr int kWaves = NT / 64;
  uint32_t hist[kBins];
  uint32_t ckey[kCandMax];
  int32_t cpos[kCandMax];
  int32_t pos[kStageK];  // kept slot -> position
  uint32_t sat_seg[kSatMax];  // saturated segments, in slot order
  uint32_t sat_cnt[kSatMax];  // their keys >= T1
  uint32_t sat_off[kSatMax];  // their first candidate
  alignas(16) uint32_t buf[kSmall];
  uint32_t res[4];
  alignas(16) uint32_t wsum[2 * kWaves];
  alignas(16) uint32_t wflag[2 * kWaves];  // per-wave flags of block_scan_flag
  alignas(16) uint32_t red[3 * (kWaves < 4 ? 4 : kWaves)];
};

// ------------------------------------------------------------ wave / block
// DPP controls: row_shr:n = 0x110 + n; row_bcast:15 = 0x142; row_bcast:31 =
// 0x143.  A lane whose DPP source is absent (or whose row is masked off)
// receives `id`, the identity of the operation.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp(uint32_t id, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, kCtrl, kRowMask, 0xF, false);
}

// Inclusive prefix over the 64 lanes of a wave, for an associative op with
// identity id.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t id, Op op) {
  x = op(x, dpp<0x111, 0xF>(id, x));
  x = op(x, dpp<0x112, 0xF>(id, x));
  x = op(x, dpp<0x114, 0xF>(id, x));
  x = op(x, dpp<0x118, 0xF>(id, x));
  x = op(x, dpp<0x142, 0xA>(id, x));
  x = op(x, dpp<0x143, 0xC>(id, x));
  return x;
}
struct Add { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct Min { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct Max { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };

// Exclusive prefix sum over the block in thread order; `tot` receives the
// total.  One barrier.  Consecutive scans alternate between the two halves
// of wsum (ph counts the scans of this thread), so a scan may start while
// slower waves still read the previous one's totals: the half it writes was
// last read before the previous scan's barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t* wsum, uint32_t& ph,
                                               uint32_t& tot) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* w = wsum + (ph & 1u) * W;
  ++ph;
  const uint32_t inc = wave_scan(x, 0u, Add());
  if (lane == 63) w[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  tot = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t v = w[i];
    tot += v;
    before += i < wave ? v : 0u;
  }
  return before + inc - x;
}

// block_scan that also ORs a per-thread flag over the block, through the
// same barrier (the result in every thread).
template <int NT>
__device__ __forceinline__ uint32_t block_scan_flag(uint32_t x, bool flag, uint32_t* wsum,
                                                    uint32_t* wflag, uint32_t& ph, uint32_t& tot,
                                                    bool& any) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* w = wsum + (ph & 1u) * W;
  uint32_t* f = wflag + (ph & 1u) * W;
  ++ph;
  const uint32_t inc = wave_scan(x, 0u, Add());
  const bool wf = __ballot(flag) != 0;
  if (lane == 63) {
    w[wave] = inc;
    f[wave] = wf ? 1u : 0u;
  }
  __syncthreads();
  uint32_t before = 0, fl = 0;
  tot = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t v = w[i];
    tot += v;
    before += i < wave ? v : 0u;
    fl |= f[i];
  }
  any = fl != 0u;
  return before + inc - x;
}

// Min, max and sum over the block (results in every thread).  One barrier;
// `red` is written once per selection.
template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t& sum,
                                             uint32_t* red) {
  constexpr int W = NT / 64;
  mn = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(mn, 0xFFFFFFFFu, Min()), 63);
  mx = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(mx, 0u, Max()), 63);
  sum = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(sum, 0u, Add()), 63);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[wave] = mn;
    red[W + wave] = mx;
    red[2 * W + wave] = sum;
  }
  __syncthreads();
  sum = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    mn = min(mn, red[i]);
    mx = max(mx, red[W + i]);
    sum += red[2 * W + i];
  }
}

__device__ __forceinline__ int bitlen32(uint32_t x) { return x ? 32 - __clz(x) : 0; }

// The need-th largest key (1-based, with multiplicity) among the keys in
// [lo, hi] that visit(f) hands to f in the threads of the block; there must
// be at least `need` of them.  On return `need` holds how many keys equal to
// the result belong to the need largest (the others are larger).  Every
// thread calls it with the same lo, hi and need; it starts and ends with
// every thread past a barrier.
template <int NT, class Visit>
__device__ __forceinline__ uint32_t select_kth(Visit visit, uint32_t lo, uint32_t hi,
                                               uint32_t& need, Smem<NT>& s, uint32_t& ph,
                                               bool zeroed = false) {
  constexpr int BPT = kBins / NT;  // bins per thread of the scan, from the top
  const int tid = threadIdx.x;
  while (lo < hi) {
    const int shift = max(0, bitlen32(hi - lo) - kBinBits);
    if (!zeroed) {  // (the caller may have cleared hist before a barrier of its own)
      for (int i = tid; i < kBins; i += NT) s.hist[i] = 0;
      __syncthreads();
    }
    zeroed = false;
    visit([&](uint32_t k) {
      if (k >= lo && k <= hi) atomicAdd(&s.hist[(k - lo) >> shift], 1u);
    });
    __syncthreads();
    // the bin b with above(b) < need <= above(b) + hist[b]
    {
      const int top = kBins - 1 - BPT * tid;
      uint32_t mine = 0;
      for (int i = 0; i < BPT; ++i) mine += s.hist[top - i];
      uint32_t tot;
      uint32_t above = block_scan<NT>(mine, s.wsum, ph, tot);
      for (int i = 0; i < BPT; ++i) {
        const uint32_t c = s.hist[top - i];
        if (above < need && need <= above + c) {
          s.res[0] = (uint32_t)(top - i);
          s.res[1] = above;
          s.res[2] = 0;
        }
        above += c;
      }
      __syncthreads();
    }
    const uint32_t b = s.res[0];
    need -= s.res[1];
    const uint32_t cnt = s.hist[b];
    const uint32_t nlo = lo + (b << shift);
    const uint32_t span = (1u << shift) - 1u;
    hi = (hi - nlo <= span) ? hi : nlo + span;
    lo = nlo;
    if (lo < hi && cnt <= (uint32_t)kSmall) {
      // rank the bin's keys directly: wave 0, one key per lane
      visit([&](uint32_t k) {
        if (k >= lo && k <= hi) s.buf[atomicAdd(&s.res[2], 1u)] = k;
      });
      __syncthreads();
      if (tid < 64) {
        const uint32_t m = s.res[2];
        const uint32_t x = (uint32_t)tid < m ? s.buf[tid] : 0u;
        uint32_t gt = 0, ge = 0;
        // every lane reads the bin's keys, sixteen at a time (LDS
        // broadcasts, issued together before their compares)
        for (uint32_t h = 0; h < m; h += 16) {
          uint4 y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = *reinterpret_cast<const uint4*>(&s.buf[h + 4 * i]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t v[4] = {y[i].x, y[i].y, y[i].z, y[i].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const bool in = h + (uint32_t)(4 * i + u) < m;
              gt += in && v[u] > x ? 1u : 0u;
              ge += in && v[u] >= x ? 1u : 0u;
            }
          }
        }
        if ((uint32_t)tid < m && gt < need && need <= ge) {  // equal keys write equal values
          s.res[0] = x;
          s.res[1] = need - gt;
        }
      }
      __syncthreads();
      const uint32_t T = s.res[0];
      need = s.res[1];
      __syncthreads();
      return T;
    }
    __syncthreads();  // the next pass rewrites hist and res
  }
  return lo;
}

// Emission bookkeeping: every key larger than T is kept, and the first
// need_eq keys equal to T in slot order.  After one block scan of each
// thread's counts (emit_begin), keep() walks the thread's keys in order.
struct Emit {
  uint32_t T, need_eq;
  uint32_t slot, eq;  // this thread's next output slot, equal keys before it
  __device__ __forceinline__ bool keep(uint32_t k) {
    const bool is_eq = k == T;
    const bool kp = k > T || (is_eq && eq < need_eq);
    eq += is_eq ? 1u : 0u;
    return kp;
  }
};
// Sets e.slot / e.eq for this thread from its counts of larger and equal
// keys (each total below 2^16).
template <int NT>
__device__ __forceinline__ void emit_begin(Emit& e, uint32_t gt, uint32_t eq, Smem<NT>& s,
                                           uint32_t& ph) {
  uint32_t tot;
  const uint32_t ex = block_scan<NT>((eq << 16) | gt, s.wsum, ph, tot);
  e.eq = ex >> 16;
  e.slot = (ex & 0xFFFFu) + min(e.eq, e.need_eq);
}

// ------------------------------------------------------------------ output
// The selection is staged as slot -> position in s.pos (K <= kStageK) and
// written out by flush(): indices, and with `roff` the byte offset of each
// kept position's row in a paged KV cache (block id from the row's block
// table `bt`, or its LDS copy `bt_lds`; -1, and DSA_DEVERR_BLOCK, for a
// block id out of range).  Slots are written as positions: the slot itself,
// or cand[slot] for a candidate-restricted row (checked against the history;
// an entry outside it is reported and written as 0).
struct Out {
  int32_t* gidx;
  int64_t* roff;
  const int32_t* cand;
  int hist;
  uint32_t* err;
  const int32_t* bt;
  const int32_t* bt_lds;
  int64_t kv_blocks, kv_block_stride, kv_row_stride;
};
__device__ __forceinline__ int out_position(const Out& o, int slot) {
  if (!o.cand) return slot;
  const int p = o.cand[slot];
  if (p >= 0 && p < o.hist) return p;
  report(o.err, DSA_DEVERR_ROW);
  return 0;
}
__device__ __forceinline__ int64_t out_row_offset(const Out& o, int p) {
  const int phys = o.bt_lds ? o.bt_lds[p >> 6] : o.bt[p >> 6];
  if (phys >= 0 && (int64_t)phys < o.kv_blocks)
    return (int64_t)phys * o.kv_block_stride + (int64_t)(p & 63) * o.kv_row_stride;
  report(o.err, DSA_DEVERR_BLOCK);
  return -1;
}
// Writes slots [0, K): the staged selection's first `count`, then -1.
template <int NT>
__device__ __forceinline__ void flush(const Out& o, int K, int count, const int32_t* staged) {
  for (int j = threadIdx.x; j < K; j += NT) {
    const int p = j < count ? out_position(o, staged[j]) : -1;
    o.gidx[j] = p;
    if (o.roff) o.roff[j] = p >= 0 ? out_row_offset(o, p) : -1;
  }
}
// Direct write of one kept slot (selections too large to stage).
__device__ __forceinline__ void put_direct(const Out& o, uint32_t slot, int s) {
  const int p = out_position(o, s);
  o.gidx[slot] = p;
  if (o.roff) o.roff[slot] = out_row_offset(o, p);
}

// ------------------------------------------------------------------ routes

// Keys of one register route, P = kRegKeys / NT per thread, in slot order
// (threads in order, entries in order); key 0 = no entry.  Full rows: entry
// j of thread t is slot P t + j.  Summary rows: thread t holds segments
// SPT t .. SPT t + SPT - 1 (kSumM entries each) and w[] their packed
// offsets; a slot is worked out only for the entries that are kept.
template <int NT>
struct Regs {
  static constexpr int P = kRegKeys / NT;
  static constexpr int SPT = P / kSumM;
  static_assert(SPT * kSumM == P && SPT * NT == kSumSegMax, "summary segments per thread");
  static_assert(P <= 64, "one bit per key in a 64-bit mask");
  using Mask = typename std::conditional<(P > 32), uint64_t, uint32_t>::type;
  uint32_t k[P];
  uint32_t w[2 * SPT];
  uint32_t nx[SPT];  // next key of each segment
  // slot of entry j
  __device__ __forceinline__ int slot(int j, int G) const {
    if (G == 0) return P * (int)threadIdx.x + j;
    const int q = j / kSumM, e = j % kSumM, wi = 2 * q + (e >> 2);
    uint32_t word = w[0];
#pragma unroll
    for (int i = 1; i < 2 * SPT; ++i) word = i == wi ? w[i] : word;
    return ((int)threadIdx.x * SPT + q) * G + (int)((word >> (8 * (e & 3))) & 0xFFu);
  }
};

__device__ __forceinline__ uint32_t popc_any(uint32_t m) { return __popc(m); }
__device__ __forceinline__ uint32_t popc_any(uint64_t m) { return __popcll(m); }

// Emits the register keys given T and the number of keys equal to T to
// keep (the first ones in slot order), into s.pos: every thread sets one
// bit per kept key, and after one block scan of the counts writes only
// those.  `sat`: this thread holds a saturated summary segment; the scan ORs
// it over the block, and when any is set nothing is written and false is
// returned (the same in every thread).  (Writing the kept keys straight to
// the output instead of staging them costs more: one narrow store per kept
// key and lane, against a few full-width ones.)
template <int NT>
__device__ __forceinline__ bool regs_emit(const Regs<NT>& r, int G, uint32_t T, uint32_t need_eq,
                                          bool sat, Smem<NT>& s, uint32_t& ph) {
  using Mask = typename Regs<NT>::Mask;
  Mask gtm = 0, eqm = 0;
#pragma unroll
  for (int j = 0; j < Regs<NT>::P; ++j) {
    gtm |= (Mask)(r.k[j] > T ? 1u : 0u) << j;
    eqm |= (Mask)(r.k[j] == T ? 1u : 0u) << j;
  }
  const uint32_t ngt = popc_any(gtm), neq = popc_any(eqm);
  uint32_t tot;
  bool any_sat;
  const uint32_t ex =
      block_scan_flag<NT>((neq << 16) | ngt, sat, s.wsum, s.wflag, ph, tot, any_sat);
  if (any_sat) return false;
  const uint32_t eq_before = ex >> 16;
  // equal keys this thread keeps, as a difference of two minima (the
  // conditional-subtract form of it lost its condition in compilation)
  const uint32_t take = min(eq_before + neq, need_eq) - min(eq_before, need_eq);
  Mask rest = eqm;
  for (uint32_t i = 0; i < take; ++i) rest &= rest - 1;  // drop the first `take` equal keys
  Mask keep = gtm | (eqm & ~rest);
  uint32_t slot = (ex & 0xFFFFu) + min(eq_before, need_eq);
  // a loop over the kept keys only, with the offsets copied to scalars first
  // (indexing the register arrays by a variable would move them to scratch)
  constexpr int SPT = Regs<NT>::SPT;
  uint32_t wv[2 * SPT];
#pragma unroll
  for (int i = 0; i < 2 * SPT; ++i) wv[i] = r.w[i];
  const int seg0 = (int)threadIdx.x * SPT;
  while (keep != 0) {
    const int j = (int)popc_any((keep & (0 - keep)) - 1);  // lowest set bit
    keep &= keep - 1;
    int p;
    if (G == 0) {
      p = Regs<NT>::P * (int)threadIdx.x + j;
    } else {
      const int wi = j >> 2;
      uint32_t word = wv[0];
#pragma unroll
      for (int i = 1; i < 2 * SPT; ++i) word = i == wi ? wv[i] : word;
      p = (seg0 + (j >> 3)) * G + (int)((word >> (8 * (j & 3))) & 0xFFu);
    }
    s.pos[slot++] = p;
  }
  return true;
}

// Streamed: histogram passes over the keys read from memory, then one
// emission pass (staged when K allows, else straight to memory).
template <int NT>
__device__ __forceinline__ void select_streamed(const float* sc, int L, int K, const Out& o,
                                                int count, Smem<NT>& s, uint32_t& ph) {
  auto visit = [&](auto f) {
    for (int i = threadIdx.x; i < L; i += NT) f(score_key(sc[i]));
  };
  uint32_t need = (uint32_t)K;
  const uint32_t T = select_kth<NT>(visit, 1u, 0xFFFFFFFFu, need, s, ph);
  // runs of NT * R slots, R consecutive per thread
  constexpr int R = 8;
  uint32_t out_before = 0, eq_before = 0;
  for (int i0 = 0; i0 < L && out_before < (uint32_t)K; i0 += NT * R) {
    const int p0 = i0 + R * (int)threadIdx.x;
    uint32_t gt = 0, eq = 0;
    for (int j = 0; j < R; ++j) {
      const uint32_t k = p0 + j < L ? score_key(sc[p0 + j]) : 0u;
      gt += k > T ? 1u : 0u;
      eq += k == T ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_scan<NT>((eq << 16) | gt, s.wsum, ph, tot);
    Emit e;
    e.T = T;
    e.need_eq = need;
    e.eq = eq_before + (ex >> 16);
    e.slot = out_before + (ex & 0xFFFFu) + min(e.eq, need) - min(eq_before, need);
    for (int j = 0; j < R; ++j) {
      const uint32_t k = p0 + j < L ? score_key(sc[p0 + j]) : 0u;
      if (k != 0u && e.keep(k)) {
        if (K <= kStageK)
          s.pos[e.slot] = p0 + j;
        else
          put_direct(o, e.slot, p0 + j);
        ++e.slot;
      }
    }
    out_before += (tot & 0xFFFFu) + min(eq_before + (tot >> 16), need) - min(eq_before, need);
    eq_before += tot >> 16;
  }
  __syncthreads();
  if (K <= kStageK) flush<NT>(o, K, count, s.pos);
}

// Whether summary segment q of this thread is saturated: its next key (the
// largest outside the summary) is >= T1.
template <int NT>
__device__ __forceinline__ bool seg_saturated(const Regs<NT>& r, int q, int L, int G, uint32_t T1) {
  const int sg = (int)threadIdx.x * Regs<NT>::SPT + q;
  return sg * G < L && r.nx[q] >= T1;
}

// Keys of saturated segment sg that are >= T1, visited by one wave in slot
// order: f(lane mask of the round, key, slot) for rounds of 64 slots.
template <class F>
__device__ __forceinline__ void sat_segment_keys(const float* sc, int L, int G, int sg, uint32_t T1,
                                                 F f) {
  const int lane = threadIdx.x & 63;
  const int s0 = sg * G, end = min(L, s0 + G);
  for (int b = s0; b < end; b += 64) {
    const int i = b + lane;
    const bool in = lane < G && i < end;
    const uint32_t k = in ? score_key(sc[i]) : 0u;
    const bool hit = in && k >= T1;
    f(__ballot(hit), hit, k, i);
  }
}

// A saturated summary row: candidates in LDS (step 4 above) into s.pos.
// `satm` marks this thread's saturated segments.  Returns false when they
// do not fit (the block agrees).
template <int NT>
__device__ __forceinline__ bool summary_saturated(const float* sc, int L, int G, const Regs<NT>& r,
                                                  uint32_t satm, uint32_t T1, uint32_t kmax, int K,
                                                  Smem<NT>& s, uint32_t& ph) {
  constexpr int kSPT = Regs<NT>::SPT, W = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  // 1. the saturated segments, listed in slot order
  uint32_t n_sat;
  const uint32_t sat_before = block_scan<NT>(__popc(satm), s.wsum, ph, n_sat);
  if (n_sat > (uint32_t)kSatMax) return false;
  {
    uint32_t i = sat_before;
#pragma unroll
    for (int q = 0; q < kSPT; ++q)
      if (satm >> q & 1u) s.sat_seg[i++] = (uint32_t)(tid * kSPT + q);
  }
  __syncthreads();
  // 2. each wave counts the keys >= T1 of its share of them
  for (uint32_t i = wave; i < n_sat; i += W) {
    uint32_t c = 0;
    sat_segment_keys(sc, L, G, (int)s.sat_seg[i], T1,
                     [&](uint64_t m, bool, uint32_t, int) { c += (uint32_t)__popcll(m); });
    if (lane == 0) s.sat_cnt[i] = c;
  }
  __syncthreads();
  // 3. candidate counts per thread, in slot order, and their offsets
  uint32_t c = 0;
  {
    uint32_t i = sat_before;
#pragma unroll
    for (int q = 0; q < kSPT; ++q) {
      if (satm >> q & 1u) {
        c += s.sat_cnt[i++];
      } else {
#pragma unroll
        for (int j = 0; j < kSumM; ++j) c += r.k[q * kSumM + j] >= T1 ? 1u : 0u;
      }
    }
  }
  uint32_t n_cand;
  uint32_t b = block_scan<NT>(c, s.wsum, ph, n_cand);
  if (n_cand > (uint32_t)kCandMax) return false;
  {
    uint32_t i = sat_before;
#pragma unroll
    for (int q = 0; q < kSPT; ++q) {
      if (satm >> q & 1u) {
        s.sat_off[i] = b;
        b += s.sat_cnt[i++];
      } else {
#pragma unroll
        for (int j = 0; j < kSumM; ++j)
          if (r.k[q * kSumM + j] >= T1) {
            s.ckey[b] = r.k[q * kSumM + j];
            s.cpos[b] = r.slot(q * kSumM + j, G);
            ++b;
          }
      }
    }
  }
  __syncthreads();
  // 4. the waves write the saturated segments' candidates at their offsets
  for (uint32_t i = wave; i < n_sat; i += W) {
    uint32_t o = s.sat_off[i];
    sat_segment_keys(sc, L, G, (int)s.sat_seg[i], T1,
                     [&](uint64_t m, bool hit, uint32_t k, int slot) {
                       if (hit) {
                         const uint32_t at = o + (uint32_t)__popcll(m & below);
                         s.ckey[at] = k;
                         s.cpos[at] = slot;
                       }
                       o += (uint32_t)__popcll(m);
                     });
  }
  __syncthreads();
  uint32_t need = (uint32_t)K;
  const uint32_t T = select_kth<NT>(
      [&](auto f) {
        for (int i = threadIdx.x; i < (int)n_cand; i += NT) f(s.ckey[i]);
      },
      T1, kmax, need, s, ph);
  // emission: thread t takes candidates qn t .. qn t + qn - 1
  const int qn = ((int)n_cand + NT - 1) / NT;
  const int i0 = min((int)n_cand, qn * tid), i1 = min((int)n_cand, i0 + qn);
  uint32_t gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    gt += s.ckey[i] > T ? 1u : 0u;
    eq += s.ckey[i] == T ? 1u : 0u;
  }
  Emit e;
  e.T = T;
  e.need_eq = need;
  emit_begin<NT>(e, gt, eq, s, ph);
  for (int i = i0; i < i1; ++i)
    if (e.keep(s.ckey[i])) s.pos[e.slot++] = s.cpos[i];
  return true;
}

// A thread's share of a row's summary: its SPT segments (SPT / 2 segment
// pairs), loaded before the row's length is known (the summary area always
// holds kSumSegMax segments per row; entries of segments past the row are
// masked once it is).  With 1024 threads each load instruction of a wave
// reads one contiguous kilobyte (sum_key_index lays the keys out so).
template <int NT>
__device__ __forceinline__ void load_summary(const uint32_t* skey, const uint8_t* soff,
                                             const uint32_t* snext, Regs<NT>& r) {
  constexpr int kSPT = Regs<NT>::SPT;
  static_assert(kSPT % 2 == 0, "whole segment pairs per thread");
#pragma unroll
  for (int i = 0; i < kSPT / 2; ++i) {
    const int pair = (int)threadIdx.x * (kSPT / 2) + i;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 a = *reinterpret_cast<const uint4*>(skey + sum_key_index(2 * pair, 4 * c));
      r.k[16 * i + 4 * c + 0] = a.x;
      r.k[16 * i + 4 * c + 1] = a.y;
      r.k[16 * i + 4 * c + 2] = a.z;
      r.k[16 * i + 4 * c + 3] = a.w;
    }
    const uint4 o = *reinterpret_cast<const uint4*>(soff + pair * 2 * kSumM);
    r.w[4 * i + 0] = o.x;
    r.w[4 * i + 1] = o.y;
    r.w[4 * i + 2] = o.z;
    r.w[4 * i + 3] = o.w;
    const uint2 n = *reinterpret_cast<const uint2*>(snext + 2 * pair);
    r.nx[2 * i] = n.x;
    r.nx[2 * i + 1] = n.y;
  }
}

// The whole selection of one row, written through `o` (every slot of
// [0, K): kept positions ascending, then -1).  `sc` is the row's score row
// (L slots, 16-byte aligned when vec); `r` holds this thread's preloaded
// share of the row's summary when has_sum (it is overwritten).  Returns
// min(K, L).  All threads of the block call it; it ends with every thread
// past a barrier.
template <int NT>
__device__ __forceinline__ int select_row(const float* sc, bool vec, int L, int K, Regs<NT>& r,
                                          bool has_sum, const Out& o, Smem<NT>& s) {
  const int tid = threadIdx.x;
  const int count = max(0, min(K, L));
  uint32_t ph = 0;  // block scans so far
  if (L <= K) {  // keep every slot
    if (K <= kStageK) {
      for (int j = tid; j < count; j += NT) s.pos[j] = j;
      __syncthreads();
      flush<NT>(o, K, count, s.pos);
    } else {
      for (int j = tid; j < K; j += NT) {
        if (j < count) {
          put_direct(o, (uint32_t)j, j);
        } else {
          o.gidx[j] = -1;
          if (o.roff) o.roff[j] = -1;
        }
      }
    }
    __syncthreads();
    return count;
  }
  constexpr int kPer = Regs<NT>::P, kSPT = Regs<NT>::SPT;
  const bool full = L <= kRegKeys && K <= kStageK;
  const bool summ = !full && has_sum && sum_row(L, K);
  if (full || summ) {
    int G = 0;
    if (full) {
      const int g0 = kPer * tid;
#pragma unroll
      for (int j = 0; j < kPer; j += 4) {
        float4 v;
        if (vec && g0 + j + 4 <= L) {
          v = *reinterpret_cast<const float4*>(sc + g0 + j);
        } else {
          v.x = g0 + j < L ? sc[g0 + j] : 0.0f;
          v.y = g0 + j + 1 < L ? sc[g0 + j + 1] : 0.0f;
          v.z = g0 + j + 2 < L ? sc[g0 + j + 2] : 0.0f;
          v.w = g0 + j + 3 < L ? sc[g0 + j + 3] : 0.0f;
        }
        r.k[j] = g0 + j < L ? score_key(v.x) : 0u;
        r.k[j + 1] = g0 + j + 1 < L ? score_key(v.y) : 0u;
        r.k[j + 2] = g0 + j + 2 < L ? score_key(v.z) : 0u;
        r.k[j + 3] = g0 + j + 3 < L ? score_key(v.w) : 0u;
      }
    } else {
      G = sum_seg(L);
      const int nseg = (L + G - 1) / G;
#pragma unroll
      for (int q = 0; q < kSPT; ++q) {
        const bool in = tid * kSPT + q < nseg;
#pragma unroll
        for (int j = 0; j < kSumM; ++j) r.k[q * 8 + j] = in ? r.k[q * 8 + j] : 0u;  // a select
      }
    }
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, n = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      kmin = min(kmin, r.k[j] != 0u ? r.k[j] : 0xFFFFFFFFu);
      kmax = max(kmax, r.k[j]);
      n += r.k[j] != 0u ? 1u : 0u;
    }
    for (int i = tid; i < kBins; i += NT) s.hist[i] = 0;  // for select_kth's first pass
    block_minmax<NT>(kmin, kmax, n, s.red);
    if (n >= (uint32_t)K) {  // always, for every row that takes these routes
      uint32_t need = (uint32_t)K;
      const uint32_t T1 = select_kth<NT>(
          [&](auto f) {
#pragma unroll
            for (int j = 0; j < kPer; ++j)
              if (r.k[j] != 0u) f(r.k[j]);
          },
          kmin, kmax, need, s, ph, true);
      uint32_t satm = 0;
      if (summ) {
#pragma unroll
        for (int q = 0; q < kSPT; ++q) satm |= (seg_saturated<NT>(r, q, L, G, T1) ? 1u : 0u) << q;
      }
      if (regs_emit<NT>(r, G, T1, need, satm != 0u, s, ph) ||
          summary_saturated<NT>(sc, L, G, r, satm, T1, kmax, K, s, ph)) {
        __syncthreads();
        flush<NT>(o, K, count, s.pos);
        __syncthreads();
        return count;
      }
    }
    __syncthreads();
  }
  select_streamed<NT>(sc, L, K, o, count, s, ph);
  if (K > kStageK) {  // padding of an unstaged selection
    for (int j = count + tid; j < K; j += NT) {
      o.gidx[j] = -1;
      if (o.roff) o.roff[j] = -1;
    }
  }
  __syncthreads();
  return count;
}

}  // namespace sel
}  // namespace dsa
