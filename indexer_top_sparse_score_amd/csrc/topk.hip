// Per-row Top-K on gfx950: one workgroup of 1024 threads per row.
//
// Method: Baidu AI Cloud, "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (keep the Top-K most
// relevant historical positions).  Readings: ties go to the lower position,
// the kept positions are written in ascending order, -1 pads to K.
//
// Scores are compared through an order-preserving 32-bit key (score_key);
// the selection is exact.  Rows of 16385 to 131072 positions (K <= 2048,
// topk_split_row) are spread over up to 32 workgroups, one per slice of 4096
// positions, and pre-select on the row's summary: the m largest keys of each
// segment of 32 to 128 positions (topk_sum_seg, topk_sum_m), written by the
// fused indexer's epilogue or, for the standalone entry point, by
// topk_summary_kernel.
//
//  1. A lower bound t on the row's K-th largest key T: the summary's keys
//     sit at distinct positions, so its own K-th largest is at most T.  One
//     2048-bin histogram of the summary over its range gives t = the lower
//     edge of the bin that holds its K-th largest key.  The segments' top
//     keys hold nearly every one of the row's top K, so t is close to T:
//     about 1.04 K keys are >= t.
//  2. Each slice compacts its keys >= t, in position order, into its
//     segment of the work area; the last slice to finish reads them all.
//  3. T is selected exactly among them, together with the number of keys
//     equal to T that are kept (the first ones in position order).
//  4. The kept positions are written in ascending order: block-wide prefix
//     sums over the compacted list, staged in LDS, then stored in one
//     coalesced pass (with the KV row offsets, from a copy of the row's block
//     table in LDS).
//
// Rows of at most 16384 positions run steps 3-4 on their keys in one
// workgroup; rows with L <= K keep every position.  A row that does not fit
// these buffers (K > 2048, more than 8192 keys >= t or more than a slice's
// share of them because of ties, or t = 0 because of NaN scores) runs the
// same selection over its keys streamed from memory.
//
// Selection (select_kth): histograms of 2048 bins laid over the current key
// range [lo, hi] narrow the range to the bin that holds the wanted rank,
// until one key value remains or the bin holds at most kSmall keys, which
// one wave then ranks directly.  Wave-level scans and reductions use DPP
// row shifts and broadcasts.

#include "dsa_common.h"

namespace dsa {
namespace {

constexpr int kT = 1024;                  // threads per workgroup
constexpr int kWaves = kT / 64;           // 16
constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;      // 2048
constexpr int kSmall = 64;                // bin size ranked directly by one wave
constexpr int kPerThread = 16;            // keys per thread of a one-workgroup row
constexpr int kMaxN = kPerThread * kT;    // 16384
constexpr int kKeysPer = 8;               // compacted keys per thread (the finish)
constexpr int kMaxKeys = kKeysPer * kT;   // 8192
constexpr int kSumPer = kSumMax / kT;     // summary keys per thread (4)
constexpr int kRunPer = kTopkSliceLen / kT;  // a slice's positions per thread (4)
static_assert(kRunPer * kT == kTopkSliceLen && kRunPer % 4 == 0, "a slice is one run per thread");
static_assert(kTopkSlices <= 64, "one wave holds the slice counts");
static_assert(kTopkSplitMaxK <= kBins, "split rows select within one staged pass");
constexpr int kBtCache = 2048;            // block-table entries cached in LDS
constexpr int kScanWords = 4 * kWaves + 1;
static_assert(kBins == 2 * kT, "find_bin gives each thread two bins");

struct Smem {
  uint32_t hist[kBins];    // histograms; afterwards slot -> kept position
  int32_t cp[kMaxKeys];    // a slice's compacted positions (for the KV prefetch)
  int32_t bt[kBtCache];    // the row's block table (rows of <= 2048 blocks)
  uint32_t buf[kSmall];
  uint32_t res[4];
  alignas(16) uint32_t wsum[kScanWords];
  alignas(16) uint32_t red[3 * kWaves];
};

__device__ __forceinline__ int bitlen32(uint32_t x) { return x ? 32 - __clz(x) : 0; }

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

// Sum of the 16 words at w (16-byte aligned) before index `upto`, and of
// all of them: four broadcast reads.
__device__ __forceinline__ uint32_t sum_words(const uint32_t* w, int upto, uint32_t& all) {
  const uint4* w4 = reinterpret_cast<const uint4*>(w);
  uint32_t before = 0;
  all = 0;
#pragma unroll
  for (int v = 0; v < kWaves / 4; ++v) {
    const uint4 q = w4[v];
    const int i = 4 * v;
    all += (q.x + q.y) + (q.z + q.w);
    before += (i < upto ? q.x : 0u) + (i + 1 < upto ? q.y : 0u) + (i + 2 < upto ? q.z : 0u) +
              (i + 3 < upto ? q.w : 0u);
  }
  return before;
}

// Exclusive prefix sum over the block in thread order; `tot` receives the
// total.  Each wave's total goes to LDS and, after one barrier, every wave
// adds up those before it.  kFree: a second barrier at the end, so `wsum`
// may be rewritten at once; without it the caller must pass a barrier
// before `wsum` is written again.
template <bool kFree = true>
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t* wsum, uint32_t& tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_scan(x, 0u, Add());
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  const uint32_t before = sum_words(wsum, wave, tot);
  if (kFree) __syncthreads();
  return before + inc - x;
}

// Exclusive prefix sums of N sequences of one value per thread, taken one
// after another (sequence 0 over threads 0..1023, then sequence 1, ...):
// ex[i] sums every earlier value of that order.  Returns the grand total.
// Wave 0 scans the N x 16 wave totals.  Starts and ends with a barrier.
template <int N>
__device__ __forceinline__ uint32_t block_scan_n(const uint32_t (&x)[N], uint32_t (&ex)[N],
                                                 uint32_t* wsum) {
  static_assert(N * kWaves <= 64, "one wave scans the wave totals");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) inc[i] = wave_scan(x[i], 0u, Add());
  __syncthreads();
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < N; ++i) wsum[i * kWaves + wave] = inc[i];
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t v = lane < N * kWaves ? wsum[lane] : 0u;
    const uint32_t c = wave_scan(v, 0u, Add());
    if (lane < N * kWaves) wsum[lane] = c - v;
    if (lane == 63) wsum[4 * kWaves] = c;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) ex[i] = wsum[i * kWaves + wave] + inc[i] - x[i];
  const uint32_t total = wsum[4 * kWaves];
  __syncthreads();
  return total;
}

// Min, max and sum over the block (results in every thread).  One barrier;
// `red` (3 x 16 words) must not be in use.
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t& sum,
                                             uint32_t* red) {
  mn = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(mn, 0xFFFFFFFFu, Min()), 63);
  mx = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(mx, 0u, Max()), 63);
  sum = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(sum, 0u, Add()), 63);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[wave] = mn;
    red[kWaves + wave] = mx;
    red[2 * kWaves + wave] = sum;
  }
  __syncthreads();
  const uint4* r4 = reinterpret_cast<const uint4*>(red);
  sum = 0;
#pragma unroll
  for (int v = 0; v < kWaves / 4; ++v) {
    const uint4 a = r4[v], b = r4[kWaves / 4 + v], c = r4[kWaves / 2 + v];
    mn = min(min(min(mn, a.x), min(a.y, a.z)), a.w);
    mx = max(max(max(mx, b.x), max(b.y, b.z)), b.w);
    sum += (c.x + c.y) + (c.z + c.w);
  }
}

// Over the 2048-bin histogram h, the bin b with above(b) < need <=
// above(b) + h[b], where above(b) counts the keys in bins above b; thread t
// owns bins 2047 - 2t and 2046 - 2t.  Results: res[0] = b, res[1] = above(b);
// res[2] is cleared (select_kth counts with it).  Requires 1 <= need <= sum
// of h.  Two barriers, the last at the end.
__device__ __forceinline__ void find_bin(const uint32_t* h, uint32_t need, uint32_t* res,
                                         uint32_t* wsum) {
  const int top = kBins - 1 - 2 * (int)threadIdx.x;
  const uint32_t c0 = h[top], c1 = h[top - 1];
  uint32_t tot;
  const uint32_t above = block_scan<false>(c0 + c1, wsum, tot);
  if (above < need && need <= above + c0) {
    res[0] = (uint32_t)top;
    res[1] = above;
    res[2] = 0;
  } else if (above + c0 < need && need <= above + c0 + c1) {
    res[0] = (uint32_t)(top - 1);
    res[1] = above + c0;
    res[2] = 0;
  }
  __syncthreads();
}

__device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi) {
  return max(0, bitlen32(hi - lo) - kBinBits);
}

// Histogram of the keys in [lo, hi] that visit(f) hands to f, on 2048 bins
// of width 2^shift from lo, and the bin b holding the need-th largest
// (res[0] = b, res[1] = keys above b).
// With kZeroed the caller has already cleared the histogram (and a barrier
// has passed since).
template <bool kZeroed = false, class Visit>
__device__ __forceinline__ void histogram_bin(Visit&& visit, uint32_t lo, uint32_t hi, int shift,
                                              uint32_t need, Smem& s) {
  if (!kZeroed) {
    for (int i = threadIdx.x; i < kBins; i += kT) s.hist[i] = 0;
    __syncthreads();
  }
  visit([&](uint32_t k) {
    if (k >= lo && k <= hi) atomicAdd(&s.hist[(k - lo) >> shift], 1u);
  });
  __syncthreads();
  find_bin(s.hist, need, s.res, s.wsum);
}

// The need-th largest key (1-based, counted with multiplicity) among the keys
// in [lo, hi] that visit(f) hands to f in the threads of the block; there
// must be at least `need` of them.  On return `need` holds how many keys
// equal to the result belong to the need largest (the others are larger).
// Every thread calls it with the same lo, hi and need.  With kZeroed the
// caller has cleared the histogram (and a barrier has passed since).
template <bool kZeroed = false, class Visit>
__device__ __forceinline__ uint32_t select_kth(Visit&& visit, uint32_t lo, uint32_t hi,
                                               uint32_t& need, Smem& s) {
  const int tid = threadIdx.x;
  bool zeroed = kZeroed;
  while (lo < hi) {
    const int shift = range_shift(lo, hi);
    if (zeroed)
      histogram_bin<true>(visit, lo, hi, shift, need, s);
    else
      histogram_bin<false>(visit, lo, hi, shift, need, s);
    zeroed = false;
    const uint32_t b = s.res[0];
    need -= s.res[1];
    const uint32_t cnt = s.hist[b];
    const uint32_t nlo = lo + (b << shift);
    const uint32_t span = (1u << shift) - 1u;
    hi = (hi - nlo <= span) ? hi : nlo + span;
    lo = nlo;
    if (lo < hi && cnt <= (uint32_t)kSmall) {
      // rank the bin's keys directly: wave 0, one key per lane.  find_bin
      // cleared the counter res[2]; res[0..1] are rewritten only after the
      // next barrier, which every thread reaches after reading them.
      visit([&](uint32_t k) {
        if (k >= lo && k <= hi) s.buf[atomicAdd(&s.res[2], 1u)] = k;
      });
      __syncthreads();
      if (tid < 64) {
        const uint32_t m = s.res[2];
        const uint32_t x = (uint32_t)tid < m ? s.buf[tid] : 0u;
        uint32_t gt = 0, ge = 0;
        for (uint32_t i = 0; i < m; ++i) {
          const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)i);
          gt += y > x ? 1u : 0u;
          ge += y >= x ? 1u : 0u;
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

// ------------------------------------------------------------------ output
// Where the kept positions go.  The emission records slot -> position in
// LDS (`pos`, the histogram's storage, free by then; K <= 2048) and flush()
// writes them out once all are known: coalesced index stores and the KV row
// offsets (block ids from the LDS copy of the block table when the row's
// table fits it).  Larger K (only on the streamed path) writes through put()
// directly.
struct Out {
  int32_t* idx;        // [K]
  int64_t* roff;       // [K] or NULL: byte offsets of the kept rows in the KV cache
  const int32_t* bt;   // the row's block table
  const int32_t* bt_lds;  // its LDS copy, or NULL
  int64_t kv_blocks, kv_block_stride, kv_row_stride;
  uint32_t* err;
  uint32_t* pos;       // LDS staging of the selection, or NULL
  // Candidate rows: the selection is over slots of the row's list, written
  // as their positions cand[slot] (NULL: slots are positions).  A position
  // outside the history (0 .. hist-1) is reported and written as 0.
  const int32_t* cand;
  int hist;
  __device__ __forceinline__ int position(int slot) const {
    if (!cand) return slot;
    const int p = cand[slot];
    if (p >= 0 && p < hist) return p;
    report(err, DSA_DEVERR_ROW);
    return 0;
  }
  __device__ __forceinline__ int64_t row_offset(int p, int phys) const {
    if (phys >= 0 && (int64_t)phys < kv_blocks)
      return (int64_t)phys * kv_block_stride + (int64_t)(p & 63) * kv_row_stride;
    report(err, DSA_DEVERR_BLOCK);
    return -1;
  }
  __device__ __forceinline__ int block_of(int p) const {
    return bt_lds ? bt_lds[p >> 6] : bt[p >> 6];
  }
  // kStaged: into `pos` (then flush()), else straight to memory
  template <bool kStaged>
  __device__ __forceinline__ void put(uint32_t slot, int p) const {
    if (kStaged) {
      pos[slot] = (uint32_t)p;
      return;
    }
    p = position(p);
    idx[slot] = p;
    if (roff) roff[slot] = row_offset(p, bt[p >> 6]);
  }
  // after the emission (and a barrier): the staged selection to memory
  __device__ __forceinline__ void flush(int K) const {
    constexpr int kPer = kBins / kT;  // slots per thread
    int p[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int slot = (int)threadIdx.x + i * kT;
      p[i] = slot < K ? position((int)pos[slot]) : 0;
      if (slot < K) idx[slot] = p[i];
    }
    if (!roff) return;
    int phys[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) phys[i] = (int)threadIdx.x + i * kT < K ? block_of(p[i]) : 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int slot = (int)threadIdx.x + i * kT;
      if (slot < K) roff[slot] = row_offset(p[i], phys[i]);
    }
  }
};

// N consecutive keys of a row starting at position i0 (entries at or past L
// are 0).  Vector loads when the row and i0 allow them.
template <int N>
__device__ __forceinline__ void load_keys(const float* sc, int i0, int L, bool vec, uint32_t (&k)[N]) {
  if (vec && (N % 4) == 0 && i0 + N <= L) {
#pragma unroll
    for (int j = 0; j < N; j += 4) {
      const float4 v = *reinterpret_cast<const float4*>(sc + i0 + j);
      k[j] = score_key(v.x);
      k[j + 1] = score_key(v.y);
      k[j + 2] = score_key(v.z);
      k[j + 3] = score_key(v.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) k[j] = i0 + j < L ? score_key(sc[i0 + j]) : 0u;
  }
}

// Emits one run of N entries per thread (threads in order, entry j of a
// thread at position pos(j)), masked to the first `n`, given T and the
// budget of keys equal to T.  `eq_before` / `out_before` carry the counts of
// earlier runs and are advanced past this one.  kLast: no other emission
// follows before a barrier (its scan then skips the trailing one).
template <int N, bool kStaged, bool kLast = false, class Pos>
__device__ __forceinline__ void emit_runs(const uint32_t (&k)[N], int n, Pos&& pos, uint32_t T,
                                          uint32_t need_eq, uint32_t& eq_before,
                                          uint32_t& out_before, const Out& o, Smem& s) {
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    gt += (j < n && k[j] > T) ? 1u : 0u;
    eq += (j < n && k[j] == T) ? 1u : 0u;
  }
  // one scan for both counts (a run holds at most 16384 entries, so each
  // half of the packed word stays below 2^16)
  uint32_t tot;
  const uint32_t ex = block_scan<!kLast>((eq << 16) | gt, s.wsum, tot);
  const uint32_t eqx = eq_before + (ex >> 16);  // equal keys before this thread
  // kept so far: every larger key, and equal keys up to the budget
  const uint32_t slot0 = out_before + (ex & 0xFFFFu) + min(eqx, need_eq) - min(eq_before, need_eq);
  out_before += (tot & 0xFFFFu) + min(eq_before + (tot >> 16), need_eq) - min(eq_before, need_eq);
  eq_before += tot >> 16;
  uint32_t slot = slot0, e = eqx;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (j < n) {
      const bool is_eq = k[j] == T;
      const bool keep = k[j] > T || (is_eq && e < need_eq);
      e += is_eq ? 1u : 0u;
      if (keep) o.template put<kStaged>(slot++, pos(j));
    }
  }
}

// ------------------------------------------------------------------- paths

// The general path: the same selection over the row's keys streamed from
// memory (several passes), then the emission run by run.
template <bool kStaged>
__device__ __forceinline__ void select_streamed(const float* sc, int L, int K, bool vec,
                                                const Out& o, Smem& s) {
  constexpr int kRun = 8;
  auto visit = [&](auto f) {
    for (int i0 = 0; i0 < L; i0 += kRun * kT) {
      const int p = i0 + kRun * (int)threadIdx.x;
      uint32_t k[kRun];
      load_keys<kRun>(sc, p, L, vec, k);
#pragma unroll
      for (int j = 0; j < kRun; ++j)
        if (p + j < L) f(k[j]);
    }
  };
  uint32_t need = (uint32_t)K;
  const uint32_t T = select_kth(visit, 0u, 0xFFFFFFFFu, need, s);
  uint32_t eq_before = 0, out_before = 0;
  for (int i0 = 0; i0 < L && out_before < (uint32_t)K; i0 += kRun * kT) {
    const int p = i0 + kRun * (int)threadIdx.x;
    uint32_t k[kRun];
    load_keys<kRun>(sc, p, L, vec, k);
    emit_runs<kRun, kStaged>(k, max(0, min(kRun, L - p)), [&](int j) { return p + j; }, T,
                             need, eq_before, out_before, o, s);
  }
}

// Steps 3-4 on the row's keys themselves, 16 per thread (rows of at most
// kMaxN positions).
__device__ __forceinline__ void select_keys(const float* sc, int L, int K, bool vec, const Out& o,
                                            Smem& s) {
  const int g0 = kPerThread * (int)threadIdx.x;
  uint32_t k[kPerThread];
  load_keys<kPerThread>(sc, g0, L, vec, k);
  const int n_mine = max(0, min(kPerThread, L - g0));
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (j < n_mine) {
      kmin = min(kmin, k[j]);
      kmax = max(kmax, k[j]);
    }
  uint32_t unused = 0;
  block_minmax(kmin, kmax, unused, s.red);
  auto visit = [&](auto f) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (j < n_mine) f(k[j]);
  };
  uint32_t need = (uint32_t)K;
  const uint32_t T = select_kth(visit, kmin, kmax, need, s);
  uint32_t eq_before = 0, out_before = 0;
  emit_runs<kPerThread, true, true>(k, n_mine, [&](int j) { return g0 + j; }, T, need, eq_before,
                                    out_before, o, s);
}

__device__ __forceinline__ Out make_out(const TopkLaunch& a, int r_local, int b) {
  Out o;
  o.idx = a.indices + (int64_t)r_local * a.K;
  o.roff = a.rowoff ? a.rowoff + (int64_t)r_local * a.K : nullptr;
  o.bt = a.rows.block_table + (int64_t)b * a.rows.max_blocks;
  o.bt_lds = nullptr;
  o.kv_blocks = a.kv.num_blocks;
  o.kv_block_stride = a.kv.block_stride;
  o.kv_row_stride = a.kv.row_stride;
  o.err = a.err;
  o.pos = nullptr;
  o.cand = nullptr;
  o.hist = 0;
  return o;
}

// Copies the row's block table to LDS when the KV row offsets are wanted and
// it fits (read while the selection runs; flush() uses it).
__device__ __forceinline__ void cache_block_table(int L, Out& o, Smem& s) {
  const int nblk = (L + kBlock - 1) / kBlock;
  if (o.roff && nblk <= kBtCache) {
    for (int i = threadIdx.x; i < nblk; i += kT) s.bt[i] = o.bt[i];
    o.bt_lds = s.bt;
  }
}

// A whole row in one workgroup: every path but the split one.  L: the score
// row's length (slots), Lh: the history's (whose block ids are cached).
__device__ __forceinline__ void row_single(const TopkLaunch& a, int r_local, int L, int Lh,
                                           Out& o, Smem& s) {
  const int tid = threadIdx.x;
  const int K = a.K;
  if (tid == 0 && a.counts) a.counts[r_local] = min(K, L);
  if (L <= K) {  // keep the whole history (nothing for an invalid row)
    for (int j = tid; j < K; j += kT) {
      if (j < L) {
        o.template put<false>((uint32_t)j, j);
      } else {
        o.idx[j] = -1;
        if (o.roff) o.roff[j] = -1;
      }
    }
    return;
  }
  const float* sc = a.scores + (int64_t)r_local * a.ld;
  if (K > kBins) {  // too many to stage: straight to memory
    select_streamed<false>(sc, L, K, a.vec, o, s);
    return;
  }
  cache_block_table(Lh, o, s);
  o.pos = s.hist;
  if (L <= kMaxN)
    select_keys(sc, L, K, a.vec, o, s);
  else
    select_streamed<true>(sc, L, K, a.vec, o, s);
  __syncthreads();
  o.flush(K);
}

// ---------------------------------------------------------- split rows
// A split row (topk_split_row) is spread over up to kTopkSlices workgroups,
// one per slice of kTopkSliceLen positions:
//  a. every workgroup computes t from the row's whole summary (the same
//     integer arithmetic on the same data, so the same t everywhere);
//  b. each keeps its slice's keys >= t and writes them, with their
//     positions and in position order, to its segment of the work area;
//  c. the last workgroup of the row to count itself in (a device-scope
//     counter, once its stores have completed) reads the segments back in
//     slice order -- position order -- selects T and the tie budget exactly
//     and writes the row out; the others warm the caches for the attention.
// Nothing waits on another workgroup.  Rows that do not take this path run
// row_single in slice 0's workgroup.

// Loads one dword of every 128-byte line of the KV rows at the positions
// cp[0..n), through the row's block table in LDS, and waits for them: only
// their arrival in the caches matters.  At most kPrefetchPer lines per
// thread (longer lists are cut), all in flight at once.
constexpr int kPrefetchPer = 8;
__device__ __forceinline__ void prefetch_rows(const TopkLaunch& a, uint32_t n, const int32_t* cp,
                                              const int32_t* bt_lds) {
  const int lines = (a.kv_row_bytes + 127) / 128;
  const uint32_t total = min(n * (uint32_t)lines, (uint32_t)(kPrefetchPer * kT));
  const uint8_t* base = static_cast<const uint8_t*>(a.kv.base);
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kPrefetchPer; ++i) {
    const uint32_t idx = threadIdx.x + (uint32_t)(i * kT);
    if (idx < total) {
      const int c = (int)(idx / (uint32_t)lines), l = (int)(idx % (uint32_t)lines);
      const int p = cp[c];
      const int phys = bt_lds[p >> 6];
      if (phys >= 0 && (int64_t)phys < a.kv.num_blocks)
        acc ^= *reinterpret_cast<const uint32_t*>(base + (int64_t)phys * a.kv.block_stride +
                                                  (int64_t)(p & 63) * a.kv.row_stride + 128 * l);
    }
  }
  asm volatile("" : : "v"(acc));  // keeps the loads, waits for them once
}

// Device-coherent store for the hand-over between a row's workgroups: an
// agent-scope atomic store, which the hardware writes through the XCD's L2
// (nothing dirty is left to write back).
__device__ __forceinline__ void store_shared(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The kRunPer scores from position i0 as raw bits (positions past L as 0);
// converted to keys only once they are needed, so nothing waits for them
// earlier.
__device__ __forceinline__ void run_scores(const float* sc, int i0, int L, bool vec,
                                           uint32_t (&x)[kRunPer]) {
  if (vec && i0 + kRunPer <= L) {
#pragma unroll
    for (int j = 0; j < kRunPer; j += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(sc + i0 + j);
      x[j] = v.x;
      x[j + 1] = v.y;
      x[j + 2] = v.z;
      x[j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRunPer; ++j) x[j] = i0 + j < L ? __float_as_uint(sc[i0 + j]) : 0u;
  }
}

__global__ __launch_bounds__(kT) void topk_split_kernel(TopkLaunch a) {
  __shared__ Smem s;
  const int tid = threadIdx.x;
  const int slice = (int)blockIdx.x;
  const int r_local = (int)blockIdx.y;
  const int K = a.K;
  // one round trip: the row's length, its summary (kSumPer keys per thread,
  // unconditional 16-byte loads: the summary area holds kSumMax per row)
  const RowIssue ri = row_issue(a.rows, a.row_begin + r_local);
  uint32_t sm[kSumPer];
  {
    const uint4 v =
        *reinterpret_cast<const uint4*>(a.tw.summ + (int64_t)r_local * kSumMax + kSumPer * tid);
    sm[0] = v.x; sm[1] = v.y; sm[2] = v.z; sm[3] = v.w;
  }
  const int Lh = row_finish(a.rows, ri);      // history length
  const int L = row_slots(a.rows, ri, Lh);    // score row length (candidate count)
  Out o = make_out(a, r_local, ri.b_ok ? ri.b : 0);
  const int32_t* crow =
      a.rows.cand ? a.rows.cand + (int64_t)(a.row_begin + r_local) * a.rows.n_cand : nullptr;
  o.cand = crow;
  o.hist = Lh;
  if (!topk_split_row(L, K)) {
    if (slice == 0) row_single(a, r_local, L, Lh, o, s);
    return;
  }
  const int S = (L + kTopkSliceLen - 1) / kTopkSliceLen;
  if (slice >= S) return;

  // this thread's run of the slice: its scores, loaded now, used after t
  const float* sc = a.scores + (int64_t)r_local * a.ld;
  const int p0 = slice * kTopkSliceLen + kRunPer * tid;
  uint32_t k[kRunPer];
  run_scores(sc, p0, L, a.vec, k);
  // and their positions (candidate rows: the list's entries, checked)
  int32_t cp[kRunPer];
  if (crow) {
    if (a.cvec && p0 + kRunPer <= L) {
#pragma unroll
      for (int j = 0; j < kRunPer; j += 4) {
        const int4 v = *reinterpret_cast<const int4*>(crow + p0 + j);
        cp[j] = v.x; cp[j + 1] = v.y; cp[j + 2] = v.z; cp[j + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRunPer; ++j) cp[j] = p0 + j < L ? crow[p0 + j] : 0;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRunPer; ++j) cp[j] = p0 + j;
  }
  for (int i = tid; i < kBins; i += kT) s.hist[i] = 0;  // for step a; block_minmax syncs
  if (slice == 0 && tid == 0 && a.counts) a.counts[r_local] = K;
  // the row's block ids for the KV row offsets: loaded now, staged in LDS
  // only by the workgroup that writes the row out
  constexpr int kBtPer = kBtCache / kT;
  const int nblk = (Lh + kBlock - 1) / kBlock;
  const bool bt_cached = o.roff && nblk <= kBtCache;
  int32_t btv[kBtPer];
#pragma unroll
  for (int j = 0; j < kBtPer; ++j) {
    const int i = tid + j * kT;
    btv[j] = bt_cached && i < nblk ? o.bt[i] : 0;
  }

  // a. t = lower edge of the bin holding the summary's K-th largest key
  //    (key 0, NaN or no position, does not count)
  const int n_sum = ((L + topk_sum_seg(L) - 1) / topk_sum_seg(L)) * topk_sum_m(L);
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, n_nz = 0;
#pragma unroll
  for (int j = 0; j < kSumPer; ++j) {
    sm[j] = kSumPer * tid + j < n_sum ? sm[j] : 0u;
    if (sm[j] != 0u) {
      kmin = min(kmin, sm[j]);
      kmax = max(kmax, sm[j]);
      ++n_nz;
    }
  }
  block_minmax(kmin, kmax, n_nz, s.red);
  uint32_t t = 0;
  if (n_nz >= (uint32_t)K) {  // else too few keys for a bound (NaN): t = 0
    t = kmin;
    if (kmin < kmax) {
      auto visit = [&](auto f) {
#pragma unroll
        for (int j = 0; j < kSumPer; ++j)
          if (sm[j] != 0u) f(sm[j]);
      };
      const int shift = range_shift(kmin, kmax);
      histogram_bin<true>(visit, kmin, kmax, shift, (uint32_t)K, s);
      t = kmin + (s.res[0] << shift);
    }
  }
  o.pos = s.hist;
  if (t == 0) {  // NaN scores at the threshold: the general path, once
    if (slice == 0) {
      __syncthreads();
      select_streamed<true>(sc, L, K, a.vec, o, s);
      __syncthreads();
      o.flush(K);
    }
    return;
  }

  // b. this slice's keys >= t (t >= 1: positions past L, key 0, never count)
  bool bad_pos = false;
#pragma unroll
  for (int j = 0; j < kRunPer; ++j) {
    k[j] = p0 + j < L ? score_key(__uint_as_float(k[j])) : 0u;
    if (crow && p0 + j < L && (cp[j] < 0 || cp[j] >= Lh)) {  // a list entry outside the history
      bad_pos = true;
      cp[j] = 0;
    }
  }
  if (bad_pos) report(a.err, DSA_DEVERR_ROW);
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kRunPer; ++j) c += k[j] >= t ? 1u : 0u;
  uint32_t n_slice;
  uint32_t at = block_scan<false>(c, s.wsum, n_slice);  // the hand-over's barriers follow
  {
    const int64_t seg = (int64_t)r_local * a.tw.cstride + (int64_t)slice * kTopkSliceLen;
#pragma unroll
    for (int j = 0; j < kRunPer; ++j)
      if (k[j] >= t) {
        store_shared(a.tw.ckey + seg + at, k[j]);
        store_shared(reinterpret_cast<uint32_t*>(a.tw.cpos) + seg + at, (uint32_t)cp[j]);
        if (at < (uint32_t)kMaxKeys) s.cp[at] = cp[j];  // for the KV prefetch
        ++at;
      }
    if (tid == 0) store_shared(a.tw.ccount + r_local * kTopkSlices + slice, n_slice);
    if (bt_cached) {  // every workgroup: the prefetch below reads it too
#pragma unroll
      for (int j = 0; j < kBtPer; ++j) s.bt[tid + j * kT] = btv[j];
    }
  }

  // c. the last slice to finish completes the row.  The segments and counts
  //    went out as device-coherent stores (written through, nothing dirty
  //    left in the L2): each wave waits until its own have completed, the
  //    barrier gathers the waves, and only then does thread 0 count the
  //    slice in (a device-scope atomic).  So no release fence, whose L2
  //    write-back cost about a microsecond per workgroup.  The workgroup
  //    that sees the count reach S invalidates its caches (an acquire fence
  //    by thread 0, before the barrier that releases the others) and reads
  //    everything back with ordinary vector loads.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // no compiler motion across the wait
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(a.tw.arrive + r_local, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const bool last = done == (uint32_t)(S - 1);
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s.res[3] = last ? 1u : 0u;
  }
  __syncthreads();
  if (s.res[3] == 0) {
    // Handed over: touch the KV rows of this slice's candidates (a superset
    // of what the row keeps), one 4-byte load per 128-byte line, so that
    // the attention's gather finds them in the caches rather than in HBM.
    if (a.kv_row_bytes > 0 && bt_cached)
      prefetch_rows(a, min(n_slice, (uint32_t)kMaxKeys), s.cp, s.bt);
    return;
  }
  if (bt_cached) o.bt_lds = s.bt;  // staged by every workgroup above
  for (int i = tid; i < kBins; i += kT) s.hist[i] = 0;  // for the selection, while loading
  // Thread t reads entries kKeysPer (t mod P) .. +kKeysPer-1 of slice t / P,
  // P = kT / S threads per slice, together with the counts (no round trip
  // between them); in thread order that is position order.  A slice with
  // more than P kKeysPer candidates makes every thread reload densely.
  const int P = kT / S;
  const int my_slice = tid / P;
  const int e0 = kKeysPer * (tid % P);
  const int64_t seg = (int64_t)r_local * a.tw.cstride + (int64_t)my_slice * kTopkSliceLen;
  const int64_t row_end = (int64_t)(r_local + 1) * a.tw.cstride;
  uint32_t kk[kKeysPer];
  int32_t pp[kKeysPer];
  // A slice's candidates end at or before the row's end of the area, so
  // entries past it are never wanted (and not read).  Segments start on
  // 16-byte boundaries: two 16-byte loads each for keys and positions.
  if (my_slice < S && seg + e0 + kKeysPer <= row_end) {
#pragma unroll
    for (int j = 0; j < kKeysPer; j += 4) {
      const uint4 kv = *reinterpret_cast<const uint4*>(a.tw.ckey + seg + e0 + j);
      const int4 pv = *reinterpret_cast<const int4*>(a.tw.cpos + seg + e0 + j);
      kk[j] = kv.x; kk[j + 1] = kv.y; kk[j + 2] = kv.z; kk[j + 3] = kv.w;
      pp[j] = pv.x; pp[j + 1] = pv.y; pp[j + 2] = pv.z; pp[j + 3] = pv.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kKeysPer; ++j) {
      const bool in = my_slice < S && seg + e0 + j < row_end;
      kk[j] = in ? a.tw.ckey[seg + e0 + j] : 0u;
      pp[j] = in ? a.tw.cpos[seg + e0 + j] : 0;
    }
  }
  // the slices' counts, lane j of every wave holding slice j's
  const int lane = tid & 63;
  const uint32_t cnt_lane = lane < S ? a.tw.ccount[r_local * kTopkSlices + lane] : 0u;
  const uint32_t n_tot = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(cnt_lane, 0u, Add()), 63);
  const uint32_t c_max = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(cnt_lane, 0u, Max()), 63);
  if (n_tot > (uint32_t)kMaxKeys) {
    // heavy ties at t: the general path
    select_streamed<true>(sc, L, K, a.vec, o, s);
  } else {
    int n;
    if (c_max <= (uint32_t)(P * kKeysPer)) {  // every slice fit its share: loaded above
      const uint32_t c_mine = (uint32_t)__shfl((int)cnt_lane, my_slice & 63);
      n = my_slice < S ? max(0, min(kKeysPer, (int)c_mine - e0)) : 0;
    } else {
      // A slice overflowed its share (the row's top keys cluster): reload
      // densely.  Thread t takes entries kKeysPer t .. +kKeysPer-1 of the
      // slices' lists laid end to end (still position order), finding each
      // entry's slice from the slices' running totals in LDS -- one more
      // round trip, on this path only.
      const uint32_t incl = wave_scan(cnt_lane, 0u, Add());  // lanes >= S: n_tot
      uint32_t* ends = s.wsum;  // ends[q] = entries in slices 0 .. q
      if (tid < kTopkSlices) ends[tid] = incl;
      __syncthreads();
      const int g0 = kKeysPer * tid;
      n = max(0, min(kKeysPer, (int)n_tot - g0));
      int q = 0;
      for (int step = kTopkSlices / 2; step >= 1; step >>= 1)  // last q with ends[q-1] <= g0
        if (q + step < kTopkSlices && (int)ends[q + step - 1] <= g0) q += step;
#pragma unroll
      for (int j = 0; j < kKeysPer; ++j) {
        const int e = g0 + j;
        if (j < n) {
          while ((int)ends[q] <= e) ++q;
          const int64_t at = (int64_t)r_local * a.tw.cstride + (int64_t)q * kTopkSliceLen +
                             (e - (q > 0 ? (int)ends[q - 1] : 0));
          kk[j] = a.tw.ckey[at];
          pp[j] = a.tw.cpos[at];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kKeysPer; ++j) kk[j] = j < n ? kk[j] : 0u;
    auto visit = [&](auto f) {
#pragma unroll
      for (int j = 0; j < kKeysPer; ++j)
        if (j < n) f(kk[j]);
    };
    uint32_t need = (uint32_t)K;
    __syncthreads();  // the cleared histogram
    const uint32_t T = select_kth<true>(visit, t, kmax, need, s);
    o.cand = nullptr;  // the segments hold positions already
    uint32_t eq_before = 0, out_before = 0;
    emit_runs<kKeysPer, true, true>(kk, n, [&](int j) { return pp[j]; }, T, need, eq_before,
                                    out_before, o, s);
  }
  __syncthreads();
  o.flush(K);
  if (tid == 0) a.tw.arrive[r_local] = 0;
}

// The summary for a standalone Top-K call: one wave per 128 positions keeps
// the m largest keys of each of their segments (segment_top).
__global__ __launch_bounds__(256) void topk_summary_kernel(TopkLaunch a) {
  int b, p;
  const int r_local = (int)blockIdx.y;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.tw.arrive[r_local] = 0;
  if (!resolve_row(a.rows, a.row_begin + r_local, b, p)) return;
  int L = p + 1;
  if (a.rows.cand) {  // the score row is the candidate list
    const int c = a.rows.cand_len[a.row_begin + r_local];
    L = c < 0 ? 0 : c > a.rows.n_cand ? a.rows.n_cand : c;
  }
  if (!topk_split_row(L, a.K)) return;
  const int lane = (int)(threadIdx.x & 63);
  const int seg = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int w0 = seg * kSumSpan;
  if (w0 >= L) return;
  const float* sc = a.scores + (int64_t)r_local * a.ld;
  const uint32_t ka = w0 + lane < L ? score_key(sc[w0 + lane]) : 0u;
  const uint32_t kb = w0 + 64 + lane < L ? score_key(sc[w0 + 64 + lane]) : 0u;
  const int m = topk_sum_m(L), G = topk_sum_seg(L);
  uint32_t out_a, out_b;
  segment_top(ka, kb, m, G, out_a, out_b);
  store_segment_top(a.tw.summ + (int64_t)r_local * kSumMax, w0, L, m, G, out_a, out_b);
}

}  // namespace

namespace {
int64_t cstride_of(int64_t max_len) { return (max_len + 63) & ~int64_t(63); }
}  // namespace

size_t topk_work_bytes(int rows, int64_t max_len) {
  if (rows <= 0) return 0;
  const size_t words = (size_t)kSumMax + 2 * (size_t)cstride_of(max_len) + kTopkSlices + 1;
  return (size_t)rows * words * sizeof(uint32_t);
}

TopkWork topk_work_carve(void* base, int rows, int64_t max_len) {
  TopkWork w;
  uint32_t* p = static_cast<uint32_t*>(base);
  w.cstride = cstride_of(max_len);
  w.summ = p;
  p += (size_t)rows * kSumMax;
  w.ckey = p;
  p += (size_t)rows * w.cstride;
  w.cpos = reinterpret_cast<int32_t*>(p);
  p += (size_t)rows * w.cstride;
  w.ccount = p;
  p += (size_t)rows * kTopkSlices;
  w.arrive = p;
  return w;
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t s) {
  if (a.num_rows <= 0) return hipSuccess;
  if (a.prep) {  // the rows' summaries (and the arrival counters cleared)
    const int64_t segs = (a.max_len + kSumSpan - 1) / kSumSpan;
    topk_summary_kernel<<<dim3((unsigned)((segs + 3) / 4), a.num_rows), 256, 0, s>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // as many slices as the longest row can use (a row that splits has at
  // most that many; the others run in slice 0)
  const int64_t slices = (a.max_len + kTopkSliceLen - 1) / kTopkSliceLen;
  const unsigned gx = (unsigned)(slices < 1 ? 1 : slices > kTopkSlices ? kTopkSlices : slices);
  topk_split_kernel<<<dim3(gx, a.num_rows), kT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
