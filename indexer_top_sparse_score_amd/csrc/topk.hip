// Per-row Top-K on gfx950, spread over the whole GPU.
//
// Method: Baidu AI Cloud, "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (keep the Top-K most
// relevant historical positions).  Readings: ties go to the lower position,
// the kept positions are written in ascending order, -1 pads to K.
//
// Scores are compared through an order-preserving 32-bit key; the selection
// is exact.  Each row is cut into slices of `slice` positions and every
// kernel runs one workgroup per (slice, row):
//
//  0. key ranges (prep kernel, or the indexer scan's epilogue in the fused
//     step): the min and max key of every 1024-position tile; the row's
//     histogram and state are cleared.
//  1. hist: histogram of the row's keys over 2048 bins of width 2^shift laid
//     from the row's min key, so the bins follow the scores' actual range.
//  2. cand: every workgroup reads the finished histogram and finds the bin
//     b* that holds the K-th largest key; keys above b* are kept for sure.
//       - b* holds a single key value T (exact ties): each slice counts its
//         keys > T and == T (tie mode);
//       - b* holds at most kCandCap keys (the usual case: a handful): each
//         slice appends them as 64-bit composites (key << 32 | ~position),
//         which are all distinct and order exactly as the selection rule
//         ranks (larger key first, then lower position);
//       - otherwise nothing (fallback).
//     The last workgroup of the row to finish (atomic arrival count) ends
//     the selection: the need-th largest composite C* (or, in the fallback,
//     a one-workgroup refinement over the row), and the output offset of
//     every slice.
//  3. compact: each slice writes its kept positions, in order, at its
//     offset: key > T, or key == T with position <= P_T (composite mode) /
//     with tie rank below the tie budget (tie mode).

#include "dsa_common.h"

namespace dsa {

// per-row state words
enum : int { kCandCount = 0, kArrived = 1, kT = 2, kPT = 3, kNeedEq = 4 };

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBinBits = 11;
static_assert((1 << kBinBits) == kTopkBins, "bins");

struct RowInfo {
  int L;       // history length (0: invalid row)
  int r_local; // row index within the call
};

__device__ __forceinline__ RowInfo row_info(const TopkLaunch& a) {
  RowInfo ri;
  ri.r_local = (int)blockIdx.y;
  int b, p;
  const int r = a.row_begin + ri.r_local;
  ri.L = resolve_row(a.rows, r, b, p) ? p + 1 : 0;
  return ri;
}

// Cross-workgroup hand-off inside one kernel, without full-L2 fences: the
// producers publish with agent-scope atomic RMWs (performed coherently for
// every XCD), wait for their completion before the arrival count, and the
// last workgroup reads them back with agent-scope loads, which skip stale
// copies in its own XCD's L2.
__device__ __forceinline__ void publish32(uint32_t* p, uint32_t v) {
  __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish64(uint64_t* p, uint64_t v) {
  __hip_atomic_exchange(reinterpret_cast<unsigned long long*>(p), (unsigned long long)v,
                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fetch64(const uint64_t* p) {
  return (uint64_t)__hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// waits until this wave's outstanding memory operations have completed
__device__ __forceinline__ void drain_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int bitlen32(uint32_t x) { return x ? 32 - __clz(x) : 0; }
__device__ __forceinline__ int bitlen64(uint64_t x) { return x ? 64 - __clzll(x) : 0; }

template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Exclusive prefix sum over the 256 threads; `tot` receives the total.
// `scratch` holds kWaves words of LDS.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* scratch,
                                                         uint32_t& tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)inc, o);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t v = scratch[w];
    before += w < wave ? v : 0u;
    tot += v;
  }
  return before + inc - x;
}

// Min/max reduction over the 256 threads (results valid in every thread).
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* scratch) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    scratch[wave] = mn;
    scratch[kWaves + wave] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mn = min(mn, scratch[w]);
    mx = max(mx, scratch[kWaves + w]);
  }
}

// The row's key range from its tiles' ranges.
__device__ __forceinline__ void row_range(const TopkLaunch& a, int r_local, int L, uint32_t& kmin,
                                          uint32_t& kmax, uint32_t* scratch) {
  const int tiles = (L + kMMTile - 1) / kMMTile;
  const uint32_t* mm = a.tw.tile_mm + (int64_t)r_local * a.tw.mm_tiles * 2;
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
  for (int t = threadIdx.x; t < tiles; t += kThreads) {
    kmin = min(kmin, mm[2 * t]);
    kmax = max(kmax, mm[2 * t + 1]);
  }
  block_minmax(kmin, kmax, scratch);
}

__device__ __forceinline__ int range_shift(uint32_t kmin, uint32_t kmax) {
  return max(0, bitlen32(kmax - kmin) - kBinBits);
}

// Finds, over a 2048-bin histogram in LDS, the bin b with
// above(b) < need <= above(b) + h[b], where above(b) counts bins > b.
// Thread t owns bins 2047-8t .. 2040-8t.  Results land in out[0] (bin) and
// out[1] (above).
__device__ __forceinline__ void find_bin(const uint32_t* h, uint32_t need, uint32_t* out,
                                         uint32_t* scratch) {
  const int t = threadIdx.x;
  const int top = kTopkBins - 1 - 8 * t;
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) mine += h[top - j];
  uint32_t tot;
  uint32_t above = block_exclusive_scan(mine, scratch, tot);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t c = h[top - j];
    if (above < need && need <= above + c) {
      out[0] = (uint32_t)(top - j);
      out[1] = above;
    }
    above += c;
  }
  __syncthreads();
}

// ----------------------------------------------------------------- 0. prep
__global__ __launch_bounds__(kThreads) void topk_prep_kernel(TopkLaunch a) {
  __shared__ uint32_t scratch[2 * kWaves];
  const RowInfo ri = row_info(a);
  if (ri.L <= a.K) return;
  const int t = blockIdx.x;
  const int start = t * kMMTile;
  if (start >= ri.L) return;
  const int end = min(ri.L, start + kMMTile);
  const float* sc = a.scores + (int64_t)ri.r_local * a.ld;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = start + threadIdx.x; i < end; i += kThreads) {
    const uint32_t k = score_key(sc[i]);
    mn = min(mn, k);
    mx = max(mx, k);
  }
  block_minmax(mn, mx, scratch);
  if (threadIdx.x == 0) {
    uint32_t* mm = a.tw.tile_mm + ((int64_t)ri.r_local * a.tw.mm_tiles + t) * 2;
    mm[0] = mn;
    mm[1] = mx;
  }
  if (t == 0) {
    uint32_t* h = a.tw.hist + (int64_t)ri.r_local * kTopkBins;
    for (int i = threadIdx.x; i < kTopkBins; i += kThreads) h[i] = 0;
    if (threadIdx.x < kStateWords) a.tw.state[(int64_t)ri.r_local * kStateWords + threadIdx.x] = 0;
  }
}

// ----------------------------------------------------------------- 1. hist
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(TopkLaunch a) {
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t scratch[2 * kWaves];
  const RowInfo ri = row_info(a);
  if (ri.L <= a.K) return;
  const int start = blockIdx.x * a.tw.slice;
  if (start >= ri.L) return;
  const int end = min(ri.L, start + a.tw.slice);
  uint32_t kmin, kmax;
  row_range(a, ri.r_local, ri.L, kmin, kmax, scratch);
  const int shift = range_shift(kmin, kmax);
  for (int i = threadIdx.x; i < kTopkBins; i += kThreads) h[i] = 0;
  __syncthreads();
  const float* sc = a.scores + (int64_t)ri.r_local * a.ld;
  for (int base = start; base < end; base += 8 * kThreads) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * kThreads + threadIdx.x;
      v[j] = i < end ? sc[i] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * kThreads + threadIdx.x;
      if (i < end) atomicAdd(&h[min((score_key(v[j]) - kmin) >> shift, (uint32_t)kTopkBins - 1)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.tw.hist + (int64_t)ri.r_local * kTopkBins;
  for (int i = threadIdx.x; i < kTopkBins; i += kThreads)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// ----------------------------------------------------------------- 2. cand

enum Mode : int { kTie = 0, kCand = 1, kFallback = 2 };

// Exact selection inside the last workgroup, composite mode: the need-th
// largest of n composites held in LDS.
__device__ uint64_t select_composite(const uint64_t* c, int n, uint32_t need, uint32_t* h,
                                     uint32_t* scratch, uint32_t* res) {
  // range of the composites
  uint64_t lo = ~0ull, hi = 0ull;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    lo = min(lo, c[i]);
    hi = max(hi, c[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, (uint64_t)__shfl_xor((long long)lo, o));
    hi = max(hi, (uint64_t)__shfl_xor((long long)hi, o));
  }
  __shared__ uint64_t red[2 * kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[wave] = lo;
    red[kWaves + wave] = hi;
  }
  __syncthreads();
  for (int w = 0; w < kWaves; ++w) {
    lo = min(lo, red[w]);
    hi = max(hi, red[kWaves + w]);
  }
  __syncthreads();
  while (lo < hi) {
    const int shift = max(0, bitlen64(hi - lo) - kBinBits);
    for (int i = threadIdx.x; i < kTopkBins; i += kThreads) h[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint64_t x = c[i];
      if (x >= lo && x <= hi)
        atomicAdd(&h[min((uint32_t)((x - lo) >> shift), (uint32_t)kTopkBins - 1)], 1u);
    }
    __syncthreads();
    find_bin(h, need, res, scratch);
    const uint32_t b = res[0];
    need -= res[1];
    const uint64_t nlo = lo + ((uint64_t)b << shift);
    const uint64_t span = (uint64_t(1) << shift) - 1;
    const uint64_t nhi = (hi - nlo < span) ? hi : nlo + span;
    lo = nlo;
    hi = nhi;
    __syncthreads();
  }
  return lo;
}

// Fallback inside the last workgroup: narrow [lo, hi] over the row's keys
// (read from global memory) until one key value T remains; returns T and the
// number of keys equal to T still to keep in `need`.
__device__ uint32_t select_in_row(const float* sc, int L, uint32_t lo, uint32_t hi,
                                  uint32_t& need, uint32_t* h, uint32_t* scratch,
                                  uint32_t* res) {
  while (lo < hi) {
    const int shift = max(0, bitlen32(hi - lo) - kBinBits);
    for (int i = threadIdx.x; i < kTopkBins; i += kThreads) h[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < L; i += kThreads) {
      const uint32_t k = score_key(sc[i]);
      if (k >= lo && k <= hi) atomicAdd(&h[min((k - lo) >> shift, (uint32_t)kTopkBins - 1)], 1u);
    }
    __syncthreads();
    find_bin(h, need, res, scratch);
    need -= res[1];
    const uint32_t nlo = lo + (res[0] << shift);
    const uint32_t span = (uint32_t)((1ull << shift) - 1);
    hi = (hi - nlo < span) ? hi : nlo + span;
    lo = nlo;
    __syncthreads();
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void topk_cand_kernel(TopkLaunch a) {
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t scratch[2 * kWaves];
  __shared__ uint32_t res[4];
  __shared__ uint64_t cl[kCandCap];
  __shared__ uint32_t sel_cnt[256];
  __shared__ uint32_t sl_a[256];
  __shared__ int last;
  const RowInfo ri = row_info(a);
  if (ri.L <= a.K) return;
  const int s = blockIdx.x;
  const int start = s * a.tw.slice;
  if (start >= ri.L) return;
  const int end = min(ri.L, start + a.tw.slice);
  const int n_sl = (ri.L + a.tw.slice - 1) / a.tw.slice;
  const int64_t rs = (int64_t)ri.r_local * a.tw.n_slices;
  uint32_t* st = a.tw.state + (int64_t)ri.r_local * kStateWords;
  const float* sc = a.scores + (int64_t)ri.r_local * a.ld;

  uint32_t kmin, kmax;
  row_range(a, ri.r_local, ri.L, kmin, kmax, scratch);
  const int shift = range_shift(kmin, kmax);
  const uint32_t* gh = a.tw.hist + (int64_t)ri.r_local * kTopkBins;
  for (int i = threadIdx.x; i < kTopkBins; i += kThreads) h[i] = gh[i];
  __syncthreads();
  find_bin(h, (uint32_t)a.K, res, scratch);
  const uint32_t bstar = res[0];
  const uint32_t above = res[1];
  const uint32_t cnt_b = h[bstar];
  const uint32_t lo_b = kmin + (bstar << shift);
  const uint32_t span = (uint32_t)((1ull << shift) - 1);
  const uint32_t hi_b = (kmax - lo_b < span) ? kmax : lo_b + span;
  const int mode = lo_b == hi_b ? kTie : (cnt_b <= (uint32_t)kCandCap ? kCand : kFallback);

  if (mode != kFallback) {
    uint32_t n_above = 0, n_eq = 0;
    const int lane = threadIdx.x & 63;
    uint64_t* cand = a.tw.cand + (int64_t)ri.r_local * kCandCap;
    for (int base = start; base < end; base += kThreads) {
      const int i = base + threadIdx.x;
      const bool ok = i < end;
      const uint32_t k = ok ? score_key(sc[i]) : 0u;
      n_above += (ok && k > hi_b) ? 1u : 0u;
      const bool in_bin = ok && k >= lo_b && k <= hi_b;
      if (mode == kTie) {
        n_eq += in_bin ? 1u : 0u;
      } else {
        const uint64_t m = __ballot(in_bin);
        uint32_t slot = 0;
        if (lane == 0 && m) slot = atomicAdd(&st[kCandCount], (uint32_t)__popcll(m));
        slot = (uint32_t)__shfl((int)slot, 0);
        const uint32_t at = slot + (uint32_t)lane_prefix(m);
        if (in_bin && at < (uint32_t)kCandCap)
          publish64(&cand[at], ((uint64_t)k << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i));
      }
    }
    uint32_t t1;
    n_above = wave_sum(n_above);
    n_eq = wave_sum(n_eq);
    __syncthreads();
    if (lane == 0) {
      scratch[threadIdx.x >> 6] = n_above;
      scratch[kWaves + (threadIdx.x >> 6)] = n_eq;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t sa = 0, se = 0;
      for (int w = 0; w < kWaves; ++w) {
        sa += scratch[w];
        se += scratch[kWaves + w];
      }
      publish32(&a.tw.s_def[rs + s], sa);
      publish32(&a.tw.s_eq[rs + s], se);
    }
    (void)t1;
  }

  // ---- arrival: the last workgroup of the row finishes the selection
  drain_memory();
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&st[kArrived], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(n_sl - 1);
  __syncthreads();
  if (!last) return;

  uint32_t need = (uint32_t)a.K - above;  // keys still to keep from inside bin b*
  uint32_t T, PT, need_eq;
  // per-slice counts in LDS: keys above the threshold, and keys equal to it
  // (tie modes) or chosen candidates (composite mode)
  for (int j = threadIdx.x; j < 256; j += kThreads) {
    sl_a[j] = j < n_sl && mode != kFallback ? fetch32(&a.tw.s_def[rs + j]) : 0u;
    sel_cnt[j] = j < n_sl && mode == kTie ? fetch32(&a.tw.s_eq[rs + j]) : 0u;
  }
  __syncthreads();
  if (mode == kCand) {
    const int n = (int)min(fetch32(&st[kCandCount]), (uint32_t)kCandCap);
    const uint64_t* cand = a.tw.cand + (int64_t)ri.r_local * kCandCap;
    for (int i = threadIdx.x; i < n; i += kThreads) cl[i] = fetch64(&cand[i]);
    __syncthreads();
    const uint64_t cstar = select_composite(cl, n, need, h, scratch, res);
    for (int i = threadIdx.x; i < n; i += kThreads)
      if (cl[i] >= cstar) {
        const uint32_t pos = 0xFFFFFFFFu - (uint32_t)cl[i];
        atomicAdd(&sel_cnt[min(pos / (uint32_t)a.tw.slice, 255u)], 1u);
      }
    __syncthreads();
    T = (uint32_t)(cstar >> 32);
    PT = 0xFFFFFFFFu - (uint32_t)cstar;
    need_eq = 0xFFFFFFFFu;
  } else {
    if (mode == kTie) {
      T = lo_b;
    } else {
      // refine inside bin b* over the whole row, then count per slice
      T = select_in_row(sc, ri.L, lo_b, hi_b, need, h, scratch, res);
      for (int j = 0; j < n_sl; ++j) {
        const int a0 = j * a.tw.slice, a1 = min(ri.L, a0 + a.tw.slice);
        uint32_t g = 0, e = 0;
        for (int i = a0 + threadIdx.x; i < a1; i += kThreads) {
          const uint32_t k = score_key(sc[i]);
          g += k > T ? 1u : 0u;
          e += k == T ? 1u : 0u;
        }
        uint32_t tg, te;
        block_exclusive_scan(g, scratch, tg);
        block_exclusive_scan(e, scratch, te);
        if (threadIdx.x == 0) {
          sl_a[j] = tg;
          sel_cnt[j] = te;
        }
      }
      __syncthreads();
    }
    need_eq = need;
    PT = 0x7FFFFFFFu;
  }
  // output offsets: slices in order; in the tie modes the budget of keys
  // equal to T is spent in position order
  const bool ties = mode != kCand;
  if (threadIdx.x == 0) {
    res[2] = 0;
    res[3] = 0;
  }
  __syncthreads();
  for (int c0 = 0; c0 < n_sl; c0 += kThreads) {
    const int j = c0 + threadIdx.x;
    const uint32_t e = (j < n_sl && ties) ? sel_cnt[j] : 0u;
    uint32_t te;
    const uint32_t eqb = res[3] + block_exclusive_scan(e, scratch, te);
    const uint32_t take = ties ? (eqb >= need_eq ? 0u : min(e, need_eq - eqb))
                               : (j < n_sl ? sel_cnt[j] : 0u);
    const uint32_t cnt = j < n_sl ? sl_a[j] + take : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan(cnt, scratch, tot);
    if (j < n_sl) {
      a.tw.s_off[rs + j] = res[2] + ex;
      a.tw.s_eqb[rs + j] = ties ? eqb : 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      res[2] += tot;
      res[3] += te;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    st[kT] = T;
    st[kPT] = PT;
    st[kNeedEq] = need_eq;
  }
}

// -------------------------------------------------------------- 3. compact
__global__ __launch_bounds__(kThreads) void topk_compact_kernel(TopkLaunch a) {
  __shared__ uint32_t scratch[2 * kWaves];
  const RowInfo ri = row_info(a);
  const int K = a.K;
  const int s = blockIdx.x;
  int32_t* out = a.indices + (int64_t)ri.r_local * K;
  if (s == 0 && threadIdx.x == 0 && a.counts) a.counts[ri.r_local] = min(K, ri.L);
  if (ri.L <= K) {
    const int a0 = s * a.tw.slice, a1 = min(ri.L, a0 + a.tw.slice);
    for (int j = a0 + threadIdx.x; j < a1; j += kThreads) out[j] = j;
    if (s == 0)
      for (int j = ri.L + threadIdx.x; j < K; j += kThreads) out[j] = -1;
    return;
  }
  const int start = s * a.tw.slice;
  if (start >= ri.L) return;
  const int end = min(ri.L, start + a.tw.slice);
  const uint32_t* st = a.tw.state + (int64_t)ri.r_local * kStateWords;
  const uint32_t T = st[kT], PT = st[kPT], need_eq = st[kNeedEq];
  const int64_t rs = (int64_t)ri.r_local * a.tw.n_slices;
  const uint32_t off0 = a.tw.s_off[rs + s];
  const uint32_t eqb0 = a.tw.s_eqb[rs + s];
  const float* sc = a.scores + (int64_t)ri.r_local * a.ld;

  // each thread owns a contiguous run of `per` positions
  const int per = (a.tw.slice + kThreads - 1) / kThreads;
  const int i0 = start + threadIdx.x * per;
  const int i1 = min(end, i0 + per);
  uint32_t n_eq = 0;
  if (need_eq != 0xFFFFFFFFu)
    for (int i = i0; i < i1; ++i) n_eq += score_key(sc[i]) == T ? 1u : 0u;
  uint32_t tot;
  uint32_t eq_rank = eqb0 + block_exclusive_scan(n_eq, scratch, tot);
  uint32_t n_sel = 0;
  {
    uint32_t er = eq_rank;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = score_key(sc[i]);
      const bool eq = k == T;
      n_sel += (k > T || (eq && (uint32_t)i <= PT && er < need_eq)) ? 1u : 0u;
      er += eq ? 1u : 0u;
    }
  }
  uint32_t at = off0 + block_exclusive_scan(n_sel, scratch, tot);
  for (int i = i0; i < i1; ++i) {
    const uint32_t k = score_key(sc[i]);
    const bool eq = k == T;
    if (k > T || (eq && (uint32_t)i <= PT && eq_rank < need_eq)) {
      if (at < (uint32_t)K) out[at] = i;
      ++at;
    }
    eq_rank += eq ? 1u : 0u;
  }
}

}  // namespace

size_t topk_work_bytes(int rows, int64_t max_len) {
  const TopkWork w = topk_work_carve(nullptr, rows, max_len);
  return (size_t)(reinterpret_cast<uintptr_t>(w.cand) + sizeof(uint64_t) * rows * kCandCap);
}

TopkWork topk_work_carve(void* base, int rows, int64_t max_len) {
  TopkWork w;
  w.mm_tiles = (int)((max_len + kMMTile - 1) / kMMTile);
  int64_t slice = 2048;
  while ((max_len + slice - 1) / slice > 256) slice += 2048;
  w.slice = (int)slice;
  w.n_slices = (int)((max_len + slice - 1) / slice);
  auto r256 = [](size_t x) { return (x + 255) & ~size_t(255); };
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* p = b + off;
    off += r256(bytes);
    return p;
  };
  w.tile_mm = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 2 * rows * w.mm_tiles));
  w.hist = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * rows * kTopkBins));
  w.state = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * rows * kStateWords));
  w.s_def = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * rows * w.n_slices));
  w.s_eq = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * rows * w.n_slices));
  w.s_off = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * rows * w.n_slices));
  w.s_eqb = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * rows * w.n_slices));
  w.cand = reinterpret_cast<uint64_t*>(take(0));
  return w;
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t s) {
  if (a.num_rows <= 0) return hipSuccess;
  if (a.prep) {
    topk_prep_kernel<<<dim3(a.tw.mm_tiles, a.num_rows), kThreads, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(a.tw.n_slices, a.num_rows);
  topk_hist_kernel<<<grid, kThreads, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  topk_cand_kernel<<<grid, kThreads, 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  topk_compact_kernel<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
