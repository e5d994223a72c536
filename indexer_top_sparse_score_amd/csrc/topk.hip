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
//     step): the min and max key of every kMMTile-position tile; the row's
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
enum : int { kCandCount = 0, kArrived = 1, kT = 2, kNeedEq = 3, kMode = 4, kLoB = 5, kAbove = 6 };

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 8;                   // positions per thread per pass
constexpr int kPass = kPer * kThreads;    // positions per pass; slices are multiples of it
constexpr int kBinBits = 11;
static_assert((1 << kBinBits) == kTopkBins, "bins");

struct RowInfo {
  int L;       // history length (0: invalid row)
  int r_local; // row index within the call
  int b;       // sequence (valid when L > 0)
};

__device__ __forceinline__ RowInfo row_info(const TopkLaunch& a) {
  RowInfo ri;
  ri.r_local = (int)blockIdx.y;
  int b = 0, p;
  const int r = a.row_begin + ri.r_local;
  ri.L = resolve_row(a.rows, r, b, p) ? p + 1 : 0;
  ri.b = b;
  return ri;
}

// Byte offset of position i's row in the paged KV cache, given its block id
// (-1, and an error report, when the id is out of range).
__device__ __forceinline__ int64_t kv_offset(const TopkLaunch& a, int i, int phys) {
  if (phys < 0 || (int64_t)phys >= a.kv.num_blocks) {
    report(a.err, DSA_DEVERR_BLOCK);
    return -1;
  }
  return (int64_t)phys * a.kv.block_stride + (int64_t)(i & 63) * a.kv.row_stride;
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

// This thread's share of the row's key range (the tiles' ranges), loaded
// two tiles per step; block_minmax finishes it.
__device__ __forceinline__ void row_range_load(const TopkLaunch& a, int r_local, int L,
                                               uint32_t& kmin, uint32_t& kmax) {
  const int tiles = (L + kMMTile - 1) / kMMTile;
  const uint32_t* mm = a.tw.tile_mm + (int64_t)r_local * a.tw.mm_tiles * 2;
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
  for (int t = threadIdx.x; t < tiles; t += 2 * kThreads) {
    const int u = min(t + kThreads, tiles - 1);
    const uint2 x = *reinterpret_cast<const uint2*>(mm + 2 * t);
    const uint2 y = *reinterpret_cast<const uint2*>(mm + 2 * u);
    kmin = min(kmin, min(x.x, y.x));
    kmax = max(kmax, max(x.y, y.y));
  }
}

// The keys of one pass (kPer per thread, coalesced; positions past `end`
// repeat the last one and are masked by the caller).
__device__ __forceinline__ void load_pass(const float* sc, int base, int end, uint32_t* k) {
#pragma unroll
  for (int j = 0; j < kPer; ++j) k[j] = score_key(sc[min(base + j * kThreads + (int)threadIdx.x, end - 1)]);
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
  const float* sc = a.scores + (int64_t)ri.r_local * a.ld;
  // the first pass's keys and the row's range are loaded together
  uint32_t k[kPer];
  load_pass(sc, start, end, k);
  uint32_t kmin, kmax;
  row_range_load(a, ri.r_local, ri.L, kmin, kmax);
  for (int i = threadIdx.x; i < kTopkBins; i += kThreads) h[i] = 0;
  block_minmax(kmin, kmax, scratch);  // its barriers also order the clearing
  const int shift = range_shift(kmin, kmax);
  for (int base = start; base < end; base += kPass) {
    if (base != start) load_pass(sc, base, end, k);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = base + j * kThreads + threadIdx.x;
      if (i < end) atomicAdd(&h[min((k[j] - kmin) >> shift, (uint32_t)kTopkBins - 1)], 1u);
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

// The need-th largest (1-based) of n <= kRankMax distinct composites in LDS:
// a composite's rank is the number of larger ones.
constexpr int kRankMax = 2 * kThreads;
__device__ uint64_t select_by_rank(const uint64_t* c, int n, uint32_t need, uint64_t* out) {
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const uint64_t x = c[i];
    uint32_t rank = 0;
    for (int j = 0; j < n; ++j) rank += c[j] > x ? 1u : 0u;
    if (rank + 1 == need) *out = x;
  }
  __syncthreads();
  return *out;
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

  // every independent load first: the first pass's keys, the row's range
  // and the finished histogram
  uint32_t k0[kPer];
  load_pass(sc, start, end, k0);
  uint32_t kmin, kmax;
  row_range_load(a, ri.r_local, ri.L, kmin, kmax);
  {
    const uint32_t* gh = a.tw.hist + (int64_t)ri.r_local * kTopkBins;
    uint32_t hv[kTopkBins / kThreads];
#pragma unroll
    for (int j = 0; j < kTopkBins / kThreads; ++j) hv[j] = gh[j * kThreads + threadIdx.x];
#pragma unroll
    for (int j = 0; j < kTopkBins / kThreads; ++j) h[j * kThreads + threadIdx.x] = hv[j];
  }
  block_minmax(kmin, kmax, scratch);  // its barriers also publish h
  const int shift = range_shift(kmin, kmax);
  find_bin(h, (uint32_t)a.K, res, scratch);
  const uint32_t bstar = res[0];
  const uint32_t above = res[1];
  const uint32_t cnt_b = h[bstar];
  const uint32_t lo_b = kmin + (bstar << shift);
  const uint32_t span = (uint32_t)((1ull << shift) - 1);
  const uint32_t hi_b = (kmax - lo_b < span) ? kmax : lo_b + span;
  const int mode = lo_b == hi_b ? kTie : (cnt_b <= (uint32_t)kCandCap ? kCand : kFallback);
  if (s == 0 && threadIdx.x == 0) {  // read by the compact kernel
    st[kMode] = (uint32_t)mode;
    st[kLoB] = lo_b;
    st[kAbove] = above;
  }

  if (mode != kFallback) {
    // One pass of kPass positions per iteration (one, for slices of 2048):
    // all loads are issued before any is used, and a wave reserves its
    // candidate slots with a single atomic for the whole pass.  Everything
    // written here is read by the next kernel, so plain stores suffice.
    uint32_t n_above = 0, n_eq = 0;
    const int lane = threadIdx.x & 63;
    uint64_t* cand = a.tw.cand + (int64_t)ri.r_local * kCandCap;
    for (int base = start; base < end; base += kPass) {
      uint32_t k[kPer];
      bool inb[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) k[j] = k0[j];
      if (base != start) load_pass(sc, base, end, k);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const bool ok = base + j * kThreads + (int)threadIdx.x < end;
        n_above += (ok && k[j] > hi_b) ? 1u : 0u;
        inb[j] = ok && k[j] >= lo_b && k[j] <= hi_b;
        n_eq += inb[j] ? 1u : 0u;
      }
      if (mode == kCand) {
        uint64_t m[kPer];
        uint32_t total = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          m[j] = __ballot(inb[j]);
          total += (uint32_t)__popcll(m[j]);
        }
        if (total != 0) {  // wave-uniform
          uint32_t slot = 0;
          if (lane == 0) slot = atomicAdd(&st[kCandCount], total);
          uint32_t at = (uint32_t)__shfl((int)slot, 0);
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            const uint32_t mine = at + (uint32_t)lane_prefix(m[j]);
            const uint32_t i = (uint32_t)(base + j * kThreads + (int)threadIdx.x);
            if (inb[j] && mine < (uint32_t)kCandCap)
              cand[mine] = ((uint64_t)k[j] << 32) | (0xFFFFFFFFu - i);
            at += (uint32_t)__popcll(m[j]);
          }
        }
      }
    }
    n_above = wave_sum(n_above);
    n_eq = wave_sum(n_eq);
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
      a.tw.s_def[rs + s] = sa;
      a.tw.s_eq[rs + s] = se;
    }
    return;  // the compact kernel finishes the selection
  }

  // ---- fallback (bin b* too full for the candidate buffer): the last
  // workgroup of the row to arrive refines the threshold over the whole row
  // and sets every slice's output offset
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&st[kArrived], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(n_sl - 1);
  __syncthreads();
  if (!last) return;

  uint32_t need = (uint32_t)a.K - above;
  const uint32_t T = select_in_row(sc, ri.L, lo_b, hi_b, need, h, scratch, res);
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
  // output offsets: slices in order, the budget of keys equal to T spent in
  // position order
  if (threadIdx.x == 0) {
    res[2] = 0;
    res[3] = 0;
  }
  __syncthreads();
  for (int c0 = 0; c0 < n_sl; c0 += kThreads) {
    const int j = c0 + threadIdx.x;
    const uint32_t e = j < n_sl ? sel_cnt[j] : 0u;
    uint32_t te;
    const uint32_t eqb = res[3] + block_exclusive_scan(e, scratch, te);
    const uint32_t take = eqb >= need ? 0u : min(e, need - eqb);
    const uint32_t cnt = j < n_sl ? sl_a[j] + take : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan(cnt, scratch, tot);
    if (j < n_sl) {
      a.tw.s_off[rs + j] = res[2] + ex;
      a.tw.s_eqb[rs + j] = eqb;
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
    st[kNeedEq] = need;
  }
}

// -------------------------------------------------------------- 3. compact
// Every workgroup first settles the selection rule for itself -- the
// threshold key T with its position cut P_T or tie budget, and its own first
// output slot -- from the per-slice counts and the candidate list (a few
// dozen composites in the usual case), so no workgroup of the previous
// kernel has to wait for the others:
//   composite mode: C* = the need-th largest candidate; keep key > T, or
//     key == T and position <= P_T; offset = keys above b* in earlier slices
//     + chosen candidates at earlier positions;
//   tie mode: T = the single key of b*; keep key > T, or key == T while
//     fewer than `need` such keys precede it; offset = keys above T in
//     earlier slices + min(need, keys equal to T in earlier slices);
//   fallback: all of it was set by the last workgroup of the cand kernel.
// Positions are then visited kPass at a time, thread t taking positions
// base + j*kThreads + t (j < kPer): every load is coalesced and issued
// before any is used.  Output order is position order, i.e. (j, wave, lane);
// ballots give the order inside a wave and per-wave counts in LDS the order
// across waves.
__global__ __launch_bounds__(kThreads) void topk_compact_kernel(TopkLaunch a) {
  __shared__ uint32_t wcnt[2][kPer][kWaves];  // per pass row and wave: [0] ties, [1] kept
  __shared__ uint64_t cl[kCandCap];
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t scratch[2 * kWaves];
  __shared__ uint32_t res[4];
  __shared__ uint64_t pick;
  __shared__ uint32_t pre[2];
  __shared__ int32_t blk[kPass / 64];  // block ids of the current pass (rowoff only)
  const RowInfo ri = row_info(a);
  const int K = a.K;
  const int s = blockIdx.x;
  int32_t* out = a.indices + (int64_t)ri.r_local * K;
  int64_t* roff = a.rowoff ? a.rowoff + (int64_t)ri.r_local * K : nullptr;
  const int32_t* bt = a.rows.block_table + (int64_t)ri.b * a.rows.max_blocks;
  if (s == 0 && threadIdx.x == 0 && a.counts) a.counts[ri.r_local] = min(K, ri.L);
  if (ri.L <= K) {
    const int a0 = s * a.tw.slice, a1 = min(ri.L, a0 + a.tw.slice);
    for (int j = a0 + threadIdx.x; j < a1; j += kThreads) {
      out[j] = j;
      if (roff) roff[j] = kv_offset(a, j, bt[j >> 6]);
    }
    if (s == 0)
      for (int j = ri.L + threadIdx.x; j < K; j += kThreads) {
        out[j] = -1;
        if (roff) roff[j] = -1;
      }
    return;
  }
  const int start = s * a.tw.slice;
  if (start >= ri.L) return;
  const int end = min(ri.L, start + a.tw.slice);
  const int n_sl = (ri.L + a.tw.slice - 1) / a.tw.slice;
  const float* sc = a.scores + (int64_t)ri.r_local * a.ld;
  const int64_t rs = (int64_t)ri.r_local * a.tw.n_slices;
  const uint32_t* st = a.tw.state + (int64_t)ri.r_local * kStateWords;
  const uint64_t* cand = a.tw.cand + (int64_t)ri.r_local * kCandCap;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // one trip for everything: this slice's first keys, the row state, every
  // slice's counts and the first kThreads candidate slots (read whether
  // filled or not: the slots always exist)
  uint32_t k0[kPer];
  load_pass(sc, start, end, k0);
  // the pass's block ids travel with its keys
  auto load_blocks = [&](int base) {
    if (roff && tid < kPass / 64) {
      const int bi = (base >> 6) + tid;
      blk[tid] = bi <= (end - 1) >> 6 ? bt[bi] : -1;
    }
  };
  load_blocks(start);
  const uint32_t mode = st[kMode];
  const uint32_t n_cand = st[kCandCount];
  static_assert(kThreads == 256, "one slice per thread");
  const uint32_t sd = tid < n_sl ? a.tw.s_def[rs + tid] : 0u;
  const uint32_t se = tid < n_sl ? a.tw.s_eq[rs + tid] : 0u;
  const uint64_t c0 = cand[tid];

  uint32_t T, PT, need_eq, off, eqb;
  if (mode == kFallback) {
    T = st[kT];
    PT = 0x7FFFFFFFu;
    need_eq = st[kNeedEq];
    off = a.tw.s_off[rs + s];
    eqb = a.tw.s_eqb[rs + s];
  } else {
    const uint32_t need = (uint32_t)K - st[kAbove];
    // keys above b* (and, tie mode, keys equal to T) in the slices before s
    uint32_t t1, t2;
    const uint32_t ex_d = block_exclusive_scan(sd, scratch, t1);
    const uint32_t ex_e = block_exclusive_scan(se, scratch, t2);
    if (tid == s) {
      pre[0] = ex_d;
      pre[1] = ex_e;
    }
    __syncthreads();
    if (mode == kTie) {
      T = st[kLoB];
      PT = 0x7FFFFFFFu;
      need_eq = need;
      eqb = pre[1];
      off = pre[0] + min(need, eqb);
    } else {
      const int n = (int)min(n_cand, (uint32_t)kCandCap);
      cl[tid] = c0;
      for (int i = kThreads + tid; i < n; i += kThreads) cl[i] = cand[i];
      __syncthreads();
      const uint64_t cstar = n <= kRankMax ? select_by_rank(cl, n, need, &pick)
                                           : select_composite(cl, n, need, h, scratch, res);
      T = (uint32_t)(cstar >> 32);
      PT = 0xFFFFFFFFu - (uint32_t)cstar;
      need_eq = 0xFFFFFFFFu;
      eqb = 0;
      // chosen candidates at positions before this slice
      uint32_t c = 0;
      for (int i = tid; i < n; i += kThreads)
        c += (cl[i] >= cstar && 0xFFFFFFFFu - (uint32_t)cl[i] < (uint32_t)start) ? 1u : 0u;
      c = wave_sum(c);
      if (lane == 0) scratch[wave] = c;
      __syncthreads();
      uint32_t before = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) before += scratch[w];
      off = pre[0] + before;
    }
  }
  const bool ties = need_eq != 0xFFFFFFFFu;

  for (int base = start; base < end; base += kPass) {
    uint32_t k[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) k[j] = k0[j];
    if (base != start) {
      load_pass(sc, base, end, k);
      load_blocks(base);  // the previous pass's readers are past its final barrier
    }
    uint64_t me[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const bool ok = base + j * kThreads + tid < end;
      me[j] = __ballot(ok && k[j] == T);
    }
    // rank among keys equal to T, in position order (tie modes only)
    uint32_t eq_rank[kPer];
    uint32_t eq_pass = 0;
    if (ties) {
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) wcnt[0][j][wave] = (uint32_t)__popcll(me[j]);
      }
      __syncthreads();
      uint32_t run = eqb;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const uint32_t c = wcnt[0][j][w];
          before += w < wave ? c : 0u;
          all += c;
        }
        eq_rank[j] = run + before + (uint32_t)lane_prefix(me[j]);
        run += all;
      }
      eq_pass = run - eqb;
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) eq_rank[j] = 0;
    }
    uint64_t ms[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t i = (uint32_t)(base + j * kThreads + tid);
      const bool ok = (int)i < end;
      const bool eq = (me[j] >> lane) & 1u;
      ms[j] = __ballot(ok && (k[j] > T || (eq && i <= PT && eq_rank[j] < need_eq)));
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) wcnt[1][j][wave] = (uint32_t)__popcll(ms[j]);
    }
    __syncthreads();
    uint32_t run = off;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      uint32_t before = 0, all = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const uint32_t c = wcnt[1][j][w];
        before += w < wave ? c : 0u;
        all += c;
      }
      const uint32_t at = run + before + (uint32_t)lane_prefix(ms[j]);
      if (((ms[j] >> lane) & 1u) && at < (uint32_t)K) {
        const int i = base + j * kThreads + tid;
        out[at] = i;
        if (roff) roff[at] = kv_offset(a, i, blk[(i - base) >> 6]);
      }
      run += all;
    }
    off = run;
    eqb += eq_pass;
    __syncthreads();  // wcnt is rewritten by the next pass
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
  int64_t slice = kPass;
  while ((max_len + slice - 1) / slice > 256) slice += kPass;
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
