// Per-row Top-K on gfx950: one workgroup of 1024 threads per row.
//
// Method: Baidu AI Cloud, "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (keep the Top-K most
// relevant historical positions).  Readings: ties go to the lower position,
// the kept positions are written in ascending order, -1 pads to K.
//
// Scores are compared through an order-preserving 32-bit key (score_key);
// the selection is exact.  A row's history is cut into groups of G
// consecutive positions (topk_group: a power of two up to 8 that leaves at
// least 2K groups), and the maximum key of every group is known before this
// kernel runs -- the fused indexer writes it in its epilogue; the standalone
// entry point runs topk_group_max_kernel first.
//
//  1. A lower bound t on the row's K-th largest key T: one 2048-bin histogram
//     of the group maxima over their range, and t = the lower edge of the bin
//     that holds the K-th largest maximum.  At least K groups have a maximum
//     >= t, so at least K keys are >= t and T >= t; every kept position lies
//     in a group whose maximum is >= t (a candidate group).  Without heavy
//     ties there are about K candidate groups holding some 1.1-1.4 K keys
//     >= t.
//  2. The candidate groups' keys are loaded and those >= t are compacted, in
//     position order, into LDS with their positions.
//  3. T is selected exactly among them, together with the number of keys
//     equal to T that are kept (the first ones in position order).
//  4. The kept positions are written in ascending order: block-wide prefix
//     sums over the compacted list, staged in LDS, then stored in one
//     coalesced pass (with the KV row offsets, from a copy of the row's block
//     table in LDS).
//
// With G = 1 the keys themselves are loaded and step 3 runs on them
// directly.  Rows with L <= K keep every position.  A row that does not fit
// these buffers (K > 2048, more than 16384 groups, more than 4096 candidate
// groups or 8192 keys >= t because of ties, or t = 0 because of NaN scores)
// runs the same selection over its keys streamed from memory.
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
constexpr int kPerThread = 16;            // group maxima (or keys) per thread
constexpr int kMaxN = kPerThread * kT;    // 16384
constexpr int kCandPer = 4;               // candidate groups per thread
constexpr int kMaxCand = kCandPer * kT;   // 4096
constexpr int kKeysPer = 8;               // compacted keys per thread
constexpr int kMaxKeys = kKeysPer * kT;   // 8192
constexpr int kBtCache = 2048;            // block-table entries cached in LDS
constexpr int kScanWords = 4 * kWaves + 1;
constexpr int kSegRead = kT / kTopkSlices;  // threads reading one slice's candidates (64)
static_assert(kSegRead * kKeysPer * kTopkSlices == kMaxKeys, "slice-major candidate layout");
static_assert(kBins == 2 * kT, "find_bin gives each thread two bins");

struct Smem {
  uint32_t hist[kBins];    // histograms; afterwards slot -> kept position
  uint32_t list[kMaxCand]; // candidate group ids, in position order
  uint32_t ck[kMaxKeys];   // compacted keys >= t, in position order
  int32_t cp[kMaxKeys];    // and their positions
  int32_t bt[kBtCache];    // the row's block table (rows of <= 2048 blocks)
  uint32_t buf[kSmall];
  uint32_t res[4];
  uint32_t wsum[kScanWords];
  uint32_t red[2 * kWaves];
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

// Exclusive prefix sum over the block in thread order; `tot` receives the
// total.  Starts and ends with a barrier, so `wsum` may be reused at once.
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t* wsum, uint32_t& tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_scan(x, 0u, Add());
  __syncthreads();
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const uint32_t v = lane < kWaves ? wsum[lane] : 0u;
    const uint32_t c = wave_scan(v, 0u, Add());
    if (lane < kWaves) wsum[lane] = c - v;
    if (lane == 63) wsum[kWaves] = c;
  }
  __syncthreads();
  const uint32_t ex = wsum[wave] + inc - x;
  tot = wsum[kWaves];
  __syncthreads();
  return ex;
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

// Min and max over the block (results in every thread).
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* red) {
  mn = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(mn, 0xFFFFFFFFu, Min()), 63);
  mx = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(mx, 0u, Max()), 63);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    red[wave] = mn;
    red[kWaves + wave] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mn = min(mn, red[w]);
    mx = max(mx, red[kWaves + w]);
  }
}

// Over the 2048-bin histogram h, the bin b with above(b) < need <=
// above(b) + h[b], where above(b) counts the keys in bins above b; thread t
// owns bins 2047 - 2t and 2046 - 2t.  Results: res[0] = b, res[1] = above(b).
// Requires 1 <= need <= sum of h.  Ends with a barrier.
__device__ __forceinline__ void find_bin(const uint32_t* h, uint32_t need, uint32_t* res,
                                         uint32_t* wsum) {
  const int top = kBins - 1 - 2 * (int)threadIdx.x;
  const uint32_t c0 = h[top], c1 = h[top - 1];
  uint32_t tot;
  const uint32_t above = block_scan(c0 + c1, wsum, tot);
  if (above < need && need <= above + c0) {
    res[0] = (uint32_t)top;
    res[1] = above;
  } else if (above + c0 < need && need <= above + c0 + c1) {
    res[0] = (uint32_t)(top - 1);
    res[1] = above + c0;
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
    __syncthreads();  // hist and res are rewritten below
    if (lo < hi && cnt <= (uint32_t)kSmall) {
      // rank the bin's keys directly: wave 0, one key per lane
      if (tid == 0) s.res[2] = 0;
      __syncthreads();
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
      p[i] = slot < K ? (int)pos[slot] : 0;
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
// earlier runs and are advanced past this one.
template <int N, bool kStaged, class Pos>
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
  const uint32_t ex = block_scan((eq << 16) | gt, s.wsum, tot);
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

// Steps 2-4 for groups of G positions.  The candidate groups' keys are
// loaded in pieces of P = G/4 (at least 1) float4 or float2 loads, lane-
// adjacent within a group so that one cache line serves its pieces: piece q
// of list entry e is taken by thread (e P + q) mod 1024 in round
// (e P + q) / 1024.  The keys >= t are compacted in (round, thread) order,
// which is position order.  Returns false, having written nothing, when
// more than kMaxKeys keys are >= t.
template <int G>
__device__ __forceinline__ bool select_groups(const float* sc, int L, int K, uint32_t t,
                                              uint32_t kmax, uint32_t n_cg, bool vec,
                                              const Out& o, Smem& s) {
  constexpr int W = G < 4 ? G : 4;      // keys per piece
  constexpr int P = G / W;              // pieces per group
  constexpr int R = kCandPer * P;       // rounds (pieces per thread)
  const int tid = threadIdx.x;
  uint32_t n_c;
  {
    int base[R];  // first position of the piece, L: none
#pragma unroll
    for (int m = 0; m < R; ++m) {
      const uint32_t q = (uint32_t)(m * kT + tid);
      const uint32_t e = q / P;
      base[m] = e < n_cg ? (int)s.list[e] * G + (int)(q % P) * W : L;
    }
    uint32_t k[R][W];
#pragma unroll
    for (int m = 0; m < R; ++m) load_keys<W>(sc, base[m], L, vec, k[m]);
    uint32_t c[R], at[R];
#pragma unroll
    for (int m = 0; m < R; ++m) {
      c[m] = 0;
#pragma unroll
      for (int j = 0; j < W; ++j) c[m] += k[m][j] >= t ? 1u : 0u;  // t >= 1: absent keys never count
    }
    static_assert(R <= 8, "rounds");
    if constexpr (R <= 4) {
      n_c = block_scan_n<R>(c, at, s.wsum);
    } else {  // two scans of four rounds
      uint32_t c0[4], c1[4], a0[4], a1[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        c0[m] = c[m];
        c1[m] = c[m + 4];
      }
      const uint32_t n0 = block_scan_n<4>(c0, a0, s.wsum);
      n_c = n0 + block_scan_n<4>(c1, a1, s.wsum);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        at[m] = a0[m];
        at[m + 4] = n0 + a1[m];
      }
    }
    if (n_c > (uint32_t)kMaxKeys) return false;
#pragma unroll
    for (int m = 0; m < R; ++m)
#pragma unroll
      for (int j = 0; j < W; ++j)
        if (k[m][j] >= t) {
          s.ck[at[m]] = k[m][j];
          s.cp[at[m]] = base[m] + j;
          ++at[m];
        }
  }
  __syncthreads();
  const int c0 = kKeysPer * tid;
  const int n = max(0, min(kKeysPer, (int)n_c - c0));
  uint32_t k[kKeysPer];
#pragma unroll
  for (int j = 0; j < kKeysPer; ++j) k[j] = j < n ? s.ck[c0 + j] : 0u;
  auto visit = [&](auto f) {
#pragma unroll
    for (int j = 0; j < kKeysPer; ++j)
      if (j < n) f(k[j]);
  };
  uint32_t need = (uint32_t)K;
  const uint32_t T = select_kth(visit, t, kmax, need, s);
  uint32_t eq_before = 0, out_before = 0;
  emit_runs<kKeysPer, true>(k, n, [&](int j) { return s.cp[c0 + j]; }, T, need, eq_before,
                            out_before, o, s);
  return true;
}

// Steps 1-4.  `gm` holds the thread's group maxima 16t .. 16t+15 (loaded
// before the row was resolved).  Returns false, having written nothing, when
// the row needs the streamed path.
__device__ __forceinline__ bool select_fast(const float* sc, int L, int K, bool vec,
                                            uint32_t (&gm)[kPerThread], const Out& o, Smem& s) {
  const int tid = threadIdx.x;
  const int G = topk_group(L, K);
  const int N = (L + G - 1) / G;
  if (N > kMaxN) return false;
  const int g0 = kPerThread * tid;
  if (G == 1) load_keys<kPerThread>(sc, g0, L, vec, gm);
  const int n_mine = max(0, min(kPerThread, N - g0));
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (j < n_mine) {
      kmin = min(kmin, gm[j]);
      kmax = max(kmax, gm[j]);
    }
  block_minmax(kmin, kmax, s.red);
  auto visit = [&](auto f) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (j < n_mine) f(gm[j]);
  };

  if (G == 1) {  // the keys themselves: select T and emit
    uint32_t need = (uint32_t)K;
    const uint32_t T = select_kth(visit, kmin, kmax, need, s);
    uint32_t eq_before = 0, out_before = 0;
    emit_runs<kPerThread, true>(gm, n_mine, [&](int j) { return g0 + j; }, T, need, eq_before,
                                out_before, o, s);
    return true;
  }

  // 1. t = lower edge of the bin holding the K-th largest group maximum
  uint32_t t = kmin;
  if (kmin < kmax) {
    const int shift = range_shift(kmin, kmax);
    histogram_bin(visit, kmin, kmax, shift, (uint32_t)K, s);
    t = kmin + (s.res[0] << shift);
  }
  // candidate groups: maxima >= t, listed in position order
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) c += (j < n_mine && gm[j] >= t) ? 1u : 0u;
  uint32_t n_cg;
  uint32_t at = block_scan(c, s.wsum, n_cg);
  // heavy ties at t, or t = 0 (NaN scores at the threshold)
  if (n_cg > (uint32_t)kMaxCand || t == 0) return false;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (j < n_mine && gm[j] >= t) s.list[at++] = (uint32_t)(g0 + j);
  __syncthreads();
  switch (G) {
    case 2: return select_groups<2>(sc, L, K, t, kmax, n_cg, vec, o, s);
    case 4: return select_groups<4>(sc, L, K, t, kmax, n_cg, vec, o, s);
    default: return select_groups<kMaxGroup>(sc, L, K, t, kmax, n_cg, vec, o, s);
  }
}

// This thread's share of a row's group maxima, 16t .. 16t+15, whatever the
// row's length turns out to be.  The loads are unconditional 16-byte ones
// (no branch, so nothing waits for them before they are used): the work
// area is padded so that kMaxN entries from any row's start are readable;
// entries past the row's groups hold other rows' or padding values and are
// never used.
__device__ __forceinline__ void load_gmax(const TopkLaunch& a, int r_local,
                                          uint32_t (&gm)[kPerThread]) {
  const uint32_t* src = a.tw.gmax + (int64_t)r_local * a.tw.gstride + kPerThread * threadIdx.x;
#pragma unroll
  for (int j = 0; j < kPerThread; j += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + j);
    gm[j] = v.x;
    gm[j + 1] = v.y;
    gm[j + 2] = v.z;
    gm[j + 3] = v.w;
  }
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

// A whole row in one workgroup: every path but the split one.
__device__ __forceinline__ void row_single(const TopkLaunch& a, int r_local, int L,
                                           uint32_t (&gm)[kPerThread], Out& o, Smem& s) {
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
  cache_block_table(L, o, s);
  o.pos = s.hist;
  if (!(K <= kMaxCand - kT && select_fast(sc, L, K, a.vec, gm, o, s)))
    select_streamed<true>(sc, L, K, a.vec, o, s);
  __syncthreads();
  o.flush(K);
}

// ---------------------------------------------------------- split rows
// A row whose group maxima are known is spread over up to kTopkSlices
// workgroups, one per slice of kTopkSliceGroups groups:
//  a. every workgroup computes t from all the row's group maxima (the same
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

// The G scores of group g as raw bits (positions past L as 0); converted to
// keys only once they are needed, so nothing waits for them earlier.
template <int G>
__device__ __forceinline__ void group_scores(const float* sc, int g, int L, bool vec,
                                             uint32_t (&x)[kMaxGroup]) {
  const int i0 = g * G;
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) x[j] = 0u;
  if (vec && G >= 4 && i0 + G <= L) {
#pragma unroll
    for (int j = 0; j < G; j += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(sc + i0 + j);
      x[j] = v.x;
      x[j + 1] = v.y;
      x[j + 2] = v.z;
      x[j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < G; ++j) x[j] = i0 + j < L ? __float_as_uint(sc[i0 + j]) : 0u;
  }
}

__global__ __launch_bounds__(kT) void topk_split_kernel(TopkLaunch a) {
  __shared__ Smem s;
  const int tid = threadIdx.x;
  const int slice = (int)blockIdx.x;
  const int r_local = (int)blockIdx.y;
  const int K = a.K;
  // one round trip: the row's length, then its group maxima
  const RowIssue ri = row_issue(a.rows, a.row_begin + r_local);
  uint32_t gm[kPerThread];
  load_gmax(a, r_local, gm);
  const int L = row_finish(a.rows, ri);
  Out o = make_out(a, r_local, ri.b_ok ? ri.b : 0);
  const int G = L > 0 ? topk_group(L, K) : 1;
  const int N = (L + G - 1) / G;
  if (!(L > K && G > 1 && K <= kBins && K <= kMaxCand - kT && N <= kMaxN)) {
    if (slice == 0) row_single(a, r_local, L, gm, o, s);
    return;
  }
  const int S = (N + kTopkSliceGroups - 1) / kTopkSliceGroups;
  if (slice >= S) return;

  // this thread's group of the slice: its keys, loaded now, used after t
  const float* sc = a.scores + (int64_t)r_local * a.ld;
  const int g = slice * kTopkSliceGroups + tid;
  uint32_t k[kMaxGroup];
  switch (G) {
    case 2: group_scores<2>(sc, g, L, a.vec, k); break;
    case 4: group_scores<4>(sc, g, L, a.vec, k); break;
    default: group_scores<kMaxGroup>(sc, g, L, a.vec, k); break;
  }
  const int n_valid = max(0, min(G, L - g * G));
  for (int i = tid; i < kBins; i += kT) s.hist[i] = 0;  // for step a; block_minmax syncs
  if (slice == 0 && tid == 0 && a.counts) a.counts[r_local] = K;
  // the row's block ids for the KV row offsets: loaded now, staged in LDS
  // only by the workgroup that writes the row out
  constexpr int kBtPer = kBtCache / kT;
  const int nblk = (L + kBlock - 1) / kBlock;
  const bool bt_cached = o.roff && nblk <= kBtCache;
  int32_t btv[kBtPer];
#pragma unroll
  for (int j = 0; j < kBtPer; ++j) {
    const int i = tid + j * kT;
    btv[j] = bt_cached && i < nblk ? o.bt[i] : 0;
  }

  // a. t = lower edge of the bin holding the K-th largest group maximum
  const int g0 = kPerThread * tid;
  const int n_mine = max(0, min(kPerThread, N - g0));
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (j < n_mine) {
      kmin = min(kmin, gm[j]);
      kmax = max(kmax, gm[j]);
    }
  block_minmax(kmin, kmax, s.red);
  uint32_t t = kmin;
  if (kmin < kmax) {
    auto visit = [&](auto f) {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j)
        if (j < n_mine) f(gm[j]);
    };
    const int shift = range_shift(kmin, kmax);
    histogram_bin<true>(visit, kmin, kmax, shift, (uint32_t)K, s);
    t = kmin + (s.res[0] << shift);
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
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) k[j] = j < n_valid ? score_key(__uint_as_float(k[j])) : 0u;
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) c += (j < G && k[j] >= t) ? 1u : 0u;
  uint32_t n_slice;
  uint32_t at = block_scan(c, s.wsum, n_slice);
  {
    const int64_t seg = (int64_t)r_local * a.tw.cstride + (int64_t)slice * kTopkSliceGroups * G;
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j)
      if (j < G && k[j] >= t) {
        store_shared(a.tw.ckey + seg + at, k[j]);
        store_shared(reinterpret_cast<uint32_t*>(a.tw.cpos) + seg + at, (uint32_t)(g * G + j));
        if (at < (uint32_t)kMaxKeys) s.cp[at] = g * G + j;  // for the KV prefetch
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
  // Thread t reads entries 8 (t mod 64) .. +7 of slice t / 64 together with
  // the counts (no round trip between them); in thread order that is
  // position order.  A slice with more than 512 candidates sends the row
  // to the general path.
  const int my_slice = tid / kSegRead;
  const int e0 = kKeysPer * (tid % kSegRead);
  const int64_t seg = (int64_t)r_local * a.tw.cstride + (int64_t)my_slice * kTopkSliceGroups * G;
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
  uint32_t cnt[kTopkSlices];
  uint32_t n_tot = 0, c_max = 0;
#pragma unroll
  for (int j = 0; j < kTopkSlices; ++j) {
    cnt[j] = j < S ? a.tw.ccount[r_local * kTopkSlices + j] : 0u;
    n_tot += cnt[j];
    c_max = max(c_max, cnt[j]);
  }
  if (n_tot > (uint32_t)kMaxKeys || c_max > (uint32_t)(kSegRead * kKeysPer)) {
    // heavy ties at t: the general path
    select_streamed<true>(sc, L, K, a.vec, o, s);
  } else {
    uint32_t c_mine = 0;
#pragma unroll
    for (int j = 0; j < kTopkSlices; ++j) c_mine = j == my_slice ? cnt[j] : c_mine;
    const int n = max(0, min(kKeysPer, (int)c_mine - e0));
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
    uint32_t eq_before = 0, out_before = 0;
    emit_runs<kKeysPer, true>(kk, n, [&](int j) { return pp[j]; }, T, need, eq_before,
                              out_before, o, s);
  }
  __syncthreads();
  o.flush(K);
  if (tid == 0) a.tw.arrive[r_local] = 0;
}

// Group maxima for a standalone Top-K call: thread -> one group of its row.
__global__ __launch_bounds__(256) void topk_group_max_kernel(TopkLaunch a) {
  int b, p;
  const int r_local = (int)blockIdx.y;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.tw.arrive[r_local] = 0;
  if (!resolve_row(a.rows, a.row_begin + r_local, b, p)) return;
  const int L = p + 1;
  if (L <= a.K) return;
  const int G = topk_group(L, a.K);
  if (G == 1) return;
  const int g = (int)(blockIdx.x * 256 + threadIdx.x);
  const int N = (L + G - 1) / G;
  if (g >= N) return;
  const float* sc = a.scores + (int64_t)r_local * a.ld + (int64_t)g * G;
  const int n = min(G, L - g * G);
  uint32_t m = 0;
  for (int j = 0; j < n; ++j) m = max(m, score_key(sc[j]));
  a.tw.gmax[(int64_t)r_local * a.tw.gstride + g] = m;
}

}  // namespace

namespace {
int64_t cstride_of(int64_t max_len) { return (max_len + 63) & ~int64_t(63); }
}  // namespace

size_t topk_work_bytes(int rows, int64_t max_len) {
  if (rows <= 0) return 0;
  const size_t words = (size_t)topk_gstride(max_len) + 2 * (size_t)cstride_of(max_len) +
                       kTopkSlices + 1;
  return ((size_t)rows * words + kMaxN) * sizeof(uint32_t);  // + load_gmax's padding
}

TopkWork topk_work_carve(void* base, int rows, int64_t max_len) {
  TopkWork w;
  uint32_t* p = static_cast<uint32_t*>(base);
  w.gstride = topk_gstride(max_len);
  w.cstride = cstride_of(max_len);
  w.gmax = p;
  p += (size_t)rows * w.gstride + kMaxN;  // load_gmax reads up to kMaxN past a row's start
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
  if (a.prep && a.max_len > 2 * a.K) {  // some row may group its positions
    const int64_t groups = (a.max_len + 1) / 2;
    topk_group_max_kernel<<<dim3((unsigned)((groups + 255) / 256), a.num_rows), 256, 0, s>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  topk_split_kernel<<<dim3(kTopkSlices, a.num_rows), kT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
