// Per-row Top-K on gfx950: an exact radix-style select of the K-th largest
// score key followed by an ordered compaction with wave ballots.
//
// Method: Baidu AI Cloud, "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (keep the Top-K most
// relevant historical positions).  Readings: ties go to the lower position,
// the kept positions are written in ascending order, -1 pads to K.
//
// One 1024-thread workgroup owns one row.
//  1. Key range: min and max of the order-preserving 32-bit keys.
//  2. Select: repeatedly histogram the keys inside the live range [lo, hi]
//     into 2048 bins laid linearly over that range, and keep the bin that
//     holds the K-th largest key.  Bins over the live range (not over fixed
//     key bits) keep the histogram spread out even when the scores crowd
//     into a few binades, which keeps LDS atomic conflicts low.  As soon as
//     the kept bin holds at most kCap keys they are copied once into LDS and
//     the remaining passes run there.  The loop ends when lo == hi: that key
//     T is the threshold, with `take` of the keys equal to T still needed.
//  3. Compaction: each wave owns a contiguous segment of positions; a count
//     pass (ballots) gives every wave its output offset and how many of the
//     keys equal to T precede it, then a write pass emits the kept positions
//     in ascending order.

#include "dsa_common.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kCap = 4096;

struct Shared {
  uint32_t hist[kBins];
  uint32_t cand_key[kCap];
  uint32_t wave_a[kWaves];
  uint32_t wave_b[kWaves];
  uint32_t wave_scan[kWaves];
  uint32_t bstar, above, ncand;
};

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}

// Inclusive prefix sum over the workgroup's 1024 threads.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t x, Shared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = (uint32_t)__shfl_up((int)x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wave_scan[wave] = x;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < wave; ++i) before += sh.wave_scan[i];
  __syncthreads();
  return x + before;
}

// Bin of key k in the live range [lo, lo + width - 1] split into kBins bins.
__device__ __forceinline__ uint32_t bin_of(uint32_t k, uint32_t lo, uint64_t width) {
  return (uint32_t)(((uint64_t)(k - lo) * kBins) / width);
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkLaunch a) {
  __shared__ Shared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.row_begin + (int)blockIdx.x;
  int b, p;
  int L = 0;
  if (resolve_row(a.rows, r, b, p)) {
    L = p + 1;
  } else if (tid == 0) {
    report(a.err, DSA_DEVERR_ROW);
  }
  const int K = a.K;
  int32_t* out = a.indices + (int64_t)(r - a.row_begin) * K;
  if (tid == 0 && a.counts) a.counts[r - a.row_begin] = min(K, L);
  if (L <= K) {
    for (int j = tid; j < K; j += kThreads) out[j] = j < L ? j : -1;
    return;
  }
  const float* sc = a.scores + (a.scores_row_offset + (int64_t)(r - a.row_begin)) * a.ld;

  // ---- 1. key range
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int i = tid; i < L; i += kThreads) {
    const uint32_t k = score_key(sc[i]);
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if (lane == 0) {
    sh.wave_a[wave] = kmin;
    sh.wave_b[wave] = kmax;
  }
  __syncthreads();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = 0; i < kWaves; ++i) {
    lo = min(lo, sh.wave_a[i]);
    hi = max(hi, sh.wave_b[i]);
  }
  __syncthreads();

  // ---- 2. select the threshold key
  uint32_t need = (uint32_t)K;  // keys still to take from inside [lo, hi]
  bool in_lds = false;
  uint32_t ncand = 0;
  while (lo < hi) {
    const uint64_t width = (uint64_t)hi - lo + 1;
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    if (in_lds) {
      for (uint32_t i = tid; i < ncand; i += kThreads) {
        const uint32_t k = sh.cand_key[i];
        if (k >= lo && k <= hi) atomicAdd(&sh.hist[bin_of(k, lo, width)], 1u);
      }
    } else {
      for (int i = tid; i < L; i += kThreads) {
        const uint32_t k = score_key(sc[i]);
        if (k >= lo && k <= hi) atomicAdd(&sh.hist[bin_of(k, lo, width)], 1u);
      }
    }
    __syncthreads();
    // suffix sums: thread t owns bins 2047-2t (higher) and 2046-2t
    const int bh = kBins - 1 - 2 * tid, bl = bh - 1;
    const uint32_t ch = sh.hist[bh], cl = sh.hist[bl];
    const uint32_t incl = block_inclusive_scan(ch + cl, sh);
    const uint32_t above_h = incl - ch - cl;  // keys in bins > bh
    if (above_h < need && need <= above_h + ch) {
      sh.bstar = bh;
      sh.above = above_h;
    } else if (above_h + ch < need && need <= above_h + ch + cl) {
      sh.bstar = bl;
      sh.above = above_h + ch;
    }
    __syncthreads();
    const uint32_t bs = sh.bstar;
    need -= sh.above;
    const uint32_t count_bs = sh.hist[bs];
    const uint32_t nlo = lo + (uint32_t)(((uint64_t)bs * width + kBins - 1) / kBins);
    const uint32_t nhi = lo + (uint32_t)((((uint64_t)bs + 1) * width + kBins - 1) / kBins) - 1;
    lo = nlo;
    hi = nhi;
    __syncthreads();
    if (!in_lds && lo < hi && count_bs <= kCap) {
      // copy the live keys into LDS once; later passes read them there
      if (tid == 0) sh.ncand = 0;
      __syncthreads();
      for (int base = 0; base < L; base += kThreads) {
        const int i = base + tid;
        uint32_t k = 0;
        bool live = false;
        if (i < L) {
          k = score_key(sc[i]);
          live = k >= lo && k <= hi;
        }
        const uint64_t m = __ballot(live);
        uint32_t slot = 0;
        if (lane == 0 && m) slot = atomicAdd(&sh.ncand, (uint32_t)__popcll(m));
        slot = (uint32_t)__shfl((int)slot, 0);
        const uint32_t at = slot + (uint32_t)lane_prefix(m);
        if (live && at < (uint32_t)kCap) sh.cand_key[at] = k;
      }
      __syncthreads();
      ncand = min(sh.ncand, (uint32_t)kCap);
      in_lds = true;
    }
  }
  const uint32_t T = lo;
  const uint32_t take = need;  // keys equal to T to keep, lowest positions first

  // ---- 3. ordered compaction
  const int seg = ((L + kWaves - 1) / kWaves + 63) & ~63;
  const int s_begin = min(L, wave * seg), s_end = min(L, s_begin + seg);
  uint32_t n_gt = 0, n_eq = 0;
  for (int base = s_begin; base < s_end; base += 64) {
    const int i = base + lane;
    const uint32_t k = i < s_end ? score_key(sc[i]) : 0u;
    const bool valid = i < s_end;
    n_gt += (uint32_t)__popcll(__ballot(valid && k > T));
    n_eq += (uint32_t)__popcll(__ballot(valid && k == T));
  }
  if (lane == 0) {
    sh.wave_a[wave] = n_gt;
    sh.wave_b[wave] = n_eq;
  }
  __syncthreads();
  uint32_t eq_before = 0, off = 0;
  for (int w = 0; w < wave; ++w) {
    const uint32_t eq_w = sh.wave_b[w];
    const uint32_t took = eq_before >= take ? 0u : min(eq_w, take - eq_before);
    off += sh.wave_a[w] + took;
    eq_before += eq_w;
  }
  uint32_t eq_seen = eq_before;
  for (int base = s_begin; base < s_end; base += 64) {
    const int i = base + lane;
    const bool valid = i < s_end;
    const uint32_t k = valid ? score_key(sc[i]) : 0u;
    const bool eq = valid && k == T;
    const uint64_t meq = __ballot(eq);
    const bool sel = (valid && k > T) || (eq && eq_seen + (uint32_t)lane_prefix(meq) < take);
    const uint64_t msel = __ballot(sel);
    const uint32_t at = off + (uint32_t)lane_prefix(msel);
    if (sel && at < (uint32_t)K) out[at] = i;
    off += (uint32_t)__popcll(msel);
    eq_seen += (uint32_t)__popcll(meq);
  }
}

}  // namespace

hipError_t launch_topk(const TopkLaunch& a, hipStream_t s) {
  if (a.num_rows <= 0) return hipSuccess;
  topk_kernel<<<a.num_rows, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
