// Index scores on gfx950: an FP8 MFMA contraction of the row's indexer query
// against every historical index key, with the ReLU gate and the head-weighted
// reduction fused into the epilogue.
//
// Method: Baidu AI Cloud, "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (score all historical
// positions, aggregate with head weights) and section 4.1 (read the paged K
// cache directly, no intermediate per-head score matrix in memory).
//
// Mapping.  One v_mfma_f32_32x32x64_f8f6f4 multiplies 32 indexer heads (M)
// by 32 positions (N) over 64 dims (K).  Heads sit on M so each lane's 16
// accumulator registers hold 16 heads of ONE position: the gate and the
// weighting are per-lane FMAs, and only one cross-lane add (the two 32-lane
// halves) finishes the head sum.  The K dimension is split over the two lane
// halves identically for the query (A) and the key (B) operands, so each lane
// loads one contiguous run of 32 * D_I / 64 bytes of its position's key row.
//
// Work split.  A workgroup (4 waves) owns a tile of kTile consecutive
// positions of one row; each wave walks 32-position sub-tiles of it with a
// one-deep register prefetch of the next sub-tile's keys.  A 32-position
// sub-tile never straddles a 64-row page, so one block-table lookup serves
// the whole wave.

#include "dsa_common.h"

namespace dsa {
namespace {

constexpr int kTile = 1024;    // positions per workgroup
constexpr int kWaves = 4;
constexpr int kSub = 32;       // positions per MFMA column block

template <int NKS>
struct KeyFrag {
  v8i k[NKS];
};

// Loads this lane's part of a key row: 32*NKS bytes at byte offset
// half*32*NKS of the row (zeros when the position is past the history or the
// page is absent).
template <int NKS>
__device__ __forceinline__ KeyFrag<NKS> load_keys(const uint8_t* row, bool ok) {
  KeyFrag<NKS> f;
  if (ok) {
    const v4i* src = reinterpret_cast<const v4i*>(row);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const v4i lo = __builtin_nontemporal_load(src + 2 * ks);
      const v4i hi = __builtin_nontemporal_load(src + 2 * ks + 1);
      f.k[ks] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) f.k[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  }
  return f;
}

// NKS = D_I / 64 K-steps; HT = 32-head tiles (ceil(H_I / 32)).
template <int NKS, int HT>
__global__ __launch_bounds__(256) void indexer_scan_kernel(IndexerLaunch a) {
  const int r = a.row_begin + (int)blockIdx.y;
  int b, p;
  if (!resolve_row(a.rows, r, b, p)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) report(a.err, DSA_DEVERR_ROW);
    return;
  }
  const int L = p + 1;
  const int tile0 = (int)blockIdx.x * kTile;
  if (tile0 >= L) return;
  const int tile_end = min(L, tile0 + kTile);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;   // head row of A, position column of B
  const int half = lane >> 5;  // which half of each 64-dim K step this lane holds
  constexpr int kRowBytes = 64 * NKS;
  constexpr int kLaneBytes = 32 * NKS;

  // A operands: the indexer query of heads ht*32 + col.
  v8i aq[HT][NKS];
  const uint8_t* qrow = a.qI + (int64_t)r * a.H_I * kRowBytes;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = ht * 32 + col;
    KeyFrag<NKS> f = load_keys<NKS>(qrow + (int64_t)head * kRowBytes + half * kLaneBytes,
                                    head < a.H_I);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) aq[ht][ks] = f.k[ks];
  }
  // Head weights of the 16 accumulator rows this lane holds:
  // register v of a 32x32 tile is row 8*(v/4) + 4*half + v%4.
  float wr[HT][16];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int head = ht * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      wr[ht][v] = head < a.H_I ? a.w[(int64_t)r * a.H_I + head] : 0.0f;
    }

  const int32_t* bt = a.rows.block_table + (int64_t)b * a.rows.max_blocks;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.kI.base);
  float* out = a.scores + (int64_t)(r - a.row_begin) * a.ld;

  auto key_row = [&](int s0, bool& page_ok) -> const uint8_t* {
    const int phys = bt[s0 >> 6];
    page_ok = phys >= 0 && (int64_t)phys < a.kI.num_blocks;
    return kbase + (int64_t)(page_ok ? phys : 0) * a.kI.block_stride +
           (int64_t)((s0 + col) & 63) * a.kI.row_stride + half * kLaneBytes;
  };

  int s0 = tile0 + wave * kSub;
  if (s0 >= tile_end) return;
  bool ok_cur;
  const uint8_t* row_cur = key_row(s0, ok_cur);
  KeyFrag<NKS> cur = load_keys<NKS>(row_cur, ok_cur && s0 + col < L);
  bool page_cur = ok_cur;

  while (true) {
    const int s1 = s0 + kWaves * kSub;
    KeyFrag<NKS> nxt;
    bool page_nxt = false;
    if (s1 < tile_end) {
      const uint8_t* row_nxt = key_row(s1, page_nxt);
      nxt = load_keys<NKS>(row_nxt, page_nxt && s1 + col < L);
    }

    float part = 0.0f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      v16f acc = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aq[ht][ks], cur.k[ks], acc,
                                                              0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 16; ++v) part += wr[ht][v] * fmaxf(acc[v], 0.0f);
    }
    part += __shfl_xor(part, 32);
    const int s = s0 + col;
    if (half == 0 && s < L) {
      // canonical +0 for a zero score; an absent page scores -inf
      out[s] = page_cur ? part + 0.0f : -__builtin_inff();
    }
    if (!page_cur && lane == 0) report(a.err, DSA_DEVERR_BLOCK);

    if (s1 >= tile_end) break;
    s0 = s1;
    cur = nxt;
    page_cur = page_nxt;
  }
}

template <int NKS, int HT>
hipError_t launch_t(const IndexerLaunch& a, hipStream_t s) {
  dim3 grid((a.max_len + kTile - 1) / kTile, a.num_rows);
  indexer_scan_kernel<NKS, HT><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerLaunch& a, hipStream_t s) {
  if (a.num_rows <= 0 || a.max_len <= 0) return hipSuccess;
  const bool two = a.H_I > 32;
  if (a.D_I == 128) return two ? launch_t<2, 2>(a, s) : launch_t<2, 1>(a, s);
  return two ? launch_t<1, 2>(a, s) : launch_t<1, 1>(a, s);
}

}  // namespace dsa
