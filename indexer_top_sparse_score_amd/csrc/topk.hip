// Per-row Top-K on gfx950 for the standalone entry point: a summary pass
// over the score rows (the same per-segment summaries the fused indexer
// writes in its epilogue), then one workgroup per row runs the exact
// selection of topk_select.h and writes the row's indices.
//
// Method: Baidu AI Cloud, "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (keep the Top-K most
// relevant historical positions).  Readings: ties go to the lower position,
// the kept positions are written in ascending order, -1 pads to K.

#include "topk_select.h"

namespace dsa {
namespace {

#ifndef DSA_TOPK_THREADS
#define DSA_TOPK_THREADS 1024
#endif
constexpr int kNT = DSA_TOPK_THREADS;  // threads of a selecting workgroup
constexpr int kBtCache = 2048;  // block-table entries cached in LDS

// One wave per 128 slots of a summary row writes that span's summary entries.
__global__ __launch_bounds__(256) void topk_summary_kernel(TopkLaunch a) {
  const int r_local = (int)blockIdx.y;
  const RowIssue ri = row_issue(a.rows, a.row_begin + r_local);
  const int Lh = row_finish(a.rows, ri);
  const int L = row_slots(a.rows, ri, Lh);
  if (!sum_row(L, a.K)) return;
  const int lane = (int)(threadIdx.x & 63);
  const int w0 = ((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * 128;
  if (w0 >= L) return;
  const float* sc = a.scores + (int64_t)r_local * a.ld;
  const uint32_t ka = w0 + lane < L ? score_key(sc[w0 + lane]) : 0u;
  const uint32_t kb = w0 + 64 + lane < L ? score_key(sc[w0 + 64 + lane]) : 0u;
  const int G = sum_seg(L);
  HalfSummary ha, hb;
  summary_halves(ka, kb, G, ha, hb);
  summary_store(ha, ka, w0, L, G, a.sum, r_local);
  summary_store(hb, kb, w0 + 64, L, G, a.sum, r_local);
}

// One row per workgroup.  The first round trip brings the row's length, its
// summary (whatever the length turns out to be) and, for row offsets, its
// block table; the selection then runs on-chip.
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(1, kNT >= 1024 ? 4 : kNT >= 512 ? 2 : 1))) void topk_select_kernel(TopkLaunch a) {
  __shared__ sel::Smem<kNT> s;
  __shared__ int32_t bt_lds[kBtCache];
  const int r_local = (int)blockIdx.x;
  const int r = a.row_begin + r_local;
  const int tid = (int)threadIdx.x;
  const RowIssue ri = row_issue(a.rows, r);
  sel::Regs<kNT> regs;
  const int64_t ro = (int64_t)r_local * kSumEntries;
  if (a.sum.key)
    sel::load_summary<kNT>(a.sum.key + ro, a.sum.off + ro, a.sum.next + (int64_t)r_local * kSumSegMax,
                           regs);
  const int32_t* bt = a.rows.block_table + (int64_t)(ri.b_ok ? ri.b : 0) * a.rows.max_blocks;
  constexpr int kBtPer = kBtCache / kNT;
  int32_t btv[kBtPer];
  const int nbt = min(a.rows.max_blocks, kBtCache);
#pragma unroll
  for (int j = 0; j < kBtPer; ++j) {
    const int i = tid + j * kNT;
    btv[j] = a.rowoff && i < nbt ? bt[i] : 0;
  }
  const int Lh = row_finish(a.rows, ri);      // history length (0: the row does not resolve)
  const int L = row_slots(a.rows, ri, Lh);    // score row length (candidate count)
  if (Lh == 0 && tid == 0) report(a.err, DSA_DEVERR_ROW);
  const bool bt_cached = a.rowoff && (Lh + kBlock - 1) / kBlock <= kBtCache;
  if (bt_cached) {
#pragma unroll
    for (int j = 0; j < kBtPer; ++j) bt_lds[tid + j * kNT] = btv[j];
  }
  __syncthreads();
  sel::Out o;
  o.gidx = a.indices + (int64_t)r_local * a.K;
  o.roff = a.rowoff ? a.rowoff + (int64_t)r_local * a.K : nullptr;
  o.cand = a.rows.cand ? a.rows.cand + (int64_t)r * a.rows.n_cand : nullptr;
  o.hist = Lh;
  o.err = a.err;
  o.bt = bt;
  o.bt_lds = bt_cached ? bt_lds : nullptr;
  o.kv_blocks = a.kv.num_blocks;
  o.kv_block_stride = a.kv.block_stride;
  o.kv_row_stride = a.kv.row_stride;
  const int n = sel::select_row<kNT>(a.scores + (int64_t)r_local * a.ld, a.vec, L, a.K, regs,
                                     a.sum.key != nullptr, o, s);
  if (tid == 0 && a.counts) a.counts[r_local] = n;
}

}  // namespace

namespace {
size_t round_up256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

size_t summary_bytes(int rows) {
  if (rows <= 0) return 0;
  return round_up256((size_t)rows * kSumEntries * sizeof(uint32_t)) +
         round_up256((size_t)rows * kSumEntries) +
         round_up256((size_t)rows * kSumSegMax * sizeof(uint32_t));
}

Summary summary_carve(void* base, int rows) {
  Summary m;
  uint8_t* p = static_cast<uint8_t*>(base);
  m.key = reinterpret_cast<uint32_t*>(p);
  p += round_up256((size_t)rows * kSumEntries * sizeof(uint32_t));
  m.off = p;
  p += round_up256((size_t)rows * kSumEntries);
  m.next = reinterpret_cast<uint32_t*>(p);
  return m;
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t s, StageEvents ev) {
  if (a.num_rows <= 0) return hipSuccess;
  if (a.prep) {
    const int64_t spans = (a.max_len + 127) / 128;
    const hipError_t e =
        launch_kernel(topk_summary_kernel, dim3((unsigned)((spans + 3) / 4), a.num_rows),
                      dim3(256), s, ev.start, nullptr, a);
    if (e != hipSuccess) return e;
    ev.start = nullptr;
  }
  return launch_kernel(topk_select_kernel, dim3(a.num_rows), dim3(kNT), s, ev.start, ev.stop, a);
}

}  // namespace dsa
