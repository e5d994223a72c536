// Index scores on gfx950: an FP8 MFMA contraction of the row's indexer query
// against every historical index key, with the ReLU gate and the head-weighted
// reduction fused into the epilogue.
//
// Method: Baidu AI Cloud, "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (score all historical
// positions, aggregate with head weights) and section 4.1 (read the paged K
// cache directly, no intermediate per-head score matrix in memory).
//
// Mapping.  One v_mfma_f32_16x16x128_f8f6f4 multiplies 16 indexer heads (M)
// by 16 positions (N) over all 128 dims (K).  Heads sit on M, so each lane's
// 4 accumulator registers hold 4 heads of ONE position: the gate and the
// weighting are per-lane FMAs, and two cross-lane adds (over the four lane
// groups) finish the head sum.  Lane group g holds bytes 16g..16g+15 and
// 64+16g..64+16g+15 of its position's key row, the same slice rule as for the
// query, so one 16-byte load instruction covers 16 rows x 64 contiguous bytes.
//
// Work split.  A workgroup (4 waves) owns a tile of kTile consecutive
// positions of one row; each wave owns a quarter of it (kSpan positions, 8
// sub-tiles of 16) and issues all of their key loads (16 KiB per wave)
// before its first MFMA.  The tile is sized so that a 4 x 128k decode batch is one round of
// workgroups at 4 waves per SIMD: every key load is in flight from the start
// and the memory pipe never drains between rounds.  A sub-tile never
// straddles a 64-row page; the tile's block ids are fetched once, one per
// lane.  The query and weights are staged once per workgroup in LDS.
// Chunked-prefill rows (an explicit row -> sequence map) take two rows per
// workgroup on one set of key loads (indexer_scan_rows_kernel below).

#include "dsa_common.h"

namespace dsa {
namespace {

#ifndef DSA_IDX_TILE
#define DSA_IDX_TILE 512
#endif
constexpr int kTile = DSA_IDX_TILE;  // positions per workgroup
constexpr int kWaves = 4;
constexpr int kSub = 16;  // positions per MFMA column block
constexpr int kSpan = kTile / kWaves;          // consecutive positions per wave
constexpr int kSubPerWave = kSpan / kSub;      // 8
static_assert(kSpan % 64 == 0, "a wave's positions are whole 64-position stores");

// This lane's 32-byte K slice of a 128-byte row (D_I = 128): the 16-byte
// pieces g and g + 4, g = lane / 16.  For D_I = 64 the slice is piece g and
// 16 zero bytes.  The same rule builds both MFMA operands, so the
// contraction pairs query and key bytes of the same dimension.
//
// `sub` (wave-uniform) points at the first of 16 key rows and `lane_off` is
// this lane's byte offset in them (its row, plus 16 bytes per slice group).
// The load is unconditional, which keeps the code free of branches so every
// wait is exact: callers point `sub` at valid memory even for an absent page
// and discard such columns afterwards.  A column of the product depends on
// its own key row alone, so rows past the sequence need no zeroing either.
template <int NKP>
__device__ __forceinline__ v8i load_slice(const uint8_t* sub, uint32_t lane_off) {
  const v4i lo = *reinterpret_cast<const v4i*>(sub + lane_off);
  const v4i hi = NKP == 2 ? *reinterpret_cast<const v4i*>(sub + lane_off + 64) : v4i{0, 0, 0, 0};
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// 16 heads x 16 positions x 128 dims of E4M3, A scaled by byte kSelA of
// scale_a and B by byte 0 of scale_b (E8M0; 127 = x1), from zero.
template <int kSelA>
__device__ __forceinline__ v4f mfma_scaled(v8i a, v8i b, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                          kSelA, scale_a, 0, scale_b);
}

// NKP = D_I / 64 pieces per lane; HT = 16-head tiles (ceil(H_I / 16)); MX:
// MXFP8 operands (one E8M0 scale per 32 dims of every query head and key
// row, Day0 section 5.1; a key block's 64 rows of scales follow its 64 code
// rows), else unscaled E4M3.
//
// Scales.  The block-scaled MFMA takes one scale byte per lane for each
// operand: lane l scales row (A) or column (B) l % 16 over the K block of
// dims [32 (l / 16), 32 (l / 16) + 32).  That block holds the first halves
// of lane groups 2j, 2j + 1 (j = l / 16 < 2) or their second halves
// (j >= 2) in the slice layout above -- a pairing of data and scales the
// hardware defines, and that this kernel only has to feed: lane (col, g)
// passes the scale of dims [32g, 32g + 32) of its head or key row.
//
// CAND: candidate-restricted rows (vLLM's DeepSeek-V4.1-Flash article,
// "Kernels"): the tile covers 512 slots of the row's candidate list rather
// than 512 consecutive positions, and every lane gathers its own key row
// (position cand[slot], block id from the table), one more round trip.
template <int NKP, int HT, bool MX, bool CAND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void indexer_scan_kernel(IndexerLaunch a) {
  const int r = a.row_begin + (int)blockIdx.y;
  const int tile0 = (int)blockIdx.x * kTile;
  const int tid = (int)(threadIdx.x & 255);  // the mask tells the compiler tid < 256
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;  // head row of A, position column of B
  const int g = lane >> 4;    // K slice group
  constexpr int kRowBytes = 64 * NKP;
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[64 * 128];
  __shared__ __attribute__((aligned(16))) float w_lds[64];
  constexpr int kNG = 2 * NKP;                 // 32-dim groups of a row (MX)
  __shared__ uint32_t qs_lds[MX ? 64 * kNG : 1];  // query scales, one per word
  __shared__ float sc_lds[kWaves][kSpan];

  // Load order matters (vector loads complete in issue order): one round
  // trip fetches the row's length, the tile's block ids and the row's query
  // and weights (once per workgroup, staged in LDS).  Every key load is
  // issued as soon as the block ids are back; the query and weights, which
  // left just after them, are put in LDS only then, so their bytes (a whole
  // query per workgroup) do not hold up the key stream.  Each sub-tile is
  // computed as soon as its own keys have landed.

  // 1. block ids of the tile's pages, one per lane (read back into scalar
  //    registers per sub-tile), fetched alongside the row's length rather
  //    than after it; query and weights into LDS, heads past H_I as zero
  constexpr int kPages = kTile / kBlock;
  static_assert(kPages <= 64, "tile spans more pages than a wave has lanes");
  // Every load of this round trip is unconditional, from a clamped
  // (always valid) address, and selected afterwards: a branch would make
  // the compiler wait for each load where it merges.
  const RowIssue ri = row_issue(a.rows, r);
  const int b = ri.b;
  const bool b_ok = ri.b_ok;
  const int32_t* bt = a.rows.block_table + (int64_t)(b_ok ? b : 0) * a.rows.max_blocks;
  // block id of the tile's page `lane` (lanes past the tile's pages, or past
  // the table's columns, read a valid entry that is never used)
  const int my_page = CAND ? 0 : bt[min(tile0 / kBlock + lane, a.rows.max_blocks - 1)];
  // candidate rows: position of the slot of each of the wave's sub-tiles
  // that this lane's column covers (clamped reads; checked after L is known)
  int cpos[CAND ? kSubPerWave : 1];
  if constexpr (CAND) {
    const int32_t* crow = a.rows.cand + (int64_t)r * a.rows.n_cand;
#pragma unroll
    for (int j = 0; j < kSubPerWave; ++j)
      cpos[j] = crow[min(tile0 + wave * kSpan + j * kSub + col, a.rows.n_cand - 1)];
  }
  // the padded query is HT*16 rows of kRowBytes <= 8 KiB: two 16-byte
  // pieces per thread (clamped reads, selected when stored)
  const int qbytes = a.H_I * kRowBytes;  // a multiple of 64
  constexpr int kQBytes = HT * 16 * kRowBytes;
  const int off0 = tid * 16, off1 = off0 + 256 * 16;
  v4i q0, q1;
  float wv;
  uint32_t qsv = 127u;
  {
    const uint8_t* qrow = a.qI + (int64_t)r * a.H_I * kRowBytes;
    q0 = *reinterpret_cast<const v4i*>(qrow + min(off0, qbytes - 16));
    q1 = *reinterpret_cast<const v4i*>(qrow + min(off1, qbytes - 16));
    wv = a.w[(int64_t)r * a.H_I + min(tid, a.H_I - 1)];
    if (MX) {  // the row's query scales
      const uint8_t* qsrow = a.qI_scale + (int64_t)r * a.H_I * kNG;
      qsv = qsrow[min(tid, a.H_I * kNG - 1)];
    }
  }
  // nothing below may be hoisted above these loads, nor they sunk below
  __builtin_amdgcn_sched_barrier(0);

  const int L = row_finish(a.rows, ri);
  if (L == 0) {
    if (blockIdx.x == 0 && threadIdx.x == 0) report(a.err, DSA_DEVERR_ROW);
    return;
  }
  // slots of the score row: L positions, or the candidate count
  const int S = CAND ? row_slots(a.rows, ri, L) : L;
  if (tile0 >= S) return;

  // 2. keys: this wave owns the kSpan positions from w0; sub-tile j starts
  //    at w0 + 16j.  Straight-line code lets the compiler wait for each
  //    sub-tile alone (vmcnt(N)) while the later loads stay in flight.
  const int w0 = tile0 + wave * kSpan;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.kI.base);
  const uint32_t lane_off = (uint32_t)(col * a.kI.row_stride + 16 * g);
  v8i keys[kSubPerWave];
  bool page_ok[kSubPerWave];
  uint32_t csw[CAND && MX ? kSubPerWave : 1];  // candidate rows: this lane's key scale word
  bool bad_pos = false, bad_blk = false;
  if constexpr (CAND) {
    // each lane's own row: a slot inside the list whose position lies in
    // the history; its block id comes from the table (one more round trip)
    int cphys[kSubPerWave];
    bool inside[kSubPerWave];
#pragma unroll
    for (int j = 0; j < kSubPerWave; ++j) {
      const bool in_list = w0 + j * kSub + col < S;
      inside[j] = in_list && cpos[j] >= 0 && cpos[j] < L;
      bad_pos = bad_pos || (in_list && !inside[j]);
      cpos[j] = inside[j] ? cpos[j] : 0;
      cphys[j] = bt[cpos[j] >> 6];
    }
#pragma unroll
    for (int j = 0; j < kSubPerWave; ++j) {
      page_ok[j] = inside[j] && cphys[j] >= 0 && (int64_t)cphys[j] < a.kI.num_blocks;
      bad_blk = bad_blk || (inside[j] && !page_ok[j]);
      const uint8_t* blk = kbase + (int64_t)(page_ok[j] ? cphys[j] : 0) * a.kI.block_stride;
      const int rr = page_ok[j] ? (cpos[j] & 63) : 0;
      keys[j] = load_slice<NKP>(blk + (int64_t)rr * a.kI.row_stride, (uint32_t)(16 * g));
      if constexpr (MX) {
        const uint8_t* sw = blk + (int64_t)kBlock * a.kI.row_stride + rr * kNG;
        if constexpr (kNG == 4)
          csw[j] = *reinterpret_cast<const uint32_t*>(sw);
        else
          csw[j] = *reinterpret_cast<const uint16_t*>(sw);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSubPerWave; ++j) {
      const int s0 = w0 + j * kSub;
      const int phys = __builtin_amdgcn_readlane(my_page, (s0 - tile0) >> 6);
      // a page past the table's columns, or with an id out of range, is absent
      page_ok[j] = s0 / kBlock < a.rows.max_blocks && phys >= 0 && (int64_t)phys < a.kI.num_blocks;
      const uint8_t* sub = kbase + (int64_t)(page_ok[j] ? phys : 0) * a.kI.block_stride +
                           (int64_t)(s0 & 63) * a.kI.row_stride;
      keys[j] = load_slice<NKP>(sub, lane_off);
    }
  }
  // MX: the scale words of the wave's key rows.  The wave's 128 positions
  // are two whole blocks (w0 is a multiple of 128), and a block keeps its
  // 64 rows' scales together after its code rows: lane l takes row l's
  // scales from block h, so word h of lane l belongs to sub-tile 4h + l / 16,
  // row l % 16, and each load is one contiguous run.  Each sub-tile fetches
  // its rows' words across lanes when it needs them, so only two registers
  // stay in flight.
  static_assert(kSubPerWave == 8 && kSpan == 2 * kBlock, "two scale words per lane cover the wave");
  uint32_t ksw[MX ? 2 : 1];
  if (MX && !CAND) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int phys = __builtin_amdgcn_readlane(my_page, ((w0 - tile0) >> 6) + h);
      const uint8_t* area = kbase + (int64_t)(page_ok[4 * h] ? phys : 0) * a.kI.block_stride +
                            (int64_t)kBlock * a.kI.row_stride;
      if constexpr (kNG == 4)
        ksw[h] = *reinterpret_cast<const uint32_t*>(area + 4 * lane);
      else
        ksw[h] = *reinterpret_cast<const uint16_t*>(area + 2 * lane);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the query and weights into LDS, heads past H_I as zero (query scales:
  // 127, i.e. x1, for padding heads)
  {
    const v4i z = v4i{0, 0, 0, 0};
    q0 = off0 < qbytes ? q0 : z;
    q1 = off1 < qbytes ? q1 : z;
    wv = tid < a.H_I ? wv : 0.0f;
    if (off0 < kQBytes) *reinterpret_cast<v4i*>(&q_lds[off0]) = q0;
    if (off1 < kQBytes) *reinterpret_cast<v4i*>(&q_lds[off1]) = q1;
    if (tid < HT * 16) w_lds[tid] = wv;
    if (MX) {
      if (tid >= a.H_I * kNG) qsv = 127u;
      if (tid < 64 * kNG) qs_lds[tid] = qsv;
    }
  }
  __syncthreads();
  // A operands (heads 16*ht + col); the head weights of this lane's
  // accumulator rows (register v of a 16x16 tile is row 4*g + v) are read
  // from LDS per use, which keeps the registers for keys in flight
  v8i aq[HT];
  // This lane's A scale for head tile ht (group g of head 16ht + col) sits in
  // byte ht of one register, and the MFMA's op-select immediate picks the
  // byte; E4M3 keeps 127 (x1) in every byte.
  int qscale = 0x7F7F7F7F;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const v4i* src = reinterpret_cast<const v4i*>(&q_lds[(16 * ht + col) * kRowBytes]);
    const v4i lo = src[g];
    const v4i hi = NKP == 2 ? src[g + 4] : v4i{0, 0, 0, 0};
    aq[ht] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if (MX && g < kNG)
      qscale = (qscale & ~(0xFF << (8 * ht))) | ((int)qs_lds[(16 * ht + col) * kNG + g] << (8 * ht));
  }
  // The wave's scores are collected in LDS and written with a few
  // full-width stores at the end, not one narrow store per sub-tile.
  float* my_sc = sc_lds[wave];
  // The Top-K's summary of this wave's slots (the kSumM largest keys of each
  // segment, with their offsets, and the segment's next key) is worked out
  // for both halves at once after the last sub-tile: the last workgroups to
  // get their keys end the kernel, and the two halves' interleaved rounds
  // take about the time of one.
  static_assert(kSpan == 128 && kSubPerWave == 8, "a wave's summary covers two halves of 64");
  const bool summ = a.sum.key && w0 < S && sum_row(S, a.topk_K);  // wave-uniform

  bool bad_page = false;
#pragma unroll
  for (int j = 0; j < kSubPerWave; ++j) {
    float part = 0.0f;
    // B scale: byte g of the key row's scale word (127, i.e. x1, for unused
    // groups and for E4M3)
    int ks = 127;
    if (MX) {
      const uint32_t word = CAND ? csw[CAND ? j : 0]
                                 : (uint32_t)__shfl((int)ksw[MX ? j / 4 : 0], 16 * (j % 4) + col);
      ks = g < kNG ? (int)((word >> (8 * g)) & 0xFFu) : 127;
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      v4f acc;
      switch (ht) {  // the op-select byte must be an immediate (ht is one once unrolled)
        case 0: acc = mfma_scaled<0>(aq[ht], keys[j], qscale, MX ? ks : 127); break;
        case 1: acc = mfma_scaled<1>(aq[ht], keys[j], qscale, MX ? ks : 127); break;
        case 2: acc = mfma_scaled<2>(aq[ht], keys[j], qscale, MX ? ks : 127); break;
        default: acc = mfma_scaled<3>(aq[ht], keys[j], qscale, MX ? ks : 127); break;
      }
      const v4f wr = *reinterpret_cast<const v4f*>(&w_lds[16 * ht + 4 * g]);
#pragma unroll
      for (int v = 0; v < 4; ++v) part += wr[v] * fmaxf(acc[v], 0.0f);
    }
    part = across_rows(part, FAdd());
    // canonical +0 for a zero score; an absent page scores -inf
    const float v = page_ok[j] ? part + 0.0f : -__builtin_inff();
    if (g == 0) my_sc[j * kSub + col] = v;
    if (!CAND) bad_page = bad_page || (w0 + j * kSub < L && !page_ok[j]);
  }
  // LDS accesses of one wave complete in order; the fence keeps the
  // compiler from moving the reads above the writes of other lanes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float* out = a.scores + (int64_t)(r - a.row_begin) * a.ld;
#pragma unroll
  for (int h = 0; h < kSpan / 64; ++h) {
    const int i = 64 * h + lane;
    if (w0 + i < S) out[w0 + i] = my_sc[i];
  }
  if (summ) {
    const int G = sum_seg(S);
    const uint32_t ka = w0 + lane < S ? score_key(my_sc[lane]) : 0u;
    const uint32_t kb = w0 + 64 + lane < S ? score_key(my_sc[64 + lane]) : 0u;
    HalfSummary ha, hb;
    summary_halves(ka, kb, G, ha, hb);
    summary_store(ha, ka, w0, S, G, a.sum, r - a.row_begin);
    summary_store(hb, kb, w0 + 64, S, G, a.sum, r - a.row_begin);
  }
  if (__builtin_amdgcn_ballot_w64(bad_page || bad_blk) && lane == 0) report(a.err, DSA_DEVERR_BLOCK);
  if (CAND && __builtin_amdgcn_ballot_w64(bad_pos) && lane == 0) report(a.err, DSA_DEVERR_ROW);
}

// The scan for chunked-prefill rows: NR consecutive rows per workgroup.
// Rows of one sequence score the same index keys, so a workgroup takes NR
// rows for its tile and runs every row's MFMAs and epilogue on one set of
// key loads: NR times fewer key bytes through L2 for the same MFMA work.  A
// row of another sequence than the workgroup's first (a pass across two
// prefill chunks) loads its own keys.  Everything else is as in
// indexer_scan_kernel (no candidate lists here).
template <int NKP, int HT, bool MX, int NR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void indexer_scan_rows_kernel(IndexerLaunch a) {
  static_assert(NR > 1, "one row per workgroup: indexer_scan_kernel");
  const int r0 = a.row_begin + (int)blockIdx.y * NR;
  const int nr = min(NR, a.row_begin + a.num_rows - r0);  // this workgroup's rows, >= 1
  const int tile0 = (int)blockIdx.x * kTile;
  const int tid = (int)(threadIdx.x & 255);  // the mask tells the compiler tid < 256
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;  // head row of A, position column of B
  const int g = lane >> 4;    // K slice group
  constexpr int kRowBytes = 64 * NKP;
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[NR][64 * 128];
  __shared__ __attribute__((aligned(16))) float w_lds[NR][64];
  constexpr int kNG = 2 * NKP;                 // 32-dim groups of a row (MX)
  __shared__ uint32_t qs_lds[NR][MX ? 64 * kNG : 1];  // query scales, one per word
  __shared__ float sc_lds[NR][kWaves][kSpan];

  // Load order matters (vector loads complete in issue order): one round
  // trip fetches the rows' lengths, the tile's block ids and the rows'
  // queries and weights (staged in LDS before the key loads go out, which
  // keeps their registers free).  Each sub-tile is computed as soon as its
  // own keys have landed.

  // 1. block ids of the tile's pages, one per lane (read back into scalar
  //    registers per sub-tile), fetched alongside the rows' lengths rather
  //    than after them; queries and weights into LDS, heads past H_I as zero
  constexpr int kPages = kTile / kBlock;
  static_assert(kPages <= 64, "tile spans more pages than a wave has lanes");
  // Every load of this round trip is unconditional, from a clamped
  // (always valid) address, and selected afterwards: a branch would make
  // the compiler wait for each load where it merges.
  RowIssue ri[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) ri[k] = row_issue(a.rows, r0 + min(k, nr - 1));
  const int b = ri[0].b;
  const bool b_ok = ri[0].b_ok;
  const int32_t* bt = a.rows.block_table + (int64_t)(b_ok ? b : 0) * a.rows.max_blocks;
  // block id of the tile's page `lane` (lanes past the tile's pages, or past
  // the table's columns, read a valid entry that is never used)
  const int my_page = bt[min(tile0 / kBlock + lane, a.rows.max_blocks - 1)];
  // the padded query is HT*16 rows of kRowBytes <= 8 KiB: two 16-byte
  // pieces per thread (clamped reads, selected when stored)
  const int qbytes = a.H_I * kRowBytes;  // a multiple of 64
  constexpr int kQBytes = HT * 16 * kRowBytes;
  const int off0 = tid * 16, off1 = off0 + 256 * 16;
  v4i q0[NR], q1[NR];
  float wv[NR];
  uint32_t qsv[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int rk = r0 + min(k, nr - 1);
    const uint8_t* qrow = a.qI + (int64_t)rk * a.H_I * kRowBytes;
    q0[k] = *reinterpret_cast<const v4i*>(qrow + min(off0, qbytes - 16));
    q1[k] = *reinterpret_cast<const v4i*>(qrow + min(off1, qbytes - 16));
    wv[k] = a.w[(int64_t)rk * a.H_I + min(tid, a.H_I - 1)];
    qsv[k] = 127u;
    if (MX) {  // the row's query scales
      const uint8_t* qsrow = a.qI_scale + (int64_t)rk * a.H_I * kNG;
      qsv[k] = qsrow[min(tid, a.H_I * kNG - 1)];
    }
  }
  // nothing below may be hoisted above these loads, nor they sunk below
  __builtin_amdgcn_sched_barrier(0);
  // the queries and weights into LDS, heads past H_I as zero (query scales:
  // 127, i.e. x1, for padding heads)
  auto stage_queries = [&]() {
    const v4i z = v4i{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const v4i x0 = off0 < qbytes ? q0[k] : z;
      const v4i x1 = off1 < qbytes ? q1[k] : z;
      const float w = tid < a.H_I ? wv[k] : 0.0f;
      if (off0 < kQBytes) *reinterpret_cast<v4i*>(&q_lds[k][off0]) = x0;
      if (off1 < kQBytes) *reinterpret_cast<v4i*>(&q_lds[k][off1]) = x1;
      if (tid < HT * 16) w_lds[k][tid] = w;
      if (MX) {
        const uint32_t qs = tid >= a.H_I * kNG ? 127u : qsv[k];
        if (tid < 64 * kNG) qs_lds[k][tid] = qs;
      }
    }
  };
  stage_queries();

  // history lengths L and score-row lengths S of the rows; a workgroup whose
  // rows all end before its tile has nothing to do
  int Lr[NR], Sr[NR];
  bool any = false;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    Lr[k] = k < nr ? row_finish(a.rows, ri[k]) : 0;
    if (k < nr && Lr[k] == 0 && blockIdx.x == 0 && threadIdx.x == 0) report(a.err, DSA_DEVERR_ROW);
    Sr[k] = Lr[k];  // slots of the score row: its positions
    any = any || tile0 < Sr[k];
  }
  if (!any) return;

  // 2. keys: this wave owns the kSpan positions from w0; sub-tile j starts
  //    at w0 + 16j.  Straight-line code lets the compiler wait for each
  //    sub-tile alone (vmcnt(N)) while the later loads stay in flight.
  const int w0 = tile0 + wave * kSpan;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.kI.base);
  const uint32_t lane_off = (uint32_t)(col * a.kI.row_stride + 16 * g);
  v8i keys[kSubPerWave];
  bool page_ok[kSubPerWave];
  // MX: the scale words of the wave's key rows.  The wave's 128 positions
  // are two whole blocks (w0 is a multiple of 128), and a block keeps its
  // 64 rows' scales together after its code rows: lane l takes row l's
  // scales from block h, so word h of lane l belongs to sub-tile 4h + l / 16,
  // row l % 16, and each load is one contiguous run.  Each sub-tile fetches
  // its rows' words across lanes when it needs them, so only two registers
  // stay in flight.
  static_assert(kSubPerWave == 8 && kSpan == 2 * kBlock, "two scale words per lane cover the wave");
  uint32_t ksw[MX ? 2 : 1];
  // the keys (and MX scale words) of a sequence whose tile block ids are
  // `page` (one per lane) in a table of max_blocks columns
  auto load_keys = [&](int page) {
#pragma unroll
    for (int j = 0; j < kSubPerWave; ++j) {
      const int s0 = w0 + j * kSub;
      const int phys = __builtin_amdgcn_readlane(page, (s0 - tile0) >> 6);
      // a page past the table's columns, or with an id out of range, is absent
      page_ok[j] = s0 / kBlock < a.rows.max_blocks && phys >= 0 && (int64_t)phys < a.kI.num_blocks;
      const uint8_t* sub = kbase + (int64_t)(page_ok[j] ? phys : 0) * a.kI.block_stride +
                           (int64_t)(s0 & 63) * a.kI.row_stride;
      keys[j] = load_slice<NKP>(sub, lane_off);
    }
    if constexpr (MX) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int phys = __builtin_amdgcn_readlane(page, ((w0 - tile0) >> 6) + h);
        const uint8_t* area = kbase + (int64_t)(page_ok[4 * h] ? phys : 0) * a.kI.block_stride +
                              (int64_t)kBlock * a.kI.row_stride;
        if constexpr (kNG == 4)
          ksw[h] = *reinterpret_cast<const uint32_t*>(area + 4 * lane);
        else
          ksw[h] = *reinterpret_cast<const uint16_t*>(area + 2 * lane);
      }
    }
  };
  load_keys(my_page);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // The wave's scores are collected in LDS, every row's before any row's
  // epilogue (the keys stay live for the next row's MFMAs, the epilogue's
  // registers come after them), and written with a few full-width stores,
  // not one narrow store per sub-tile.
  static_assert(kSpan == 128 && kSubPerWave == 8, "a wave's summary covers two halves of 64");
  bool bad_page = false;
  // row k of the workgroup (one that needs this tile): its scores on the
  // loaded keys into LDS
  auto score_row = [&](int k) __attribute__((always_inline)) {
    const int L = Lr[k];
    float* my_sc = sc_lds[k][wave];
    // A operands (heads 16*ht + col); the head weights of this lane's
    // accumulator rows (register v of a 16x16 tile is row 4*g + v) are read
    // from LDS per use, which keeps the registers for keys in flight
    v8i aq[HT];
    // This lane's A scale for head tile ht (group g of head 16ht + col) sits
    // in byte ht of one register, and the MFMA's op-select immediate picks
    // the byte; E4M3 keeps 127 (x1) in every byte.
    int qscale = 0x7F7F7F7F;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const v4i* src = reinterpret_cast<const v4i*>(&q_lds[k][(16 * ht + col) * kRowBytes]);
      const v4i lo = src[g];
      const v4i hi = NKP == 2 ? src[g + 4] : v4i{0, 0, 0, 0};
      aq[ht] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (MX && g < kNG)
        qscale = (qscale & ~(0xFF << (8 * ht))) | ((int)qs_lds[k][(16 * ht + col) * kNG + g] << (8 * ht));
    }
#pragma unroll
    for (int j = 0; j < kSubPerWave; ++j) {
      float part = 0.0f;
      // B scale: byte g of the key row's scale word (127, i.e. x1, for
      // unused groups and for E4M3)
      int ks = 127;
      if (MX) {
        const uint32_t word = (uint32_t)__shfl((int)ksw[MX ? j / 4 : 0], 16 * (j % 4) + col);
        ks = g < kNG ? (int)((word >> (8 * g)) & 0xFFu) : 127;
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        v4f acc;
        switch (ht) {  // the op-select byte must be an immediate (ht is one once unrolled)
          case 0: acc = mfma_scaled<0>(aq[ht], keys[j], qscale, MX ? ks : 127); break;
          case 1: acc = mfma_scaled<1>(aq[ht], keys[j], qscale, MX ? ks : 127); break;
          case 2: acc = mfma_scaled<2>(aq[ht], keys[j], qscale, MX ? ks : 127); break;
          default: acc = mfma_scaled<3>(aq[ht], keys[j], qscale, MX ? ks : 127); break;
        }
        const v4f wr = *reinterpret_cast<const v4f*>(&w_lds[k][16 * ht + 4 * g]);
#pragma unroll
        for (int v = 0; v < 4; ++v) part += wr[v] * fmaxf(acc[v], 0.0f);
      }
      part = across_rows(part, FAdd());
      // canonical +0 for a zero score; an absent page scores -inf
      const float v = page_ok[j] ? part + 0.0f : -__builtin_inff();
      if (g == 0) my_sc[j * kSub + col] = v;
      bad_page = bad_page || (w0 + j * kSub < L && !page_ok[j]);
    }
  };
  // row k's epilogue: its scores out, and the Top-K's summary of this
  // wave's slots (the kSumM largest keys of each segment, with their
  // offsets, and the segment's next key), both halves at once
  auto finish_row = [&](int k) __attribute__((always_inline)) {
    const int S = Sr[k];
    const int rk = r0 + k;
    const float* my_sc = sc_lds[k][wave];
    const bool summ = a.sum.key && w0 < S && sum_row(S, a.topk_K);  // wave-uniform
    float* out = a.scores + (int64_t)(rk - a.row_begin) * a.ld;
#pragma unroll
    for (int h = 0; h < kSpan / 64; ++h) {
      const int i = 64 * h + lane;
      if (w0 + i < S) out[w0 + i] = my_sc[i];
    }
    if (summ) {
      const int G = sum_seg(S);
      const uint32_t ka = w0 + lane < S ? score_key(my_sc[lane]) : 0u;
      const uint32_t kb = w0 + 64 + lane < S ? score_key(my_sc[64 + lane]) : 0u;
      HalfSummary ha, hb;
      summary_halves(ka, kb, G, ha, hb);
      summary_store(ha, ka, w0, S, G, a.sum, rk - a.row_begin);
      summary_store(hb, kb, w0 + 64, S, G, a.sum, rk - a.row_begin);
    }
  };
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    if (k < nr && tile0 < Sr[k]) {  // (workgroup-uniform)
      // a row of another sequence: its own block ids, then its own keys
      if (k > 0 && !(ri[k].b_ok && ri[k].b == b && b_ok)) {
        const int32_t* btk = a.rows.block_table + (int64_t)ri[k].b * a.rows.max_blocks;
        load_keys(btk[min(tile0 / kBlock + lane, a.rows.max_blocks - 1)]);
      }
      score_row(k);
    }
  }
  // LDS accesses of one wave complete in order; the fence keeps the
  // compiler from moving the reads above the writes of other lanes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int k = 0; k < NR; ++k)
    if (k < nr && tile0 < Sr[k]) finish_row(k);
  if (__builtin_amdgcn_ballot_w64(bad_page) && lane == 0) report(a.err, DSA_DEVERR_BLOCK);
}

// Rows per workgroup for chunked-prefill rows (an explicit row -> sequence
// map) with E4M3 operands; MXFP8 operands (two more live registers per lane)
// and every other batch run one row per workgroup.
#ifndef DSA_IDX_PREFILL_ROWS
#define DSA_IDX_PREFILL_ROWS 2
#endif
constexpr int kPrefillRows = DSA_IDX_PREFILL_ROWS;

template <int NKP, int HT, bool MX>
hipError_t launch_t(const IndexerLaunch& a, hipStream_t s, StageEvents ev) {
  const int tiles = (a.max_len + kTile - 1) / kTile;
  if constexpr (!MX && kPrefillRows > 1) {
    if (!a.rows.cand && a.rows.row_seq && a.num_rows > 1)
      return launch_kernel(indexer_scan_rows_kernel<NKP, HT, false, kPrefillRows>,
                           dim3(tiles, (a.num_rows + kPrefillRows - 1) / kPrefillRows),
                           dim3(256), s, ev.start, ev.stop, a);
  }
  return launch_kernel(a.rows.cand ? indexer_scan_kernel<NKP, HT, MX, true>
                                   : indexer_scan_kernel<NKP, HT, MX, false>,
                       dim3(tiles, a.num_rows), dim3(256), s, ev.start, ev.stop, a);
}

template <bool MX>
hipError_t launch_mx(const IndexerLaunch& a, hipStream_t s, StageEvents ev) {
  const int ht = (a.H_I + 15) / 16;
  if (a.D_I == 128) {
    switch (ht) {
      case 1: return launch_t<2, 1, MX>(a, s, ev);
      case 2: return launch_t<2, 2, MX>(a, s, ev);
      case 3: return launch_t<2, 3, MX>(a, s, ev);
      default: return launch_t<2, 4, MX>(a, s, ev);
    }
  }
  switch (ht) {
    case 1: return launch_t<1, 1, MX>(a, s, ev);
    case 2: return launch_t<1, 2, MX>(a, s, ev);
    case 3: return launch_t<1, 3, MX>(a, s, ev);
    default: return launch_t<1, 4, MX>(a, s, ev);
  }
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerLaunch& a, hipStream_t s, StageEvents ev) {
  if (a.num_rows <= 0 || a.max_len <= 0) return hipSuccess;
  return a.qI_scale ? launch_mx<true>(a, s, ev) : launch_mx<false>(a, s, ev);
}

}  // namespace dsa
