// Internal declarations shared by the gfx950 kernels and the C-ABI front end.
// Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

constexpr int kBlock = 64;  // tokens per cache page

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

// Row -> (sequence, position) map and the block table, as kernels see it.
struct RowMap {
  const int32_t* seq_lens;
  const int32_t* block_table;
  const int32_t* row_seq;  // NULL: row r -> sequence r
  const int32_t* row_pos;  // NULL: position seq_lens[b] - 1
  int32_t num_seqs;
  int32_t max_blocks;
  // Candidate-restricted rows: row r scores only the positions
  // cand[r * n_cand + c], c < cand_len[r] (ascending); NULL: every position.
  const int32_t* cand;
  const int32_t* cand_len;
  int32_t n_cand;
};

// Resolves row r.  Returns false (and leaves b, p unspecified) when the
// sequence id or the position is out of range; the caller then treats the
// row as having no history and reports DSA_DEVERR_ROW.
__device__ __forceinline__ bool resolve_row(const RowMap& m, int r, int& b, int& p) {
  b = m.row_seq ? m.row_seq[r] : r;
  if (b < 0 || b >= m.num_seqs) return false;
  const int len = m.seq_lens[b];
  p = m.row_pos ? m.row_pos[r] : len - 1;
  if (p < 0 || p >= len || p >= m.max_blocks * kBlock) return false;
  return true;
}

// Row resolution split in two, for kernels whose first round trip should
// carry everything: row_issue loads the row's length and position without
// branches (an absent row_pos reads a valid dummy) and keeps them in vector
// registers -- the empty asm hides their uniformity, so the compiler does
// not move them to scalar registers, and wait for them, at once;
// row_finish applies resolve_row's checks and returns the history length
// L = p + 1, or 0 for a row that does not resolve.  Only a row_seq lookup
// (chunked prefill rows) costs a round trip of its own.
struct RowIssue {
  int b, len_v, pos_v, clen_v;
  bool b_ok;
};
__device__ __forceinline__ RowIssue row_issue(const RowMap& m, int r) {
  typedef __attribute__((address_space(1))) const int32_t gint;  // global, not flat
  RowIssue q;
  q.b = m.row_seq ? m.row_seq[r] : r;
  q.b_ok = q.b >= 0 && q.b < m.num_seqs;
  gint* len_at = (gint*)(m.seq_lens + (q.b_ok ? q.b : 0));
  gint* pos_at = (gint*)(m.row_pos ? m.row_pos + r : m.seq_lens);
  gint* clen_at = (gint*)(m.cand_len ? m.cand_len + r : m.seq_lens);
  asm volatile("" : "+v"(len_at), "+v"(pos_at), "+v"(clen_at));
  q.len_v = *len_at;
  q.pos_v = *pos_at;
  q.clen_v = *clen_at;
  return q;
}
__device__ __forceinline__ int row_finish(const RowMap& m, const RowIssue& q) {
  const int len = __builtin_amdgcn_readfirstlane(q.len_v);
  const int p = m.row_pos ? __builtin_amdgcn_readfirstlane(q.pos_v) : len - 1;
  if (!q.b_ok || p < 0 || p >= len || p >= m.max_blocks * kBlock) return 0;
  return p + 1;
}
// Length of the row's score row: its candidate count (clamped to
// 0 .. n_cand) for a candidate-restricted row, else its history length L
// (0 for a row that does not resolve).
__device__ __forceinline__ int row_slots(const RowMap& m, const RowIssue& q, int L) {
  if (!m.cand || L == 0) return L;
  const int c = __builtin_amdgcn_readfirstlane(q.clen_v);
  return c < 0 ? 0 : c > m.n_cand ? m.n_cand : c;
}

__device__ __forceinline__ void report(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

// Order-preserving 32-bit key of a float32 score: larger score, larger key;
// -0 and +0 share a key; NaN gets 0 and ranks below every number.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag == 0) u = 0;
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return mag > 0x7F800000u ? 0u : k;
}

// ----------------------------------------------------- cross-lane, registers
// Reductions over lanes without an LDS round trip.  v_permlane16_swap
// exchanges 16-lane rows 0<->1 and 2<->3, v_permlane32_swap the two wave
// halves: with both operands the same value the returned pair holds this
// lane's value and its partner's, so op(pair) is the same in both lanes.
// Within a row, DPP quad permutes and the half-row and row mirrors pair
// lanes 1, 2, 4 and 8 apart (each step combines two disjoint groups).
struct FMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct FAdd { __device__ float operator()(float a, float b) const { return a + b; } };
template <class Op>
__device__ __forceinline__ float xor16(float x, Op op) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
template <class Op>
__device__ __forceinline__ float xor32(float x, Op op) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
// op over the four 16-lane rows (lanes l, l^16, l^32, l^48), in every lane
template <class Op>
__device__ __forceinline__ float across_rows(float x, Op op) {
  return xor32(xor16(x, op), op);
}
// op over all 64 lanes, in every lane
template <class Op>
__device__ __forceinline__ float across_wave(float x, Op op) {
  x = op(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_f<0x141>(x));  // row_half_mirror
  x = op(x, dpp_f<0x140>(x));  // row_mirror
  return across_rows(x, op);
}

// Number of set bits of `mask` below this lane (wave64).
__device__ __forceinline__ int lane_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are validated by
// the front end before these run.

// ------------------------------------------------------ Top-K work area
// The Top-K's pre-selection.  A row's positions are cut into segments of G
// = topk_sum_seg(L) positions (32 to 128, at most 1024 segments up to
// 131072 positions); the m = topk_sum_m(L) largest keys of each segment
// form the row's summary, 3072 to kSumMax keys for the rows that use it
// (topk_split_row: more than 16384 positions, so more than 512 segments).
// The summary's keys sit at distinct positions, so its K-th largest is a
// lower bound on the row's K-th largest score;
// with about two summary keys per row key kept, and about two kept keys per
// segment, the segments' top keys hold nearly all of the row's top K and
// the bound is close.  The fused indexer and the standalone summary pass
// call the same functions, so they agree on every row.
constexpr int kSumSpan = 128;           // positions per indexer wave (one or more segments)
constexpr int kSumSegs = 1024;          // segments per row, at most (up to 131072 positions)
constexpr int kSumMax = 4096;           // summary keys per row, at most
constexpr int kSumCap = 8;              // keys per segment, at most
__host__ __device__ inline int topk_sum_seg(int L) {
  int G = 32;
  while (G < kSumSpan && (L + G - 1) / G > kSumSegs) G <<= 1;
  return G;
}
__host__ __device__ inline int topk_sum_m(int L) {
  const int G = topk_sum_seg(L);
  const int nseg = (L + G - 1) / G;
  if (nseg <= 0) return 0;
  const int m = kSumMax / nseg;
  return m < kSumCap ? m : kSumCap;
}
constexpr int kTopkSlices = 32;         // workgroups per row, at most
constexpr int kTopkSliceLen = 4096;     // positions per slice
constexpr int kTopkSplitMaxK = 2048;
// Rows that the Top-K spreads over slices (and that get a summary).  Rows
// of up to 16384 positions are faster in one workgroup, which holds 16 keys
// per thread.
__host__ __device__ inline bool topk_split_row(int L, int K) {
  return K <= kTopkSplitMaxK && L > 16384 && L <= kTopkSlices * kTopkSliceLen;
}

// Maximum of an unsigned value over aligned groups of G lanes (16, 32 or
// 64, wave-uniform), in every lane of the group.
__device__ __forceinline__ uint32_t group_max_u32(uint32_t x, int G) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));  // row_mirror
  if (G >= 32) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((uint32_t)p[0], (uint32_t)p[1]);
  }
  if (G >= 64) {
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = max((uint32_t)p[0], (uint32_t)p[1]);
  }
  return x;
}

// The m largest keys of each segment of G positions of a wave's 128 (key a
// of lane l: position l, key b: position 64 + l), with multiplicity: m
// rounds of a group maximum, each taking out one instance (the lowest lane
// of the group that holds it).  G = 128: one segment over both keys, lane
// i < m gets its (i+1)-th largest in out_a.  G <= 64: segments of G lanes
// in each key; lane G s + i, i < m, gets segment s's (i+1)-th largest of
// the a keys in out_a and of the b keys in out_b.  G and m are wave-uniform.
__device__ __forceinline__ void segment_top(uint32_t ka, uint32_t kb, int m, int G, uint32_t& out_a,
                                            uint32_t& out_b) {
  const int lane = (int)(threadIdx.x & 63);
  out_a = out_b = 0u;
  if (G >= kSumSpan) {
    for (int i = 0; i < m; ++i) {
      const uint32_t v = max(ka, kb);
      const uint32_t M = group_max_u32(v, 64);
      const uint64_t hit = __ballot(v == M);
      if (lane == (int)__builtin_ctzll(hit)) {
        if (ka == M)
          ka = 0u;
        else
          kb = 0u;
      }
      out_a = lane == i ? M : out_a;
    }
    return;
  }
  const int base = lane & ~(G - 1);
  const uint64_t gmask = G == 64 ? ~0ull : ((1ull << G) - 1ull) << base;
  for (int i = 0; i < m; ++i) {
    const uint32_t Ma = group_max_u32(ka, G), Mb = group_max_u32(kb, G);
    const uint64_t ha = __ballot(ka == Ma) & gmask, hb = __ballot(kb == Mb) & gmask;
    if (lane == (int)__builtin_ctzll(ha)) ka = 0u;
    if (lane == (int)__builtin_ctzll(hb)) kb = 0u;
    out_a = lane - base == i ? Ma : out_a;
    out_b = lane - base == i ? Mb : out_b;
  }
}

// Writes a wave's summary keys (segment_top's results for the 128 positions
// from w0, of a score row of S positions) into the row's summary `summ`.
__device__ __forceinline__ void store_segment_top(uint32_t* summ, int w0, int S, int m, int G,
                                                  uint32_t out_a, uint32_t out_b) {
  const int lane = (int)(threadIdx.x & 63);
  if (G >= kSumSpan) {
    if (lane < m && w0 < S) summ[(w0 / G) * m + lane] = out_a;
    return;
  }
  const int i = lane & (G - 1), s_lane = lane / G;
  if (i < m && w0 + G * s_lane < S) summ[(w0 / G + s_lane) * m + i] = out_a;
  if (i < m && w0 + 64 + G * s_lane < S) summ[((w0 + 64) / G + s_lane) * m + i] = out_b;
}

// The Top-K's work area, carved from the caller's workspace:
//  - summ [rows][kSumMax]: each row's summary (segment s's keys at
//    s * m .. s * m + m - 1);
//  - ckey, cpos [rows][cstride]: the candidate keys and positions that the
//    workgroups of a row's slices hand to the one that finishes the row
//    (slice j's entries start at j * kTopkSliceLen);
//  - ccount [rows][kTopkSlices]: how many candidates each slice left;
//  - arrive [rows]: slices of the row done so far.  Whichever kernel writes
//    the summary for a call (the fused indexer, or the standalone summary
//    pass) zeroes it first.
struct TopkWork {
  uint32_t* summ;
  uint32_t* ckey;
  int32_t* cpos;
  int64_t cstride;
  uint32_t* ccount;
  uint32_t* arrive;
};
// bytes of the work area for `rows` rows of history up to max_len
size_t topk_work_bytes(int rows, int64_t max_len);
// carves the work area out of `base` (256-byte aligned)
TopkWork topk_work_carve(void* base, int rows, int64_t max_len);

struct IndexerLaunch {
  RowMap rows;
  const uint8_t* qI;
  const uint8_t* qI_scale;  // MXFP8: [rows][H_I][D_I/32] E8M0; NULL: unscaled E4M3
  const float* w;
  dsa_paged kI;
  float* scores;
  int64_t ld;
  uint32_t* err;
  int32_t H_I, D_I;
  int32_t row_begin, num_rows;  // rows [row_begin, row_begin + num_rows)
  int32_t max_len;              // upper bound of any row's history length
  TopkWork tw;                  // summaries for a Top-K of topk_K that follows,
  int32_t topk_K;               // or nothing when tw.summ is NULL
};
hipError_t launch_indexer_scores(const IndexerLaunch& a, hipStream_t s);

struct TopkLaunch {
  RowMap rows;
  const float* scores;  // row r reads scores[(r - row_begin) * ld]
  int64_t ld;
  int32_t* indices;     // [num_rows][K]
  int32_t* counts;      // [num_rows] or NULL
  uint32_t* err;
  int32_t K;
  int32_t row_begin, num_rows;
  int32_t max_len;
  TopkWork tw;
  bool prep;            // compute the summaries here (no fused indexer before)
  bool vec;             // every score row is 16-byte aligned (ld % 4 == 0)
  bool cvec;            // every candidate row is 16-byte aligned (n_cand % 4 == 0)
  // Optional: also write each kept position's byte offset in the paged KV
  // cache `kv` (block table -> physical block), -1 for padding and for
  // positions whose block id is out of range, to rowoff[num_rows][K].
  int64_t* rowoff;
  dsa_paged kv;
  // With rowoff: bytes of a KV row the attention that follows reads (0: none).
  // The Top-K then touches every candidate's row once it has handed its
  // slice over, so that the attention's gather finds them in the caches.
  int32_t kv_row_bytes;
};
hipError_t launch_topk(const TopkLaunch& a, hipStream_t s);

struct AttnLaunch {
  RowMap rows;
  const uint16_t* q;
  dsa_paged k, v;
  bool latent;  // v aliases k (same base and strides)
  const int32_t* indices;
  int64_t indices_row_offset;  // indices row of row_begin
  const int64_t* rowoff;       // optional [num_rows][K] byte offsets of the selected
                               // rows (latent layout), -1 = absent; replaces the
                               // index -> block table lookup
  uint16_t* out;
  float* lse;
  void* partial;   // workspace for split-key partials, or NULL when n_chunks == 1
  uint32_t* err;
  int32_t H_q, D_qk, D_v, K;
  float scale;
  int32_t row_begin, num_rows;
  int32_t n_chunks;
};
// Chunks the index list of each row is split into for the kernel that the
// layout (latent or not) selects, and the most either layout may use (for
// workspace sizes, which do not know the layout).
int attn_chunks(int num_rows, int H_q, int D_qk, int K, bool latent);
int attn_chunks_max(int num_rows, int H_q, int D_qk, int K);
size_t attn_partial_bytes(int num_rows, int H_q, int D_v, int n_chunks);
hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s);

}  // namespace dsa
