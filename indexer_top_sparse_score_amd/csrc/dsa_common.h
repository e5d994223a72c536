// Internal declarations shared by the gfx950 kernels and the C-ABI front end.
// Nothing here is exported.
#pragma once

#include <hip/hip_ext.h>
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
// -0 and +0 share a key; NaN gets 1 and ranks below every number (the keys
// of numbers are at least 0x007FFFFF).  Key 0 stands for "no slot".
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag == 0) u = 0;
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return mag > 0x7F800000u ? 1u : k;
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

// ------------------------------------------------------ Top-K summaries
// A row of more than 16384 and at most 131072 slots (with K <= 2048) gets a
// summary from the indexer's epilogue, or from the standalone summary pass:
// its slots are cut into segments of G = sum_seg(L) slots (16, 32 or 64:
// the smallest that makes at most 2048 segments), and for each segment
//  - the kSumM largest keys with their offsets in the segment, in slot
//    order (key 0 fills the entries of a segment shorter than kSumM), and
//  - the largest key not among them (the segment's next key; 0 if none).
// Equal keys are taken together, so ties can put more than kSumM keys among
// the largest; such a segment keeps its first kSumM of them and gets the
// largest key value as its next key, which makes the selection re-read it.
// The selection (topk_select.h) works from it.  With K <= 2048 a segment
// holds on average G K / L <= 2 of the row's K largest keys, so its next key
// seldom reaches the selection threshold; when it does, the selection
// re-reads that segment's scores.
constexpr int kSumM = 8;                        // entries per segment
constexpr int kSumSegMax = 2048;                // segments per row, at most
constexpr int kSumEntries = kSumM * kSumSegMax; // 16384 per row
constexpr int kSumMinLen = 16385;
constexpr int kSumMaxLen = 131072;
constexpr int kSumMaxK = 2048;
__host__ __device__ inline int sum_seg(int L) {
  int G = 16;
  while (G < 64 && (L + G - 1) / G > kSumSegMax) G <<= 1;
  return G;
}
__host__ __device__ inline bool sum_row(int L, int K) {
  return K <= kSumMaxK && L >= kSumMinLen && L <= kSumMaxLen;
}

// The summaries of a pass of rows, carved from a workspace: keys
// [rows][kSumEntries] (uint32, laid out by sum_key_index), offsets
// [rows][kSumSegMax][kSumM] (uint8), next keys [rows][kSumSegMax] (uint32).
//
// Key layout within a row: segments go in pairs (2p, 2p + 1), whose 16
// entries j = 8 (sg & 1) + e form four chunks of four keys; chunk c of pair
// p sits at (c * kSumSegMax / 2 + p) * 4.  A selecting workgroup of 1024
// threads holds one pair per thread, so each of its four key loads reads
// 16 contiguous bytes per lane, a kilobyte per wave.
__host__ __device__ inline int sum_key_index(int sg, int e) {
  const int j = ((sg & 1) << 3) | e;
  return (((j >> 2) * (kSumSegMax / 2) + (sg >> 1)) << 2) | (j & 3);
}
struct Summary {
  uint32_t* key;
  uint8_t* off;
  uint32_t* next;
};
size_t summary_bytes(int rows);
Summary summary_carve(void* base, int rows);

// Maximum over aligned groups of G lanes (16, 32 or 64) of two values at
// once, x and y, each in every lane of its group.  Within a row of 16 lanes
// four DPP steps per value, interleaved so that each fills the other's wait
// states.  Across rows one v_permlane16_swap of x with y leaves, after a
// max, x's pair-of-rows maxima in the even rows and y's in the odd rows (row
// 2i + v holds the max of rows 2i, 2i + 1 of value v); for G = 64 a
// v_permlane32_swap folds the two halves of the wave the same way.  A last
// v_permlane16_swap spreads the even rows to every lane (x) and the odd rows
// (y).
template <int G>
__device__ __forceinline__ void group_max2_u32(uint32_t& x, uint32_t& y) {
  static_assert(G == 16 || G == 32 || G == 64, "segment size");
#define DSA_GMAX_DPP(ctrl)                                                                   \
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, ctrl, 0xF, 0xF, false));     \
  y = max(y, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)y, ctrl, 0xF, 0xF, false));
  DSA_GMAX_DPP(0xB1)   // quad_perm [1,0,3,2]
  DSA_GMAX_DPP(0x4E)   // quad_perm [2,3,0,1]
  DSA_GMAX_DPP(0x141)  // row_half_mirror
  DSA_GMAX_DPP(0x140)  // row_mirror
#undef DSA_GMAX_DPP
  if constexpr (G >= 32) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    uint32_t c = max((uint32_t)p[0], (uint32_t)p[1]);
    if constexpr (G == 64) {
      const auto q = __builtin_amdgcn_permlane32_swap(c, c, false, false);
      c = max((uint32_t)q[0], (uint32_t)q[1]);
    }
    const auto r = __builtin_amdgcn_permlane16_swap(c, c, false, false);
    x = (uint32_t)r[0];
    y = (uint32_t)r[1];
  }
}

// The summary of one half of a wave's 128 slots (64 slots, one per lane),
// as this lane's share: whether its key is taken, its rank among the taken
// keys of its segment, how many were taken there, and the segment's next
// key.  G = sum_seg(S) lanes form a segment.
struct HalfSummary {
  bool taken;
  int rank, count;
  uint32_t next;
};
__device__ __forceinline__ HalfSummary summary_finish(bool t, uint32_t rest_max, int G) {
  const int lane = (int)(threadIdx.x & 63);
  const int base = lane & ~(G - 1);
  const uint64_t gmask = G == 64 ? ~0ull : ((1ull << G) - 1ull) << base;
  const uint64_t m = __ballot(t) & gmask;
  HalfSummary hs;
  hs.taken = t;
  hs.rank = lane_prefix(m);
  hs.count = __popcll(m);
  hs.next = hs.count > kSumM ? ~0u : rest_max;
  return hs;
}
// Both halves' summaries; ka and kb are the keys of this lane's slot in
// each half (0 past the row; keys of slots are at least 1).  kSumM rounds
// each take, in every segment, all keys equal to the largest key left;
// then the next key is the largest key not taken.  Registers only.
template <int G>
__device__ __forceinline__ void summary_halves_g(uint32_t ka, uint32_t kb, HalfSummary& ha,
                                                 HalfSummary& hb) {
  bool ta = false, tb = false;
#pragma unroll
  for (int i = 0; i < kSumM; ++i) {
    uint32_t ma = ka, mb = kb;
    group_max2_u32<G>(ma, mb);
    const bool ea = ka != 0u && ka == ma, eb = kb != 0u && kb == mb;
    ta = ta || ea;
    tb = tb || eb;
    ka = ea ? 0u : ka;
    kb = eb ? 0u : kb;
  }
  group_max2_u32<G>(ka, kb);
  ha = summary_finish(ta, ka, G);
  hb = summary_finish(tb, kb, G);
}
__device__ __forceinline__ void summary_halves(uint32_t ka, uint32_t kb, int G, HalfSummary& ha,
                                               HalfSummary& hb) {
  if (G == 64)
    summary_halves_g<64>(ka, kb, ha, hb);
  else if (G == 32)
    summary_halves_g<32>(ka, kb, ha, hb);
  else
    summary_halves_g<16>(ka, kb, ha, hb);
}

// Writes a half's summary: slots h0 .. h0 + 63 (h0 a multiple of 64, the
// half's first slot) of row `row` of a row of S slots, this lane's key k.
// The taken keys go out in slot order (the first kSumM of them), then zero
// entries up to kSumM.
__device__ __forceinline__ void summary_store(const HalfSummary& hs, uint32_t k, int h0, int S,
                                              int G, const Summary& sum, int64_t row) {
  const int lane = (int)(threadIdx.x & 63);
  const int base = lane & ~(G - 1), i = lane - base;
  if (h0 + base >= S) return;
  const int sg = (h0 + base) / G;
  uint32_t* kd = sum.key + row * kSumEntries;
  uint8_t* od = sum.off + row * kSumEntries + sg * kSumM;
  if (hs.taken && hs.rank < kSumM) {
    kd[sum_key_index(sg, hs.rank)] = k;
    od[hs.rank] = (uint8_t)i;
  }
  if (i >= hs.count && i < kSumM) {
    kd[sum_key_index(sg, i)] = 0u;
    od[i] = 0;
  }
  if (i == 0) sum.next[row * kSumSegMax + sg] = hs.next;
}

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
  Summary sum;                  // summaries for a Top-K of topk_K that follows,
  int32_t topk_K;               // or nothing when sum.key is NULL
};
// Optional timing of a launch: `start` takes the time its (first) kernel
// begins and `stop` the time its (last) kernel ends, stamped by the
// dispatch itself (hipExtLaunchKernel), so no marker sits between kernels.
struct StageEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// kernel<<<g, b, 0, s>>>(args...), through hipExtLaunchKernel when either
// event is set.
template <class... A>
hipError_t launch_kernel(void (*kernel)(A...), dim3 g, dim3 b, hipStream_t s, hipEvent_t start,
                         hipEvent_t stop, A... args) {
  if (!start && !stop) {
    kernel<<<g, b, 0, s>>>(args...);
    return hipGetLastError();
  }
  void* argv[] = {static_cast<void*>(&args)...};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), g, b, argv, 0, s, start, stop,
                            0);
}

hipError_t launch_indexer_scores(const IndexerLaunch& a, hipStream_t s, StageEvents ev = {});

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
  Summary sum;          // the rows' summaries
  bool prep;            // write the summaries here (no fused indexer before)
  bool vec;             // every score row is 16-byte aligned (ld % 4 == 0)
  // Optional: also write each kept position's byte offset in the paged KV
  // cache `kv` (block table -> physical block), -1 for padding and for
  // positions whose block id is out of range, to rowoff[num_rows][K].
  int64_t* rowoff;
  dsa_paged kv;
};
hipError_t launch_topk(const TopkLaunch& a, hipStream_t s, StageEvents ev = {});

struct AttnLaunch {
  RowMap rows;
  const uint16_t* q;
  dsa_paged k, v;
  bool latent;  // v aliases k (same base and strides)
  bool kv8;     // the (latent) cache holds E4M3 rows with tile scales (DSA_KV_FP8)
  // The selection: indices [.][K] (row row_begin + i at row indices_row_offset
  // + i); or, for the latent layout, the kept rows' byte offsets in the KV
  // cache as the Top-K wrote them (rowoff [num_rows][K], -1 = absent),
  // which replace the index -> block table lookup.
  const int32_t* indices;
  int64_t indices_row_offset;
  const int64_t* rowoff;
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
// layout (latent or not) and the cache format (kv8: FP8 rows) select, and
// the most any of them may use (for workspace sizes, which do not know the
// layout or the format).
int attn_chunks(int num_rows, int H_q, int D_qk, int K, bool latent, bool kv8);
int attn_chunks_max(int num_rows, int H_q, int D_qk, int K);
size_t attn_partial_bytes(int num_rows, int H_q, int D_v, int n_chunks);
// whether launch_sparse_attn reads row offsets (AttnLaunch.rowoff) for this
// shape and layout
bool attn_uses_rowoff(int D_qk, int D_v, bool latent);
// `ev` times the attention kernel, `merge` the split-key merge (with one
// chunk per row there is no merge kernel: both its events are recorded on
// the stream right after the attention)
hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s, StageEvents ev = {},
                              StageEvents merge = {});

}  // namespace dsa
