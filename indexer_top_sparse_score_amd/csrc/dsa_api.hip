// C-ABI front end of libdsa.so: argument validation, workspace sizing and
// the launch sequence of each entry point.  Validation touches no HIP API,
// so every error code can be produced on a machine without a GPU.

#include <cmath>
#include <cstdint>
#include <mutex>

#include "dsa_common.h"
#include "prolog.h"

namespace dsa {
namespace {

constexpr size_t kHeader = 256;                    // error word + reserved
// Fused step: score rows (and summaries) kept per pass of rows.  Chunked
// prefill batches of thousands of rows are cut into passes whose score slab
// stays within the 256 MB Infinity Cache.
constexpr size_t kScoresBudget = size_t(128) << 20;

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int check_rows(const dsa_problem* p) {
  if (!p) return DSA_ERR_INVALID;
  if (p->num_rows < 0 || p->num_seqs < 1 || p->max_blocks < 1) return DSA_ERR_INVALID;
  if (!p->seq_lens || !p->block_table) return DSA_ERR_INVALID;
  if (!aligned(p->seq_lens, 4) || !aligned(p->block_table, 4)) return DSA_ERR_INVALID;
  if ((p->row_seq && !aligned(p->row_seq, 4)) || (p->row_pos && !aligned(p->row_pos, 4)))
    return DSA_ERR_INVALID;
  if (p->block_size != DSA_BLOCK_SIZE) return DSA_ERR_UNSUPPORTED;
  if (p->max_blocks > (1 << 24)) return DSA_ERR_UNSUPPORTED;
  if (!p->cand != !p->cand_len) return DSA_ERR_INVALID;  // both or neither
  if (p->cand && (p->n_cand < 1 || !aligned(p->cand, 16) || !aligned(p->cand_len, 4)))
    return DSA_ERR_INVALID;
  if (p->cand && p->n_cand > (1 << 24)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

int check_indexer_shape(const dsa_problem* p) {
  if (p->H_I < 1 || p->D_I < 1) return DSA_ERR_INVALID;
  if (p->H_I > 64) return DSA_ERR_UNSUPPORTED;
  if (p->D_I != 64 && p->D_I != 128) return DSA_ERR_UNSUPPORTED;
  if (p->indexer_format == DSA_INDEXER_E4M3) {
    if (p->qI_scale) return DSA_ERR_INVALID;
  } else if (p->indexer_format == DSA_INDEXER_MXFP8) {
    if (!p->qI_scale) return DSA_ERR_INVALID;
  } else {
    return DSA_ERR_INVALID;
  }
  return DSA_OK;
}

int check_attn_shape(const dsa_problem* p) {
  if (p->H_q < 1 || p->D_qk < 1 || p->D_v < 1 || p->K < 1) return DSA_ERR_INVALID;
  if (!std::isfinite(p->scale)) return DSA_ERR_INVALID;
  if (p->H_q > 128) return DSA_ERR_UNSUPPORTED;
  // a row's index list is split into at most 64 chunks of at most 256 slots
  if (p->K > DSA_MAX_ATTN_K) return DSA_ERR_UNSUPPORTED;
  const bool small = p->D_qk == 64 && p->D_v == 64;
  const bool mla = p->D_qk == 576 && p->D_v == 512;
  if (!small && !mla) return DSA_ERR_UNSUPPORTED;
  if (p->kv_format != DSA_KV_BF16 && p->kv_format != DSA_KV_FP8) return DSA_ERR_INVALID;
  if (p->kv_format == DSA_KV_FP8 && !mla) return DSA_ERR_UNSUPPORTED;  // latent 576/512 only
  return DSA_OK;
}

int check_paged(const dsa_paged& c, int64_t row_bytes) {
  if (!c.base || !aligned(c.base, 16)) return DSA_ERR_INVALID;
  if (c.num_blocks < 1 || c.block_stride <= 0 || c.row_stride <= 0) return DSA_ERR_INVALID;
  if (c.block_stride % 16 || c.row_stride % 16) return DSA_ERR_INVALID;
  if (c.row_stride < row_bytes) return DSA_ERR_INVALID;
  // kernels address the rows of one block with 32-bit offsets
  if (c.row_stride > (int64_t(1) << 24)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

// The index-key cache: D_I code bytes per row; MXFP8 blocks also hold the
// 64 rows' scales (D_I / 32 bytes each) after the code rows.
int check_kI(const dsa_problem* p, const dsa_paged& kI) {
  int st = check_paged(kI, p->D_I);
  if (st != DSA_OK) return st;
  if (p->indexer_format == DSA_INDEXER_MXFP8 &&
      kI.block_stride < 64 * kI.row_stride + 2 * (int64_t)p->D_I)
    return DSA_ERR_INVALID;
  return DSA_OK;
}

// The prolog writes MXFP8 operands: the indexer shape with that format.
int check_prolog_shape(const dsa_problem* p) {
  if (p->indexer_format != DSA_INDEXER_MXFP8) return DSA_ERR_INVALID;
  if (p->H_I < 1 || p->D_I < 1) return DSA_ERR_INVALID;
  if (p->H_I > 64) return DSA_ERR_UNSUPPORTED;
  if (p->D_I != 64 && p->D_I != 128) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return DSA_ERR_INVALID;
  return DSA_OK;
}

RowMap row_map(const dsa_problem* p) {
  RowMap m;
  m.seq_lens = p->seq_lens;
  m.block_table = p->block_table;
  m.row_seq = p->row_seq;
  m.row_pos = p->row_pos;
  m.num_seqs = p->num_seqs;
  m.max_blocks = p->max_blocks;
  m.cand = p->cand;
  m.cand_len = p->cand_len;
  m.n_cand = p->cand ? p->n_cand : 0;
  return m;
}

// Length of a score row: the candidate list's, or the longest history.
int64_t max_len(const dsa_problem* p) {
  return p->cand ? (int64_t)p->n_cand : (int64_t)p->max_blocks * DSA_BLOCK_SIZE;
}

// Row stride of the fused step's score slab: a multiple of 64 floats, so
// every row is 256-byte aligned.
int64_t slab_ld(const dsa_problem* p) { return (max_len(p) + 63) & ~int64_t(63); }


// Whether any row of the problem can have a summary (more than 16384 slots).
bool needs_summary(const dsa_problem* p) { return max_len(p) >= kSumMinLen && p->K <= kSumMaxK; }

int rows_per_pass(const dsa_problem* p, size_t budget = kScoresBudget) {
  const size_t per_row = (size_t)slab_ld(p) * sizeof(float) +
                         (needs_summary(p) ? (size_t)kSumEntries * 5 : 0);
  size_t rp = budget / per_row;
  // a multiple of 128 rows when there is room for more: the attention of 16
  // rows and more runs two workgroups per row, so 128 rows fill one round
  // of the 256 CUs (390 rows per pass left 12 workgroups alone in a fourth
  // round)
  if (rp > 128) rp = rp / 128 * 128;
  if (rp < 1) rp = 1;
  if (rp > (size_t)p->num_rows) rp = (size_t)p->num_rows;
  return (int)rp;
}

bool is_latent(const dsa_paged& k, const dsa_paged& v) {
  return k.base == v.base && k.block_stride == v.block_stride && k.row_stride == v.row_stride;
}

int status_of(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

struct DecodeLayout {
  int rp;
  size_t idx_off, roff_off, scores_off, sum_off, part_off, total;
};

// Workspace of the fused step, per pass of rows: the selection, the selected
// rows' byte offsets in the KV cache (for the latent layout; reserved for
// every shape so that the size does not depend on the caches' strides), the
// float32 score slab, the rows' Top-K summaries and the attention's
// split-key partials.
DecodeLayout decode_layout(const dsa_problem* p, size_t budget = kScoresBudget) {
  DecodeLayout d;
  d.rp = rows_per_pass(p, budget);
  const int nc = attn_chunks_max(d.rp, p->H_q, p->D_qk, p->K);
  d.idx_off = kHeader;
  d.roff_off = d.idx_off + round256((size_t)d.rp * p->K * sizeof(int32_t));
  d.scores_off = d.roff_off + round256((size_t)d.rp * p->K * sizeof(int64_t));
  d.sum_off = d.scores_off + round256((size_t)d.rp * slab_ld(p) * sizeof(float));
  d.part_off = d.sum_off + round256(needs_summary(p) ? summary_bytes(d.rp) : 0);
  d.total = d.part_off + round256(attn_partial_bytes(d.rp, p->H_q, p->D_v, nc));
  return d;
}

int check_attn_args(const dsa_problem* p, const uint16_t* q, const dsa_paged& k,
                           const dsa_paged& v, uint16_t* out, float* lse) {
  int st = check_attn_shape(p);
  if (st != DSA_OK) return st;
  if (!q || !out) return DSA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(out, 16) || (lse && !aligned(lse, 4))) return DSA_ERR_INVALID;
  if (p->kv_format == DSA_KV_FP8) {
    // E4M3 rows of D_qk codes serving as K and V (the latent layout), each
    // block's 64 rows of float32 tile scales after its code rows
    if (p->D_qk != 576 || p->D_v != 512) return DSA_ERR_UNSUPPORTED;
    if (!is_latent(k, v)) return DSA_ERR_INVALID;
    if ((st = check_paged(k, p->D_qk)) != DSA_OK) return st;
    const int64_t tiles = (p->D_qk + 127) / 128;
    if (k.block_stride < 64 * k.row_stride + 64 * 4 * tiles) return DSA_ERR_INVALID;
    // the attention kernel keeps a gathered row as (block id, row) in 32 bits
    if (k.num_blocks > (int64_t(1) << 26)) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
  }
  if (p->kv_format != DSA_KV_BF16) return DSA_ERR_INVALID;
  if ((st = check_paged(k, 2 * (int64_t)p->D_qk)) != DSA_OK) return st;
  if ((st = check_paged(v, 2 * (int64_t)p->D_v)) != DSA_OK) return st;
  // the latent kernel keeps each gathered row's offset in 32 bits of 16-byte
  // units: its cache spans at most 64 GiB
  if (is_latent(k, v) && (int64_t)k.num_blocks * k.block_stride > (int64_t(1) << 36))
    return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

// The layout the attention kernels gather by DMA: rows shared by K and V
// (bf16, or FP8 codes with their tile scales).
bool dma_latent(const dsa_problem*, const dsa_paged& k, const dsa_paged& v) {
  return is_latent(k, v);
}

AttnLaunch attn_launch(const dsa_problem* p, const uint16_t* q, dsa_paged k, dsa_paged v,
                              uint16_t* out, float* lse, uint32_t* err) {
  AttnLaunch a;
  a.rows = row_map(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.latent = is_latent(k, v);
  a.kv8 = p->kv_format == DSA_KV_FP8;
  a.indices = nullptr;
  a.indices_row_offset = 0;
  a.rowoff = nullptr;
  a.out = out;
  a.lse = lse;
  a.partial = nullptr;
  a.err = err;
  a.H_q = p->H_q;
  a.D_qk = p->D_qk;
  a.D_v = p->D_v;
  a.K = p->K;
  a.scale = p->scale;
  a.row_begin = 0;
  a.num_rows = p->num_rows;
  a.n_chunks = 1;
  return a;
}

// Validation shared by both fused-step entry points (everything but the
// workspace).
int check_decode_args(const dsa_problem* p, const uint8_t* qI, const float* w,
                      const dsa_paged& kI, const uint16_t* q, const dsa_paged& k,
                      const dsa_paged& v, uint16_t* out, float* lse, int32_t* indices_out,
                      int32_t* counts_out) {
  int st = check_rows(p);
  if (st != DSA_OK) return st;
  if ((st = check_indexer_shape(p)) != DSA_OK) return st;
  if ((st = check_attn_args(p, q, k, v, out, lse)) != DSA_OK) return st;
  if (!qI || !w || !aligned(qI, 16) || !aligned(w, 4)) return DSA_ERR_INVALID;
  if ((st = check_kI(p, kI)) != DSA_OK) return st;
  if ((indices_out && !aligned(indices_out, 4)) || (counts_out && !aligned(counts_out, 4)))
    return DSA_ERR_INVALID;
  return DSA_OK;
}

// The fused step itself, on a workspace `base` laid out as `d`; device-side
// errors are OR-ed into *err.  With `ev` (eight events), the last pass of
// rows stamps the start and end of its scan (ev[0], ev[1]), selection
// (ev[2], ev[3]), attention (ev[4], ev[5]) and merge (ev[6], ev[7]).
int decode_run(const dsa_problem* p, const uint8_t* qI, const float* w, dsa_paged kI,
               const uint16_t* q, dsa_paged k, dsa_paged v, uint16_t* out, float* lse,
               int32_t* indices_out, int32_t* counts_out, char* base, const DecodeLayout& d,
               uint32_t* err, hipStream_t s, const hipEvent_t* ev = nullptr) {
  int st = DSA_OK;
  float* scores = reinterpret_cast<float*>(base + d.scores_off);
  const int64_t ld = slab_ld(p);
  const Summary sum = needs_summary(p) ? summary_carve(base + d.sum_off, d.rp)
                                       : Summary{nullptr, nullptr, nullptr};
  const bool use_rowoff = attn_uses_rowoff(p->D_qk, p->D_v, dma_latent(p, k, v));
  int64_t* roff = reinterpret_cast<int64_t*>(base + d.roff_off);

  // Four launches per pass of rows: indexer scan (scores and summaries),
  // Top-K selection, sparse attention, split-key merge.
  for (int row0 = 0; row0 < p->num_rows; row0 += d.rp) {
    const int nr = p->num_rows - row0 < d.rp ? p->num_rows - row0 : d.rp;
    int32_t* idx = indices_out ? indices_out + (int64_t)row0 * p->K
                               : reinterpret_cast<int32_t*>(base + d.idx_off);
    const hipEvent_t* tev = ev && row0 + nr >= p->num_rows ? ev : nullptr;
    auto stage = [&](int i) {
      StageEvents e;
      if (tev) e = StageEvents{tev[2 * i], tev[2 * i + 1]};
      return e;
    };

    IndexerLaunch ia;
    ia.rows = row_map(p);
    ia.qI = qI;
    ia.w = w;
    ia.kI = kI;
    ia.scores = scores;
    ia.ld = ld;
    ia.err = err;
    ia.H_I = p->H_I;
    ia.D_I = p->D_I;
    ia.qI_scale = p->qI_scale;
    ia.row_begin = row0;
    ia.num_rows = nr;
    ia.max_len = (int32_t)max_len(p);
    ia.sum = sum;
    ia.topk_K = p->K;
    if ((st = status_of(launch_indexer_scores(ia, s, stage(0)))) != DSA_OK) return st;

    TopkLaunch ta;
    ta.rows = row_map(p);
    ta.scores = scores;
    ta.ld = ld;
    ta.indices = idx;
    ta.counts = counts_out ? counts_out + row0 : nullptr;
    ta.err = err;
    ta.K = p->K;
    ta.row_begin = row0;
    ta.num_rows = nr;
    ta.max_len = (int32_t)max_len(p);
    ta.sum = sum;
    ta.prep = false;  // the indexer wrote the summaries
    ta.vec = true;    // 256-byte aligned slab, ld a multiple of 64
    ta.rowoff = use_rowoff ? roff : nullptr;
    ta.kv = k;
    if ((st = status_of(launch_topk(ta, s, stage(1)))) != DSA_OK) return st;

    AttnLaunch aa = attn_launch(p, q, k, v, out, lse, err);
    aa.indices = idx;
    aa.indices_row_offset = 0;
    aa.rowoff = use_rowoff ? roff : nullptr;
    aa.row_begin = row0;
    aa.num_rows = nr;
    // the workspace holds partials for the larger of the two layouts' counts
    aa.n_chunks = attn_chunks(d.rp, p->H_q, p->D_qk, p->K, aa.latent, aa.kv8);
    aa.partial = aa.n_chunks > 1 ? static_cast<void*>(base + d.part_off) : nullptr;
    if ((st = status_of(launch_sparse_attn(aa, s, stage(2), stage(3)))) != DSA_OK) return st;
  }
  return DSA_OK;
}


// ------------------------------------------------- allocation-free entry point
// The library's own scratch for dsa_decode_step_static: a file-scope device
// array, one copy on every GPU the library runs on, held until the process
// ends.  Host code never uses the array's name as an address: its device
// address on the current GPU comes from hipGetSymbolAddress, once per
// device.
static __device__ __align__(256) uint8_t scratch[DSA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev >= 0 && dev < kMaxDevices && g_scratch_ptr[dev]) {
    *out = g_scratch_ptr[dev];
    return DSA_OK;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DSA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) g_scratch_ptr[dev] = static_cast<char*>(ptr);
  *out = static_cast<char*>(ptr);
  return DSA_OK;
}

// The fused step's layout with a score budget small enough that the whole
// workspace fits the scratch (fewer rows per pass), or false when even one
// row per pass does not fit.
bool static_layout(const dsa_problem* p, DecodeLayout& d) {
  for (size_t budget = kScoresBudget; budget >= 4096; budget /= 2) {
    d = decode_layout(p, budget);
    if (d.total <= (size_t)DSA_STATIC_SCRATCH_BYTES) return true;
    if (d.rp == 1) break;
  }
  return false;
}

}  // namespace
}  // namespace dsa

using namespace dsa;

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t dsa_workspace_size(const dsa_problem* p, int op) {
  if (check_rows(p) != DSA_OK) return 0;
  switch (op) {
    case DSA_OP_INDEXER_SCORES:
      return check_indexer_shape(p) == DSA_OK ? kHeader : 0;
    case DSA_OP_TOPK:
      if (p->K < 1) return 0;
      return kHeader + round256(needs_summary(p) ? summary_bytes(p->num_rows) : 0);
    case DSA_OP_SPARSE_ATTN: {
      if (check_attn_shape(p) != DSA_OK) return 0;
      const int nc = attn_chunks_max(p->num_rows, p->H_q, p->D_qk, p->K);
      return kHeader + round256(attn_partial_bytes(p->num_rows, p->H_q, p->D_v, nc));
    }
    case DSA_OP_DECODE_STEP:
      if (check_indexer_shape(p) != DSA_OK || check_attn_shape(p) != DSA_OK) return 0;
      if (p->num_rows == 0) return kHeader;
      return decode_layout(p).total;
    case DSA_OP_INDEXER_PROLOG:
      return check_prolog_shape(p) == DSA_OK ? kHeader : 0;
    default:
      return 0;
  }
}

int dsa_indexer_prolog(const dsa_problem* p, int32_t D_x, float eps, const uint16_t* x,
                       const uint16_t* w_q, const uint16_t* w_g, const uint16_t* k_new,
                       const uint16_t* k_gamma, uint8_t* qI, uint8_t* qI_scale, float* w,
                       dsa_paged kI, void* ws, size_t ws_bytes, void* stream) {
  int st = check_rows(p);
  if (st != DSA_OK) return st;
  if ((st = check_prolog_shape(p)) != DSA_OK) return st;
  if (D_x < 32 || D_x % 32) return DSA_ERR_INVALID;
  if (D_x > 65536) return DSA_ERR_UNSUPPORTED;
  if (!std::isfinite(eps) || eps < 0.0f) return DSA_ERR_INVALID;
  if (!x || !w_q || !w_g || !k_new || !k_gamma || !qI || !qI_scale || !w) return DSA_ERR_INVALID;
  if (!aligned(x, 16) || !aligned(w_q, 16) || !aligned(w_g, 16) || !aligned(qI, 16) ||
      !aligned(k_new, 4) || !aligned(k_gamma, 4) || !aligned(w, 4))
    return DSA_ERR_INVALID;
  if ((st = check_kI(p, kI)) != DSA_OK) return st;
  if ((st = check_ws(ws, ws_bytes, kHeader)) != DSA_OK) return st;
  if (p->num_rows == 0) return DSA_OK;
  PrologLaunch a;
  a.rows = row_map(p);
  a.rows.cand = nullptr;  // the prolog writes each row's own position
  a.rows.cand_len = nullptr;
  a.rows.n_cand = 0;
  a.x = x;
  a.w_q = w_q;
  a.w_g = w_g;
  a.k_new = k_new;
  a.k_gamma = k_gamma;
  a.qI = qI;
  a.qI_scale = qI_scale;
  a.w = w;
  a.kI = static_cast<uint8_t*>(const_cast<void*>(kI.base));
  a.kI_block_stride = kI.block_stride;
  a.kI_row_stride = kI.row_stride;
  a.kI_num_blocks = kI.num_blocks;
  a.err = static_cast<uint32_t*>(ws);
  a.num_rows = p->num_rows;
  a.D_x = D_x;
  a.H_I = p->H_I;
  a.D_I = p->D_I;
  a.eps = eps;
  return status_of(launch_indexer_prolog(a, static_cast<hipStream_t>(stream)));
}

int dsa_indexer_scores(const dsa_problem* p, const uint8_t* qI, const float* w, dsa_paged kI,
                       float* scores, int64_t ld_scores, void* ws, size_t ws_bytes,
                       void* stream) {
  int st = check_rows(p);
  if (st != DSA_OK) return st;
  if ((st = check_indexer_shape(p)) != DSA_OK) return st;
  if (!qI || !w || !scores) return DSA_ERR_INVALID;
  if (!aligned(qI, 16) || !aligned(w, 4) || !aligned(scores, 4)) return DSA_ERR_INVALID;
  if ((st = check_kI(p, kI)) != DSA_OK) return st;
  if (ld_scores < max_len(p)) return DSA_ERR_INVALID;
  if ((st = check_ws(ws, ws_bytes, kHeader)) != DSA_OK) return st;
  if (p->num_rows == 0) return DSA_OK;
  IndexerLaunch a;
  a.rows = row_map(p);
  a.qI = qI;
  a.w = w;
  a.kI = kI;
  a.scores = scores;
  a.ld = ld_scores;
  a.err = static_cast<uint32_t*>(ws);
  a.H_I = p->H_I;
  a.D_I = p->D_I;
  a.qI_scale = p->qI_scale;
  a.row_begin = 0;
  a.num_rows = p->num_rows;
  a.max_len = (int32_t)max_len(p);
  a.sum = Summary{nullptr, nullptr, nullptr};
  a.topk_K = 0;
  return status_of(launch_indexer_scores(a, static_cast<hipStream_t>(stream)));
}

int dsa_topk(const dsa_problem* p, const float* scores, int64_t ld_scores, int32_t* indices,
             int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  int st = check_rows(p);
  if (st != DSA_OK) return st;
  if (p->K < 1) return DSA_ERR_INVALID;
  if (!scores || !indices) return DSA_ERR_INVALID;
  if (!aligned(scores, 4) || !aligned(indices, 4) || (counts && !aligned(counts, 4)))
    return DSA_ERR_INVALID;
  if (ld_scores < max_len(p)) return DSA_ERR_INVALID;
  if ((st = check_ws(ws, ws_bytes, dsa_workspace_size(p, DSA_OP_TOPK))) != DSA_OK) return st;
  if (p->num_rows == 0) return DSA_OK;
  TopkLaunch a;
  a.rows = row_map(p);
  a.scores = scores;
  a.ld = ld_scores;
  a.indices = indices;
  a.counts = counts;
  a.err = static_cast<uint32_t*>(ws);
  a.K = p->K;
  a.row_begin = 0;
  a.num_rows = p->num_rows;
  a.max_len = (int32_t)max_len(p);
  a.sum = needs_summary(p) ? summary_carve(static_cast<char*>(ws) + kHeader, p->num_rows)
                           : Summary{nullptr, nullptr, nullptr};
  a.prep = a.sum.key != nullptr;
  a.vec = aligned(scores, 16) && ld_scores % 4 == 0;
  a.rowoff = nullptr;
  a.kv = dsa_paged{};
  return status_of(launch_topk(a, static_cast<hipStream_t>(stream)));
}

int dsa_sparse_attn(const dsa_problem* p, const uint16_t* q, dsa_paged k, dsa_paged v,
                    const int32_t* indices, uint16_t* out, float* lse, void* ws,
                    size_t ws_bytes, void* stream) {
  int st = check_rows(p);
  if (st != DSA_OK) return st;
  if ((st = check_attn_args(p, q, k, v, out, lse)) != DSA_OK) return st;
  if (!indices || !aligned(indices, 4)) return DSA_ERR_INVALID;
  if ((st = check_ws(ws, ws_bytes, dsa_workspace_size(p, DSA_OP_SPARSE_ATTN))) != DSA_OK)
    return st;
  if (p->num_rows == 0) return DSA_OK;
  AttnLaunch a = attn_launch(p, q, k, v, out, lse, static_cast<uint32_t*>(ws));
  a.indices = indices;
  a.n_chunks = attn_chunks(p->num_rows, p->H_q, p->D_qk, p->K, a.latent, a.kv8);
  a.partial = a.n_chunks > 1
                  ? static_cast<void*>(static_cast<char*>(ws) + kHeader)
                  : nullptr;
  return status_of(launch_sparse_attn(a, static_cast<hipStream_t>(stream)));
}

int dsa_decode_step(const dsa_problem* p, const uint8_t* qI, const float* w, dsa_paged kI,
                    const uint16_t* q, dsa_paged k, dsa_paged v, uint16_t* out, float* lse,
                    int32_t* indices_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                    void* stream) {
  int st = check_decode_args(p, qI, w, kI, q, k, v, out, lse, indices_out, counts_out);
  if (st != DSA_OK) return st;
  if ((st = check_ws(ws, ws_bytes, dsa_workspace_size(p, DSA_OP_DECODE_STEP))) != DSA_OK)
    return st;
  if (p->num_rows == 0) return DSA_OK;
  char* base = static_cast<char*>(ws);
  return decode_run(p, qI, w, kI, q, k, v, out, lse, indices_out, counts_out, base,
                    decode_layout(p), reinterpret_cast<uint32_t*>(base),
                    static_cast<hipStream_t>(stream));
}

int dsa_decode_step_timed(const dsa_problem* p, const uint8_t* qI, const float* w, dsa_paged kI,
                          const uint16_t* q, dsa_paged k, dsa_paged v, uint16_t* out, float* lse,
                          int32_t* indices_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                          void* const* events, void* stream) {
  if (!events) return DSA_ERR_INVALID;
  hipEvent_t ev[8];
  for (int i = 0; i < 8; ++i) {
    if (!events[i]) return DSA_ERR_INVALID;
    ev[i] = static_cast<hipEvent_t>(events[i]);
  }
  int st = check_decode_args(p, qI, w, kI, q, k, v, out, lse, indices_out, counts_out);
  if (st != DSA_OK) return st;
  if ((st = check_ws(ws, ws_bytes, dsa_workspace_size(p, DSA_OP_DECODE_STEP))) != DSA_OK)
    return st;
  if (p->num_rows == 0) return DSA_OK;
  char* base = static_cast<char*>(ws);
  return decode_run(p, qI, w, kI, q, k, v, out, lse, indices_out, counts_out, base,
                    decode_layout(p), reinterpret_cast<uint32_t*>(base),
                    static_cast<hipStream_t>(stream), ev);
}

int dsa_decode_step_static(const dsa_problem* p, const uint8_t* qI, const float* w,
                           dsa_paged kI, const uint16_t* q, dsa_paged k, dsa_paged v,
                           uint16_t* out, float* lse, int32_t* indices_out, int32_t* counts_out,
                           uint32_t* err, void* stream) {
  int st = check_decode_args(p, qI, w, kI, q, k, v, out, lse, indices_out, counts_out);
  if (st != DSA_OK) return st;
  if (err && !aligned(err, 4)) return DSA_ERR_INVALID;
  if (p->num_rows == 0) return DSA_OK;
  // the fused step's layout with passes of rows small enough for the scratch
  DecodeLayout d;
  if (!static_layout(p, d)) return DSA_ERR_WORKSPACE;
  char* base = nullptr;
  if ((st = static_scratch(&base)) != DSA_OK) return st;
  // with no error word of the caller's, device-side errors go to the
  // scratch's header word, which nothing reads
  return decode_run(p, qI, w, kI, q, k, v, out, lse, indices_out, counts_out, base, d,
                    err ? err : reinterpret_cast<uint32_t*>(base),
                    static_cast<hipStream_t>(stream));
}

}  // extern "C"
