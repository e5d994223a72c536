/*
 * dsa.h -- C ABI of the MI355X (gfx950) indexer -> Top-K -> sparse-attention
 * library (libdsa.so).
 *
 * The method (Baidu AI Cloud, "Day0 Inference Support and Performance
 * Optimization for New Architecture LLMs", section 2.2): a lightweight
 * indexer scores each query row against every historical position, the
 * per-head scores are aggregated with per-head weights, the Top-K positions
 * are kept, and the sparse attention core reads only those KV rows.  The
 * indexer reads the paged K cache directly (section 4.1); the attention core
 * gathers the selected rows of the main KV cache from the indexer's position
 * list (section 4.2); the fused call takes the FP8 indexer query, the index
 * keys and the head weights and returns positions (section 4.3).
 * One KV latent row is shared by every query head ("SPLASH: Switching
 * Parallel Layouts of Attention with Seamless Handoff for LLM Serving",
 * section 2).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor argument is a DEVICE pointer owned by the caller.  The
 *   library never allocates, frees or retains memory, never synchronises
 *   and never reads device memory from the host.  Calls enqueue kernels on
 *   `stream` (a hipStream_t; NULL = the null stream) and return at once;
 *   they are capturable into a hipGraph.
 * - Validation is synchronous and happens before anything is enqueued: a
 *   negative dsa_status comes back and nothing runs.  A failed kernel launch
 *   returns DSA_ERR_HIP.  Faults during execution surface on the caller's
 *   next synchronisation.  Nothing is printed and no exception crosses the
 *   ABI.
 * - The library keeps no state; calls are reentrant.  Calls that overlap in
 *   time need separate workspaces.
 * - Row r of the problem is a query at absolute position p_r of sequence
 *   b_r.  Its history is positions 0 .. p_r inclusive (L_r = p_r + 1): the
 *   current token's own index key and KV row are already in the caches.
 *   Decode passes row_seq = row_pos = NULL (row r is sequence r at position
 *   seq_lens[r] - 1); chunked prefill passes both arrays.
 * - Paging: position s of sequence b lives in physical block
 *   block_table[b * max_blocks + s / 64], row s % 64.  The index-key cache and
 *   the KV cache share the block table.
 * - Device-side checks: a row whose sequence or position is out of range, a
 *   block id outside [0, num_blocks) or an attention index outside [-1, p_r]
 *   is never dereferenced.  The row, page or index is treated as absent and a
 *   DSA_DEVERR_* bit is OR-ed into the 32-bit error word at byte 0 of the
 *   workspace.  The word is sticky: the caller zeroes the workspace once after
 *   allocating it and may read the word back after synchronising.
 * - Alignment: qI, q, out and cache bases 16 bytes; cache strides multiples
 *   of 16 bytes; scores, w, lse, indices, counts 4 bytes; workspace 256.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define DSA_API __attribute__((visibility("default")))
#else
#define DSA_API
#endif

#define DSA_ABI_VERSION 8
#define DSA_BLOCK_SIZE 64
#define DSA_MAX_ATTN_K 16384 /* largest K of dsa_sparse_attn / dsa_decode_step */
#define DSA_STATIC_SCRATCH_BYTES (64u << 20) /* scratch of dsa_decode_step_static, per GPU */

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID = -1,     /* a NULL, misaligned, negative or inconsistent argument */
  DSA_ERR_UNSUPPORTED = -2, /* valid, but a shape this build does not implement      */
  DSA_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than dsa_workspace_size()    */
  DSA_ERR_HIP = -4          /* a kernel launch failed                                 */
} dsa_status;

/* bits of the sticky device error word at byte 0 of the workspace */
#define DSA_DEVERR_ROW 1u   /* row's sequence / position out of range: row treated as empty */
#define DSA_DEVERR_BLOCK 2u /* block id outside [0, num_blocks): page treated as absent      */
#define DSA_DEVERR_INDEX 4u /* attention index outside [-1, p_r]: index skipped              */

/* A paged cache: [num_blocks][64 rows][row bytes], rows at any stride. */
typedef struct {
  const void* base;     /* device address of physical block 0, row 0            */
  int64_t block_stride; /* bytes from one physical block to the next             */
  int64_t row_stride;   /* bytes from one row (token) to the next inside a block;
                           above 2^24: DSA_ERR_UNSUPPORTED                       */
  int64_t num_blocks;   /* number of physical blocks addressable from base       */
} dsa_paged;

/* Shapes and the row -> (sequence, position) map, shared by every call. */
typedef struct {
  int32_t num_seqs;           /* sequences in the batch (>= 1)                         */
  int32_t num_rows;           /* query rows (0 = nothing to do)                         */
  const int32_t* seq_lens;    /* [num_seqs] tokens in each sequence's caches            */
  const int32_t* block_table; /* [num_seqs][max_blocks] physical block ids              */
  int32_t max_blocks;         /* columns of block_table (>= 1)                          */
  int32_t block_size;         /* tokens per block; must be 64                           */
  const int32_t* row_seq;     /* [num_rows] sequence of each row, or NULL (row r -> r)  */
  const int32_t* row_pos;     /* [num_rows] position p_r, or NULL (seq_lens[b] - 1)     */
  int32_t H_I;                /* indexer heads, 1..64                                   */
  int32_t D_I;                /* indexer head dim, 64 or 128                            */
  int32_t H_q;                /* attention query heads, 1..128                          */
  int32_t D_qk;               /* attention q/k dim: 64 or 576                           */
  int32_t D_v;                /* attention v / output dim: 64 (with D_qk 64) or 512     */
  int32_t K;                  /* positions kept per row, >= 1 (attention: at most
                                 DSA_MAX_ATTN_K, else DSA_ERR_UNSUPPORTED)               */
  float scale;                /* attention logit scale, finite (e.g. 1/sqrt(D_qk))      */
  int32_t indexer_format;     /* DSA_INDEXER_E4M3 or DSA_INDEXER_MXFP8                  */
  const uint8_t* qI_scale;    /* MXFP8: [num_rows][H_I][D_I / 32] E8M0 scales of qI;
                                 NULL for E4M3                                          */
  /* Candidate-restricted indexer (vLLM's DeepSeek-V4.1-Flash article,
     "Kernels": later indexer layers score only a fixed set of candidate
     positions).  NULL cand: every row scores its whole history.          */
  const int32_t* cand;        /* [num_rows][n_cand] candidate positions of each row,
                                 ascending, each in 0 .. p_r                            */
  const int32_t* cand_len;    /* [num_rows] valid leading entries of each list, clamped
                                 to 0 .. n_cand; entries past it are not read           */
  int32_t n_cand;             /* row length of cand (>= 1 with cand)                    */
  int32_t kv_format;          /* DSA_KV_BF16 or DSA_KV_FP8 (see dsa_sparse_attn)        */
} dsa_problem;

/* indexer operand formats (dsa_problem.indexer_format) */
enum {
  DSA_INDEXER_E4M3 = 0,  /* unscaled E4M3 codes                                         */
  DSA_INDEXER_MXFP8 = 1  /* E4M3 codes with one E8M0 scale per group of 32 dims (Day0,
                            section 5.1); see dsa_indexer_scores                        */
};

/* KV cache formats (dsa_problem.kv_format) */
enum {
  DSA_KV_BF16 = 0, /* bf16 rows                                                          */
  DSA_KV_FP8 = 1   /* E4M3 rows with one float32 scale per tile of 128 elements (Day0,
                      section 5.2); latent 576/512 layout only; see dsa_sparse_attn     */
};

/* which call dsa_workspace_size() sizes */
enum {
  DSA_OP_INDEXER_SCORES = 0,
  DSA_OP_TOPK = 1,
  DSA_OP_SPARSE_ATTN = 2,
  DSA_OP_DECODE_STEP = 3,
  DSA_OP_INDEXER_PROLOG = 4
};

/* Bytes of workspace `op` needs for problem `p` (a multiple of 256, at least
 * 256), or 0 when the problem is invalid or unsupported.  Host-only. */
DSA_API size_t dsa_workspace_size(const dsa_problem* p, int op);

/*
 * Index scores (Day0 article, section 2.2, first two steps):
 *   scores[r * ld_scores + s] = sum_h w[r, h] * max(0, sum_d qI[r, h, d] * kI[s, d])
 * for s = 0 .. p_r, in float32; a zero score is stored as +0.
 *   qI      E4M3 (OCP FN) codes, [num_rows][H_I][D_I], row-major
 *   w       float32 head weights, [num_rows][H_I]
 *   kI      paged index-key cache, one D_I-byte E4M3 row per position,
 *           shared by all indexer heads
 *   scores  float32 [num_rows][ld_scores]; ld_scores >= 64 * max_blocks.
 *           Entries s > p_r are neither read nor written.
 * FP8 products are exact and accumulate in float32, so integer-valued inputs
 * whose partial sums stay below 2**24 give exact scores in any order.
 *
 * With indexer_format = DSA_INDEXER_MXFP8 (Day0 article, section 5.1: one
 * shared scale per group of 32 dims of Q and of K), the dims are cut into
 * groups g of 32 and each group of a query head and of a key row carries an
 * E8M0 scale byte e (the value 2**(e - 127); e = 255 is not allowed):
 *   sum_d qI[r, h, d] * kI[s, d]  becomes
 *   sum_g 2**(eq[r, h, g] + ek[s, g] - 254) * sum_{d in g} qI[r, h, d] * kI[s, d]
 *   eq      p->qI_scale, [num_rows][H_I][D_I / 32]
 *   ek      the scale area of each kI block, after its 64 rows of codes:
 *           ek[s, g] of the position s in row i of block b is the byte at
 *           b * block_stride + 64 * row_stride + i * (D_I / 32) + g, so a
 *           block holds 64 * row_stride bytes of codes and then 2 * D_I
 *           bytes of scales (block_stride >= 64 * row_stride + 2 * D_I,
 *           else DSA_ERR_INVALID).  The code rows keep their alignment and
 *           the scales of 64 positions are one contiguous run.
 * Power-of-two scales keep every product exact.
 *
 * With candidates (p->cand), row r scores its list instead: for slots
 * c = 0 .. cand_len[r] - 1, scores[r * ld_scores + c] is the score of
 * position cand[r][c], and ld_scores >= n_cand.  A list that is not
 * ascending inside 0 .. p_r gives unspecified scores for the offending
 * slots (a position outside the history sets DSA_DEVERR_ROW), never an
 * access outside the caches.
 */
DSA_API int dsa_indexer_scores(const dsa_problem* p, const uint8_t* qI, const float* w, dsa_paged kI,
                       float* scores, int64_t ld_scores, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * Top-K (Day0 article, section 2.2, third step): for each row keep the
 * min(K, L_r) positions with the largest score among scores[r, 0 .. p_r];
 * equal scores go to the lower position; -0 equals +0; NaN ranks last.
 *   indices  int32 [num_rows][K]: the kept positions in ascending order,
 *            then -1 up to K
 *   counts   int32 [num_rows] = min(K, L_r), or NULL
 * With candidates (p->cand) a row's scores are per slot (as
 * dsa_indexer_scores writes them), L_r = cand_len[r], and the kept slots are
 * written as their positions cand[r][c]: ascending, ties to the lower
 * position.
 */
DSA_API int dsa_topk(const dsa_problem* p, const float* scores, int64_t ld_scores, int32_t* indices,
             int32_t* counts, void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse MQA (Day0 article, sections 2.2 and 4.2): for each row and query
 * head h, softmax attention over the KV rows named in indices[r, 0 .. K-1]
 * (entries of -1 are skipped):
 *   logit_j = scale * sum_d q[r, h, d] * k_j[d]
 *   out[r, h, :] = sum_j exp(logit_j - m) v_j / sum_j exp(logit_j - m)
 *   lse[r, h]    = m + ln(sum_j exp(logit_j - m))       (natural log)
 * with m the largest logit.  A row with no valid index gives out = 0 and
 * lse = -inf.
 *   q        bf16 [num_rows][H_q][D_qk]
 *   k        paged cache of bf16 rows of D_qk elements
 *   v        paged cache of bf16 rows whose first D_v elements are V; pass
 *            the k descriptor again for the latent layout (V = the leading
 *            D_v columns of each K row; the cache, num_blocks * block
 *            stride bytes, may then span at most 64 GiB, else
 *            DSA_ERR_UNSUPPORTED)
 *   indices  int32 [num_rows][K]
 *   out      bf16 [num_rows][H_q][D_v]; lse float32 [num_rows][H_q] or NULL
 * Products are bf16 x bf16 with float32 accumulation; softmax in float32.
 *
 * With kv_format = DSA_KV_FP8 (Day0 article, section 5.2: FP8 KV quantised
 * per token in tiles of 128 elements), D_qk = 576, D_v = 512, and k and v
 * are the same descriptor (the latent layout, else DSA_ERR_INVALID).  A row
 * holds 576 E4M3 (OCP FN) codes at row_stride; the 64 rows of a block are
 * followed by their float32 tile scales, row i's five at
 * b * block_stride + 64 * row_stride + 20 * i (block_stride >= 64 *
 * row_stride + 1280, else DSA_ERR_INVALID).  Element d of a row has the
 * value code[d] * scale[d / 128]: four tiles of 128 and a last one of 64.
 * The kernel decodes each gathered element to bf16 (rounded to nearest
 * even) before the bf16 products.  NaN codes are not valid input.
 */
DSA_API int dsa_sparse_attn(const dsa_problem* p, const uint16_t* q, dsa_paged k, dsa_paged v,
                    const int32_t* indices, uint16_t* out, float* lse, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * The whole step, fused (Day0 article, sections 4.1-4.3): index scores,
 * Top-K and sparse MQA for every row, with the same results as calling the
 * three entry points above in turn.  Scores stay in the workspace.
 *   indices_out  int32 [num_rows][K] copy of the selection, or NULL
 *   counts_out   int32 [num_rows], or NULL
 * Other arguments as above.
 */
DSA_API int dsa_decode_step(const dsa_problem* p, const uint8_t* qI, const float* w, dsa_paged kI,
                    const uint16_t* q, dsa_paged k, dsa_paged v, uint16_t* out, float* lse,
                    int32_t* indices_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * dsa_decode_step with per-stage timing, for benchmarks: the same launches
 * and results, plus eight caller-created HIP events (hipEvent_t, passed as
 * void*) that the last pass of rows stamps with the start and end times of
 * its stages, taken by the kernel dispatches themselves:
 *   events[0], [1]  indexer scan        events[2], [3]  Top-K selection
 *   events[4], [5]  sparse attention    events[6], [7]  split-key merge
 * (with no merge kernel, [6] and [7] are recorded right after the attention),
 * so hipEventElapsedTime(events[2i], events[2i + 1]) is the duration of
 * stage i.  Not meant for graph capture.  events NULL, or any of the eight
 * NULL: DSA_ERR_INVALID and nothing runs.  Other arguments and errors as
 * dsa_decode_step.
 */
DSA_API int dsa_decode_step_timed(const dsa_problem* p, const uint8_t* qI, const float* w,
                                  dsa_paged kI, const uint16_t* q, dsa_paged k, dsa_paged v,
                                  uint16_t* out, float* lse, int32_t* indices_out,
                                  int32_t* counts_out, void* ws, size_t ws_bytes,
                                  void* const* events, void* stream);

/*
 * The fused step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Results are those of dsa_decode_step.
 * The call itself allocates nothing: the library keeps one scratch array of
 * DSA_STATIC_SCRATCH_BYTES on every GPU it runs on (reserved when the library
 * is loaded, held until the process ends) and lays the step out in it,
 * cutting the rows into smaller passes when needed.  A problem whose layout
 * does not fit even one row per pass returns DSA_ERR_WORKSPACE and nothing
 * runs.  The first call on a device looks the array's address up (a HIP
 * runtime query, no allocation).
 *   err  optional device pointer to a caller-owned uint32 into which the
 *        DSA_DEVERR_* bits are OR-ed (sticky, as the workspace error word of
 *        dsa_decode_step; the caller zeroes it); NULL: not reported
 * Every call on a GPU shares that GPU's scratch, and the scratch keeps the
 * last call's contents (nothing in it needs to start at zero): calls that
 * overlap in time on one GPU -- on different streams, or from different
 * threads -- race and give undefined results.  Serialise them.
 */
DSA_API int dsa_decode_step_static(const dsa_problem* p, const uint8_t* qI, const float* w,
                                   dsa_paged kI, const uint16_t* q, dsa_paged k, dsa_paged v,
                                   uint16_t* out, float* lse, int32_t* indices_out,
                                   int32_t* counts_out, uint32_t* err, void* stream);

/*
 * The indexer prolog (Day0 article, section 4.3: Q projection, K
 * normalisation, per-group Q quantisation and head-weight projection ahead
 * of the fused call), producing the MXFP8 operands of section 5.1 with bf16
 * projections (section 5.3).  For every row r, in one launch:
 *   q[r]  = W_q x[r]          x bf16 [num_rows][D_x], w_q bf16 [H_I * D_I][D_x]
 *                             (row h * D_I + d gives head h, dim d)
 *   qI, qI_scale = MXFP8(q[r]) per head and group of 32 dims:
 *                             qI E4M3 [num_rows][H_I][D_I],
 *                             qI_scale E8M0 [num_rows][H_I][D_I / 32]
 *   w[r]  = W_g x[r]          w_g bf16 [H_I][D_x]; w float32 [num_rows][H_I]
 *   y     = k_gamma * k_new[r] / sqrt(mean(k_new[r]^2) + eps)
 *                             k_new bf16 [num_rows][D_I] (the row's own index
 *                             key before normalisation), k_gamma bf16 [D_I]
 *   MXFP8(y) is written into kI at the row's position p_r of sequence b_r:
 *   codes at row p_r % 64 of block block_table[b_r][p_r / 64], scales in
 *   that block's scale area (the MXFP8 page layout of dsa_indexer_scores).
 * Products are bf16 x bf16 with float32 accumulation.  Readings: q, y and w
 * are bf16 tensors (the float32 result rounded to nearest even; w holds its
 * bf16 values); a group of 32 values v shares the scale
 * 2^(floor(log2 max|v|) - 8) (OCP microscaling; 2^-127 for an all-zero
 * group) and each code is v over the scale rounded to nearest even in E4M3,
 * saturated at +-448, keeping v's sign.
 *   p        shapes, rows and block table as for the other calls;
 *            indexer_format must be DSA_INDEXER_MXFP8 (else DSA_ERR_INVALID);
 *            the attention fields and K are not read
 *   D_x      input width, a multiple of 32 in 32 .. 65536
 *            (else DSA_ERR_INVALID / DSA_ERR_UNSUPPORTED above 65536)
 *   eps      finite, >= 0
 *   kI       the index-key cache, written (its base is cast to writable)
 * Alignment: x, w_q, w_g, qI 16 bytes; k_new, k_gamma, w 4 bytes.
 * Workspace: dsa_workspace_size(p, DSA_OP_INDEXER_PROLOG) bytes (the error
 * word).  A row that does not resolve or whose block id is out of range
 * writes nothing to kI and sets DSA_DEVERR_ROW / DSA_DEVERR_BLOCK; its qI,
 * qI_scale and w are still written.
 */
DSA_API int dsa_indexer_prolog(const dsa_problem* p, int32_t D_x, float eps, const uint16_t* x,
                               const uint16_t* w_q, const uint16_t* w_g, const uint16_t* k_new,
                               const uint16_t* k_gamma, uint8_t* qI, uint8_t* qI_scale,
                               float* w, dsa_paged kI, void* ws, size_t ws_bytes, void* stream);

/* Static text for a dsa_status value ("unknown status" otherwise). */
DSA_API const char* dsa_status_string(int status);

/* DSA_ABI_VERSION of the loaded library. */
DSA_API int dsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
