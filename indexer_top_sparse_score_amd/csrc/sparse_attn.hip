// Sparse MQA on gfx950: gather the selected KV rows through the block table
// and run an online-softmax attention over them with bf16 MFMA and float32
// accumulation.
//
// Method: Baidu AI Cloud, "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (the attention core
// reads only the selected KV rows) and section 4.2 (gather from the main KV
// cache by the indexer's position list); one KV latent row serves every query
// head ("SPLASH: Switching Parallel Layouts of Attention with Seamless
// Handoff for LLM Serving", section 2); float32 accumulation as in
// "Bandwidth-Aware LLM Inference on Heterogeneous Many-Core
// Supercomputers", section III.B.4.
//
// Work split.  A workgroup of NW waves x 16 query heads covers one chunk of
// a row's index list.  A prologue turns every index of the chunk into a row
// address (index -> block table -> byte offset) in LDS.  The chunk is then
// walked 32 keys at a time through two LDS buffers: the gathered rows are
// staged key-major (for the logits) and transposed (for P.V); while one
// sub-block is on the MFMA pipe, the next one's row loads are in flight.
// Per wave and 32 keys:
//   S^T[32 keys x 16 heads] = K[32 x D_qk] . Q^T     (v_mfma_f32_16x16x32_bf16,
//                                                    Q^T held in registers)
//   online softmax per head (exp2 domain), in registers
//   O^T[D_v x 16 heads]   += V^T[D_v x 32] . P^T    (P^T straight from the S^T
//                                                    accumulators, no LDS trip)
// The contraction index of P.V is permuted so that each lane's P^T operand is
// exactly the 8 logits its S^T accumulators already hold; the V^T operand is
// read with the same permutation.
// When a row's index list is split over several chunks, each chunk writes
// its (max, sum, unnormalised O) in float32 and a second kernel merges them
// by log-sum-exp.

#include "dsa_common.h"

#ifndef DSA_ATTN_MAX_CHUNKS
#define DSA_ATTN_MAX_CHUNKS 16
#endif
#ifndef DSA_ATTN_LATENT_DMA
#define DSA_ATTN_LATENT_DMA 1
#endif
#ifndef DSA_ATTN_KDEPTH
#define DSA_ATTN_KDEPTH 8  // K fragment reads in flight ahead of their MFMAs
#endif
#ifndef DSA_ATTN_NBUF
#define DSA_ATTN_NBUF 3
#endif
#ifndef DSA_ATTN_TARGET_WGS
#define DSA_ATTN_TARGET_WGS 256
#endif
#ifndef DSA_ATTN_KSPLIT
#define DSA_ATTN_KSPLIT 2  // key halves per latent workgroup when rows are split into chunks
#endif
#ifndef DSA_ATTN_MERGE_TILES
#define DSA_ATTN_MERGE_TILES 4  // 16-dim tiles per merge workgroup (32 threads each)
#endif

namespace dsa {
namespace {

constexpr int kSB = 32;        // keys per sub-block
constexpr int kHPW = 16;       // heads per wave
constexpr int kMaxChunk = 256; // index slots per workgroup (staged kernel)
constexpr int kMaxChunkLat = 2048;  // index slots per workgroup (latent kernel)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Split-key partials of a call, float32:
//  - (max, sum) as float2 [rows][chunks][H_q]: the chunk's reference max of
//    the log2-scaled logits (-inf for an empty chunk) and its sum of
//    exponentials against it;
//  - the chunk's unnormalised output O = sum_j 2^(t_j - max) v_j, per
//    (row, chunk) in blocks of 16 heads: [HB][DV/16][16 heads][16 dims], HB =
//    ceil(H_q / 16).  This is the order in which a wave's O^T accumulators
//    sit in its lanes, so each 16-dim tile of a wave is one contiguous 1 KB
//    store.
__host__ __device__ inline size_t part_stats_bytes(int rows, int chunks, int H_q) {
  return ((size_t)rows * chunks * H_q * sizeof(float2) + 255) & ~size_t(255);
}
__host__ __device__ inline int64_t part_block_floats(int H_q, int DV) {
  return (int64_t)((H_q + 15) / 16) * 16 * DV;
}
__device__ __forceinline__ float2* part_stats(const AttnLaunch& a, int row_local, int chunk) {
  return reinterpret_cast<float2*>(a.partial) + ((int64_t)row_local * a.n_chunks + chunk) * a.H_q;
}
__device__ __forceinline__ float* part_out(const AttnLaunch& a, int row_local, int chunk, int DV) {
  return reinterpret_cast<float*>(static_cast<char*>(a.partial) +
                                  part_stats_bytes(a.num_rows, a.n_chunks, a.H_q)) +
         ((int64_t)row_local * a.n_chunks + chunk) * part_block_floats(a.H_q, DV);
}

// A wave's partial: lane (grp, cidx) holds O^T[16mt + 4grp + v][head0 + cidx]
// in o[mt][v]; lsum is the head's whole sum (reduced across the lane groups).
template <int MT>
__device__ __forceinline__ void write_partial(const AttnLaunch& a, int row_local, int chunk,
                                              int head0, int lane, const v4f* o, float m2,
                                              float lsum) {
  const int cidx = lane & 15, grp = lane >> 4;
  float* dst = part_out(a, row_local, chunk, 16 * MT) + (int64_t)(head0 / 16) * (MT * 256) +
               cidx * 16 + 4 * grp;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) __builtin_nontemporal_store(o[mt], reinterpret_cast<v4f*>(dst + mt * 256));
  if (grp == 0 && head0 + cidx < a.H_q)
    part_stats(a, row_local, chunk)[head0 + cidx] =
        float2{lsum > 0.0f ? m2 : -__builtin_inff(), lsum};
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)bf16_bits(lo) | ((uint32_t)bf16_bits(hi) << 16);
}

// Column position of key quad q (keys 4q..4q+3) in row `row` of the
// transposed V tile.  The XOR with row/16 spreads the transposing writes --
// 64 lanes writing rows 8 apart -- over every bank; the P.V reads, 16
// consecutive rows per instruction, stay conflict-free.
__device__ __forceinline__ int vt_quad(int q, int row) { return q ^ ((row >> 4) & 7); }

// x, or zero when keep is false (per-word masks: a select on the whole
// vector type would go through private memory)
__device__ __forceinline__ uint4 keep_or_zero(const uint4& x, bool keep) {
  const uint32_t m = keep ? 0xFFFFFFFFu : 0u;
  return uint4{x.x & m, x.y & m, x.z & m, x.w & m};
}

// 32-bit word c of a 16-byte register group
__device__ __forceinline__ uint32_t word(const uint4& x, int c) {
  return c == 0 ? x.x : c == 1 ? x.y : c == 2 ? x.z : x.w;
}

// Epilogue of one wave: lane (grp, cidx) holds O^T[16mt + 4grp + v][head]
// in o[mt][v], the head's reference max m2 (log2 units) and its sum of
// exponentials.  One chunk: out = O / sum (bf16) and lse; several: the
// chunk's float32 partial.
template <int MT>
__device__ __forceinline__ void write_result(const AttnLaunch& a, int r, int row_local, int chunk,
                                             int head, int grp, const v4f* o, float m2, float lsum) {
  constexpr int DV = 16 * MT;
  if (a.n_chunks > 1) {
    write_partial<MT>(a, row_local, chunk, head - (head & 15), (int)(threadIdx.x & 63), o, m2,
                      lsum);
    return;
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  uint16_t* dst = a.out + ((int64_t)r * a.H_q + head) * DV + 4 * grp;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    uint2 w;
    w.x = pack2(o[mt][0] * inv, o[mt][1] * inv);
    w.y = pack2(o[mt][2] * inv, o[mt][3] * inv);
    *reinterpret_cast<uint2*>(dst + 16 * mt) = w;
  }
  if (grp == 0 && a.lse)
    a.lse[(int64_t)r * a.H_q + head] = lsum > 0.0f ? (m2 + log2f(lsum)) * kLn2 : -__builtin_inff();
}

// The single-chunk result written through LDS, so that every global store
// is a whole 1 KB head row (64 lanes x 16 B) rather than 16 scattered 32-byte
// pieces: the wave's 16 x 512 bf16 go to `stage` (16 rows, pitch 1040 B to
// spread the banks) and come back one head row per instruction.  `stage` is
// this wave's own 16.25 KB of LDS; nothing else may use it meanwhile.
__device__ __forceinline__ void write_out_staged(const AttnLaunch& a, int r, int head0, int lane,
                                                 const v4f* o, float m2, float lsum,
                                                 uint8_t* stage) {
  constexpr int DV = 512, MT = DV / 16, kPitch = 2 * DV + 16;
  const int cidx = lane & 15, grp = lane >> 4;
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    uint2 w;
    w.x = pack2(o[mt][0] * inv, o[mt][1] * inv);
    w.y = pack2(o[mt][2] * inv, o[mt][3] * inv);
    *reinterpret_cast<uint2*>(stage + cidx * kPitch + 2 * (16 * mt + 4 * grp)) = w;
  }
  uint16_t* dst = a.out + ((int64_t)r * a.H_q + head0) * DV;
  const int nh = min(kHPW, a.H_q - head0);
#pragma unroll
  for (int h = 0; h < kHPW; ++h)
    if (h < nh)
      *reinterpret_cast<uint4*>(dst + (int64_t)h * DV + 8 * lane) =
          *reinterpret_cast<const uint4*>(stage + h * kPitch + 16 * lane);
  const int head = head0 + cidx;
  if (grp != 0 || cidx >= nh) return;
  if (a.lse)
    a.lse[(int64_t)r * a.H_q + head] = lsum > 0.0f ? (m2 + log2f(lsum)) * kLn2 : -__builtin_inff();
}

struct AttnGrid {
  int n_hg;     // head groups
  int n_units;  // rows * chunks
  int chunk;    // index slots per chunk (multiple of kSB, <= kMaxChunk)
};

// Maps a workgroup to (unit, head group).  Workgroups are dealt round-robin
// to the 8 XCDs (id & 7); XCD x takes the contiguous unit range
// [x*U, x*U + U), U = ceil(units / 8), head groups innermost.  So the head
// groups of a (row, chunk) unit share its gathered rows, and the chunks of
// a row share its queries, through one XCD's L2.
__device__ __forceinline__ bool decode_wg(const AttnGrid& g, int& unit, int& hg) {
  const int id = (int)blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int per_xcd = (g.n_units + 7) / 8;
  hg = slot % g.n_hg;
  unit = xcd * per_xcd + slot / g.n_hg;
  return unit < g.n_units;
}

template <int DQK, int DV, bool LATENT, int NW>
struct Cfg {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kHG = kHPW * NW;  // heads per workgroup
  static constexpr int KP = DQK + 8;     // key-major LDS pitch (elements)
  static constexpr int VP = kSB + 4;     // dims-major LDS pitch (elements)
  static constexpr int KS = DQK / 32;    // MFMA steps for the logits
  static constexpr int MT = DV / 16;     // O^T row tiles
  // staging jobs per sub-block: V^T jobs = (8-dim group, 4-key quad) pairs;
  // K jobs = the 16-byte pieces of the K rows not covered by V^T jobs
  static constexpr int kVJobs = (DV / 8) * (kSB / 4);
  static constexpr int kVJ = (kVJobs + kThreads - 1) / kThreads;
  static constexpr int kKPieces = LATENT ? (DQK - DV) / 8 : DQK / 8;
  static constexpr int kKJobs = kSB * kKPieces;
  static constexpr int kKJ = (kKJobs + kThreads - 1) / kThreads;
  // kKPieces as a divisor (with no K pieces beyond V, kKJ is 0 and it is
  // never used)
  static constexpr int kKDiv = kKPieces > 0 ? kKPieces : 1;
  static constexpr int kKsElems = kSB * KP;
  static constexpr int kVtElems = DV * VP;
};

// A staging job's raw data: 8 bf16 elements (16 bytes).
template <class C>
struct Staged {
  uint4 v[C::kVJ > 0 ? C::kVJ : 1][4];
  uint4 k[C::kKJ > 0 ? C::kKJ : 1];
};

// Eight FP8 KV elements -- 8 E4M3 codes and the float32 scale of their
// tile -- as packed bf16: decoded (the hardware conversion is the OCP E4M3
// one), times the scale and rounded to bf16.  `keep` false gives zeros (an
// absent row).
struct Raw8 {
  uint2 x;
  float s;
};
__device__ __forceinline__ uint4 raw_bf16x8(const Raw8& r, bool keep) {
  float f[8];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const int word = (int)(w ? r.x.y : r.x.x);
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
    f[4 * w + 0] = lo[0];
    f[4 * w + 1] = lo[1];
    f[4 * w + 2] = hi[0];
    f[4 * w + 3] = hi[1];
  }
  const float sc = keep ? r.s : 0.0f;
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)  // one packed round-to-nearest-even conversion per pair
    w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{f[2 * i] * sc, f[2 * i + 1] * sc}), b2));
  return uint4{w[0], w[1], w[2], w[3]};
}

// KV8: the latent cache holds E4M3 code rows, and a block keeps its 64 rows'
// float32 tile scales after its code rows (row i's kKvTiles scales at
// 64 * row_stride + 4 * kKvTiles * i); element d belongs to tile d / 128.
constexpr int kKvTile = 128;
constexpr int kKvDim = 576;  // the FP8 cache's rows: the 576-wide latent
constexpr int kKvTiles = (kKvDim + kKvTile - 1) / kKvTile;  // 5

template <int DQK, int DV, bool LATENT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void sparse_attn_kernel(AttnLaunch a, AttnGrid g) {
  using C = Cfg<DQK, DV, LATENT, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::kKsElems];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][C::kVtElems];
  __shared__ int64_t koff[kMaxChunk];
  // separate V: V row offsets
  __shared__ int64_t voff[LATENT ? 1 : kMaxChunk];

  int unit, hg;
  if (!decode_wg(g, unit, hg)) return;
  const int r = a.row_begin + unit / a.n_chunks;
  const int chunk = unit % a.n_chunks;
  const int row_local = r - a.row_begin;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cidx = lane & 15, grp = lane >> 4;

  int b = 0, p = -1;
  if (!resolve_row(a.rows, r, b, p)) {
    p = -1;
    if (chunk == 0 && hg == 0 && tid == 0) report(a.err, DSA_DEVERR_ROW);
  }
  const int slot0 = chunk * g.chunk;
  const int n_slots = max(0, min(a.K, slot0 + g.chunk) - slot0);
  const int nsb = (n_slots + kSB - 1) / kSB;

  // ---- prologue: every index of the chunk -> row byte offsets
  {
    const int32_t* idx_row = a.indices + (a.indices_row_offset + row_local) * (int64_t)a.K;
    const int32_t* bt = a.rows.block_table + (int64_t)b * a.rows.max_blocks;
    for (int i = tid; i < nsb * kSB; i += C::kThreads) {
      int64_t ko = -1, vo = -1;
      if (i < n_slots && p >= 0) {
        const int idx = idx_row[slot0 + i];
        if (idx >= 0 && idx <= p) {
          const int phys = bt[idx >> 6];
          const bool okk = phys >= 0 && (int64_t)phys < a.k.num_blocks;
          const bool okv = LATENT || (phys >= 0 && (int64_t)phys < a.v.num_blocks);
          if (okk && okv) {
            ko = (int64_t)phys * a.k.block_stride + (int64_t)(idx & 63) * a.k.row_stride;
            vo = (int64_t)phys * a.v.block_stride + (int64_t)(idx & 63) * a.v.row_stride;
          } else {
            report(a.err, DSA_DEVERR_BLOCK);
          }
        } else if (idx != -1) {
          report(a.err, DSA_DEVERR_INDEX);
        }
      }
      koff[i] = ko;
      if (!LATENT) voff[i] = vo;
    }
  }

  // Q^T operand: this lane's head, 8 dims per MFMA step
  const int head = hg * C::kHG + wave * kHPW + cidx;
  const bool head_ok = head < a.H_q;
  v8s qb[C::KS];
  {
    const uint16_t* qrow = a.q + ((int64_t)r * a.H_q + (head_ok ? head : 0)) * DQK + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const v8s x = *reinterpret_cast<const v8s*>(qrow + 32 * ks);
      qb[ks] = head_ok ? x : v8s{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  __syncthreads();

  const uint8_t* kbase = static_cast<const uint8_t*>(a.k.base);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v.base);

  // ---- staging: global -> registers (issue), registers -> LDS (land).
  // Loads are unconditional (an absent row reads row 0 of block 0, which
  // always exists) and raw; rows that are absent are zeroed only when they
  // land, so nothing waits on the loads while the previous sub-block runs.
  auto issue = [&](int sb, Staged<C>& st) {
    const int base = sb * kSB;
#pragma unroll
    for (int i = 0; i < C::kVJ; ++i) {
      const int job = tid + i * C::kThreads;
      const int dg = job % (DV / 8), kq = (job / (DV / 8)) % (kSB / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t off = (LATENT ? koff : voff)[base + 4 * kq + j];
        st.v[i][j] = *reinterpret_cast<const uint4*>((LATENT ? kbase : vbase) + (off >= 0 ? off : 0) +
                                                     dg * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < C::kKJ; ++i) {
      const int job = tid + i * C::kThreads;
      const int key = (job / C::kKDiv) % kSB, piece = job % C::kKDiv;
      const int64_t off = koff[base + key];
      const int d0 = (LATENT ? DV : 0) + 8 * piece;
      st.k[i] = *reinterpret_cast<const uint4*>(kbase + (off >= 0 ? off : 0) + d0 * 2);
    }
  };
  auto land = [&](Staged<C>& st, int sb, int buf) {
    const int base = sb * kSB;
    uint16_t* ks = Ks[buf];
    uint16_t* vt = Vt[buf];
#pragma unroll
    for (int i = 0; i < C::kVJ; ++i) {
      const int job = tid + i * C::kThreads;
      // every thread owns a job when the jobs divide evenly: no guard
      const bool mine = C::kVJ * C::kThreads == C::kVJobs || job < C::kVJobs;
      const int dg = job % (DV / 8), kq = (job / (DV / 8)) % (kSB / 4);
      uint4 vv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vv[j] = keep_or_zero(st.v[i][j], (LATENT ? koff : voff)[base + 4 * kq + j] >= 0);
      if (mine) {
      if (LATENT) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint4*>(&ks[(4 * kq + j) * C::KP + 8 * dg]) = vv[j];
      }
      // transpose: vv[j] holds dims 8dg..8dg+7 of key 4kq+j; row 8dg+dd of
      // V^T takes element dd of each of the 4 keys
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const uint32_t a0 = word(vv[0], dd >> 1), a1 = word(vv[1], dd >> 1);
        const uint32_t a2 = word(vv[2], dd >> 1), a3 = word(vv[3], dd >> 1);
        uint2 t;
        t.x = (dd & 1) ? (a0 >> 16) | (a1 & 0xFFFF0000u) : (a0 & 0xFFFFu) | (a1 << 16);
        t.y = (dd & 1) ? (a2 >> 16) | (a3 & 0xFFFF0000u) : (a2 & 0xFFFFu) | (a3 << 16);
        const int row = 8 * dg + dd;
        *reinterpret_cast<uint2*>(&vt[row * C::VP + 4 * vt_quad(kq, row)]) = t;
      }
      }
    }
#pragma unroll
    for (int i = 0; i < C::kKJ; ++i) {
      const int job = tid + i * C::kThreads;
      const bool mine = C::kKJ * C::kThreads == C::kKJobs || job < C::kKJobs;
      const int key = (job / C::kKDiv) % kSB, piece = job % C::kKDiv;
      const int d0 = (LATENT ? DV : 0) + 8 * piece;
      if (mine) *reinterpret_cast<uint4*>(&ks[key * C::KP + d0]) = keep_or_zero(st.k[i], koff[base + key] >= 0);
    }
  };

  v4f o[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) o[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m2 = -__builtin_inff();  // running max of the log2-scaled logits
  float lsum = 0.0f;             // this lane's share of the running sum
  const float c2 = a.scale * kLog2e;

  Staged<C> st;
  if (nsb > 0) issue(0, st);
  for (int sb = 0; sb < nsb; ++sb) {
    const int buf = sb & 1;
    // Buffer `buf` was last read in sub-block sb-2; every wave finished that
    // before passing the barrier of sub-block sb-1, so it is free to fill.
    land(st, sb, buf);
    __syncthreads();
    if (sb + 1 < nsb) issue(sb + 1, st);
    // validity of the sub-block's 32 keys, as a wave-uniform mask
    const uint32_t valid =
        (uint32_t)__ballot(lane < kSB && koff[sb * kSB + (lane & (kSB - 1))] >= 0);
    if (valid == 0) continue;

    const uint16_t* ks = Ks[buf];
    const uint16_t* vt = Vt[buf];
    // ---- logits S^T (keys x heads): two 16-key tiles
    v4f s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = &ks[(16 * kt + cidx) * C::KP + 8 * grp];
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk) {
        const v8s ka = *reinterpret_cast<const v8s*>(krow + 32 * kk);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(v8bf, ka), __builtin_bit_cast(v8bf, qb[kk]), acc, 0, 0, 0);
      }
      s[kt] = acc;
    }
    // ---- online softmax for this lane's head over keys 16kt + 4grp + v
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = 16 * kt + 4 * grp + v;
        const float x = ((valid >> key) & 1u) ? s[kt][v] * c2 : -__builtin_inff();
        s[kt][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = across_rows(mx, FMax());
    // Lazy rescaling: the reference max m2 only moves when some head's max
    // exceeds it by more than 8 (log2 units), so the exponentials below stay
    // <= 2^8 and the accumulators are rescaled rarely.  Any reference gives
    // the same softmax; lse uses the same reference.
    const float m_new = fmaxf(m2, mx);  // finite: the sub-block has a valid key
    if (__ballot(m_new > m2 + 8.0f)) {
      const float alpha = exp2f(m2 - m_new);  // 0 while nothing has accumulated
      lsum *= alpha;
      if (m2 != -__builtin_inff()) {
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) o[mt] *= alpha;
      }
      m2 = m_new;
    }
    float pv[8];
    float psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = exp2f(s[kt][v] - m2);
        pv[kt * 4 + v] = e;
        psum += e;
      }
    lsum += psum;
    // ---- O^T += V^T . P^T ; contraction slot e of lane group grp is
    //      key 4grp+e (e < 4) or 16+4grp+(e-4) (e >= 4)
    const v8bf pb = __builtin_bit_cast(
        v8bf, (uint4){pack2(pv[0], pv[1]), pack2(pv[2], pv[3]), pack2(pv[4], pv[5]),
                      pack2(pv[6], pv[7])});
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      const int row = 16 * mt + cidx;
      const uint16_t* vrow = &vt[row * C::VP];
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * vt_quad(grp, row));
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 4 * vt_quad(4 + grp, row));
      const v8bf va = __builtin_bit_cast(v8bf, (uint4){lo.x, lo.y, hi.x, hi.y});
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[mt], 0, 0, 0);
    }
  }

  lsum = across_rows(lsum, FAdd());
  if (!head_ok) return;

  write_result<C::MT>(a, r, row_local, chunk, head, grp, o, m2, lsum);
}

// ---------------------------------------------------------------------------
// Latent rows (576 bf16 = 1152 B; V = the first 512 elements): the gathered
// rows move HBM -> LDS by DMA (global_load_lds, 16 B per lane, no staging
// registers), NBUF sub-blocks deep, and both MFMA operands are read from the
// one key-major tile: the K rows as they are for the logits, and V^T through
// the transposing LDS read (ds_read_b64_tr_b16).
//
// Tile of a sub-block: 32 rows x 72 pieces of 16 B, piece p of row r at
// slot r*72 + (p ^ (r & 7)) -- the XOR keeps both the logit reads (16 rows,
// same piece) and the transposing reads (4 rows x 4 dim groups) within two
// lanes per bank.  DMA instruction i of a sub-block fills slots 64i..64i+63
// (lane l -> slot 64i + l), so each wave issues exactly kDmaPerWave of them
// per sub-block and waits on them with a fixed vmcnt.
//
// Transposing read: within each 16-lane group, lane j names 4 consecutive
// bf16 e_j[0..3]; lane i receives e_{i/4 + 4k}[i % 4] for k = 0..3.  With
// lane j naming row 4g + j/4 (key) and dims 16mt + 4(j%4) .. +3, lane i of
// group g gets V[4g + k][16mt + i], k = 0..3: the A operand of
// O^T += V^T . P^T in the contraction order the S^T accumulators hold.
namespace lat {
constexpr int kDqk = 576, kDv = 512;
constexpr int kPieces = kDqk * 2 / 16;             // 72
constexpr int kTileBytes = kSB * kPieces * 16;     // 36864
constexpr int kDmaPerSB = kSB * kPieces / 64;      // 36 DMA instructions per sub-block
constexpr int kKS = kDqk / 32;                     // 18
constexpr int kMT = kDv / 16;                      // 32
__device__ __forceinline__ int slot(int row, int piece) { return row * kPieces + (piece ^ (row & 7)); }
}  // namespace lat

typedef short v4s __attribute__((ext_vector_type(4)));

// One 16-byte-per-lane DMA, global -> LDS (lane l lands at lds + 16 l).
// Issued through inline asm on purpose: with the builtin, the compiler makes
// every later LDS read wait for all DMAs in flight (vmcnt(0)), since it
// cannot tell the buffers apart, which would serialise the prefetch.  The
// caller orders the tile accesses itself (wait_vm + barrier).  M0 carries
// the LDS address and is restored; the s_nop is the wait state an M0 write
// needs before an LDS DMA reads it.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// One 4-byte-per-lane DMA, global -> LDS (lane l lands at lds + 4 l), as
// dma16.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// Waits until at most `groups` groups of PER DMA instructions are in flight.
template <int PER>
__device__ __forceinline__ void wait_vm(int groups) {
  static_assert(3 * PER <= 63, "vmcnt field");
  switch (groups) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory"); break;
  }
}

// KV8 (the FP8 latent cache: E4M3 code rows, each with five float32 tile
// scales in its block's scale area): a step's 64 code rows (576 B each) and
// their scales move HBM -> LDS by DMA into a ring of two steps, 18 KB of
// codes per sub-block instead of 36 KB of bf16; once a step has landed, the
// workgroup decodes it into the bf16 tiles above (code value x its tile's
// scale, rounded to bf16 -- the same values the register-staged kernel
// makes), and the MFMA loop runs on them unchanged.
//
// KSPLIT: the key halves of a workgroup.  With KSPLIT = 2 the kNW waves are
// kNW / 2 head waves (16 heads each) times two key halves: both halves share
// every staged sub-block, half 0 takes the even sub-blocks of the chunk and
// half 1 the odd ones, and at the end half 1 hands its accumulators to half
// 0 through LDS, which merges them by log-sum-exp.  Twice the waves per
// staged byte, and the same partial per workgroup.
template <int NBUF, int kNW, int KSPLIT, bool KV8 = false>
__global__ __launch_bounds__(64 * kNW, 1) void sparse_attn_latent_kernel(AttnLaunch a, AttnGrid g) {
  using namespace lat;
  constexpr int NT = 64 * kNW;
  constexpr int kHW = kNW / KSPLIT;  // head waves
  constexpr int kDmaPerWave = kDmaPerSB / kNW;
  // KV8: per step and wave, code DMAs (16 B per lane) for kSB * KSPLIT rows
  // of 36 pieces, and scale DMAs (4 B per lane) for those rows' 8-float
  // slots (5 used)
  constexpr int kRowsStep = kSB * KSPLIT;
  constexpr int kCodePieces = kKvDim / 16;  // 36
  constexpr int kCodeDma = KV8 ? kRowsStep * kCodePieces / 64 / kNW : 0;
  constexpr int kScaleDma = KV8 ? kRowsStep * 8 / 64 / kNW : 0;
  constexpr int kPerStep = KV8 ? kCodeDma + kScaleDma : KSPLIT * kDmaPerWave;  // DMA instructions per wave per step
  constexpr int kCodeBytes = kRowsStep * kKvDim, kStepBytes = kCodeBytes + kRowsStep * 32;
  constexpr int kCodeSteps = KV8 ? 2 : 0;                        // the code ring, in steps
  constexpr int kAhead = KV8 ? kCodeSteps : NBUF / KSPLIT;       // steps staged at once
  static_assert(kDmaPerSB % kNW == 0, "DMA instructions per wave");
  static_assert(!KV8 || (kRowsStep * kCodePieces % (64 * kNW) == 0 && kRowsStep * 8 % (64 * kNW) == 0 &&
                         KSPLIT == 2 && NBUF == KSPLIT && kRowsStep / kNW * kCodePieces == 64 * kCodeDma),
                "FP8 steps: whole DMA instructions per wave, one tile per key half");
  static_assert(KSPLIT == 1 || KSPLIT == 2, "key halves");
  static_assert(NBUF % KSPLIT == 0 && kAhead >= 2 && (kAhead - 1) * kPerStep <= 63, "vmcnt");
  constexpr int kLdsBytes = NBUF * kTileBytes + kCodeSteps * kStepBytes;
  // epilogue staging of the head waves, after the merge area (KSPLIT = 2)
  constexpr int kMergeBytes = KSPLIT == 2 ? kHW * 64 * (kMT * 16 + 8) : 0;
  static_assert(kMergeBytes + kHW * 16 * (2 * kDv + 16) <= kLdsBytes,
                "merge and epilogue staging fit the tiles");
  // the tiles, then (KV8) the code ring; the merge and the epilogue reuse it all
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  auto tile = [&](int i) { return lds + i * kTileBytes; };
  // each slot's row offset in the cache in 16-byte units (the front end
  // keeps the cache below 64 GiB for this kernel), ~0u for an absent row;
  // KV8: the row's (block id << 6 | row in block) instead
  __shared__ __attribute__((aligned(16))) uint32_t koff[kMaxChunkLat];

  int unit, hg;
  if (!decode_wg(g, unit, hg)) return;
  const int r = a.row_begin + unit / a.n_chunks;
  const int chunk = unit % a.n_chunks;
  const int row_local = r - a.row_begin;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave % kHW, kh = wave / kHW;  // head wave, key half
  const int cidx = lane & 15, grp = lane >> 4;

  const int slot0 = chunk * g.chunk;
  const int n_slots = max(0, min(a.K, slot0 + g.chunk) - slot0);
  // sub-blocks, rounded up to whole steps (a padding sub-block is all
  // absent rows and adds nothing)
  const int nsb = (n_slots + kSB * KSPLIT - 1) / (kSB * KSPLIT) * KSPLIT;
  const int nst = nsb / KSPLIT;

  // ---- prologue: every index slot of the chunk -> row byte offset (-1:
  //      absent).  Ready-made when the Top-K wrote them (-1 for a row that
  //      does not resolve, which that kernel has reported): one round trip,
  //      and nothing else is loaded before it, so the first DMAs go out as
  //      soon as it is back.
  if (a.rowoff) {
    const int64_t* ro = a.rowoff + (int64_t)row_local * a.K + slot0;
    for (int i = tid; i < nsb * kSB; i += NT) {
      const int64_t o = i < n_slots ? ro[i] : -1;
      if constexpr (KV8) {  // o = block * block_stride + row * row_stride
        uint32_t kf = ~0u;
        if (o >= 0) {
          const int64_t blk = o / a.k.block_stride;
          kf = (uint32_t)(blk << 6) | (uint32_t)((o - blk * a.k.block_stride) / a.k.row_stride);
        }
        koff[i] = kf;
      } else {
        koff[i] = o >= 0 ? (uint32_t)(o >> 4) : ~0u;
      }
    }
  } else {
    int b = 0, p = -1;
    if (!resolve_row(a.rows, r, b, p)) {
      p = -1;
      if (chunk == 0 && hg == 0 && tid == 0) report(a.err, DSA_DEVERR_ROW);
    }
    const int32_t* idx_row = a.indices + (a.indices_row_offset + row_local) * (int64_t)a.K;
    const int32_t* bt = a.rows.block_table + (int64_t)b * a.rows.max_blocks;
    for (int i = tid; i < nsb * kSB; i += NT) {
      int64_t ko = -1;
      if (i < n_slots && p >= 0) {
        const int idx = idx_row[slot0 + i];
        if (idx >= 0 && idx <= p) {
          const int phys = bt[idx >> 6];
          if (phys >= 0 && (int64_t)phys < a.k.num_blocks)
            ko = KV8 ? ((int64_t)phys << 6) | (idx & 63)
                     : (int64_t)phys * a.k.block_stride + (int64_t)(idx & 63) * a.k.row_stride;
          else
            report(a.err, DSA_DEVERR_BLOCK);
        } else if (idx != -1) {
          report(a.err, DSA_DEVERR_INDEX);
        }
      }
      koff[i] = ko >= 0 ? (uint32_t)(KV8 ? ko : ko >> 4) : ~0u;
    }
  }

  __syncthreads();

  const uint8_t* kbase = static_cast<const uint8_t*>(a.k.base);
  // DMA of sub-block sb: this wave's instructions t = 0..kDmaPerWave-1 fill
  // slots 64*(wave*kDmaPerWave + t) + lane.  Absent rows read row 0 of block
  // 0 (which always exists) and are zeroed after they land.
  // (All row offsets are read before the first DMA: the DMA's asm is a
  // compiler memory barrier, so reads interleaved with it would each wait.)
  // A wave's DMAs of a sub-block cover its rows kRowsPW * wave .. + kRowsPW
  // - 1 (kRowsPW rows x 72 pieces = kDmaPerWave x 64 slots): their offsets
  // come in with a few broadcast LDS reads, and instruction t, whose lanes
  // span at most two of those rows (64 slots < 72 pieces), picks its row's
  // offset with one select.
  constexpr int kRowsPW = kSB / kNW;
  static_assert(kRowsPW * kPieces == kDmaPerWave * 64 && kRowsPW % 4 == 0, "rows per wave");
  auto issue = [&](int sb) {
    uint8_t* buf = tile(sb % NBUF);
    uint32_t kr[kRowsPW];
#pragma unroll
    for (int i = 0; i < kRowsPW; i += 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(&koff[sb * kSB + kRowsPW * wave + i]);
      kr[i] = x.x;
      kr[i + 1] = x.y;
      kr[i + 2] = x.z;
      kr[i + 3] = x.w;
    }
    const uint8_t* src[kDmaPerWave];
#pragma unroll
    for (int t = 0; t < kDmaPerWave; ++t) {
      const int sl = 64 * t + lane;  // slot within this wave's rows
      const int j = sl / kPieces;    // a_t or a_t + 1
      const int at = 64 * t / kPieces;
      const int piece = (sl - j * kPieces) ^ ((kRowsPW * wave + j) & 7);
      const uint32_t o16 = (at + 1 < kRowsPW && j > at) ? kr[at + 1 < kRowsPW ? at + 1 : at] : kr[at];
      src[t] = kbase + (o16 != ~0u ? (int64_t)o16 << 4 : 0) + 16 * piece;
    }
    const uint32_t lds0 =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(buf + 1024 * wave * kDmaPerWave));
#pragma unroll
    for (int t = 0; t < kDmaPerWave; ++t) dma16(src[t], lds0 + 1024 * t);
  };
  auto zero_absent = [&](int sb) {
    uint8_t* buf = tile(sb % NBUF);
#pragma unroll
    for (int t = 0; t < kDmaPerWave; ++t) {
      const int i = wave * kDmaPerWave + t;
      const int sl = 64 * i + lane;
      if (koff[sb * kSB + sl / kPieces] == ~0u)
        *reinterpret_cast<uint4*>(buf + 16 * sl) = uint4{0u, 0u, 0u, 0u};
    }
  };

  // the first step's sub-blocks requested, then Q^T (this lane's head, 8
  // dims per MFMA step), then the rest of the lookahead: what the first
  // MFMAs need is queued ahead of what they do not
  // KV8: the DMAs of step st into ring slot st % kCodeSteps.  Code
  // instruction i fills the step's 16-byte code slots 64i .. 64i + 63 (slot
  // s: row s / 36, piece s % 36); scale instruction j fills its float slots
  // 64j .. 64j + 63 (row d / 8, scale d % 8; slots 5..7 of a row repeat
  // scale 4 and go unused).  Each wave's instructions cover its own kRW
  // rows, whose (block, row) come in with a few broadcast LDS reads before
  // the first DMA.  Absent rows read block 0 and are zeroed when decoded.
  auto issue8 = [&](int st) {
    constexpr int kRW = kRowsStep / kNW;
    uint8_t* ring = lds + NBUF * kTileBytes + (st % (kCodeSteps > 0 ? kCodeSteps : 1)) * kStepBytes;
    uint32_t kf[kRW];
#pragma unroll
    for (int i = 0; i < kRW; i += 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(&koff[st * kRowsStep + kRW * wave + i]);
      kf[i] = x.x;
      kf[i + 1] = x.y;
      kf[i + 2] = x.z;
      kf[i + 3] = x.w;
    }
    auto row_base = [&](uint32_t f) -> int64_t {  // where the row's block starts
      return f == ~0u ? 0 : (int64_t)(f >> 6) * a.k.block_stride;
    };
    const uint8_t* csrc[kCodeDma > 0 ? kCodeDma : 1];
#pragma unroll
    for (int t = 0; t < kCodeDma; ++t) {
      const int sl = 64 * t + lane;       // slot within this wave's rows
      const int j = sl / kCodePieces;     // at, at + 1 or at + 2
      const int at = 64 * t / kCodePieces;
      const uint32_t f = j == at ? kf[at] : j == at + 1 ? kf[at + 1 < kRW ? at + 1 : at]
                                                         : kf[at + 2 < kRW ? at + 2 : at];
      const int64_t off = f == ~0u ? 0 : row_base(f) + (int64_t)(f & 63) * a.k.row_stride;
      csrc[t] = kbase + off + 16 * (sl - j * kCodePieces);
    }
    const uint8_t* ssrc[kScaleDma > 0 ? kScaleDma : 1];
#pragma unroll
    for (int t = 0; t < kScaleDma; ++t) {
      uint32_t f = kf[8 * t];  // the row: 8 t + lane / 8 of this wave's
#pragma unroll
      for (int q = 1; q < 8; ++q)
        if ((lane >> 3) == q) f = kf[8 * t + q < kRW ? 8 * t + q : 8 * t];
      const int k = min(lane & 7, kKvTiles - 1);
      const int64_t off = f == ~0u ? 0
                                   : row_base(f) + kBlock * a.k.row_stride +
                                         (int64_t)(f & 63) * (4 * kKvTiles) + 4 * k;
      ssrc[t] = kbase + off;
    }
    const uint32_t c0 =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ring + 1024 * kCodeDma * wave));
    const uint32_t s0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(ring + kCodeBytes + 256 * kScaleDma * wave));
#pragma unroll
    for (int t = 0; t < kCodeDma; ++t) dma16(csrc[t], c0 + 1024 * t);
#pragma unroll
    for (int t = 0; t < kScaleDma; ++t) dma4(ssrc[t], s0 + 256 * t);
  };
  // KV8: step st's codes decoded into the bf16 tiles (its key half x's rows
  // into tile x), code value x tile scale rounded to bf16; absent rows zero.
  // Thread t decodes row t / kTPR, pieces t % kTPR + kTPR j: one row's
  // offsets and validity per thread, and for each j a wave reads and writes
  // 16 rows' worth of whole 16-lane runs.
  auto convert8 = [&](int st) {
    constexpr int kTPR = NT / kRowsStep;          // threads per row
    constexpr int kN = kPieces / kTPR;            // bf16 pieces per thread
    static_assert(!KV8 || (NT % kRowsStep == 0 && kPieces % kTPR == 0), "whole pieces per thread");
    const uint8_t* ring = lds + NBUF * kTileBytes + (st % (kCodeSteps > 0 ? kCodeSteps : 1)) * kStepBytes;
    const int row = tid / kTPR, p0 = tid % kTPR, rr = row & (kSB - 1);
    static_assert(!KV8 || (kTPR == 4 && kKvTile / 8 == 16), "piece p0 + 4 j lies in scale tile j / 4");
    const uint8_t* src = ring + row * kKvDim + 8 * p0;
    const float* sc = reinterpret_cast<const float*>(ring + kCodeBytes) + row * 8;
    uint8_t* dst = tile(row / kSB) + 16 * (rr * kPieces);
    const bool keep = koff[st * kRowsStep + row] != ~0u;
    float s5[kKvTiles];
#pragma unroll
    for (int t = 0; t < kKvTiles; ++t) s5[t] = sc[t];
    constexpr int kB = 6;  // code reads in flight
    static_assert(!KV8 || kN % kB == 0, "whole batches");
#pragma unroll
    for (int j0 = 0; j0 < kN; j0 += kB) {
      uint2 c[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) c[u] = *reinterpret_cast<const uint2*>(src + 8 * kTPR * (j0 + u));
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int j = j0 + u, p = p0 + kTPR * j;
        Raw8 rw;
        rw.x = c[u];
        rw.s = s5[j / 4];
        *reinterpret_cast<uint4*>(dst + 16 * (p ^ (rr & 7))) = raw_bf16x8(rw, keep);
      }
    }
  };
  auto issue_step = [&](int st) {
    if constexpr (KV8) {
      issue8(st);
    } else {
#pragma unroll
      for (int x = 0; x < KSPLIT; ++x) issue(st * KSPLIT + x);
    }
  };
  // Q of the workgroup's heads is one contiguous run of rows, staged once
  // per workgroup by DMA into the last kQT tile buffers (as sub-blocks of
  // keys are, same swizzle) and read from there as each wave's Q^T operand;
  // the steps that fill those buffers are requested after the reads.
  // Loading Q^T per wave straight from memory instead would fetch it once
  // per key half, in 16-row gathers.
  constexpr int kHG = kHPW * kHW;  // heads per workgroup
  constexpr int kQT = kHG / kSB;   // tile buffers they take
  static_assert(kHG % kSB == 0 && kQT < NBUF, "the workgroup's heads fill whole tiles");
  // (KV8: the steps go to the code ring, none to a Q buffer; they are
  // requested after Q, and the wait for Q lets them stay in flight)
  constexpr int kStepQ = KV8 ? 0 : (NBUF - kQT) / KSPLIT;  // first step that writes a Q buffer
  const int head0_wg = hg * kHG;
  for (int x = 0; x < min(kStepQ, nst); ++x) issue_step(x);
  {
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(a.q + (int64_t)r * a.H_q * kDqk);
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      const uint8_t* src[kDmaPerWave];
#pragma unroll
      for (int t = 0; t < kDmaPerWave; ++t) {
        const int sl = 64 * (wave * kDmaPerWave + t) + lane;
        const int row = sl / kPieces;
        const int piece = (sl - row * kPieces) ^ (row & 7);
        const int h = head0_wg + kSB * qt + row;
        src[t] = qbase + (int64_t)(h < a.H_q ? h : 0) * (2 * kDqk) + 16 * piece;  // (rows past H_q go unused)
      }
      const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(tile(NBUF - kQT + qt) + 1024 * wave * kDmaPerWave));
#pragma unroll
      for (int t = 0; t < kDmaPerWave; ++t) dma16(src[t], lds0 + 1024 * t);
    }
  }
  if constexpr (KV8) {
    for (int x = 0; x < min(kAhead, nst); ++x) issue_step(x);
    wait_vm<kPerStep>(min(kAhead, nst));
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  const int head = head0_wg + hw * kHPW + cidx;
  const bool head_ok = head < a.H_q;
  v8s qb[kKS];
  {
    const int qr = hw * kHPW + cidx;  // row among the workgroup's heads
    const uint8_t* qrow = tile(NBUF - kQT + qr / kSB) + 16 * ((qr % kSB) * kPieces);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const v8s x = *reinterpret_cast<const v8s*>(qrow + 16 * ((grp + 4 * ks) ^ (qr & 7)));
      qb[ks] = head_ok ? x : v8s{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  __syncthreads();  // every wave holds its Q^T: the buffers are free
  if constexpr (!KV8)
    for (int x = kStepQ; x < min(kAhead, nst); ++x) issue_step(x);
  const float c2 = a.scale * kLog2e;

  // Per-lane tile offsets.  Logits: lane (grp, cidx) reads row 16kt + cidx,
  // piece 4kk + grp; the XOR touches only the low 3 bits of the piece, so
  // the piece's slot is 8(kk/2) + ((4(kk&1) + grp) ^ (row & 7)).  P.V: lane
  // reads rows rlo, rlo + 16 and piece 2mt + h, i.e. slot
  // 8(mt/4) + ((2(mt&3) + h) ^ (rlo & 7)), plus `within` bytes.
  constexpr int kRow16 = 16 * kPieces * 16;  // bytes of 16 tile rows
  const int r7 = cidx & 7;
  const int s_even = 16 * (cidx * kPieces + (grp ^ r7));
  const int s_odd = 16 * (cidx * kPieces + ((4 + grp) ^ r7));
  int v_base[4];
  {
    const int rlo = 4 * grp + (cidx >> 2);
    const int h = (cidx & 3) >> 1, within = (cidx & 1) * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) v_base[q] = 16 * (rlo * kPieces + ((2 * q + h) ^ (rlo & 7))) + within;
  }

  // Softmax reference.  The exponentials are taken against a fixed
  // per-head reference m2, so the accumulators are only ever touched by
  // MFMAs (a rescale would need every accumulator in VGPRs).  First pass:
  // m2 = the head's max over the first sub-block with a valid key (one
  // cross-lane reduction; the sub-blocks after it need none).  Should a later
  // logit exceed it by more than kSlack (log2 units; exponentials stay
  // <= 2^kSlack otherwise), the workgroup runs the chunk again with m2 = the
  // true chunk max, which the first pass has collected lane by lane.  Any
  // reference gives the same softmax; lse uses the same one.
  constexpr float kSlack = 16.0f;
  v4f o[kMT];
  float m2 = -__builtin_inff();
  float lsum = 0.0f;   // this lane's share of the sum of exponentials
  float m_fix = -__builtin_inff();
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) o[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    m2 = m_fix;
    lsum = 0.0f;
    float m_lane = -__builtin_inff();  // max over this lane's logits
    bool over = false;                 // (wave) a logit exceeded m2 + kSlack

    // Steps of KSPLIT sub-blocks (one per key half).  kAhead steps are
    // requested up front (before the pass loop for the first pass); step st
    // >= 1 requests step st + kAhead - 1 into the buffers freed by step st-1.
    if (pass > 0)
      for (int x = 0; x < min(kAhead, nst); ++x) issue_step(x);
    for (int st = 0; st < nst; ++st) {
      // steps requested after this one: all but the first kAhead were
      // requested one step ahead
      // (KV8 requests step st + kAhead as soon as step st is decoded, so
      // kAhead - 1 later steps are in flight here)
      const int issued_to = KV8 ? min(nst - 1, st + kAhead - 1)
                                : st == 0 ? min(kAhead, nst) - 1 : min(nst - 1, st + kAhead - 2);
      wait_vm<kPerStep>(issued_to - st);
      if constexpr (!KV8) {
#pragma unroll
        for (int x = 0; x < KSPLIT; ++x) {
          const int sbx = st * KSPLIT + x;
          const bool any_absent =
              __ballot(lane < kSB && koff[sbx * kSB + (lane & (kSB - 1))] == ~0u) != 0;
          if (any_absent) zero_absent(sbx);
        }
      }
      // every wave's DMAs of this step have landed, and every wave is done
      // with the buffers the next DMAs overwrite (last read in step st-1)
      __syncthreads();
      if constexpr (KV8) {
        // decode the step into the tiles the MFMAs read; its ring slot is
        // then free for step st + kAhead
        convert8(st);
        __syncthreads();
        if (st + kAhead < nst) issue_step(st + kAhead);
      } else {
        if (st >= 1 && st + kAhead - 1 < nst) issue_step(st + kAhead - 1);
      }
      const int sb = st * KSPLIT + kh;  // this wave's sub-block
      const uint32_t valid =
          (uint32_t)__ballot(lane < kSB && koff[sb * kSB + (lane & (kSB - 1))] != ~0u);

      // No early exit below: every sub-block runs its MFMAs (a sub-block
      // without a valid key, or after an overrun, adds P = 0), so the
      // accumulators have one producer and stay in AGPRs across the loop.
      const uint8_t* buf = tile(sb % NBUF);
      // ---- logits S^T (keys x heads): two 16-key tiles; every read is one
      //      of two per-lane bases plus an immediate offset
      // The two tiles' MFMA chains alternate (step i: tile i % 2, dims
      // 32(i / 2)), so consecutive MFMAs are independent, and the fragment
      // reads run kDepth steps ahead.  The fences pin this order: left
      // alone, the scheduler issues each read just before its MFMA and the
      // LDS latency is exposed on every step.
      v4f s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      {
        constexpr int kSteps = 2 * kKS, kDepth = DSA_ATTN_KDEPTH;
        auto frag = [&](int i) {
          const int kk = i >> 1, kt = i & 1;
          return *reinterpret_cast<const v8s*>(buf + ((kk & 1) ? s_odd : s_even) + 128 * (kk >> 1) +
                                               kt * kRow16);
        };
        v8s f[kDepth];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kDepth; ++i) f[i] = frag(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
          s[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf, f[i % kDepth]), __builtin_bit_cast(v8bf, qb[i >> 1]), s[i & 1],
              0, 0, 0);
          if (i + kDepth < kSteps) f[i % kDepth] = frag(i + kDepth);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- softmax for this lane's head over keys 16kt + 4grp + v, in log2
      //      units: x = logit * scale * log2(e), t = x - m2.  Absent keys
      //      (only in sub-blocks with padding or missing pages) are masked to
      //      -inf after the scaling, so any finite scale (zero and negative
      //      included) leaves them out.
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[kt][v] *= c2;
      if (valid != 0xFFFFFFFFu) {  // wave-uniform
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (!((valid >> (16 * kt + 4 * grp + v)) & 1u)) s[kt][v] = -__builtin_inff();
      }
      if (m2 == -__builtin_inff()) {  // wave-uniform: every head sees the same keys
        float mx = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[kt][v]);
        m2 = across_rows(mx, FMax());  // -inf only without a valid key
      }
      float pv[8];
      float psum = 0.0f;
      bool hot = false;  // a logit above m2 + kSlack
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float t = s[kt][v] - m2;  // -inf for masked keys
          hot = hot || t > kSlack;
          m_lane = fmaxf(m_lane, s[kt][v]);
          pv[kt * 4 + v] = t;
        }
      over = over || __ballot(hot) != 0;
      // past an overrun the pass only collects the lane maxima; a sub-block
      // before the first valid key (m2 still -inf, t NaN) adds nothing
      const bool skip = over || m2 == -__builtin_inff();  // wave-uniform
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float e = skip ? 0.0f : __builtin_amdgcn_exp2f(pv[j]);  // exp2(-inf) = 0
        pv[j] = e;
        psum += e;
      }
      lsum += psum;
      const v8bf pb = __builtin_bit_cast(
          v8bf, (uint4){pack2(pv[0], pv[1]), pack2(pv[2], pv[3]), pack2(pv[4], pv[5]),
                        pack2(pv[6], pv[7])});
      // ---- O^T += V^T . P^T, V^T read transposed from the key-major tile;
      //      rows rlo and rlo + 16 share their swizzle, so every read is one
      //      of four per-lane bases plus an immediate offset
      {
        // V^T fragments read kDepth MFMAs ahead, order pinned as above
        constexpr int kDepth = 8;
        auto vfrag = [&](int mt) {
          const uint8_t* at = buf + v_base[mt & 3] + 128 * (mt >> 2);
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)at);
          const v4s hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(at + kRow16));
          return v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        v8s f[kDepth];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < kDepth; ++mt) f[mt] = vfrag(mt);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, f[mt % kDepth]), pb,
                                                          o[mt], 0, 0, 0);
          if (mt + kDepth < kMT) f[mt % kDepth] = vfrag(mt + kDepth);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // the last iteration waited for every DMA; the barrier also makes the
    // buffers free for a second pass
    if (!__syncthreads_or(over)) break;
    m_fix = across_rows(m_lane, FMax());
  }

  lsum = across_rows(lsum, FAdd());
  // every wave is past the last barrier and every DMA has landed: the tile
  // buffers are free for the merge and the epilogue staging
  if constexpr (KSPLIT == 2) {
    // half 1 -> LDS: lane-major v4f per 16-dim tile, then (m2, lsum)
    uint8_t* mbase = lds + hw * (64 * (kMT * 16 + 8));
    v4f* mo = reinterpret_cast<v4f*>(mbase);
    float2* mls = reinterpret_cast<float2*>(mbase + 64 * kMT * 16);
    if (kh == 1) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) mo[mt * 64 + lane] = o[mt];
      mls[lane] = float2{m2, lsum};
    }
    __syncthreads();
    if (kh == 1) return;
    // half 0 merges: each half's exponentials are against its own reference
    const float2 other = mls[lane];
    const float M = fmaxf(m2, other.x);
    const float f0 = m2 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m2 - M);
    const float f1 = other.x == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(other.x - M);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const v4f b = mo[mt * 64 + lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) o[mt][v] = o[mt][v] * f0 + b[v] * f1;
    }
    lsum = lsum * f0 + other.y * f1;
    m2 = M;
  }
  const int head0 = hg * (kHPW * kHW) + hw * kHPW;
  if (head0 >= a.H_q) return;
  if (a.n_chunks > 1) {
    write_partial<kMT>(a, row_local, chunk, head0, lane, o, m2, lsum);
    return;
  }
  // the head waves' staging (16.25 KB each) sits after the merge area
  write_out_staged(a, r, head0, lane, o, m2, lsum,
                   lds + kMergeBytes + hw * (16 * (2 * kDv + 16)));
}

// Merges the chunks of each (row, head) by log-sum-exp: with M the largest
// chunk max, chunk c weighs g_c = 2^(max_c - M), and out = sum_c g_c O_c /
// sum_c g_c sum_c.  A workgroup of 32 MTW threads takes one row, one block
// of 16 heads and MTW of its 16-dim tiles; thread t holds 8 consecutive
// floats of that slice of every chunk's partial (tile t / 32, head
// (t / 2) % 16, dims 8 (t % 2) .. +7), loaded kBatch chunks per round trip
// (kBatch: the chunk count rounded up to a power of two, at most 16, so no
// load repeats a chunk).  Small workgroups make many of them: the merge is a
// streaming read.
template <int DV, int MTW, int kBatch>
__global__ __launch_bounds__(32 * MTW) void attn_combine_kernel(AttnLaunch a) {
  constexpr int MT = DV / 16;
  static_assert(MT % MTW == 0, "tiles per workgroup");
  const int row_local = (int)blockIdx.x;
  const int r = a.row_begin + row_local;
  const int hb = (int)blockIdx.y;
  const int tid = (int)threadIdx.x;
  const int mt_l = tid >> 5, hl = (tid >> 1) & 15, d0 = (tid & 1) * 8;
  if (mt_l >= MTW) return;
  const int mt = (int)blockIdx.z * MTW + mt_l;
  const int head = hb * 16 + hl;
  const bool head_ok = head < a.H_q;
  const int n = a.n_chunks;
  const int64_t cstride = part_block_floats(a.H_q, DV);
  const float* p0 = part_out(a, row_local, 0, DV) + (int64_t)hb * (MT * 256) + mt * 256 + hl * 16 + d0;
  const float2* st0 = part_stats(a, row_local, 0) + (head_ok ? head : 0);
  // one round trip per batch of chunks (partials and statistics together);
  // the running max M moves batch by batch, rescaling what has accumulated
  float M = -__builtin_inff();
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  float Ls = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kBatch) {
    v4f x[kBatch][2];
    float2 st[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = min(c0 + u, n - 1);
      x[u][0] = *reinterpret_cast<const v4f*>(p0 + c * cstride);
      x[u][1] = *reinterpret_cast<const v4f*>(p0 + c * cstride + 4);
      st[u] = st0[(int64_t)c * a.H_q];
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (c0 + u < n) Mb = fmaxf(Mb, st[u].x);
    if (Mb > M) {  // (never true while every chunk so far is empty)
      const float f = M == -__builtin_inff() ? 0.0f : exp2f(M - Mb);
      Ls *= f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= f;
      M = Mb;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      // empty chunks (max -inf) and chunks past n weigh 0
      const float wu = (c0 + u < n && st[u].x != -__builtin_inff()) ? exp2f(st[u].x - M) : 0.0f;
      Ls += wu * st[u].y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += x[u][0][i] * wu;
        acc[4 + i] += x[u][1][i] * wu;
      }
    }
  }
  if (!head_ok) return;
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  uint4 w;
  w.x = pack2(acc[0] * inv, acc[1] * inv);
  w.y = pack2(acc[2] * inv, acc[3] * inv);
  w.z = pack2(acc[4] * inv, acc[5] * inv);
  w.w = pack2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(a.out + ((int64_t)r * a.H_q + head) * DV + 16 * mt + d0) = w;
  if (a.lse && blockIdx.z == 0 && mt_l == 0 && d0 == 0)
    a.lse[(int64_t)r * a.H_q + head] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : -__builtin_inff();
}

// Waves (16 heads each) per workgroup.  The latent 576/512 kernel uses
// DSA_ATTN_LAT_WAVES (one workgroup per CU, as its tiles take most of the
// LDS: two waves make twice the workgroups of four, filling every CU for
// few rows); the staged kernel four, except for small heads and few of them.
#ifndef DSA_ATTN_LAT_WAVES
#define DSA_ATTN_LAT_WAVES 2
#endif
//
// From kWideRows rows on, bf16 latent rows take 64-head workgroups instead
// (four head waves, no key split: sparse_attn_latent_kernel<4, 4, 1>): each
// gathered row is then staged by half as many workgroups, which outweighs
// the larger partials once many rows fill the chip (measured on 32 rows x
// 32k: attention + merge 49.6 -> 47.2 us; 64 ragged rows up to 128k: 90.9
// -> 78.4 us; 4096 prefill rows: attention 254 -> 201 us per pass), while
// with 4 rows the key split of the 32-head workgroup is worth more (12.6
// against 13.6 us).  FP8 rows keep the 32-head kernel, the only one that
// decodes them.
constexpr int kWideRows = 16;
int waves_for(int H_q, int D_qk, bool latent, int num_rows, bool kv8) {
  if (D_qk == 576 && latent && DSA_ATTN_LATENT_DMA)
    return !kv8 && num_rows >= kWideRows ? 4 : DSA_ATTN_LAT_WAVES;
  return (H_q > kHPW || D_qk > 64) ? 4 : 1;
}

bool uses_latent_kernel(int D_qk, bool latent) {
  return D_qk == 576 && latent && DSA_ATTN_LATENT_DMA;
}

template <int DQK, int DV, int NW>
hipError_t launch_t(const AttnLaunch& a, hipStream_t s, StageEvents ev, StageEvents merge) {
  AttnGrid g;
  g.n_hg = (a.H_q + kHPW * NW - 1) / (kHPW * NW);
  g.n_units = a.num_rows * a.n_chunks;
  const int per = (a.K + a.n_chunks - 1) / a.n_chunks;
  g.chunk = (per + kSB - 1) / kSB * kSB;
  const int grid = (g.n_units + 7) / 8 * 8 * g.n_hg;
  void (*kernel)(AttnLaunch, AttnGrid) = nullptr;
  int threads = 64 * NW;
  if constexpr (DQK == lat::kDqk && NW > 1) {
    if (uses_latent_kernel(DQK, a.latent)) {
      // four head waves (64-head workgroups, from 16 rows on): no key
      // split, four sub-block buffers
      kernel = NW == 4 ? sparse_attn_latent_kernel<4, 4, 1> : sparse_attn_latent_kernel<DSA_ATTN_NBUF, NW, 1>;
      if constexpr (NW == 2) {
        // two head waves times two key halves (four waves: every SIMD of
        // the CU busy), for split and whole rows alike
        if (DSA_ATTN_KSPLIT == 2) {
          kernel = sparse_attn_latent_kernel<4, 4, 2>;
          threads = 256;
        }
        // the FP8 cache: codes staged by DMA, decoded into two bf16 tiles
        if (a.kv8) {
          kernel = sparse_attn_latent_kernel<2, 4, 2, true>;
          threads = 256;
        }
      }
    }
  }
  // (the 576-wide staged kernel only ever runs with four waves)
  if constexpr (DQK != lat::kDqk || NW == 4) {
    if (!kernel && !a.kv8)
      kernel = a.latent ? sparse_attn_kernel<DQK, DV, true, NW> : sparse_attn_kernel<DQK, DV, false, NW>;
  }
  // FP8 rows only ever run the two-head-wave kernel, which decodes them
  if (!kernel || (a.kv8 && NW != 2)) return hipErrorInvalidConfiguration;
  hipError_t e = launch_kernel(kernel, dim3(grid), dim3(threads), s, ev.start, ev.stop, a, g);
  if (e != hipSuccess) return e;
  if (a.n_chunks == 1) {
    if (merge.start && (e = hipEventRecord(merge.start, s)) != hipSuccess) return e;
    if (merge.stop && (e = hipEventRecord(merge.stop, s)) != hipSuccess) return e;
    return hipSuccess;
  }
  constexpr int MT = DV / 16, MTW = MT < DSA_ATTN_MERGE_TILES ? MT : DSA_ATTN_MERGE_TILES;
  void (*combine)(AttnLaunch) = a.n_chunks <= 2   ? attn_combine_kernel<DV, MTW, 2>
                                : a.n_chunks <= 4 ? attn_combine_kernel<DV, MTW, 4>
                                : a.n_chunks <= 8 ? attn_combine_kernel<DV, MTW, 8>
                                                  : attn_combine_kernel<DV, MTW, 16>;
  return launch_kernel(combine, dim3(a.num_rows, (a.H_q + 15) / 16, MT / MTW), dim3(32 * MTW), s,
                       merge.start, merge.stop, a);
}

}  // namespace

int attn_chunks(int num_rows, int H_q, int D_qk, int K, bool latent, bool kv8) {
  if (num_rows <= 0) return 1;
  const int hpw = kHPW * waves_for(H_q, D_qk, latent, num_rows, kv8);
  const int n_hg = (H_q + hpw - 1) / hpw;
  const int want = (DSA_ATTN_TARGET_WGS + num_rows * n_hg - 1) / (num_rows * n_hg);
  const int cap = uses_latent_kernel(D_qk, latent) ? kMaxChunkLat : kMaxChunk;
  const int least = (K + cap - 1) / cap;  // chunks must fit the kernel's slots
  const int most = max(least, min(DSA_ATTN_MAX_CHUNKS, (K + kSB - 1) / kSB));
  return min(64, max(least, min(want, most)));
}

size_t attn_partial_bytes(int num_rows, int H_q, int D_v, int n_chunks) {
  if (n_chunks <= 1) return 0;
  return part_stats_bytes(num_rows, n_chunks, H_q) +
         (size_t)num_rows * n_chunks * part_block_floats(H_q, D_v) * sizeof(float);
}

int attn_chunks_max(int num_rows, int H_q, int D_qk, int K) {
  // (FP8 rows, in 32-head workgroups, never take more chunks than bf16 rows)
  return max(attn_chunks(num_rows, H_q, D_qk, K, true, false),
             attn_chunks(num_rows, H_q, D_qk, K, false, false));
}

bool attn_uses_rowoff(int D_qk, int D_v, bool latent) {
  return D_v == lat::kDv && uses_latent_kernel(D_qk, latent);
}

hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s, StageEvents ev,
                              StageEvents merge) {
  if (a.num_rows <= 0) return hipSuccess;
  switch (waves_for(a.H_q, a.D_qk, a.latent, a.num_rows, a.kv8) * 1000 + a.D_qk) {
    case 2576: return launch_t<576, 512, 2>(a, s, ev, merge);
    case 4576: return launch_t<576, 512, 4>(a, s, ev, merge);
    case 4064: return launch_t<64, 64, 4>(a, s, ev, merge);
    default: return launch_t<64, 64, 1>(a, s, ev, merge);
  }
}

}  // namespace dsa
