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
// its (max, sum, unnormalised O) and a second kernel merges them by
// log-sum-exp.

#include "dsa_common.h"

#ifndef DSA_ATTN_MAX_CHUNKS
#define DSA_ATTN_MAX_CHUNKS 16
#endif
#ifndef DSA_ATTN_TARGET_WGS
#define DSA_ATTN_TARGET_WGS 256
#endif

namespace dsa {
namespace {

constexpr int kSB = 32;        // keys per sub-block
constexpr int kHPW = 16;       // heads per wave
constexpr int kMaxChunk = 256; // index slots per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// floats per (row, chunk, head) partial record: O[DV], max, sum, 2 pad
__host__ __device__ constexpr int part_stride(int dv) { return dv + 4; }

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

struct AttnGrid {
  int n_hg;     // head groups
  int n_units;  // rows * chunks
  int chunk;    // index slots per chunk (multiple of kSB, <= kMaxChunk)
};

// Maps a workgroup to (unit, head group) so that the head groups of one
// (row, chunk) unit land on the same XCD (workgroups are dealt round-robin
// to the 8 XCDs) and share the gathered rows through that XCD's L2.
__device__ __forceinline__ bool decode_wg(const AttnGrid& g, int& unit, int& hg) {
  const int id = (int)blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  hg = slot % g.n_hg;
  unit = (slot / g.n_hg) * 8 + xcd;
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
  static constexpr int kKsElems = kSB * KP;
  static constexpr int kVtElems = DV * VP;
};

template <class C>
struct Staged {
  uint4 v[C::kVJ > 0 ? C::kVJ : 1][4];
  uint4 k[C::kKJ > 0 ? C::kKJ : 1];
};

template <int DQK, int DV, bool LATENT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void sparse_attn_kernel(AttnLaunch a, AttnGrid g) {
  using C = Cfg<DQK, DV, LATENT, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::kKsElems];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][C::kVtElems];
  __shared__ int64_t koff[kMaxChunk];
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
        st.v[i][j] = *reinterpret_cast<const uint4*>((LATENT ? kbase : vbase) +
                                                     (off >= 0 ? off : 0) + dg * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < C::kKJ; ++i) {
      const int job = tid + i * C::kThreads;
      const int key = (job / C::kKPieces) % kSB, piece = job % C::kKPieces;
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
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st.v[i][j] = keep_or_zero(st.v[i][j], (LATENT ? koff : voff)[base + 4 * kq + j] >= 0);
      if (mine) {
      if (LATENT) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint4*>(&ks[(4 * kq + j) * C::KP + 8 * dg]) = st.v[i][j];
      }
      // transpose: st.v[i][j] holds dims 8dg..8dg+7 of key 4kq+j; row
      // 8dg+dd of V^T takes element dd of each of the 4 keys
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const uint32_t a0 = word(st.v[i][0], dd >> 1), a1 = word(st.v[i][1], dd >> 1);
        const uint32_t a2 = word(st.v[i][2], dd >> 1), a3 = word(st.v[i][3], dd >> 1);
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
      const int key = (job / C::kKPieces) % kSB, piece = job % C::kKPieces;
      const int d0 = (LATENT ? DV : 0) + 8 * piece;
      if (mine)
        *reinterpret_cast<uint4*>(&ks[key * C::KP + d0]) = keep_or_zero(st.k[i], koff[base + key] >= 0);
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
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
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

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (!head_ok) return;

  if (a.n_chunks == 1) {
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    uint16_t* orow = a.out + ((int64_t)r * a.H_q + head) * DV + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      uint2 w;
      w.x = pack2(o[mt][0] * inv, o[mt][1] * inv);
      w.y = pack2(o[mt][2] * inv, o[mt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * mt) = w;
    }
    if (a.lse && grp == 0)
      a.lse[(int64_t)r * a.H_q + head] = lsum > 0.0f ? (m2 + log2f(lsum)) * kLn2 : -__builtin_inff();
  } else {
    float* part = a.partial +
                  (((int64_t)row_local * a.n_chunks + chunk) * a.H_q + head) * part_stride(DV);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
      *reinterpret_cast<v4f*>(part + 16 * mt + 4 * grp) = o[mt];
    if (grp == 0) {
      part[DV] = m2;
      part[DV + 1] = lsum;
    }
  }
}

// Merges the per-chunk (max, sum, unnormalised O) of each (row, head): one
// wave per head; lane c holds chunk c's statistics.
template <int DV>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnLaunch a) {
  constexpr int PER = DV / 64;  // dims per lane
  const int row_local = blockIdx.x;
  const int r = a.row_begin + row_local;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (head >= a.H_q) return;
  const int n = a.n_chunks;  // <= 64
  const float* part0 = a.partial + ((int64_t)row_local * n * a.H_q + head) * part_stride(DV);
  const int64_t cstride = (int64_t)a.H_q * part_stride(DV);
  const float mc = lane < n ? part0[lane * cstride + DV] : -__builtin_inff();
  const float lc = lane < n ? part0[lane * cstride + DV + 1] : 0.0f;
  float M = mc;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  float Ls = 0.0f;
  if (M != -__builtin_inff()) {
    const float f = mc == -__builtin_inff() ? 0.0f : exp2f(mc - M);
    Ls = lc * f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) Ls += __shfl_xor(Ls, o);
    int c = 0;
    for (; c + 4 <= n; c += 4) {
      float x[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < PER; ++i) x[u][i] = part0[(c + u) * cstride + lane * PER + i];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float fu = __shfl(f, c + u);
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += x[u][i] * fu;
      }
    }
    for (; c < n; ++c) {
      const float fu = __shfl(f, c);
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += part0[c * cstride + lane * PER + i] * fu;
    }
  }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  uint16_t* orow = a.out + ((int64_t)r * a.H_q + head) * DV + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[i] = bf16_bits(acc[i] * inv);
  if (a.lse && lane == 0)
    a.lse[(int64_t)r * a.H_q + head] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : -__builtin_inff();
}

// four waves (64 heads, one wave per SIMD and so the whole register file
// each) per workgroup, except for small heads and few of them
int waves_for(int H_q, int D_qk) { return (H_q > kHPW || D_qk > 64) ? 4 : 1; }

template <int DQK, int DV, int NW>
hipError_t launch_t(const AttnLaunch& a, hipStream_t s) {
  AttnGrid g;
  g.n_hg = (a.H_q + kHPW * NW - 1) / (kHPW * NW);
  g.n_units = a.num_rows * a.n_chunks;
  const int per = (a.K + a.n_chunks - 1) / a.n_chunks;
  g.chunk = (per + kSB - 1) / kSB * kSB;
  const int grid = (g.n_units + 7) / 8 * 8 * g.n_hg;
  if (a.latent)
    sparse_attn_kernel<DQK, DV, true, NW><<<grid, 64 * NW, 0, s>>>(a, g);
  else
    sparse_attn_kernel<DQK, DV, false, NW><<<grid, 64 * NW, 0, s>>>(a, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_chunks == 1) return e;
  attn_combine_kernel<DV><<<dim3(a.num_rows, (a.H_q + 3) / 4), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int attn_chunks(int num_rows, int H_q, int D_qk, int K) {
  if (num_rows <= 0) return 1;
  const int hpw = kHPW * waves_for(H_q, D_qk);
  const int n_hg = (H_q + hpw - 1) / hpw;
  const int want = (DSA_ATTN_TARGET_WGS + num_rows * n_hg - 1) / (num_rows * n_hg);
  const int least = (K + kMaxChunk - 1) / kMaxChunk;  // chunks must fit kMaxChunk slots
  const int most = max(least, min(DSA_ATTN_MAX_CHUNKS, (K + kSB - 1) / kSB));
  return min(64, max(least, min(want, most)));
}

size_t attn_partial_bytes(int num_rows, int H_q, int D_v, int n_chunks) {
  if (n_chunks <= 1) return 0;
  return (size_t)num_rows * n_chunks * H_q * part_stride(D_v) * sizeof(float);
}

hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s) {
  if (a.num_rows <= 0) return hipSuccess;
  if (a.D_qk == 576) return launch_t<576, 512, 4>(a, s);
  return waves_for(a.H_q, a.D_qk) == 4 ? launch_t<64, 64, 4>(a, s) : launch_t<64, 64, 1>(a, s);
}

}  // namespace dsa
