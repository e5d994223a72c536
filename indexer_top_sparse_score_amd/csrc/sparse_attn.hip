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
// Work split.  A workgroup = 4 waves x 16 query heads = 64 heads of one row,
// over one chunk of the row's index list.  The chunk is walked 32 keys at a
// time: the 32 selected rows are gathered with 16-byte coalesced loads into
// LDS twice -- key-major for the logits and transposed (dims-major) for P.V.
// Per wave and 32 keys:
//   S^T[32 keys x 16 heads] = K[32 x D_qk] . Q^T     (v_mfma_f32_16x16x32_bf16,
//                                                    Q^T held in registers)
//   online softmax per head (exp2 domain), in registers
//   O^T[D_v x 16 heads]   += V^T[D_v x 32] . P^T    (P^T straight from the S^T
//                                                    accumulators, no LDS trip)
// The contraction index of P.V is permuted so that each lane's P^T operand is
// exactly the 8 logits its S^T accumulators already hold; the V^T operand is
// read with the same permutation.
// When the index list is split over several chunks, each chunk writes its
// (max, sum, unnormalised O) and a second kernel merges them by log-sum-exp.

#include "dsa_common.h"

namespace dsa {
namespace {

constexpr int kSB = 32;      // keys per sub-block
constexpr int kHPW = 16;     // heads per wave
constexpr int kWaves = 4;
constexpr int kHG = kHPW * kWaves;  // heads per workgroup
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

struct AttnGrid {
  int n_hg;     // head groups of 64
  int n_units;  // rows * chunks
  int chunk;    // index slots per chunk (multiple of kSB)
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

template <int DQK, int DV, bool LATENT>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(AttnLaunch a, AttnGrid g) {
  constexpr int KP = DQK + 8;    // key-major LDS pitch (elements)
  constexpr int VP = kSB + 4;    // dims-major LDS pitch (elements)
  constexpr int KS = DQK / 32;   // MFMA steps for the logits
  constexpr int MT = DV / 16;    // O^T row tiles
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kSB * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DV * VP];
  __shared__ int64_t koff[kSB];
  __shared__ int64_t voff[kSB];
  __shared__ uint32_t vmask;

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
  const int slot1 = min(a.K, slot0 + g.chunk);

  // Q^T operand: this lane's head, 8 dims per MFMA step
  const int head = hg * kHG + wave * kHPW + cidx;
  const bool head_ok = head < a.H_q;
  v8s qb[KS];
  {
    const uint16_t* qrow = a.q + ((int64_t)r * a.H_q + (head_ok ? head : 0)) * DQK + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (head_ok) {
        qb[ks] = *reinterpret_cast<const v8s*>(qrow + 32 * ks);
      } else {
        qb[ks] = v8s{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }

  v4f o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m2 = -__builtin_inff();  // running max of the log2-scaled logits
  float lsum = 0.0f;             // this lane's share of the running sum
  const float c2 = a.scale * kLog2e;

  const int32_t* idx_row = a.indices + (a.indices_row_offset + row_local) * (int64_t)a.K;
  const int32_t* bt = a.rows.block_table + (int64_t)b * a.rows.max_blocks;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k.base);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v.base);

  for (int s0 = slot0; s0 < slot1; s0 += kSB) {
    // ---- resolve the 32 selected positions to row addresses
    if (tid < kSB) {
      const int slot = s0 + tid;
      int64_t ko = -1, vo = -1;
      if (slot < slot1 && p >= 0) {
        const int idx = idx_row[slot];
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
      koff[tid] = ko;
      voff[tid] = vo;
      const uint64_t m = __ballot(ko >= 0);
      if (tid == 0) vmask = (uint32_t)m;
    }
    __syncthreads();

    // ---- gather into LDS (key-major Ks, dims-major Vt)
    if (LATENT) {
      // V = the first DV columns of each K row: one load feeds both copies.
      // Thread = (dims 8dg..8dg+7) x (keys 4kq..4kq+3), two passes of 4 keys.
      const int dg = tid & 63;
      if (dg < DV / 8) {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          const int kq = (tid >> 6) + 4 * pass;
          uint4 d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t off = koff[4 * kq + j];
            d[j] = off >= 0 ? *reinterpret_cast<const uint4*>(kbase + off + dg * 16)
                            : uint4{0, 0, 0, 0};
            *reinterpret_cast<uint4*>(&Ks[(4 * kq + j) * KP + 8 * dg]) = d[j];
          }
          const uint16_t* e = reinterpret_cast<const uint16_t*>(d);  // e[j*8 + dim]
#pragma unroll
          for (int dd = 0; dd < 8; ++dd) {
            uint2 t;
            t.x = e[0 * 8 + dd] | ((uint32_t)e[1 * 8 + dd] << 16);
            t.y = e[2 * 8 + dd] | ((uint32_t)e[3 * 8 + dd] << 16);
            *reinterpret_cast<uint2*>(&Vt[(8 * dg + dd) * VP + 4 * kq]) = t;
          }
        }
      }
      // columns DV..DQK-1 (the part only the logits use)
      constexpr int kRest = (DQK - DV) / 8;  // 16-byte pieces per row
      if constexpr (kRest > 0)
      for (int c = tid; c < kSB * kRest; c += 256) {
        const int key = c / kRest, piece = c % kRest;
        const int64_t off = koff[key];
        *reinterpret_cast<uint4*>(&Ks[key * KP + DV + 8 * piece]) =
            off >= 0 ? *reinterpret_cast<const uint4*>(kbase + off + DV * 2 + piece * 16)
                     : uint4{0, 0, 0, 0};
      }
    } else {
      constexpr int kPieces = DQK / 8;
      for (int c = tid; c < kSB * kPieces; c += 256) {
        const int key = c / kPieces, piece = c % kPieces;
        const int64_t off = koff[key];
        *reinterpret_cast<uint4*>(&Ks[key * KP + 8 * piece]) =
            off >= 0 ? *reinterpret_cast<const uint4*>(kbase + off + piece * 16)
                     : uint4{0, 0, 0, 0};
      }
      constexpr int kDG = DV / 8;
      for (int t = tid; t < kDG * 8; t += 256) {
        const int dg = t % kDG, kq = t / kDG;  // dims 8dg.., keys 4kq..
        uint4 d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t off = voff[4 * kq + j];
          d[j] = off >= 0 ? *reinterpret_cast<const uint4*>(vbase + off + dg * 16)
                          : uint4{0, 0, 0, 0};
        }
        const uint16_t* e = reinterpret_cast<const uint16_t*>(d);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          uint2 w2;
          w2.x = e[0 * 8 + dd] | ((uint32_t)e[1 * 8 + dd] << 16);
          w2.y = e[2 * 8 + dd] | ((uint32_t)e[3 * 8 + dd] << 16);
          *reinterpret_cast<uint2*>(&Vt[(8 * dg + dd) * VP + 4 * kq]) = w2;
        }
      }
    }
    __syncthreads();

    const uint32_t valid = vmask;
    if (valid != 0) {
      // ---- logits S^T (keys x heads): two 16-key tiles
      v4f s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* krow = &Ks[(16 * kt + cidx) * KP + 8 * grp];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const v8s ka = *reinterpret_cast<const v8s*>(krow + 32 * ks);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf, ka), __builtin_bit_cast(v8bf, qb[ks]), acc, 0, 0, 0);
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
      const float m_new = fmaxf(m2, mx);
      const bool live = m_new != -__builtin_inff();
      const float alpha = live ? exp2f(m2 - m_new) : 1.0f;
      float pv[8];
      float psum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float e = live ? exp2f(s[kt][v] - m_new) : 0.0f;
          pv[kt * 4 + v] = e;
          psum += e;
        }
      lsum = lsum * alpha + psum;
      m2 = m_new;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
      }
      // ---- O^T += V^T . P^T ; contraction slot e of lane group grp is
      //      key 4grp+e (e < 4) or 16+4grp+(e-4) (e >= 4)
      const v8bf pb = __builtin_bit_cast(
          v8bf, (uint4){pack2(pv[0], pv[1]), pack2(pv[2], pv[3]), pack2(pv[4], pv[5]),
                        pack2(pv[6], pv[7])});
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint16_t* vrow = &Vt[(16 * mt + cidx) * VP];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * grp);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * grp);
        const v8bf va = __builtin_bit_cast(v8bf, (uint4){lo.x, lo.y, hi.x, hi.y});
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[mt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (!head_ok) return;

  if (a.n_chunks == 1) {
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    uint16_t* orow = a.out + ((int64_t)r * a.H_q + head) * DV + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint2 w;
      w.x = pack2(o[mt][0] * inv, o[mt][1] * inv);
      w.y = pack2(o[mt][2] * inv, o[mt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * mt) = w;
    }
    if (a.lse && grp == 0)
      a.lse[(int64_t)r * a.H_q + head] = lsum > 0.0f ? (m2 + log2f(lsum)) * kLn2 : -__builtin_inff();
  } else {
    float* part = a.partial + (((int64_t)row_local * a.n_chunks + chunk) * a.H_q + head) * part_stride(DV);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<v4f*>(part + 16 * mt + 4 * grp) = o[mt];
    if (grp == 0) {
      part[DV] = m2;
      part[DV + 1] = lsum;
    }
  }
}

// Merges the per-chunk (max, sum, unnormalised O) of each (row, head).
template <int DV>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnLaunch a) {
  constexpr int PER = DV / 64;  // dims per lane
  const int row_local = blockIdx.x;
  const int r = a.row_begin + row_local;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (head >= a.H_q) return;
  const float* part0 = a.partial + ((int64_t)row_local * a.n_chunks * a.H_q + head) * part_stride(DV);
  const int64_t cstride = (int64_t)a.H_q * part_stride(DV);
  float M = -__builtin_inff();
  for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, part0[c * cstride + DV]);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  float Ls = 0.0f;
  if (M != -__builtin_inff()) {
    for (int c = 0; c < a.n_chunks; ++c) {
      const float* pc = part0 + c * cstride;
      const float mc = pc[DV];
      if (mc == -__builtin_inff()) continue;
      const float f = exp2f(mc - M);
      Ls += pc[DV + 1] * f;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += pc[lane * PER + i] * f;
    }
  }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  uint16_t* orow = a.out + ((int64_t)r * a.H_q + head) * DV + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[i] = bf16_bits(acc[i] * inv);
  if (a.lse && lane == 0)
    a.lse[(int64_t)r * a.H_q + head] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : -__builtin_inff();
}

template <int DQK, int DV>
hipError_t launch_t(const AttnLaunch& a, hipStream_t s) {
  AttnGrid g;
  g.n_hg = (a.H_q + kHG - 1) / kHG;
  g.n_units = a.num_rows * a.n_chunks;
  const int per = (a.K + a.n_chunks - 1) / a.n_chunks;
  g.chunk = (per + kSB - 1) / kSB * kSB;
  const int grid = (g.n_units + 7) / 8 * 8 * g.n_hg;
  if (a.latent)
    sparse_attn_kernel<DQK, DV, true><<<grid, 256, 0, s>>>(a, g);
  else
    sparse_attn_kernel<DQK, DV, false><<<grid, 256, 0, s>>>(a, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_chunks == 1) return e;
  attn_combine_kernel<DV><<<dim3(a.num_rows, (a.H_q + 3) / 4), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int attn_chunks(int num_rows, int H_q, int K) {
  if (num_rows <= 0) return 1;
  const int n_hg = (H_q + kHG - 1) / kHG;
  const int want = (256 + num_rows * n_hg - 1) / (num_rows * n_hg);
  const int most = max(1, min(16, (K + 2 * kSB - 1) / (2 * kSB)));
  return max(1, min(want, most));
}

size_t attn_partial_bytes(int num_rows, int H_q, int D_v, int n_chunks) {
  if (n_chunks <= 1) return 0;
  return (size_t)num_rows * n_chunks * H_q * part_stride(D_v) * sizeof(float);
}

hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s) {
  if (a.num_rows <= 0) return hipSuccess;
  if (a.D_qk == 576) return launch_t<576, 512>(a, s);
  return launch_t<64, 64>(a, s);
}

}  // namespace dsa
