// Indexer prolog on gfx950 (Baidu AI Cloud, "Day0 Inference Support and
// Performance Optimization for New Architecture LLMs", section 4.3): the Q
// projection with its per-group MXFP8 quantisation (section 5.1), the
// head-weight projection, and the RMS normalisation and quantisation of each
// row's new index key, written into the paged index-key cache.
//
// The page overlaps these small operators on three streams.  They are
// independent of one another, so here they are one dispatch whose grid is cut
// into three ranges of workgroups, one per operator, and the quantisation is
// the projection's epilogue: no intermediate tensor goes through memory and
// there is one launch instead of five.
//
// Projections: bf16 products, float32 accumulation (v_mfma_f32_16x16x32_bf16,
// A = 16 weight rows x 32 inputs, B = 32 inputs x 16 rows of x).  A
// workgroup owns 32 output features -- one quantisation group of one head,
// or 32 head weights -- for 16 NT rows.  Its KS waves split the input width;
// each streams its slice of the 32 weight rows straight into A operands (a
// load is 16 rows x 64 contiguous bytes) and accumulates the whole tile; the
// partial tiles are summed through LDS.  The weights are read once per tile
// of rows: for decode batches of at most 16 rows, once.
//
// Arithmetic of the outputs (readings of the page): q, the normalised key
// and the head weights are bf16 tensors, each the float32 result rounded to
// nearest even; a group of 32 values shares the scale 2^(floor(log2 amax) -
// 8) (the OCP microscaling rule, 8 being E4M3's largest exponent; 2^-127 for
// an all-zero group), and each code is its value over the scale rounded to
// nearest even in E4M3 and saturated at +-448.

#include "dsa_common.h"
#include "prolog.h"

namespace dsa {
namespace {

// x rounded to nearest even at bf16's 8 significant bits (finite x): adding
// 0x7FFF plus the kept part's last bit carries exactly past a tie to even.
__device__ __forceinline__ float bf16_round_f(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xFFFF0000u);
}

// E4M3 (OCP FN) code of x, rounded to nearest even, magnitudes from 448 up
// saturated to 448, the sign bit x's own.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (code 8 is 2^-6)
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // 2^e <= a < 2^(e+1)
    uint32_t m = (uint32_t)rintf((ldexpf(a, -e) - 1.0f) * 8.0f);
    if (m == 8u) {
      m = 0u;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | m;
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code | sign;
}

// The group's shared exponent from its largest magnitude (float bits):
// floor(log2 amax) - 8, clamped to E8M0's -127 .. 127; zero and subnormal
// maxima give -127.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 8;
  return e < -127 ? -127 : e > 127 ? 127 : e;
}

// Maximum over the 16 lanes of this lane's row.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  return x;
}
// Maximum over the aligned 32 lanes (two rows) holding this lane.
__device__ __forceinline__ float lanes32_max(float x) { return xor16(row16_max(x), FMax{}); }

// Workgroup -> unit of a range of n units, dealt so that the units each XCD
// runs are consecutive (workgroups go to the 8 XCDs in turn): tiles of rows
// that share a feature group share its weight rows through one L2.
__device__ __forceinline__ int xcd_unit(int bid, int n) {
  const int per = n / 8, rem = n % 8, x = bid % 8, slot = bid / 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + slot;
}

// The new key of row r (one wave): RMS-normalised with gamma, rounded to
// bf16, MXFP8-quantised and written at the row's slot of the key cache.
__device__ __forceinline__ void key_norm_row(const PrologLaunch& a, int r, int lane) {
  int b, p;
  if (!resolve_row(a.rows, r, b, p)) {
    if (lane == 0) report(a.err, DSA_DEVERR_ROW);
    return;
  }
  const int page = a.rows.block_table[(int64_t)b * a.rows.max_blocks + p / kBlock];
  if (page < 0 || page >= a.kI_num_blocks) {
    if (lane == 0) report(a.err, DSA_DEVERR_BLOCK);
    return;
  }
  const uint16_t* kr = a.k_new + (int64_t)r * a.D_I;
  float k0, k1 = 0.0f, g0, g1 = 0.0f;
  if (a.D_I == 128) {  // two elements per lane: 2l, 2l + 1
    const uint32_t kv = *reinterpret_cast<const uint32_t*>(kr + 2 * lane);
    const uint32_t gv = *reinterpret_cast<const uint32_t*>(a.k_gamma + 2 * lane);
    k0 = __uint_as_float(kv << 16);
    k1 = __uint_as_float(kv & 0xFFFF0000u);
    g0 = __uint_as_float(gv << 16);
    g1 = __uint_as_float(gv & 0xFFFF0000u);
  } else {  // D_I = 64: element l
    k0 = __uint_as_float((uint32_t)kr[lane] << 16);
    g0 = __uint_as_float((uint32_t)a.k_gamma[lane] << 16);
  }
  const float ss = across_wave(k0 * k0 + k1 * k1, FAdd{});
  const float inv = 1.0f / sqrtf(ss / (float)a.D_I + a.eps);
  const float y0 = bf16_round_f(k0 * inv * g0), y1 = bf16_round_f(k1 * inv * g1);
  // a group of 32 elements is 16 lanes (D_I = 128) or 32 lanes (D_I = 64)
  const float m = fmaxf(fabsf(y0), fabsf(y1));
  const float amax = a.D_I == 128 ? row16_max(m) : lanes32_max(m);
  const int se = mx_shared_exp(amax);
  uint8_t* blk = a.kI + (int64_t)page * a.kI_block_stride;
  uint8_t* crow = blk + (int64_t)(p % kBlock) * a.kI_row_stride;
  uint8_t* srow = blk + (int64_t)kBlock * a.kI_row_stride + (p % kBlock) * (a.D_I / 32);
  if (a.D_I == 128) {
    const uint32_t c = e4m3_code(ldexpf(y0, -se)) | (e4m3_code(ldexpf(y1, -se)) << 8);
    *reinterpret_cast<uint16_t*>(crow + 2 * lane) = (uint16_t)c;
    if ((lane & 15) == 0) srow[lane >> 4] = (uint8_t)(se + 127);
  } else {
    crow[lane] = (uint8_t)e4m3_code(ldexpf(y0, -se));
    if ((lane & 31) == 0) srow[lane >> 5] = (uint8_t)(se + 127);
  }
}

// One output of a projection, by the 32 consecutive lanes that hold a
// feature group of one row (feature f0 + feat, value v): q values go out as
// MXFP8 codes with the group's scale, head weights as float32.
__device__ __forceinline__ void store_output(const PrologLaunch& a, bool is_q, int r, int fgroup,
                                             int feat, float v) {
  const int F = a.H_I * a.D_I, f0 = 32 * fgroup;
  const float vb = bf16_round_f(v);
  if (is_q) {
    const int se = mx_shared_exp(lanes32_max(fabsf(vb)));
    if (r < a.num_rows) {
      a.qI[(int64_t)r * F + f0 + feat] = (uint8_t)e4m3_code(ldexpf(vb, -se));
      if (feat == 0) a.qI_scale[(int64_t)r * (F / 32) + fgroup] = (uint8_t)(se + 127);
    }
  } else if (r < a.num_rows && f0 + feat < a.H_I) {
    a.w[(int64_t)r * a.H_I + f0 + feat] = vb;
  }
}

template <int NT, int KS>
__global__ __launch_bounds__(64 * KS) void prolog_kernel(PrologLaunch a) {
  constexpr int kRows = 16 * NT;                 // rows per tile
  constexpr int kU = NT == 1 ? 8 : 4;            // 32-wide input steps per batch of loads
  __shared__ float red[KS][2 * NT * 256];        // the waves' partial tiles
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int F = a.H_I * a.D_I;
  const int rtiles = (a.num_rows + kRows - 1) / kRows;
  const int nq = (F / 32) * rtiles, ng = ((a.H_I + 31) / 32) * rtiles;
  const int bid = blockIdx.x;

  if (bid >= nq + ng) {  // K normalisation and quantisation: one wave per row
    const int r = (bid - nq - ng) * KS + wave;
    if (r < a.num_rows) key_norm_row(a, r, lane);
    return;
  }

  // ---- a projection tile: 32 features x kRows rows
  const bool is_q = bid < nq;
  const int unit = is_q ? xcd_unit(bid, nq) : bid - nq;
  const int fgroup = unit / rtiles, rtile = unit % rtiles;
  const int f0 = 32 * fgroup, r0 = kRows * rtile;
  const uint16_t* W = is_q ? a.w_q : a.w_g;
  const int nfeat = is_q ? F : a.H_I;
  const int cidx = lane & 15, kg = lane >> 4;
  const uint16_t* wrow[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int f = min(f0 + 16 * mt + cidx, nfeat - 1);  // past the last feature: unused
    wrow[mt] = W + (int64_t)f * a.D_x + 8 * kg;
  }
  const uint16_t* xrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = min(r0 + 16 * nt + cidx, a.num_rows - 1);  // past the last row: unused
    xrow[nt] = a.x + (int64_t)r * a.D_x + 8 * kg;
  }
  const int nsteps = a.D_x / 32;
  const int per = (nsteps + KS - 1) / KS;
  const int s0 = wave * per, s1 = min(nsteps, s0 + per);
  v4f acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = s0; s < s1; s += kU) {
    v8s av[kU][2], bv[kU][NT];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int k = 32 * min(s + u, s1 - 1);  // a step past the slice reloads its last one
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) av[u][mt] = *reinterpret_cast<const v8s*>(wrow[mt] + k);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bv[u][nt] = *reinterpret_cast<const v8s*>(xrow[nt] + k);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (s + u < s1) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(v8bf, av[u][mt]), __builtin_bit_cast(v8bf, bv[u][nt]),
                acc[mt][nt], 0, 0, 0);
      }
    }
  }
  // lane l, register i of tile (mt, nt) holds feature 16 mt + 4 (l / 16) + i
  // of the tile, row 16 nt + l % 16
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][(mt * NT + nt) * 256 + 64 * i + lane] = acc[mt][nt][i];
  __syncthreads();

  // epilogue: 32 consecutive threads hold the 32 features of one row
  const int feat = tid & 31, within = feat & 15, mt = feat >> 4;
  const int src_lane_hi = 16 * (within >> 2), ireg = within & 3;
#pragma unroll
  for (int rl = tid >> 5; rl < kRows; rl += 2 * KS) {
    const int nt = rl >> 4;
    const int idx = (mt * NT + nt) * 256 + 64 * ireg + src_lane_hi + (rl & 15);
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < KS; ++w) v += red[w][idx];
    store_output(a, is_q, r0 + rl, fgroup, feat, v);
  }
}

// Decode batches of at most R rows: the projections as
// matrix-vector products on the vector ALUs, so that every weight load is
// one contiguous kilobyte (lane l reads 8 consecutive inputs of one weight
// row) -- the access HBM and the address units serve best -- instead of the
// 16 rows x 64 bytes an MFMA operand needs.  A workgroup of 16 waves owns
// one q group of 32 features, 2 per wave.  Per chunk of
// inputs each wave issues all its weight loads at once (2 features x 4096
// inputs: 16 KB in flight per wave, 256 KB per CU), the chunk's R rows of x
// are staged in LDS meanwhile, and each lane keeps float32 partial sums for
// its 2 features x R rows, reduced across the wave at the end.
__device__ __forceinline__ void bf16x8_to_f32(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <int R>
__global__ __launch_bounds__(1024) void prolog_gemv_kernel(PrologLaunch a) {
  constexpr int kWaves = 16, kFW = 2;  // waves, q features per wave
  constexpr int KC = 32768 / R < 4096 ? 32768 / R : 4096;  // inputs per chunk (<= 64 KB of x in LDS)
  constexpr int kXP = R * KC / 8 / (64 * kWaves);          // 16-byte pieces of x per thread
  constexpr int kJ = KC / 512;         // 512-input loads per feature and chunk
  __shared__ __attribute__((aligned(16))) uint16_t xs[R * KC];
  __shared__ float res[32][R + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int F = a.H_I * a.D_I;
  const int nq = F / 32;
  const int bid = blockIdx.x;
  // Workgroup b < nq owns q group b.  The head weights and the new keys ride
  // along in the first workgroups -- head weight b for b < H_I (its kJ
  // 512-input slices of a chunk spread over waves 0 .. kJ - 1, one load
  // each), then key row b - H_I in wave 0 -- so a 64 x 128 indexer's 256
  // workgroups are the whole launch, one round on the chip's 256 CUs, with
  // no tail of workgroups after them (extra ones only when H_I + rows > nq).
  const bool has_q = bid < nq;
  const int gh = bid < a.H_I ? bid : -1;
  const int kr = bid >= a.H_I && bid < a.H_I + a.num_rows ? bid - a.H_I : -1;
  const bool gw = wave < kJ && gh >= 0;  // this wave adds slice `wave` of head weight gh
  __shared__ float gpart[kJ][R];
  const int fgroup = has_q ? bid : 0;
  const uint16_t* wr[kFW];  // this lane's weight rows
#pragma unroll
  for (int f = 0; f < kFW; ++f) wr[f] = a.w_q + (int64_t)(32 * fgroup + kFW * wave + f) * a.D_x;
  const uint16_t* wg = a.w_g + (int64_t)(gh >= 0 ? gh : 0) * a.D_x;
  float acc[kFW][R], accg[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    accg[r] = 0.0f;
#pragma unroll
    for (int f = 0; f < kFW; ++f) acc[f][r] = 0.0f;
  }

  static_assert(R * KC / 8 == kXP * 64 * kWaves && kJ <= kWaves, "whole pieces of x per thread");
  for (int c0 = 0; c0 < a.D_x && (has_q || gh >= 0); c0 += KC) {
    const int kc = min(KC, a.D_x - c0);  // a multiple of 32
    // this thread's pieces of the chunk's rows of x, loaded first so
    // that waiting for them does not wait for the weights behind them
    // (every load is issued unconditionally -- a piece past the chunk or
    // past the last row reads a valid address, and its value is dropped
    // only where it is used -- so that the waits count loads exactly)
    uint4 xv[kXP];
    int xo[kXP];
    bool xok[kXP];
#pragma unroll
    for (int t = 0; t < kXP; ++t) {
      const int i = tid + 64 * kWaves * t, r = i / (KC / 8), k8 = i % (KC / 8);
      xok[t] = r < a.num_rows && 8 * k8 < kc;
      xo[t] = r * KC + 8 * k8;
      xv[t] = *reinterpret_cast<const uint4*>(a.x + (xok[t] ? (int64_t)r * a.D_x + c0 + 8 * k8 : 0));
    }
    // load j of a feature covers inputs c0 + 512 j + 8 lane + 0..7 (lanes
    // past the chunk read its first piece and skip it below); the sums take
    // the loads in issue order as they arrive
    uint4 wv[kJ][kFW], wgv;
    const int goff = 512 * wave + 8 * lane < kc ? c0 + 512 * wave + 8 * lane : c0;
    if (gw) wgv = *reinterpret_cast<const uint4*>(wg + goff);
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int off = 512 * j + 8 * lane < kc ? c0 + 512 * j + 8 * lane : c0;
#pragma unroll
      for (int f = 0; f < kFW; ++f) wv[j][f] = *reinterpret_cast<const uint4*>(wr[f] + off);
    }
    __syncthreads();  // the previous chunk's x reads are done
#pragma unroll
    for (int t = 0; t < kXP; ++t)
      *reinterpret_cast<uint4*>(xs + xo[t]) = xok[t] ? xv[t] : uint4{0u, 0u, 0u, 0u};
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int kk = 512 * j + 8 * lane;
      if (kk < kc) {
        float wf[kFW][8];
#pragma unroll
        for (int f = 0; f < kFW; ++f) bf16x8_to_f32(wv[j][f], wf[f]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float xf[8];
          bf16x8_to_f32(*reinterpret_cast<const uint4*>(xs + r * KC + kk), xf);
#pragma unroll
          for (int f = 0; f < kFW; ++f)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[f][r] = fmaf(wf[f][e], xf[e], acc[f][r]);
        }
      }
    }
    if (gw && 512 * wave + 8 * lane < kc) {  // this wave's slice of the head weight
      float gf[8];
      bf16x8_to_f32(wgv, gf);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float xf[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(xs + r * KC + 512 * wave + 8 * lane), xf);
#pragma unroll
        for (int e = 0; e < 8; ++e) accg[r] = fmaf(gf[e], xf[e], accg[r]);
      }
    }
  }
  if (gw) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = across_wave(accg[r], FAdd{});
      if (lane == 0) gpart[wave][r] = v;
    }
  }
  __syncthreads();
  if (wave == 0) {
    if (gh >= 0 && lane < R && lane < a.num_rows) {  // the slices in order
      float v = 0.0f;
#pragma unroll
      for (int j = 0; j < kJ; ++j) v += gpart[j][lane];
      a.w[(int64_t)lane * a.H_I + gh] = bf16_round_f(v);
    }
    if (kr >= 0) key_norm_row(a, kr, lane);
  }
  if (!has_q) return;
#pragma unroll
  for (int f = 0; f < kFW; ++f)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = across_wave(acc[f][r], FAdd{});
      if (lane == 0) res[kFW * wave + f][r] = v;
    }
  __syncthreads();
  if (tid < 32 * R) {  // whole waves: 32 R is a multiple of 64
    const int r = tid >> 5, feat = tid & 31;
    store_output(a, true, r, fgroup, feat, res[feat][r]);
  }
}

// Batches of many rows (chunked prefill): the projections as an LDS-tiled
// GEMM.  A workgroup of 4 waves owns 128 features x 128 rows.  Per stage of
// 64 inputs the weight tile (128 features x 64) and the x tile (128 rows x
// 64) move HBM -> LDS by DMA (global_load_lds, 16 B per lane, 8 instructions
// per wave), two stages deep; the 16-byte pieces of tile row r sit at piece
// p ^ (r & 7), so the operand reads (16 rows at one piece) spread over the
// banks.  Each wave computes 64 features x 64 rows (4 x 4 MFMA tiles) from
// LDS: every byte fetched from L2 feeds 64 rows or features instead of 16.
namespace gemm {
constexpr int kBM = 128, kBN = 128, kBK = 64;         // features, rows, inputs per stage
constexpr int kPieces = kBK * 2 / 16;                  // 16-byte pieces per tile row
constexpr int kTileBytes = kBM * kBK * 2;              // 16 KB
constexpr int kStageBytes = 2 * kTileBytes;            // the W tile, then the x tile
constexpr int kDmaPerWave = kStageBytes / 1024 / 4;    // 8
static_assert(kBM == kBN, "one tile shape for both operands");
}  // namespace gemm

// One 16-byte-per-lane DMA, global -> LDS (lane l lands at lds + 16 l).  In
// inline asm so that the compiler's LDS reads do not all wait for every DMA
// in flight; the kernel orders the tiles itself (waitcnt + barrier).  M0
// carries the LDS address and is restored; the s_nop is the wait state an M0
// write needs before an LDS DMA reads it.
__device__ __forceinline__ void gemm_dma16(const void* src, uint32_t lds) {
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

__global__ __launch_bounds__(256) void prolog_gemm_kernel(PrologLaunch a) {
  using namespace gemm;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cidx = lane & 15, grp = lane >> 4;
  const int F = a.H_I * a.D_I;
  const int nqt = (F + kBM - 1) / kBM, ngt = (a.H_I + kBM - 1) / kBM;
  const int rtiles = (a.num_rows + kBN - 1) / kBN;
  const int nproj = (nqt + ngt) * rtiles;
  const int bid = blockIdx.x;
  if (bid >= nproj) {  // K normalisation and quantisation: one wave per row
    const int r = (bid - nproj) * 4 + wave;
    if (r < a.num_rows) key_norm_row(a, r, lane);
    return;
  }
  // units in (feature tile, row tile) order, dealt so that each XCD runs
  // consecutive units: the row tiles of a feature tile share its weights in
  // one L2
  const int unit = xcd_unit(bid, nproj);
  const int ft = unit / rtiles, rt = unit % rtiles;
  const bool is_q = ft < nqt;
  const uint16_t* W = is_q ? a.w_q : a.w_g;
  const int nfeat = is_q ? F : a.H_I;
  const int f0 = kBM * (is_q ? ft : ft - nqt), r0 = kBN * rt;
  const int nst = (a.D_x + kBK - 1) / kBK;

  // DMA of stage st: instruction i = kDmaPerWave wave + t fills the stage's
  // slots 64 i .. 64 i + 63: tile i / 16 (0: weights, 1: x), row sl / 8 and
  // LDS piece sl % 8 of it (sl = 64 (i % 16) + lane).  Rows past the last
  // feature or row read the last one (unused); inputs past D_x (a last stage
  // of 32) read the stage's first piece (unused).
  const uint8_t* src_row[kDmaPerWave];
  int src_piece[kDmaPerWave];
#pragma unroll
  for (int t = 0; t < kDmaPerWave; ++t) {
    const int i = kDmaPerWave * wave + t, sl = 64 * (i % 16) + lane;
    const int row = sl / kPieces, pc = sl % kPieces;
    const bool wt = i < 16;
    const int g = wt ? min(f0 + row, nfeat - 1) : min(r0 + row, a.num_rows - 1);
    src_row[t] = reinterpret_cast<const uint8_t*>((wt ? W : a.x) + (int64_t)g * a.D_x);
    src_piece[t] = pc ^ (row & 7);
  }
  auto issue = [&](int st) {
    const int k0 = kBK * st;
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds + (st & 1) * kStageBytes + 1024 * kDmaPerWave * wave));
#pragma unroll
    for (int t = 0; t < kDmaPerWave; ++t) {
      const int k = k0 + 8 * src_piece[t];
      gemm_dma16(src_row[t] + 2 * (k < a.D_x ? k : k0), base + 1024 * t);
    }
  };

  // this wave's 64 x 64 sub-tile and its operand read offsets
  const int fw = 64 * (wave & 1), rw = 64 * (wave >> 1);
  v4f acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

  issue(0);
  if (nst > 1) issue(1);
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's DMAs of stage st have landed
    const uint8_t* wt = lds + (st & 1) * kStageBytes;
    const uint8_t* xt = wt + kTileBytes;
    const int nks = min(2, (a.D_x - kBK * st) / 32);  // 32-input MFMA steps in the stage
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks < nks) {
        v8s af[4], bf[4];
        const int pc = 4 * ks + grp;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int ra = fw + 16 * m + cidx, rb = rw + 16 * m + cidx;
          af[m] = *reinterpret_cast<const v8s*>(wt + 16 * (ra * kPieces + (pc ^ (ra & 7))));
          bf[m] = *reinterpret_cast<const v8s*>(xt + 16 * (rb * kPieces + (pc ^ (rb & 7))));
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(v8bf, af[mt]), __builtin_bit_cast(v8bf, bf[nt]), acc[mt][nt], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done with buffer st & 1
    if (st + 2 < nst) issue(st + 2);
  }

  // epilogue: lane (grp, cidx), register i of tile (mt, nt) holds feature
  // f0 + fw + 16 mt + 4 grp + i of row r0 + rw + 16 nt + cidx; a q group of 32
  // features is the tile pair (2 p, 2 p + 1), spread over the 4 lanes of
  // equal cidx
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int r = r0 + rw + 16 * nt + cidx;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int fg = f0 + fw + 32 * pg;  // the group's first feature
      float vb[2][4];
      float m = 0.0f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vb[h][i] = bf16_round_f(acc[2 * pg + h][nt][i]);
          m = fmaxf(m, fabsf(vb[h][i]));
        }
      if (is_q) {
        const int se = mx_shared_exp(across_rows(m, FMax{}));
        if (r < a.num_rows && fg < F) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) c |= e4m3_code(ldexpf(vb[h][i], -se)) << (8 * i);
            *reinterpret_cast<uint32_t*>(a.qI + (int64_t)r * F + fg + 16 * h + 4 * grp) = c;
          }
          if (grp == 0) a.qI_scale[(int64_t)r * (F / 32) + fg / 32] = (uint8_t)(se + 127);
        }
      } else if (r < a.num_rows) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int f = fg + 16 * h + 4 * grp + i;
            if (f < a.H_I) a.w[(int64_t)r * a.H_I + f] = vb[h][i];
          }
      }
    }
  }
}

}  // namespace

hipError_t launch_indexer_prolog(const PrologLaunch& a, hipStream_t s) {
  const int F = a.H_I * a.D_I;
  const int ngemv = max(F / 32, a.H_I + a.num_rows);
  // (measured at 4096 inputs, 64 x 128: 4 rows 19.9 us on the vector ALUs
  // against 25.7 us on the MFMA tile; at 8 rows the vector-ALU kernel's
  // registers spill)
  if (a.num_rows <= 4) {
    prolog_gemv_kernel<4><<<ngemv, 1024, 0, s>>>(a);
  } else if (a.num_rows <= 16) {
    constexpr int NT = 1, KS = 8;
    const int n = F / 32 + (a.H_I + 31) / 32 + (a.num_rows + KS - 1) / KS;
    prolog_kernel<NT, KS><<<n, 64 * KS, 0, s>>>(a);
  } else {
    using namespace gemm;
    const int rt = (a.num_rows + kBN - 1) / kBN;
    const int n = ((F + kBM - 1) / kBM + (a.H_I + kBM - 1) / kBM) * rt + (a.num_rows + 3) / 4;
    prolog_gemm_kernel<<<n, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dsa
