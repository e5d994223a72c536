// CPU oracle of the indexer -> Top-K -> sparse-attention step, in plain C++.
//
// TEST INFRASTRUCTURE ONLY.  This is the slow, obviously correct statement of
// what the hot path computes.  Only the test-suite, the package smoke check
// and the CPU-baseline leg of the benchmark load it (through oracle/cpp.py).
// It shares no code, header, table or constant with the HIP library, and
// neither one includes the other.
//
// Each step follows Baidu AI Cloud's "Day0 Inference Support and Performance
// Optimization for New Architecture LLMs", section 2.2 (score every
// historical position, aggregate the per-head scores with head weights, keep
// the Top-K positions, attend over only those rows), with the paged caches of
// sections 4.1-4.2 and the MXFP8 indexer format of section 5.1.  Readings of
// what the pages leave open (ReLU gate, tie rule, ascending output, latent V,
// history inclusive of the current token) are stated where they are used.
//
// Arithmetic is binary64.  The per-head dot products of E4M3 codes are exact
// (products of 4-bit-mantissa values summed over at most a few hundred terms
// fit in 53 bits; power-of-two group scales keep them exact); the weighted
// head sum runs in ascending head order and is rounded once to binary32.
// Top-K is a full sort.  Attention is the softmax definition over the
// gathered rows (THInfer, eq. 9, restricted to the selected set).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

namespace {

// ------------------------------------------------------------------ formats
// OCP E4M3 "FN": sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
// holds subnormals m * 2^-9; 0x7F and 0xFF are NaN; no infinities.
double e4m3_value(uint8_t code) {
  const double sign = (code & 0x80) ? -1.0 : 1.0;
  const int e = (code >> 3) & 0xF, m = code & 0x7;
  if (e == 0xF && m == 0x7) return std::nan("");
  if (e == 0) return sign * m * std::ldexp(1.0, -9);
  return sign * (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
}

struct E4M3Table {
  double v[256];
  E4M3Table() {
    for (int c = 0; c < 256; ++c) v[c] = e4m3_value((uint8_t)c);
  }
};
const E4M3Table& e4m3() {
  static const E4M3Table t;
  return t;
}

// E8M0 scale byte (OCP microscaling): 2^(e - 127); 255 is NaN.
double e8m0_value(uint8_t e) { return e == 255 ? std::nan("") : std::ldexp(1.0, (int)e - 127); }

// bfloat16: the upper half of a binary32.
double bf16_value(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// FP8 KV cache (Day0 article, section 5.2: FP8, quantised per token and head
// in tiles of 128 elements).  Readings: E4M3 codes, one binary32 scale per
// tile, value = code value * scale; a row of D elements has ceil(D / 128)
// tiles, the last one shorter when 128 does not divide D.
constexpr int kKvTile = 128;
int kv_tiles(int D) { return (D + kKvTile - 1) / kKvTile; }
double kv_fp8_value(uint8_t code, float scale) { return e4m3().v[code] * (double)scale; }

// Order-preserving key of a binary32 score: larger score, larger key; -0 and
// +0 share a key; NaN gets 0 and ranks below every number.
uint32_t score_key(float s) {
  if (std::isnan(s)) return 0u;
  if (s == 0.0f) s = 0.0f;
  uint32_t u;
  std::memcpy(&u, &s, 4);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------ indexer prolog
// Day0 article, section 4.3 (Q projection, K normalisation, per-group Q
// quantisation, head-weight projection), with the MXFP8 format of section
// 5.1 and bf16 projections (section 5.3).  Readings: the prolog's tensors (q,
// the normalised key, g) are bf16 activations, each the exact value rounded
// once to nearest even; the K normalisation is RMS normalisation with a bf16
// weight; the group scale follows the OCP microscaling conversion.

// Nearest-even rounding of v to bfloat16 (8 significant bits; below 2^-126
// the fixed 2^-133 grid of the subnormals).  std::nearbyint rounds half to
// even in the default rounding mode.
uint16_t bf16_round_bits(double v) {
  int e;
  std::frexp(v, &e);  // v = f 2^e, 0.5 <= |f| < 1
  const int qe = std::max(e, -125) - 8;
  const double r = std::ldexp(std::nearbyint(std::ldexp(v, -qe)), qe);
  const float f = (float)r;  // exact: r has at most 8 significant bits
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

// E4M3 code of v: the magnitude (saturated at 448) is split into exponent and
// a 3-bit mantissa rounded half to even; subnormals are multiples of 2^-9.
// The sign bit is v's own, also when the magnitude rounds to zero.
uint8_t e4m3_round_code(double v) {
  const double a = std::min(std::fabs(v), 448.0);
  int code;
  if (a < std::ldexp(1.0, -6)) {
    code = (int)std::nearbyint(std::ldexp(a, 9));  // 0..8; 8 is 2^-6, code 0x08
  } else {
    int E;
    std::frexp(a, &E);
    int e = E - 1;  // 2^e <= a < 2^(e+1)
    int m = (int)std::nearbyint((std::ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8) {
      m = 0;
      ++e;
    }
    code = ((e + 7) << 3) | m;
    if (code > 0x7E) code = 0x7E;
  }
  return (uint8_t)(code | (std::signbit(v) ? 0x80 : 0));
}

// One group of n values: the shared scale byte and the codes.  The scale is
// 2^(floor(log2 max|v|) - 8), 8 being E4M3's largest exponent, clamped to
// E8M0's 2^-127 .. 2^127 (2^-127 for an all-zero group).
void mx_quantize_group(const double* v, int n, uint8_t* codes, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(v[i]));
  int shared = -127;
  if (amax > 0.0) {
    int E;
    std::frexp(amax, &E);
    shared = std::min(127, std::max(-127, E - 1 - 8));
  }
  *scale = (uint8_t)(shared + 127);
  for (int i = 0; i < n; ++i) codes[i] = e4m3_round_code(std::ldexp(v[i], -shared));
}

// Sum of products of two bf16 rows in binary64 with Neumaier's compensation,
// so the rounding of the result to bf16 sees the exact sum in all but
// pathological cases (integer inputs are exact either way).
double dot_bf16(const uint16_t* a, const uint16_t* b, int n) {
  double s = 0.0, c = 0.0;
  for (int i = 0; i < n; ++i) {
    const double t = bf16_value(a[i]) * bf16_value(b[i]);  // exact
    const double u = s + t;
    c += std::fabs(s) >= std::fabs(t) ? (s - u) + t : (t - u) + s;
    s = u;
  }
  return s + c;
}

// Runs fn(i) for i in [0, n) on up to `threads` host threads.
template <class F>
void parallel_for(int64_t n, int threads, F fn) {
  if (threads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  const int t = (int)std::min<int64_t>(threads, n);
  std::vector<std::thread> pool;
  for (int k = 0; k < t; ++k)
    pool.emplace_back([&, k] {
      for (int64_t i = k; i < n; i += t) fn(i);
    });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// Value of every E4M3 code (for pins against other decoders).
void orc_e4m3_table(double* out) {
  for (int c = 0; c < 256; ++c) out[c] = e4m3().v[c];
}

void orc_score_keys(const float* s, int64_t n, uint32_t* keys) {
  for (int64_t i = 0; i < n; ++i) keys[i] = score_key(s[i]);
}

// Index scores of one query row against n key rows (Day0 article, section
// 2.2): I[s] = sum_h w[h] * max(0, dot_h[s]), dot_h[s] = sum_d qI[h,d] kI[s,d].
//   qI [H][D] E4M3 codes, w [H] binary32, kI [n][D] E4M3 codes (gathered).
//   MXFP8 (qs, ks non-NULL; section 5.1): dims in groups of 32 share an E8M0
//   scale, qs [H][D/32], ks [n][D/32]; each group's partial dot is scaled by
//   both groups' scales before the groups are summed.
// Reading: the ReLU gate acts per head before the weighting.  One shared key
// row per position serves every head.  A zero score is stored as +0.
void orc_indexer_scores(const uint8_t* qI, const float* w, const uint8_t* kI, const uint8_t* qs,
                        const uint8_t* ks, int H, int D, int64_t n, float* out, int threads) {
  const double* t = e4m3().v;
  const int G = D / 32;
  std::vector<double> q((size_t)H * D);
  for (size_t i = 0; i < q.size(); ++i) q[i] = t[qI[i]];
  const int64_t chunk = 256;
  parallel_for((n + chunk - 1) / chunk, threads, [&](int64_t c) {
    std::vector<double> k(D);
    for (int64_t s = c * chunk; s < std::min(n, (c + 1) * chunk); ++s) {
      for (int d = 0; d < D; ++d) k[d] = t[kI[s * D + d]];
      double total = 0.0;
      for (int h = 0; h < H; ++h) {
        double dot = 0.0;
        if (!qs) {
          for (int d = 0; d < D; ++d) dot += q[(size_t)h * D + d] * k[d];
        } else {
          for (int g = 0; g < G; ++g) {
            double part = 0.0;
            for (int d = 32 * g; d < 32 * g + 32; ++d) part += q[(size_t)h * D + d] * k[d];
            dot += part * e8m0_value(qs[h * G + g]) * e8m0_value(ks[s * G + g]);
          }
        }
        total += (double)w[h] * std::max(0.0, dot);
      }
      out[s] = (float)total + 0.0f;
    }
  });
}

// Top-K of one row's n scores (Day0 article, section 2.2): the min(K, n)
// slots with the largest score; readings: equal scores go to the lower slot,
// NaN ranks last, the kept slots are written in ascending order and -1 pads
// to K.  A full sort by (key descending, slot ascending).  Returns the count.
int64_t orc_topk(const float* scores, int64_t n, int64_t K, int32_t* idx) {
  std::vector<int64_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::vector<uint32_t> key(n);
  for (int64_t i = 0; i < n; ++i) key[i] = score_key(scores[i]);
  std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    return key[a] != key[b] ? key[a] > key[b] : a < b;
  });
  const int64_t count = std::min(K, n);
  std::vector<int64_t> kept(order.begin(), order.begin() + count);
  std::sort(kept.begin(), kept.end());
  for (int64_t j = 0; j < K; ++j) idx[j] = j < count ? (int32_t)kept[j] : -1;
  return count;
}

// Softmax attention of one query row (H heads, bf16 q [H][Dqk]) over n
// gathered rows of decoded values: logit[h,j] = scale sum_d q[h,d] k[j,d];
// o[h] = sum_j exp(logit - m) v[j] / sum_j exp(logit - m); lse[h] = m +
// ln(sum).  With no rows: o = 0 and lse = -inf.  k [n][Dqk], v [n][Dv].
static void attention_values(const uint16_t* q, const double* k, const double* v, int64_t n,
                             int H, int Dqk, int Dv, double scale, double* o, double* lse, int threads) {
  parallel_for(H, threads, [&](int64_t h) {
    double* oh = o + h * Dv;
    for (int d = 0; d < Dv; ++d) oh[d] = 0.0;
    if (n == 0) {
      lse[h] = -INFINITY;
      return;
    }
    std::vector<double> logit(n);
    for (int64_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int d = 0; d < Dqk; ++d) dot += bf16_value(q[h * Dqk + d]) * k[j * Dqk + d];
      logit[j] = scale * dot;
    }
    const double m = *std::max_element(logit.begin(), logit.end());
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      const double p = std::exp(logit[j] - m);
      l += p;
      for (int d = 0; d < Dv; ++d) oh[d] += p * v[j * Dv + d];
    }
    for (int d = 0; d < Dv; ++d) oh[d] /= l;
    lse[h] = m + std::log(l);
  });
}

// attention_values with bf16 rows: k [n][Dqk], v [n][Dv] (bf16 bits).
void orc_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t n, int H,
                   int Dqk, int Dv, double scale, double* o, double* lse, int threads) {
  std::vector<double> kd((size_t)n * Dqk), vd((size_t)n * Dv);
  for (size_t i = 0; i < kd.size(); ++i) kd[i] = bf16_value(k[i]);
  for (size_t i = 0; i < vd.size(); ++i) vd[i] = bf16_value(v[i]);
  attention_values(q, kd.data(), vd.data(), n, H, Dqk, Dv, scale, o, lse, threads);
}

// Decoded values of n FP8 KV rows: codes [n][D] (E4M3), scales
// [n][ceil(D / 128)] -> out [n][D].
void orc_kv_fp8_decode(const uint8_t* codes, const float* scales, int64_t n, int D, double* out) {
  const int T = kv_tiles(D);
  for (int64_t j = 0; j < n; ++j)
    for (int d = 0; d < D; ++d)
      out[j * D + d] = kv_fp8_value(codes[j * D + d], scales[j * T + d / kKvTile]);
}

// The same attention by brute force over every one of the n rows of a
// history, with the unselected ones masked to -inf before the softmax
// (selected: n flags).  A different route to orc_attention's result.
void orc_masked_dense_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const uint8_t* selected, int64_t n, int H, int Dqk, int Dv,
                                double scale, double* o, double* lse) {
  for (int h = 0; h < H; ++h) {
    std::vector<double> s(n);
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int d = 0; d < Dqk; ++d) dot += bf16_value(q[h * Dqk + d]) * bf16_value(k[j * Dqk + d]);
      s[j] = selected[j] ? scale * dot : -INFINITY;
      m = std::max(m, s[j]);
    }
    double l = 0.0;
    for (int d = 0; d < Dv; ++d) o[h * Dv + d] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      const double e = std::isinf(s[j]) ? 0.0 : std::exp(s[j] - m);
      l += e;
      for (int d = 0; d < Dv; ++d) o[h * Dv + d] += e * bf16_value(v[j * Dv + d]);
    }
    for (int d = 0; d < Dv; ++d) o[h * Dv + d] /= l;
    lse[h] = m + std::log(l);
  }
}

// The inputs of a whole step, in the layouts of the caches (raw bits).
struct OrcStep {
  int32_t num_rows, num_seqs, max_blocks, num_blocks;
  const int32_t* seq_lens;     // [num_seqs]
  const int32_t* block_table;  // [num_seqs][max_blocks]
  const int32_t* row_seq;      // [num_rows] or NULL: row r -> sequence r
  const int32_t* row_pos;      // [num_rows] or NULL: seq_lens[b] - 1
  int32_t H_I, D_I;
  const uint8_t* qI;           // [num_rows][H_I][D_I]
  const float* w;              // [num_rows][H_I]
  const uint8_t* kI;           // [num_blocks][64][D_I]
  const uint8_t* qI_scale;     // [num_rows][H_I][D_I/32] or NULL
  const uint8_t* kI_scale;     // [num_blocks][64][D_I/32] or NULL
  const int32_t* cand;         // [num_rows][n_cand] or NULL
  const int32_t* cand_len;     // [num_rows]
  int32_t n_cand;
  int32_t H_q, D_qk, D_v, K;
  double scale;
  const uint16_t* q;           // [num_rows][H_q][D_qk]
  const uint16_t* k;           // [num_blocks][64][D_qk] (bf16 KV cache)
  const uint16_t* v;           // [num_blocks][64][D_v] or NULL: V = the first D_v of each K row
  const uint8_t* k8;           // FP8 KV cache instead of k, v: [num_blocks][64][D_qk] E4M3
  const float* k8_scale;       //   codes and [num_blocks][64][ceil(D_qk/128)] tile scales;
                               //   latent layout (V = the first D_v of each decoded row)
};

// The step for the rows listed (n_sel of them, row ids), in order:
//   indices [n_sel][K], counts [n_sel], out [n_sel][H_q][D_v], lse [n_sel][H_q],
//   scores  [n_sel][ld] (or NULL; NaN past each row's history).
// Row r's history is positions 0 .. p_r inclusive (reading: the current
// token's key is already in the cache); position s lives in block
// block_table[b][s / 64], row s % 64 (Day0 article, sections 4.1-4.2).  A
// candidate-restricted row scores only its list's first cand_len[r] entries
// (vLLM's DeepSeek-V4.1-Flash article, "Kernels") and keeps the Top-K slots
// of the list, written as their positions.  Returns 0, or -1 for a row whose
// sequence or position is out of range.
int orc_decode_step(const OrcStep* p, const int32_t* rows, int n_sel, int32_t* indices,
                    int64_t* counts, double* out, double* lse, float* scores, int64_t ld,
                    int threads) {
  const int B = 64;
  for (int i = 0; i < n_sel; ++i) {
    const int r = rows[i];
    const int b = p->row_seq ? p->row_seq[r] : r;
    if (b < 0 || b >= p->num_seqs) return -1;
    const int pos = p->row_pos ? p->row_pos[r] : p->seq_lens[b] - 1;
    if (pos < 0 || pos >= p->seq_lens[b] || pos >= p->max_blocks * B) return -1;
    const int32_t* bt = p->block_table + (int64_t)b * p->max_blocks;
    // the history this row scores
    std::vector<int64_t> hist;
    if (p->cand) {
      const int32_t* c = p->cand + (int64_t)r * p->n_cand;
      const int n = std::max(0, std::min(p->cand_len[r], p->n_cand));
      for (int j = 0; j < n; ++j) {
        if (c[j] < 0 || c[j] > pos || (j > 0 && c[j] <= c[j - 1])) return -1;
        hist.push_back(c[j]);
      }
    } else {
      hist.resize(pos + 1);
      std::iota(hist.begin(), hist.end(), 0);
    }
    const int64_t n = (int64_t)hist.size();
    // gather the index keys (and their scales) of the history
    const int D = p->D_I, G = D / 32;
    std::vector<uint8_t> kI((size_t)n * D), ks(p->kI_scale ? (size_t)n * G : 0);
    for (int64_t j = 0; j < n; ++j) {
      const int64_t row = (int64_t)bt[hist[j] / B] * B + hist[j] % B;
      std::memcpy(&kI[(size_t)j * D], p->kI + row * D, D);
      if (p->kI_scale) std::memcpy(&ks[(size_t)j * G], p->kI_scale + row * G, G);
    }
    std::vector<float> sc(n);
    orc_indexer_scores(p->qI + (int64_t)r * p->H_I * D, p->w + (int64_t)r * p->H_I, kI.data(),
                       p->qI_scale ? p->qI_scale + (int64_t)r * p->H_I * G : nullptr,
                       p->kI_scale ? ks.data() : nullptr, p->H_I, D, n, sc.data(), threads);
    if (scores) {
      float* srow = scores + (int64_t)i * ld;
      for (int64_t j = 0; j < ld; ++j) srow[j] = j < n ? sc[j] : std::nanf("");
    }
    int32_t* idx = indices + (int64_t)i * p->K;
    counts[i] = orc_topk(sc.data(), n, p->K, idx);
    // slots -> positions (candidate slots are in position order, so the
    // order and the tie rule carry over)
    for (int64_t j = 0; j < counts[i]; ++j) idx[j] = (int32_t)hist[idx[j]];
    // gather the selected KV rows and attend
    const int64_t m = counts[i];
    const uint16_t* qr = p->q + (int64_t)r * p->H_q * p->D_qk;
    double* o_r = out + (int64_t)i * p->H_q * p->D_v;
    double* lse_r = lse + (int64_t)i * p->H_q;
    if (p->k8) {  // FP8 cache: decode each gathered row, V = its first D_v values
      const int T = kv_tiles(p->D_qk);
      std::vector<double> kd((size_t)m * p->D_qk), vd((size_t)m * p->D_v);
      for (int64_t j = 0; j < m; ++j) {
        const int64_t row = (int64_t)bt[idx[j] / B] * B + idx[j] % B;
        orc_kv_fp8_decode(p->k8 + row * p->D_qk, p->k8_scale + row * T, 1, p->D_qk,
                          &kd[(size_t)j * p->D_qk]);
        for (int d = 0; d < p->D_v; ++d) vd[(size_t)j * p->D_v + d] = kd[(size_t)j * p->D_qk + d];
      }
      attention_values(qr, kd.data(), vd.data(), m, p->H_q, p->D_qk, p->D_v, p->scale, o_r, lse_r,
                       threads);
      continue;
    }
    std::vector<uint16_t> kr((size_t)m * p->D_qk), vr((size_t)m * p->D_v);
    for (int64_t j = 0; j < m; ++j) {
      const int64_t row = (int64_t)bt[idx[j] / B] * B + idx[j] % B;
      std::memcpy(&kr[(size_t)j * p->D_qk], p->k + row * p->D_qk, 2 * (size_t)p->D_qk);
      if (p->v)
        std::memcpy(&vr[(size_t)j * p->D_v], p->v + row * p->D_v, 2 * (size_t)p->D_v);
      else  // latent layout (reading): V is the first D_v elements of the K row
        std::memcpy(&vr[(size_t)j * p->D_v], p->k + row * p->D_qk, 2 * (size_t)p->D_v);
    }
    orc_attention(qr, kr.data(), vr.data(), m, p->H_q, p->D_qk, p->D_v, p->scale, o_r, lse_r,
                  threads);
  }
  return 0;
}

// Bit-level pieces of the prolog, for pins against other routines.
void orc_bf16_round(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_round_bits(v[i]);
}
void orc_e4m3_round(const double* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_round_code(v[i]);
}
// MXFP8 quantisation of rows of n values (n a multiple of 32).
void orc_mx_quantize(const double* v, int64_t rows, int n, uint8_t* codes, uint8_t* scales) {
  for (int64_t r = 0; r < rows; ++r)
    for (int g = 0; g < n / 32; ++g)
      mx_quantize_group(v + r * n + 32 * g, 32, codes + r * n + 32 * g, scales + r * (n / 32) + g);
}

// The indexer prolog for `rows` rows (Day0 article, section 4.3):
//   q = W_q x            x [rows][D_x] bf16, w_q [H_I * D_I][D_x] bf16
//   qI, qs = MXFP8(bf16(q)) per head and group of 32
//   g = W_g x            w_g [H_I][D_x] bf16; w = bf16(g) stored as binary32
//   y = gamma * k / sqrt(mean(k^2) + eps), k [rows][D_I] bf16, gamma [D_I]
//   kI, ks = MXFP8(bf16(y))
// Outputs: q binary64 [rows][H_I * D_I], q_bf16, qI [rows][H_I * D_I],
// qs [rows][H_I * D_I / 32], w [rows][H_I], k_bf16 [rows][D_I], kI
// [rows][D_I], ks [rows][D_I / 32].
void orc_prolog(const uint16_t* x, const uint16_t* w_q, const uint16_t* w_g, const uint16_t* k,
                const uint16_t* gamma, double eps, int rows, int D_x, int H_I, int D_I, double* q,
                uint16_t* q_bf16, uint8_t* qI, uint8_t* qs, float* w, uint16_t* k_bf16,
                uint8_t* kI, uint8_t* ks, int threads) {
  const int F = H_I * D_I;
  parallel_for(rows, threads, [&](int64_t r) {
    const uint16_t* xr = x + r * D_x;
    std::vector<double> qv(F);
    for (int f = 0; f < F; ++f) {
      q[r * F + f] = dot_bf16(w_q + (int64_t)f * D_x, xr, D_x);
      q_bf16[r * F + f] = bf16_round_bits(q[r * F + f]);
      qv[f] = bf16_value(q_bf16[r * F + f]);
    }
    for (int gi = 0; gi < F / 32; ++gi)
      mx_quantize_group(&qv[32 * gi], 32, qI + r * F + 32 * gi, qs + r * (F / 32) + gi);
    for (int h = 0; h < H_I; ++h)
      w[r * H_I + h] = (float)bf16_value(bf16_round_bits(dot_bf16(w_g + (int64_t)h * D_x, xr, D_x)));
    double ss = 0.0;
    for (int d = 0; d < D_I; ++d) {
      const double kd = bf16_value(k[r * D_I + d]);
      ss += kd * kd;
    }
    const double inv = 1.0 / std::sqrt(ss / D_I + eps);
    std::vector<double> yv(D_I);
    for (int d = 0; d < D_I; ++d) {
      k_bf16[r * D_I + d] = bf16_round_bits(bf16_value(gamma[d]) * bf16_value(k[r * D_I + d]) * inv);
      yv[d] = bf16_value(k_bf16[r * D_I + d]);
    }
    for (int gi = 0; gi < D_I / 32; ++gi)
      mx_quantize_group(&yv[32 * gi], 32, kI + r * D_I + 32 * gi, ks + r * (D_I / 32) + gi);
  });
}

}  // extern "C"
