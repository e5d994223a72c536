"""Pins of the CPU oracle against things other than itself.

The pages print no worked numeric example for any step of the path, so every
pin here is a closed form, a brute-force route that does not share the
oracle's code path, a library routine, or an invariant that a plausible slip
(a dropped term, a wrong sign or index, a transposed operand, a misplaced
gate, a wrong tie rule) breaks.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.formats import E4M3_TABLE
from tests.helpers import ORACLES, run_oracle
from workloads import make_batch, oracle_arrays, small_workload


@pytest.fixture(params=sorted(ORACLES))
def orc(request):
    """Each pin runs on both oracle routes: the numpy statement and the plain
    C++ one (written separately; neither calls the other)."""
    return ORACLES[request.param]


# ----------------------------------------------------------------- formats

def test_e4m3_closed_form_codes():
    # values worked out by hand from the E4M3 field layout (s eeee mmm, bias 7)
    cases = {
        0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x44: 3.0, 0x48: 4.0, 0x4A: 5.0,
        0x4C: 6.0, 0x4E: 7.0, 0x50: 8.0, 0x30: 0.5, 0x7E: 448.0, 0xFE: -448.0,
        0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0xB8: -1.0,
        0x3C: 1.5, 0x77: 240.0,
    }
    for code, val in cases.items():
        assert oracle.e4m3_to_f64([code])[0] == val, hex(code)
    neg_zero = oracle.e4m3_to_f64([0x80])[0]
    assert neg_zero == 0.0 and math.copysign(1.0, neg_zero) < 0
    assert np.isnan(E4M3_TABLE[0x7F]) and np.isnan(E4M3_TABLE[0xFF])
    assert np.isfinite(np.delete(E4M3_TABLE, [0x7F, 0xFF])).all()


def test_e4m3_matches_torch_decoder():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.e4m3_to_f64(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert (both_nan | (ref == mine)).all()
    assert (np.signbit(ref) == np.signbit(mine))[~both_nan].all()


def test_e4m3_ordering_and_integers():
    pos = E4M3_TABLE[0x00:0x7F]
    assert (np.diff(pos) > 0).all()                         # codes 0..0x7E strictly increasing
    assert (E4M3_TABLE[0x80:0xFF] == -pos).all()            # sign-magnitude mirror
    ints = torch.arange(-8, 9, dtype=torch.float32)
    codes = ints.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (oracle.e4m3_to_f64(codes) == ints.numpy()).all()


def test_bf16_decoder():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0000: 0.0, 0x7F80: np.inf,
             0x3E80: 0.25, 0x0001: 2.0 ** -133}
    for bits, val in cases.items():
        assert oracle.bf16_to_f64([bits])[0] == val, hex(bits)
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 50000).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]               # no inf/NaN
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert (oracle.bf16_to_f64(bits) == ref).all()


# ----------------------------------------------------------- index scores

def _e4m3(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_scores_one_hot_keys_closed_form(orc):
    # key s = c_s * e_{d_s}: the dot product collapses to c_s * q[h, d_s], so
    # I[s] = sum_h w_h * max(0, c_s * q[h, d_s]).  H_I != D_I so a transposed
    # operand cannot pass.
    rng = np.random.default_rng(1)
    H, D, L = 5, 16, 40
    q = rng.integers(-8, 9, (H, D))
    w = rng.integers(0, 4, H).astype(np.float32)
    d_s = rng.integers(0, D, L)
    c_s = rng.choice([-3, -1, 1, 2, 4], L)
    k = np.zeros((L, D))
    k[np.arange(L), d_s] = c_s
    got = orc.indexer_scores_row(_e4m3(q), w, _e4m3(k))
    for s in range(L):
        want = 0.0
        for h in range(H):
            want += float(w[h]) * max(0.0, float(c_s[s]) * float(q[h, d_s[s]]))
        assert got[s] == np.float32(want), s


def test_scores_gate_is_per_head(orc):
    # two heads of opposite sign on one key: a gate applied after the head sum
    # would give max(0, 3*4 - 2*4) = 4; the per-head gate gives 3*4 = 12.
    q = np.zeros((2, 4)); q[0, 0] = 4; q[1, 0] = -4
    k = np.zeros((1, 4)); k[0, 0] = 1
    w = np.array([3.0, 2.0], np.float32)
    assert orc.indexer_scores_row(_e4m3(q), w, _e4m3(k))[0] == 12.0
    # every head gated off, with a negative weight: the score is +0
    w2 = np.array([-1.0, -2.0], np.float32)
    z = orc.indexer_scores_row(_e4m3(-np.abs(q)), w2, _e4m3(k))[0]
    assert z == 0 and not np.signbit(z)


def test_scores_linear_identity(orc):
    # max(0, x) - max(0, -x) = x, so I(q) - I(-q) = sum_h w_h q_h . k_s
    # = k_s . (sum_h w_h q_h): weights folded into the query first, a
    # different association than the oracle's (per-head dots, then weights).
    rng = np.random.default_rng(2)
    H, D, L = 7, 64, 300
    q = rng.integers(-8, 9, (H, D)).astype(np.float64)
    k = rng.integers(-8, 9, (L, D)).astype(np.float64)
    w = rng.integers(0, 4, H).astype(np.float32)
    plus = orc.indexer_scores_row(_e4m3(q), w, _e4m3(k)).astype(np.float64)
    minus = orc.indexer_scores_row(_e4m3(-q), w, _e4m3(k)).astype(np.float64)
    folded = (w.astype(np.float64)[:, None] * q).sum(axis=0)      # [D]
    want = (k * folded[None, :]).sum(axis=1)
    assert (plus - minus == want).all()


def test_scores_integer_mode_exact_and_invariant(orc):
    rng = np.random.default_rng(3)
    H, D, L = 64, 128, 200
    q = rng.integers(-8, 9, (H, D))
    k = rng.integers(-8, 9, (L, D))
    w = rng.integers(0, 4, H).astype(np.float32)
    s = orc.indexer_scores_row(_e4m3(q), w, _e4m3(k))
    assert (s == np.round(s)).all()
    # exact integer arithmetic as an independent route
    dots = [[sum(int(a) * int(b) for a, b in zip(q[h], k[j])) for j in range(L)] for h in range(H)]
    want = [sum(int(w[h]) * max(0, dots[h][j]) for h in range(H)) for j in range(L)]
    assert (s.astype(np.int64) == np.array(want)).all()
    # doubling every weight doubles every score exactly
    assert (orc.indexer_scores_row(_e4m3(q), 2 * w, _e4m3(k)) == 2 * s).all()
    # permuting heads together with their weights changes nothing
    perm = rng.permutation(H)
    assert (orc.indexer_scores_row(_e4m3(q[perm]), w[perm], _e4m3(k)) == s).all()


def _f32_nearest(x):
    """float32 nearest to the rational x, ties to even (exact arithmetic)."""
    c = np.float32(float(x))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda f: (abs(Fraction(float(f)) - x),
                                     int(np.array(f, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_scores_gaussian_are_the_exact_value_rounded_once(orc):
    # Every E4M3 value is an integer multiple of 2**-9, so with integer codes
    # Q = 512 q and Kc = 512 k each head's dot product is (Q @ Kc^T) / 2**18
    # exactly, in int64.  The weighted head sum is then formed in exact
    # rational arithmetic and rounded to the nearest float32.  The oracle
    # rounds a binary64 sum once, so it must give the same float32 unless the
    # exact value sits within binary64 noise of a float32 rounding boundary.
    g = torch.Generator().manual_seed(4)
    qc = torch.randn(64, 128, generator=g).to(torch.float8_e4m3fn)
    kc = torch.randn(300, 128, generator=g).to(torch.float8_e4m3fn)
    w = (torch.rand(64, generator=g) * 3).numpy()
    qv = qc.view(torch.uint8).numpy()
    kv = kc.view(torch.uint8).numpy()
    Qi = (E4M3_TABLE[qv] * 512).astype(np.int64)
    Ki = (E4M3_TABLE[kv] * 512).astype(np.int64)
    assert (Qi == E4M3_TABLE[qv] * 512).all() and (Ki == E4M3_TABLE[kv] * 512).all()
    dots = Qi @ Ki.T                                        # [64, 300], units of 2**-18
    wf = [Fraction(float(x)) for x in w]
    got = orc.indexer_scores_row(qv, w, kv)
    near_boundary = 0
    for s in range(kv.shape[0]):
        exact = sum(wf[h] * int(dots[h, s]) for h in range(64) if dots[h, s] > 0) / 2 ** 18
        want = _f32_nearest(exact)
        if got[s] != want:
            # only allowed next to a rounding boundary, one ulp away
            lo, hi = sorted([float(got[s]), float(want)])
            mid = (Fraction(lo) + Fraction(hi)) / 2
            assert np.nextafter(np.float32(lo), np.float32(np.inf)) == np.float32(hi)
            assert abs(exact - mid) <= abs(exact) * Fraction(1, 2 ** 45), s
            near_boundary += 1
    assert near_boundary <= 1


# ----------------------------------------------------- MXFP8 index scores

def test_e8m0_closed_form_codes():
    # E8M0 scale byte e stands for 2**(e - 127) (OCP microscaling reading)
    cases = {0: 2.0 ** -127, 1: 2.0 ** -126, 126: 0.5, 127: 1.0, 128: 2.0, 130: 8.0,
             254: 2.0 ** 127}
    for code, val in cases.items():
        assert oracle.e8m0_to_f64([code])[0] == val, code
    assert np.isnan(oracle.e8m0_to_f64([255])[0])
    # doubling per code step, over the whole finite range
    v = oracle.e8m0_to_f64(np.arange(255, dtype=np.uint8))
    assert (v[1:] == 2 * v[:-1]).all()


def _mx_case(rng, H=6, D=128, L=50):
    q = rng.integers(-4, 5, (H, D))
    k = rng.integers(-4, 5, (L, D))
    sq = rng.integers(125, 130, (H, D // 32)).astype(np.uint8)
    sk = rng.integers(125, 130, (L, D // 32)).astype(np.uint8)
    w = rng.integers(0, 4, H).astype(np.float32)
    return q, k, sq, sk, w


def test_mx_scores_unit_scales_reduce_to_e4m3(orc):
    # every scale 127 (x1): the MXFP8 score is the pinned unscaled score
    rng = np.random.default_rng(11)
    q, k, _, _, w = _mx_case(rng)
    ones_q = np.full((q.shape[0], q.shape[1] // 32), 127, np.uint8)
    ones_k = np.full((k.shape[0], k.shape[1] // 32), 127, np.uint8)
    got = orc.indexer_scores_row(_e4m3(q), w, _e4m3(k), ones_q, ones_k)
    assert (got == orc.indexer_scores_row(_e4m3(q), w, _e4m3(k))).all()


def test_mx_scores_one_hot_keys_closed_form(orc):
    # key s = c_s * e_{d_s} with scale byte b on the group of d_s: the head's
    # dot product is c_s * q[h, d_s] * 2**(eq[h, d_s // 32] + b - 254)
    rng = np.random.default_rng(12)
    H, D, L = 5, 128, 40
    q = rng.integers(-4, 5, (H, D))
    sq = rng.integers(124, 131, (H, D // 32)).astype(np.uint8)
    w = rng.integers(0, 4, H).astype(np.float32)
    d_s = rng.integers(0, D, L)
    c_s = rng.choice([-3, -1, 1, 2, 4], L)
    k = np.zeros((L, D))
    k[np.arange(L), d_s] = c_s
    sk = rng.integers(124, 131, (L, D // 32)).astype(np.uint8)
    got = orc.indexer_scores_row(_e4m3(q), w, _e4m3(k), sq, sk)
    for s in range(L):
        g = d_s[s] // 32
        want = 0.0
        for h in range(H):
            scale = 2.0 ** (int(sq[h, g]) + int(sk[s, g]) - 254)
            want += float(w[h]) * max(0.0, float(c_s[s]) * float(q[h, d_s[s]]) * scale)
        assert got[s] == np.float32(want), s


def test_mx_scores_code_scale_trade_and_group_locality(orc):
    rng = np.random.default_rng(13)
    q, k, sq, sk, w = _mx_case(rng)
    base = orc.indexer_scores_row(_e4m3(q), w, _e4m3(k), sq, sk)
    # halving a group's codes (kept even so halves stay integers) while
    # raising that group's scale by one step leaves every score unchanged;
    # the trade only holds if the scale multiplies exactly its own 32 dims
    q2, sq2 = 2 * (q // 2), sq.copy()
    base2 = orc.indexer_scores_row(_e4m3(q2), w, _e4m3(k), sq2, sk)
    for g in range(q.shape[1] // 32):
        qh, sqh = q2.copy(), sq2.copy()
        qh[:, 32 * g:32 * (g + 1)] //= 2
        sqh[:, g] += 1
        assert (orc.indexer_scores_row(_e4m3(qh), w, _e4m3(k), sqh, sk) == base2).all(), g
    # a key group's scale one step up doubles exactly that group's share of
    # every head's dot product: check through the linear identity of the gate
    # (I(q) - I(-q) = sum_h w_h dot_h), group by group with integer arithmetic
    lin = lambda qq, sk_: (orc.indexer_scores_row(_e4m3(qq), w, _e4m3(k), sq, sk_).astype(np.float64)
                           - orc.indexer_scores_row(_e4m3(-qq), w, _e4m3(k), sq, sk_).astype(np.float64))
    d0 = lin(q, sk)
    for g in range(q.shape[1] // 32):
        sk_up = sk.copy()
        sk_up[:, g] += 1
        dims = slice(32 * g, 32 * (g + 1))
        share = sum(float(w[h]) * (q[h, dims] * k[:, dims]).sum(axis=1).astype(np.float64)
                    * 2.0 ** (sq[h, g].astype(np.int64) + sk[:, g].astype(np.int64) - 254)
                    for h in range(q.shape[0]))
        assert (lin(q, sk_up) - d0 == share).all(), g
    assert base.dtype == np.float32


def test_mx_scores_integer_mode_exact(orc):
    # integer codes in [-4, 4], scales 2**-2 .. 2**2: exact rational
    # arithmetic (Python ints over a common 2**-8 denominator) as the route
    rng = np.random.default_rng(14)
    q, k, sq, sk, w = _mx_case(rng, H=16, L=60)
    s = orc.indexer_scores_row(_e4m3(q), w, _e4m3(k), sq, sk)
    H, L = q.shape[0], k.shape[0]
    want = []
    for j in range(L):
        tot = 0
        for h in range(H):
            dot = 0  # in units of 2**-8
            for g in range(q.shape[1] // 32):
                part = int((q[h, 32 * g:32 * (g + 1)] * k[j, 32 * g:32 * (g + 1)]).sum())
                dot += part * 2 ** (int(sq[h, g]) + int(sk[j, g]) - 254 + 8)
            tot += int(w[h]) * max(0, dot)
        want.append(tot / 256.0)
    assert (s.astype(np.float64) == np.array(want)).all()


# ------------------------------------------------------------------ Top-K

def test_score_keys_order(orc):
    vals = np.array([-np.inf, -3.4e38, -1.0, -1e-40, -0.0, 0.0, 1e-45, 1e-40, 1.0, 2.0,
                     3.4e38, np.inf], dtype=np.float32)
    keys = orc.score_keys(vals).astype(np.int64)
    assert (np.diff(keys)[[0, 1, 2, 3]] > 0).all()
    assert keys[4] == keys[5]                                # -0 and +0 tie
    assert (np.diff(keys)[5:] > 0).all()
    assert orc.score_keys(np.array([np.nan], np.float32))[0] == 0
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    kx = orc.score_keys(x).astype(np.int64)
    i, j = rng.integers(0, len(x), (2, 20000))
    assert ((x[i] < x[j]) == (kx[i] < kx[j])).all()


def _topk_brute(values, K):
    # Python's own sort on the float values: largest first, ties to the lower index
    order = sorted(range(len(values)), key=lambda i: (-float(values[i]), i))
    chosen = sorted(order[:min(K, len(values))])
    return chosen + [-1] * (K - len(chosen))


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force(seed, orc):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 400))
    K = int(rng.integers(1, 80))
    if seed % 3 == 0:
        vals = rng.integers(-5, 6, L).astype(np.float32)            # heavy ties
    elif seed % 3 == 1:
        vals = rng.standard_normal(L).astype(np.float32)
    else:
        vals = rng.choice(np.array([-np.inf, -2.0, -0.0, 0.0, 1.0, 7.0, np.inf], np.float32), L)
    idx, n = orc.topk_row(vals, K)
    assert n == min(K, L)
    assert idx.tolist() == _topk_brute(vals, K)


def test_topk_closed_forms(orc):
    idx, n = orc.topk_row(np.full(100, 3.0, np.float32), 10)
    assert n == 10 and idx.tolist() == list(range(10))             # all equal: lowest positions
    idx, n = orc.topk_row(np.arange(5, dtype=np.float32), 8)
    assert n == 5 and idx.tolist() == [0, 1, 2, 3, 4, -1, -1, -1]  # K >= L: everything
    vals = np.zeros(1000, np.float32)
    planted = [3, 77, 500, 999]
    vals[planted] = [5, 9, 7, 6]
    idx, n = orc.topk_row(vals, 4)
    assert idx.tolist() == planted                                  # ascending positions
    vals[[10, 20]] = -0.0                                           # -0 ties +0: lower positions win
    idx, _ = orc.topk_row(vals, 6)
    assert idx.tolist() == [0, 1, 3, 77, 500, 999]


# -------------------------------------------------------------- attention

def _bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_attention_sparse_equals_masked_dense(orc):
    rng = np.random.default_rng(6)
    H, D, Dv, L = 8, 64, 48, 90
    q, k, v = _bf16(rng.standard_normal((H, D))), _bf16(rng.standard_normal((L, D))), \
        _bf16(rng.standard_normal((L, Dv)))
    sel = np.sort(rng.choice(L, 30, replace=False))
    o, lse = orc.sparse_attn_row(q, k[sel], v[sel], 0.125)
    mask = np.zeros(L, bool); mask[sel] = True
    o2, lse2 = orc.masked_dense_attn_row(q, k, v, mask, 0.125)
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-13) and np.allclose(lse, lse2, rtol=1e-13)
    logits = 0.125 * oracle.bf16_to_f64(q) @ oracle.bf16_to_f64(k[sel]).T
    assert np.allclose(lse, scipy.special.logsumexp(logits, axis=1), rtol=1e-13)


def test_attention_closed_forms(orc):
    rng = np.random.default_rng(7)
    H, D, Dv, n = 4, 32, 16, 12
    q, k, v = _bf16(rng.standard_normal((H, D))), _bf16(rng.standard_normal((n, D))), \
        _bf16(rng.standard_normal((n, Dv)))
    vf = oracle.bf16_to_f64(v)
    o, lse = orc.sparse_attn_row(q, k[5:6], v[5:6], 0.3)         # one row: o = v_s
    assert np.allclose(o, np.broadcast_to(vf[5], o.shape), rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.3 * oracle.bf16_to_f64(q) @ oracle.bf16_to_f64(k[5]), rtol=1e-14)
    const = _bf16(np.full((n, Dv), 1.5))
    o, _ = orc.sparse_attn_row(q, k, const, 0.3)                 # constant V
    assert np.allclose(o, 1.5, rtol=0, atol=1e-14)
    o, lse = orc.sparse_attn_row(_bf16(np.zeros((H, D))), k, v, 0.3)   # q = 0: mean of V
    assert np.allclose(o, np.broadcast_to(vf.mean(axis=0), o.shape), atol=1e-14)
    assert np.allclose(lse, math.log(n))
    o, lse = orc.sparse_attn_row(q, k[:0], v[:0], 0.3)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_dense_causal_matches_torch_sdpa():
    rng = np.random.default_rng(8)
    H, D, Dv, L = 6, 64, 32, 77
    q, k, v = _bf16(rng.standard_normal((H, D))), _bf16(rng.standard_normal((L, D))), \
        _bf16(rng.standard_normal((L, Dv)))
    scale = 1 / 8
    got = oracle.dense_causal_attn_row(q, k, v, scale)
    tq = torch.from_numpy(oracle.bf16_to_f64(q))[None, :, None, :]
    tk = torch.from_numpy(oracle.bf16_to_f64(k))[None, None].expand(1, H, L, D)
    tv = torch.from_numpy(oracle.bf16_to_f64(v))[None, None].expand(1, H, L, Dv)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0, :, 0].numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ FP8 KV cache
# Day0 article, section 5.2: FP8 KV rows quantised per token in tiles of 128
# elements, one scale per tile; 576 = 4 * 128 + 64 gives a shorter last tile.

_KV_TILES = [(0, 128), (128, 256), (256, 384), (384, 512), (512, 576)]


def test_kv_fp8_decode_closed_forms(orc):
    D = 576
    codes = np.zeros((2, D), np.uint8)
    codes[0, :] = 0x38                      # 1.0 everywhere
    codes[1, 0], codes[1, 127] = 0x7E, 0xB8    # 448, -1.0: first and last of tile 0
    codes[1, 128], codes[1, 511] = 0x40, 0x01  # 2.0 (tile 1), 2**-9 (last of tile 3)
    codes[1, 512], codes[1, 575] = 0x3C, 0xC0  # 1.5, -2.0: first and last of the 64-wide tile
    scales = np.array([[1, 2, 4, 8, 16], [0.5, 3.0, 0.25, 1024.0, 0.125]], np.float32)
    got = orc.kv_fp8_to_f64(codes, scales)
    row0 = np.concatenate([np.full(hi - lo, 2.0 ** t) for t, (lo, hi) in enumerate(_KV_TILES)])
    assert np.array_equal(got[0], row0)
    row1 = np.zeros(D)
    row1[0], row1[127], row1[128], row1[511] = 224.0, -0.5, 6.0, 2.0
    row1[512], row1[575] = 0.1875, -0.25
    assert np.array_equal(got[1], row1)


def test_kv_fp8_scale_of_one_tile_moves_only_its_elements(orc):
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 0x7E, size=(4, 576)).astype(np.uint8)   # finite codes
    codes[:, ::2] |= 0x80                                             # and negative ones
    sc = rng.uniform(0.5, 2.0, size=(4, 5)).astype(np.float32)
    base = orc.kv_fp8_to_f64(codes, sc)
    for t, (lo, hi) in enumerate(_KV_TILES):
        sc2 = sc.copy()
        sc2[:, t] *= 2
        got = orc.kv_fp8_to_f64(codes, sc2)
        assert np.array_equal(got[:, lo:hi], 2 * base[:, lo:hi])
        rest = np.ones(576, bool)
        rest[lo:hi] = False
        assert np.array_equal(got[:, rest], base[:, rest])


def test_kv_fp8_step_equals_the_bf16_step_on_the_same_values(orc):
    # power-of-two tile scales keep every decoded value exact in bfloat16:
    # the FP8 step must then match the already pinned bf16 step bit for bit
    wl = small_workload("f", lengths=[5, 300, 2100], mode="int", K=128, kv_fmt="fp8",
                        table="shuffled")
    arr = oracle_arrays(make_batch(wl, seed=11))
    rng = np.random.default_rng(12)
    sc = np.exp2(rng.integers(-8, 3, size=arr["k_scale_cache"].shape)).astype(np.float32)
    vals = orc.kv_fp8_to_f64(arr["k_cache"], sc)
    f32 = vals.astype(np.float32)
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f64(bits), vals)
    r8 = run_oracle(dict(arr, k_scale_cache=sc), impl=orc)
    r16 = run_oracle(dict(arr, k_cache=bits, k_scale_cache=None), impl=orc)
    assert np.array_equal(r8["indices"], r16["indices"])
    assert np.array_equal(r8["out"], r16["out"]) and np.array_equal(r8["lse"], r16["lse"])


# ------------------------------------------------------------- end to end

def _tiny(**kw):
    base = dict(H_I=4, D_I=64, H_q=8, D_qk=64, D_v=64, K=64, scale=0.125, mode="int")
    base.update(kw)
    return base


def test_decode_step_K_at_least_L_is_dense_causal(orc):
    # with K >= every history length the sparse step is dense causal attention
    wl = small_workload("t", lengths=[1, 37, 64, 65, 130], latent=True, **_tiny(K=256, D_qk=96))
    arr = oracle_arrays(make_batch(wl, seed=9))
    res = run_oracle(arr, impl=orc)
    for i in range(5):
        b, p = arr["row_seq"][i], arr["row_pos"][i]
        hist = np.arange(p + 1)
        assert res["counts"][i] == p + 1
        assert res["indices"][i][:p + 1].tolist() == hist.tolist()
        k_all = oracle.gather_positions(arr["k_cache"], arr["block_table"][b], hist)
        dense = oracle.dense_causal_attn_row(arr["q"][i], k_all, k_all[:, :64], wl.scale)
        assert np.allclose(res["out"][i], dense, rtol=1e-12, atol=1e-12)


def test_decode_step_block_table_shuffle_invariance(orc):
    wl = small_workload("t", lengths=[300, 129, 700], latent=False, **_tiny(K=40))
    a = oracle_arrays(make_batch(wl, seed=10, table="identity"))
    b = oracle_arrays(make_batch(wl, seed=10, table="shuffled"))
    # same values, different physical placement: re-place b's blocks where a has them
    assert not (a["block_table"] == b["block_table"]).all()
    for key in ("kI_cache", "k_cache", "v_cache"):
        moved = np.empty_like(b[key])
        for s in range(3):
            nb = (a["seq_lens"][s] + 63) // 64
            moved[b["block_table"][s, :nb]] = a[key][a["block_table"][s, :nb]]
        b[key] = moved
    ra, rb = run_oracle(a, impl=orc), run_oracle(b, impl=orc)
    assert (ra["indices"] == rb["indices"]).all()
    assert all((x == y).all() for x, y in zip(ra["scores"], rb["scores"]))
    assert (ra["out"] == rb["out"]).all()


def test_decode_step_row_alone_equals_row_in_batch_and_prefill_rows(orc):
    wl = small_workload("t", lengths=[500, 260, 900], **_tiny(K=32, D_qk=96, latent=True))
    batch = make_batch(wl, seed=11)
    full = run_oracle(oracle_arrays(batch), impl=orc)
    one = run_oracle(oracle_arrays(batch, rows=[2]), impl=orc)
    assert (one["indices"][0] == full["indices"][2]).all()
    assert (one["out"][0] == full["out"][2]).all()
    # a chunked-prefill row at position p sees exactly positions 0..p
    pre = small_workload("p", lengths=[400], prefill_rows=16, **_tiny(K=32))
    arr = oracle_arrays(make_batch(pre, seed=12))
    res = run_oracle(arr, impl=orc)
    assert arr["row_pos"].tolist() == list(range(384, 400))
    for i in range(16):
        assert len(res["scores"][i]) == arr["row_pos"][i] + 1
        assert res["indices"][i].max() <= arr["row_pos"][i]


# ----------------------------------------------------- candidate-restricted
def _with_cand(arr, cand_rows):
    """arr with explicit candidate lists (ascending, -1 padded)."""
    n = max(1, max(len(c) for c in cand_rows))
    cand = np.full((len(cand_rows), n), -1, dtype=np.int32)
    for i, c in enumerate(cand_rows):
        cand[i, :len(c)] = c
    out = dict(arr)
    out["cand"] = cand
    out["cand_len"] = np.array([len(c) for c in cand_rows], dtype=np.int32)
    return out


def test_candidates_covering_the_history_reduce_to_the_full_step(orc):
    wl = small_workload("t", lengths=[37, 200, 700], **_tiny(K=50))
    arr = oracle_arrays(make_batch(wl, seed=21))
    full = run_oracle(arr, impl=orc)
    cand = run_oracle(_with_cand(arr, [np.arange(L) for L in (37, 200, 700)]), impl=orc)
    assert (full["indices"] == cand["indices"]).all()
    assert (full["counts"] == cand["counts"]).all()
    assert np.array_equal(full["out"], cand["out"]) and np.array_equal(full["lse"], cand["lse"])
    for a, b in zip(full["scores"], cand["scores"]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_candidate_scores_and_top_k_by_brute_force(seed, orc):
    # scores at the candidates are the full scores at those positions; the
    # kept set is the K best candidates (score, then lower position), written
    # ascending, by a plain sort over the candidate list
    wl = small_workload("t", lengths=[900, 333], **_tiny(K=40, mode="gauss"))
    arr = oracle_arrays(make_batch(wl, seed=seed))
    rng = np.random.default_rng(seed)
    rows = [np.sort(rng.choice(900, 150, replace=False)), np.sort(rng.choice(333, 30, replace=False))]
    full = run_oracle(arr, impl=orc)
    got = run_oracle(_with_cand(arr, rows), impl=orc)
    for i, c in enumerate(rows):
        sc = np.asarray(full["scores"][i])[c]
        assert np.array_equal(np.asarray(got["scores"][i]), sc)
        best = sorted(range(len(c)), key=lambda j: (-float(sc[j]), int(c[j])))[:40]
        want = np.sort(c[best])
        n = min(40, len(c))
        assert got["counts"][i] == n
        assert (got["indices"][i][:n] == want).all() and (got["indices"][i][n:] == -1).all()


def test_candidates_outside_the_kept_set_do_not_matter(orc):
    # dropping candidates that are not kept leaves the selection and the
    # attention unchanged; an empty list keeps nothing
    wl = small_workload("t", lengths=[500], **_tiny(K=20, mode="gauss"))
    arr = oracle_arrays(make_batch(wl, seed=8))
    c = np.arange(0, 500, 3)
    a = run_oracle(_with_cand(arr, [c]), impl=orc)
    kept = a["indices"][0][:20]
    b = run_oracle(_with_cand(arr, [np.union1d(kept, c[::5])]), impl=orc)
    assert (a["indices"] == b["indices"]).all()
    assert np.allclose(a["out"], b["out"], rtol=0, atol=1e-12)
    e = run_oracle(_with_cand(arr, [np.array([], dtype=np.int64)]), impl=orc)
    assert e["counts"][0] == 0 and (e["indices"][0] == -1).all() and (e["out"][0] == 0).all()


def test_candidates_must_be_ascending_positions_of_the_history():
    with pytest.raises(ValueError):
        oracle.row_history(10, np.array([3, 2]), 2)
    with pytest.raises(ValueError):
        oracle.row_history(10, np.array([3, 11]), 2)
    assert (oracle.row_history(10, np.array([3, 7, -1]), 2) == [3, 7]).all()
