"""Pins of the oracle's indexer prolog (q and head-weight projections, RMS
normalisation of the new key, MXFP8 quantisation per group of 32) against
things other than itself: library conversions (torch's bf16 and float8 RNE
casts, torch's rms_norm), exact rational brute force, closed forms from the
format definitions, and invariants.  Every pin runs on both oracle routes.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import E4M3_TABLE
from tests.helpers import ORACLES
from workloads import make_prolog_inputs, prolog_arrays


@pytest.fixture(params=sorted(ORACLES))
def orc(request):
    return ORACLES[request.param]


def _bits_of(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16(values):
    """bf16 bits of values that bf16 holds exactly."""
    return _bits_of(torch.tensor(np.asarray(values, np.float32)).to(torch.bfloat16))


# ------------------------------------------------------------ bf16 rounding

def test_bf16_round_matches_torch_on_float32_values(orc):
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
                        rng.standard_normal(1000)]).astype(np.float32)
    want = _bits_of(torch.from_numpy(v).to(torch.bfloat16))
    assert np.array_equal(orc.bf16_round(v.astype(np.float64)), want)


def test_bf16_round_closed_forms(orc):
    # 8 significant bits: spacing 2**-7 just above 1
    cases = [(1.0, 0x3F80), (1.0 + 2.0 ** -8, 0x3F80),               # tie -> even
             (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),                 # just past the tie
             (1.0 + 3 * 2.0 ** -8, 0x3F82),                          # tie -> even (up)
             (-(1.0 + 2.0 ** -8), 0xBF80), (0.0, 0x0000), (-0.0, 0x8000),
             (256.0 + 1.0, 0x4380), (256.0 + 3.0, 0x4382)]           # integers past 256
    got = orc.bf16_round(np.array([v for v, _ in cases]))
    assert [int(x) for x in got] == [b for _, b in cases]


# ------------------------------------------------------------ E4M3 rounding

def test_e4m3_round_matches_torch_in_range(orc):
    rng = np.random.default_rng(4)
    finite = E4M3_TABLE[:0x7F]
    mids = (finite[:-1] + finite[1:]) / 2                 # exact midpoints: ties
    v = np.concatenate([rng.uniform(-448, 448, 3000), rng.standard_normal(3000) * 2.0 ** -7,
                        mids, -mids, finite, -finite]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_round(v.astype(np.float64)), want)


def test_e4m3_round_saturates_and_keeps_sign(orc):
    v = np.array([448.0, 449.0, 464.0, 480.0, 1e9, -500.0, -2.0 ** -12, 2.0 ** -12, -0.0])
    got = [int(c) for c in orc.e4m3_round(v)]
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80]


def test_e4m3_round_is_the_nearest_code_by_exact_arithmetic(orc):
    # brute force over every finite code with exact rationals
    rng = np.random.default_rng(5)
    vals = np.concatenate([rng.uniform(-20, 20, 60), rng.uniform(-0.02, 0.02, 40)])
    got = orc.e4m3_round(vals)
    for x, c in zip(vals, got):
        fx = Fraction(float(x))
        best = None
        for code in range(0x7F):
            mag = Fraction(float(E4M3_TABLE[code]))
            d = abs(abs(fx) - mag)
            key = (d, code % 2)          # nearest, then the even code
            if best is None or key < best[0]:
                best = (key, code)
        want = best[1] | (0x80 if x < 0 else 0)
        assert int(c) == want, (x, hex(int(c)), hex(want))


# -------------------------------------------------------- MXFP8 quantisation

def test_mx_quantize_closed_forms(orc):
    g = np.zeros((5, 32))
    g[0, :] = 1.0                         # amax 1 = 2**0: scale 2**-8, code of 256
    g[1, 0], g[1, 1] = 1.75, -0.5         # amax 1.75: 448 and -128 (2**7: 0x70, signed 0xF0)
    g[2, 0] = 1.99                        # 509.44 saturates at 448
    g[3, 5] = -3.0                        # amax 3: scale 2**-7, -384 (code 0xFC)
    codes, scales = orc.mx_quantize(g)    # row 4 all zero
    assert [int(s) for s in scales[:, 0]] == [119, 119, 119, 120, 0]
    assert np.all(codes[0] == 0x78)                                    # 256 = 2**8
    assert codes[1, 0] == 0x7E and codes[1, 1] == 0xF0 and np.all(codes[1, 2:] == 0)
    assert codes[2, 0] == 0x7E
    assert codes[3, 5] == 0xFC and np.all(np.delete(codes[3], 5) == 0)
    assert np.all(codes[4] == 0)


def test_mx_quantize_error_bound_and_power_of_two_invariance(orc):
    rng = np.random.default_rng(6)
    v = rng.standard_normal((40, 128)) * 10.0 ** rng.integers(-6, 6, (40, 1))
    codes, scales = orc.mx_quantize(v)
    deq = oracle.mx_dequantize(codes, scales)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=-1)
    r = np.abs(v) / X                     # magnitude in units of the scale, < 512
    assert np.all(r < 512)
    half_ulp = np.where(r < 2.0 ** -6, 2.0 ** -10, np.exp2(np.floor(np.log2(np.maximum(r, 2.0 ** -6))) - 4))
    err = np.abs(deq - v) / X
    assert np.all((err <= half_ulp) | (r >= 448))
    # the group's largest magnitude lands in [256, 448]
    amax_code = np.abs(E4M3_TABLE[codes]).reshape(40, 4, 32).max(axis=-1)
    assert np.all((amax_code >= 256) & (amax_code <= 448))
    # scaling one group by 2**j moves its scale by j and keeps every code
    v2 = v.copy()
    v2[:, 32:64] *= 2.0 ** 5
    c2, s2 = orc.mx_quantize(v2)
    assert np.array_equal(c2, codes)
    assert np.array_equal(s2[:, 1].astype(int), scales[:, 1].astype(int) + 5)
    assert np.array_equal(np.delete(s2, 1, axis=1), np.delete(scales, 1, axis=1))


# ----------------------------------------------------------- RMS norm

def test_rms_norm_matches_torch(orc):
    rng = np.random.default_rng(7)
    k = rng.standard_normal((6, 128))
    gamma = 1.0 + 0.1 * rng.standard_normal(128)
    want = torch.nn.functional.rms_norm(torch.from_numpy(k), (128,), torch.from_numpy(gamma),
                                        eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(k, gamma, 1e-6), want, rtol=1e-14, atol=0)


def test_prolog_key_norm_closed_form(orc):
    # a key of equal magnitudes c: y = gamma * sign(k) / sqrt(1 + eps / c**2);
    # with eps = 0 and gamma a power of two the bf16 result is exact
    D = 64
    k = np.where(np.arange(D) % 3 == 0, -4.0, 4.0)
    gamma = np.where(np.arange(D) % 2 == 0, 2.0, 0.5)
    arr = _tiny_inputs(rows=1, D_x=32, H_I=1, D_I=D)
    arr["k_new"] = _bf16(k)[None, :]
    arr["k_gamma"] = _bf16(gamma)
    res = orc.indexer_prolog(**arr, eps=0.0, H_I=1, D_I=D)
    want = gamma * np.sign(k)
    assert np.array_equal(oracle.formats.bf16_to_f64(res["k_bf16"][0]), want)
    # group amax 2 = 2**1: scale 2**-7, codes 256 (2**8: 0x78) and 64 (2**6: 0x68) with signs
    assert [int(s) for s in res["kI_scale"][0]] == [120, 120]
    c = np.where(gamma == 2.0, 0x78, 0x68) | np.where(k < 0, 0x80, 0)
    assert np.array_equal(res["kI"][0], c.astype(np.uint8))


# ---------------------------------------------------------- projections

def _tiny_inputs(rows, D_x, H_I, D_I, mode="int", seed=1):
    return prolog_arrays(make_prolog_inputs(rows, H_I, D_I, D_x=D_x, mode=mode, seed=seed))


def test_prolog_one_hot_x_selects_weight_columns(orc):
    H_I, D_I, D_x = 2, 64, 96
    arr = _tiny_inputs(rows=3, D_x=D_x, H_I=H_I, D_I=D_I, mode="gauss")
    x = np.zeros((3, D_x))
    cols = [0, 17, 95]
    for r, j in enumerate(cols):
        x[r, j] = 1.0
    arr["x"] = _bf16(x)
    res = orc.indexer_prolog(**arr, eps=1e-6, H_I=H_I, D_I=D_I)
    for r, j in enumerate(cols):
        assert np.array_equal(res["q_bf16"][r].reshape(-1), arr["w_q"][:, j])
        assert np.array_equal(res["w"][r], oracle.formats.bf16_to_f64(arr["w_g"][:, j]).astype(np.float32))


def test_prolog_integer_mode_by_exact_integer_arithmetic(orc):
    H_I, D_I, D_x, rows = 2, 64, 160, 3
    arr = _tiny_inputs(rows=rows, D_x=D_x, H_I=H_I, D_I=D_I, mode="int", seed=2)
    res = orc.indexer_prolog(**arr, eps=1e-6, H_I=H_I, D_I=D_I)
    xi = oracle.formats.bf16_to_f64(arr["x"]).astype(int).tolist()
    wq = oracle.formats.bf16_to_f64(arr["w_q"]).astype(int).tolist()
    wg = oracle.formats.bf16_to_f64(arr["w_g"]).astype(int).tolist()
    for r in range(rows):
        q = [sum(a * b for a, b in zip(wq[f], xi[r])) for f in range(H_I * D_I)]
        g = [sum(a * b for a, b in zip(wg[h], xi[r])) for h in range(H_I)]
        # integers of magnitude < 256 are exact in bf16 here
        assert max(abs(v) for v in q + g) < 256
        assert np.array_equal(oracle.formats.bf16_to_f64(res["q_bf16"][r].reshape(-1)), q)
        assert np.array_equal(res["w"][r].astype(np.float64), g)
        # their MXFP8 form is within half an E4M3 step of each integer, or
        # saturated at 448 scale units (group maxima land in [256, 512))
        deq = oracle.mx_dequantize(res["qI"][r].reshape(-1), res["qI_scale"][r].reshape(-1))
        X = np.repeat(np.exp2(res["qI_scale"][r].reshape(-1).astype(float) - 127), 32)
        qa = np.array(q, float)
        units = np.abs(qa) / X
        assert np.all(units < 512)
        sat = units >= 448
        assert np.array_equal(deq[sat], np.sign(qa[sat]) * 448 * X[sat])
        half = np.exp2(np.floor(np.log2(np.maximum(units, 2.0 ** -6))) - 4) * X
        assert np.all(np.abs(deq - qa)[~sat] <= half[~sat])


def test_prolog_heads_and_groups_are_independent(orc):
    # permuting the heads of W_q permutes the heads of qI and qI_scale
    H_I, D_I, D_x = 4, 64, 64
    arr = _tiny_inputs(rows=2, D_x=D_x, H_I=H_I, D_I=D_I, mode="gauss", seed=3)
    base = orc.indexer_prolog(**arr, eps=1e-6, H_I=H_I, D_I=D_I)
    perm = [2, 0, 3, 1]
    wq = arr["w_q"].reshape(H_I, D_I, D_x)[perm].reshape(H_I * D_I, D_x)
    res = orc.indexer_prolog(**dict(arr, w_q=wq), eps=1e-6, H_I=H_I, D_I=D_I)
    assert np.array_equal(res["qI"], base["qI"][:, perm])
    assert np.array_equal(res["qI_scale"], base["qI_scale"][:, perm])
    # doubling x doubles q and g exactly: codes unchanged, scales + 1
    x2 = _bits_of(torch.from_numpy(arr["x"].view(np.int16)).view(torch.bfloat16).float()
                  .mul(2).to(torch.bfloat16))
    res2 = orc.indexer_prolog(**dict(arr, x=x2), eps=1e-6, H_I=H_I, D_I=D_I)
    assert np.array_equal(res2["qI"], base["qI"])
    assert np.array_equal(res2["qI_scale"].astype(int), base["qI_scale"].astype(int) + 1)
    assert np.array_equal(res2["w"], 2 * base["w"])
    assert np.array_equal(res2["kI"], base["kI"])   # the key does not see x


def test_prolog_routes_agree():
    arr = _tiny_inputs(rows=5, D_x=256, H_I=8, D_I=128, mode="gauss", seed=4)
    a = oracle.indexer_prolog(**arr, eps=1e-6, H_I=8, D_I=128)
    b = oracle.cpp.indexer_prolog(**arr, eps=1e-6, H_I=8, D_I=128, threads=3)
    for key in ("q_bf16", "qI", "qI_scale", "w", "k_bf16", "kI", "kI_scale"):
        assert np.array_equal(np.asarray(a[key]).reshape(-1), np.asarray(b[key]).reshape(-1)), key
