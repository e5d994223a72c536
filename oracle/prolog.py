"""The indexer prolog, written out in binary64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Baidu AI Cloud's "Day0 Inference Support and Performance Optimization for New
Architecture LLMs", section 4.3, lists the indexer's input preparation: a Q
projection ``q = W_q x``, a K normalisation of the new key, a per-group
quantisation of q, and a head-weight projection ``g = W_g x``; the fused
scoring / Top-K call then takes the quantised q, the keys and g.  Section 5.1
fixes the indexer's format (MXFP8: every 32 values share one scale, Q and K
alike) and section 5.3 keeps the projections in bf16.

Readings of what the page leaves open (each stated where it is used):

* x, W_q, W_g and the new key are bf16; products are exact and are summed in
  binary64 (exact for integer inputs), and every prolog output that the page
  calls a tensor (q,
  the normalised key, g) is a bf16 activation: the exact value rounded once,
  to nearest even, to bf16.  The quantiser then works on those bf16 values.
* "K normalisation" is RMS normalisation with a learned bf16 weight gamma:
  ``y_d = gamma_d * k_d / sqrt(mean_d(k_d^2) + eps)``.
* ``quant_per_group`` is the OCP microscaling conversion: for each group of
  32, the shared scale is ``2**(floor(log2(max|v|)) - 8)`` (8 is the largest
  exponent of an E4M3 value), clamped to the E8M0 range ``2**-127 ..
  2**127``, ``2**-127`` for an all-zero group; each element's code is its
  value over the scale rounded to nearest even in E4M3, saturated at +-448,
  keeping the sign of a value that rounds to zero.
* The head weights g are stored as float32 (the fused call's ``w``), holding
  their bf16 values exactly.
"""

import numpy as np

from .formats import E4M3_TABLE

#: values per shared scale (Day0 article, section 5.1)
MX_GROUP = 32

#: E4M3's largest exponent (448 = 1.75 * 2**8) and largest finite value
_E4M3_EMAX = 8
_E4M3_MAX = 448.0


def bf16_round(values) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of binary64 values, rounded to nearest
    even (8 significant bits; subnormals below 2**-126 on a fixed 2**-133
    grid).  Values beyond the bf16 range are not expected here and raise."""
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("finite values only")
    m, e = np.frexp(v)                       # v = m * 2**e, 0.5 <= |m| < 1
    quantum_exp = np.maximum(e, -125) - 8    # spacing of bf16 values near v
    r = np.rint(np.ldexp(v, -quantum_exp))   # rint: ties to even
    out = np.ldexp(r, quantum_exp)
    if np.any(np.abs(out) >= 2.0 ** 128):
        raise ValueError("outside the bf16 range")
    bits = out.astype(np.float32).view(np.uint32) >> np.uint32(16)
    return bits.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


# positive finite E4M3 codes 0x00 .. 0x7E, in increasing value order
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3_TABLE[:0x7F]


def e4m3_round(values) -> np.ndarray:
    """E4M3 (OCP FN) codes of binary64 values: nearest value, ties to the even
    code (the code's last bit is the mantissa's), magnitudes from 448 up
    saturate to 448, and the sign bit is the value's own (so a negative value
    that rounds to zero gives 0x80)."""
    v = np.asarray(values, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("NaN has no code here")
    a = np.minimum(np.abs(v), _E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")       # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    neg = np.signbit(v)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def mx_quantize(values, group=MX_GROUP):
    """Per-group MXFP8 quantisation along the last axis (its length a multiple
    of ``group``): (codes uint8 [..., n], scales uint8 E8M0 [..., n / group])
    with code value * 2**(scale - 127) approximating each value."""
    v = np.asarray(values, dtype=np.float64)
    n = v.shape[-1]
    if n % group:
        raise ValueError("length must be a multiple of the group")
    g = v.reshape(*v.shape[:-1], n // group, group)
    amax = np.abs(g).max(axis=-1)
    _, e = np.frexp(amax)                     # amax = m * 2**e, floor(log2 amax) = e - 1
    shared = np.where(amax > 0, e - 1 - _E4M3_EMAX, -127)
    shared = np.clip(shared, -127, 127)
    codes = e4m3_round(np.ldexp(g, -shared[..., None]))
    return codes.reshape(v.shape), (shared + 127).astype(np.uint8)


def mx_dequantize(codes, scales, group=MX_GROUP) -> np.ndarray:
    """Values of MXFP8 groups (exact): code value times 2**(scale - 127)."""
    c = E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
    s = np.asarray(scales, dtype=np.int64) - 127
    return np.ldexp(c, np.repeat(s, group, axis=-1))


def rms_norm(k, gamma, eps) -> np.ndarray:
    """RMS normalisation along the last axis with weight gamma (binary64)."""
    k = np.asarray(k, dtype=np.float64)
    ms = np.mean(k * k, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * k / np.sqrt(ms + float(eps))


def indexer_prolog(*, x, w_q, w_g, k_new, k_gamma, eps, H_I, D_I):
    """The prolog for a batch of rows (Day0 article, section 4.3).

    x uint16 bf16 [rows, D_x]; w_q bf16 [H_I * D_I, D_x]; w_g bf16 [H_I, D_x];
    k_new bf16 [rows, D_I] (each row's own index key, before normalisation);
    k_gamma bf16 [D_I].  Returns q (binary64) and q_bf16, qI E4M3
    [rows, H_I, D_I], qI_scale E8M0 [rows, H_I, D_I / 32], w float32
    [rows, H_I], the normalised key k_bf16 [rows, D_I] and its MXFP8 codes
    kI [rows, D_I] and scales kI_scale [rows, D_I / 32]."""
    if D_I % MX_GROUP:
        raise ValueError("D_I must be a multiple of the group")
    xf = bf16_bits_to_f64(x)
    rows = xf.shape[0]
    q = xf @ bf16_bits_to_f64(w_q).T                 # Q projection, summed in binary64
    q_bf16 = bf16_round(q)
    qI, qs = mx_quantize(bf16_bits_to_f64(q_bf16).reshape(rows, H_I, D_I))
    g = xf @ bf16_bits_to_f64(w_g).T                 # head-weight projection
    g_bf16 = bf16_round(g)
    y = rms_norm(bf16_bits_to_f64(k_new), bf16_bits_to_f64(k_gamma), eps)
    k_bf16 = bf16_round(y)
    kI, ks = mx_quantize(bf16_bits_to_f64(k_bf16))
    return {"q": q, "q_bf16": q_bf16, "qI": qI, "qI_scale": qs,
            "w": bf16_bits_to_f64(g_bf16).astype(np.float32),
            "k_y": y, "k_bf16": k_bf16, "kI": kI, "kI_scale": ks}
