"""Storage formats of the hot path's inputs, decoded from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* FP8 E4M3, OCP "FN" flavour -- the FP8 the indexer and KV cache are stored in
  (Baidu Day0 article, sections 5.1-5.2; "FP8 E4M3" KV in the SPLASH summary,
  section 5): 1 sign bit, a 4-bit exponent with bias 7 and a 3-bit mantissa.
  Exponent field 0 holds subnormals m * 2**-9.  The two codes whose exponent
  and mantissa bits are all ones (0x7F and 0xFF) are NaN; there is no
  infinity, so the largest finite magnitude is 1.75 * 2**8 = 448.
* bfloat16: the upper 16 bits of an IEEE-754 binary32 value.
* E8M0 scale bytes of the MXFP8 indexer format (Day0 article, section 5.1:
  one shared scale per group of 32 values).  The page does not state the
  encoding; the reading taken is the OCP microscaling one: byte e stands for
  2**(e - 127), and e = 255 is NaN.
* The FP8 KV cache (Day0 article, section 5.2: FP8 storage quantised per
  token, per head, in tiles of 128 elements).  Readings: the codes are E4M3;
  each tile carries one binary32 scale and an element's value is its code's
  value times its tile's scale; a row of D elements has ceil(D / 128) tiles,
  the last one shorter when 128 does not divide D (576 = 4 * 128 + 64).
"""

import numpy as np


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return float("nan")
    if exponent == 0:
        return sign * mantissa * 2.0 ** -9
    return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)


#: value of every one of the 256 E4M3 codes, as binary64
E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode an array of E4M3 byte codes to binary64 (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_to_f64(codes) -> np.ndarray:
    """Decode an array of E8M0 scale bytes to binary64 (exact): 2**(e - 127),
    NaN for 255."""
    e = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    out = np.exp2(e - 127.0)
    out[np.asarray(codes) == 255] = np.nan
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """Decode an array of bfloat16 bit patterns (uint16) to binary64 (exact)."""
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


#: elements per scale tile of the FP8 KV cache (Day0 article, section 5.2)
KV_TILE = 128


def kv_tiles(dim: int) -> int:
    """Scale tiles of an FP8 KV row of ``dim`` elements."""
    return (int(dim) + KV_TILE - 1) // KV_TILE


def kv_fp8_to_f64(codes, scales) -> np.ndarray:
    """Decode FP8 KV rows to binary64 (exact): codes uint8 [..., D] (E4M3),
    scales float32 [..., kv_tiles(D)]; element d is e4m3(code[d]) times the
    scale of tile d // 128."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32).astype(np.float64)
    d = codes.shape[-1]
    if scales.shape[-1] != kv_tiles(d):
        raise ValueError("one scale per tile of 128 elements")
    per_elem = np.repeat(scales, KV_TILE, axis=-1)[..., :d]
    return e4m3_to_f64(codes) * per_elem
