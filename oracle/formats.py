"""Storage formats, written out from their definitions (oracle side).

TEST INFRASTRUCTURE ONLY.  See ``oracle/__init__.py``.

Formats (the element and scale types the pages' support tables name:
"Grouped GEMM + Quant (SM100)", §Data Types, tables of ab_dtype / sf_dtype):

* E4M3 ("float8_e4m3fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits.
  Exponent field 0 holds subnormals m/8 * 2^-6; S.1111.111 is NaN; there is
  no infinity; the largest finite magnitude is 448 (the q_max the
  quantisation step of the same page names for E4M3).
* E5M2 ("float8_e5m2"): sign, 5 exponent bits (bias 15), 2 mantissa bits,
  the upper byte of an IEEE binary16: exponent field 0 holds subnormals
  m/4 * 2^-14, field 31 is infinity (m = 0) or NaN; largest finite 57344.
* E2M1 ("float4_e2m1fn_x2", two per byte): sign, 2 exponent bits (bias 1),
  1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E8M0 ("float8_e8m0fnu"): a bare biased exponent, value 2^(x-127); 0xFF is NaN.
* BF16: the upper 16 bits of an IEEE binary32.

Decoders return float64.  Encoders take a real value and return the code of
the nearest representable value, ties to the code with an even mantissa
(round-half-even), saturating to the largest finite magnitude ("satfinite").
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_e4m3(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def decode_e5m2(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = (c & 0x3).astype(np.float64)
    val = np.where(e == 0, (m / 4.0) * 2.0 ** -14, (1.0 + m / 4.0) * np.exp2(e.astype(np.float64) - 15.0))
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


def decode_e2m1(nibbles) -> np.ndarray:
    c = np.asarray(nibbles).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    val = np.where(e == 0, m / 2.0, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return sign * val


def unpack_e2m1x2(packed) -> np.ndarray:
    """(..., K/2) bytes -> (..., K) nibbles; the even K element is the low nibble."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def decode_e8m0(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64) & 0xFF
    return np.where(c == 0xFF, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def decode_bf16(bits) -> np.ndarray:
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):       # NaN payloads convert as NaN
        return b.view(np.float32).astype(np.float64)


# non-negative finite E4M3 values in code order 0x00..0x7E (strictly increasing)
_E4M3_POS = decode_e4m3(np.arange(0x7F))


def encode_e4m3(values) -> np.ndarray:
    """Nearest E4M3 code, ties to even mantissa, |v| > 448 saturates to 448."""
    v = np.asarray(values, dtype=np.float64)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")      # first value >= mag
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag == 0, 0, code)
    code = code | np.where((v < 0) & (code != 0), 0x80, 0)
    return code.astype(np.uint8)


def encode_bf16(values) -> np.ndarray:
    """Nearest BF16 (8 significant bits), ties to even, from a float64 value."""
    v = np.asarray(values, dtype=np.float64)
    mant, ex = np.frexp(v)                  # v = mant * 2^ex, |mant| in [0.5, 1)
    quantum_exp = np.maximum(ex - 8, -133)  # 8 significant bits; BF16 subnormal step 2^-133
    r = np.ldexp(np.rint(np.ldexp(v, -quantum_exp)), quantum_exp)   # rint: half to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
