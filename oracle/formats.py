"""Number formats used by the caches: OCP fp8 e4m3fn and bfloat16.

Oracle (test infrastructure). Written from the format definitions, not from
any library's conversion code:

* OCP 8-bit floating point, E4M3 ("fn" variant: no infinities, one NaN
  pattern per sign, S.1111.111; largest finite 448; exponent bias 7;
  subnormals when the exponent field is zero). This is the fp8 type the
  latent-KV cache uses when it is stored in fp8 ("dsa_backend.py (sglang
  main)", ``_forward_flashmla_kv``: the cache is fp8 with page size 64 and
  is produced by ``quantize_k_cache``).
* bfloat16: the upper 16 bits of an IEEE binary32.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Decode e4m3fn byte codes (uint8 array) to float64, exactly.

    value = (-1)^s * 2^(e-7) * (1 + m/8)   for e in 1..15 (except the NaN code)
    value = (-1)^s * 2^(-6)  * (m/8)       for e == 0 (subnormal or zero)
    code 0x7F / 0xFF = NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    nan = (c & 0x7F) == 0x7F
    return np.where(nan, np.nan, val)


def _positive_table():
    """All non-negative finite e4m3fn values, indexed by code 0x00..0x7E."""
    return e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode_rne_sat(x):
    """Encode float values to e4m3fn codes: round to nearest, ties to even,
    saturating to +-448 (no NaN is ever produced for finite input).

    Plain definition: for |x| pick the representable non-negative value
    nearest to |x|; at an exact midpoint pick the one whose code is even (the
    code's low bit is the mantissa's low bit); magnitudes at or above 448 give
    448. The sign bit is copied (so -0.0 encodes as 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("e4m3 encoder: NaN input")
    table = _positive_table()  # strictly increasing with the code
    a = np.abs(x)
    hi = np.searchsorted(table, a, side="left")  # first code with value >= a
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_hi = table[hi] - a
    d_lo = a - table[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(a >= table[-1], len(table) - 1, code)  # saturate to 448
    sign = np.signbit(x).astype(np.int64)
    return (code | (sign << 7)).astype(np.uint8)


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f32_bits_to_f64(raw_le_bytes):
    """Little-endian float32 bytes (uint8 array, last dim multiple of 4) to
    float64."""
    r = np.ascontiguousarray(np.asarray(raw_le_bytes, dtype=np.uint8))
    return r.view("<f4").astype(np.float64)
