"""Exact decoders and RNE encoders for E2M1, E4M3 (FN), E8M0 and BF16.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Definitions (OCP Microscaling Formats (MX) v1.0, element and scale formats;
named on the pages as "NVFP4"/"nvfp4_e2m1", "FP8 E4M3" and "MXFP"):

* E2M1: 4 bits s|e:2|m:1, exponent bias 1, no Inf/NaN.
  e == 0: value = m * 0.5 (subnormal); else (1 + m/2) * 2**(e-1).
* E4M3 (FN variant): 8 bits s|e:4|m:3, bias 7, no Inf.
  e == 0: value = (m/8) * 2**-6; else (1 + m/8) * 2**(e-7);
  s.1111.111 is NaN, so the largest finite magnitude is 0x7E = 448.
* E8M0: 8-bit unsigned biased exponent, value 2**(c-127); 0xFF is NaN.
* BF16: the top 16 bits of an IEEE binary32.

Encoders round a non-negative magnitude to the nearest representable value,
ties to the code with an even last bit (IEEE round-to-nearest-even), and
saturate anything above the largest finite value to it ("satfinite").  They
are written as a nearest-neighbour search over the representable grid, which
is the definition of rounding, not a bit trick.
"""

import numpy as np


# ---------------------------------------------------------------- decoders --

def e2m1_value(code: int) -> float:
    """Value of one E2M1 code (low 4 bits of ``code``)."""
    code &= 0xF
    s, e, m = code >> 3, (code >> 1) & 0x3, code & 0x1
    mag = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


def e4m3_value(code: int) -> float:
    """Value of one E4M3 (FN) code; NaN for 0x7F / 0xFF."""
    code &= 0xFF
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e8m0_value(code: int) -> float:
    """Value of one E8M0 code: 2**(code-127); NaN for 0xFF."""
    code &= 0xFF
    return float("nan") if code == 0xFF else 2.0 ** (code - 127)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def decode_e2m1(codes) -> np.ndarray:
    """Unpacked E2M1 codes (any integer array, low nibble used) -> float64."""
    return E2M1_TABLE[np.asarray(codes).astype(np.int64) & 0xF]


def decode_e4m3(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes).astype(np.int64) & 0xFF]


def decode_e8m0(codes) -> np.ndarray:
    return E8M0_TABLE[np.asarray(codes).astype(np.int64) & 0xFF]


def decode_bf16(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN payloads stay NaN
        return b.view(np.float32).astype(np.float64)


def decode_f16(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64, exactly, from the bit
    fields: sign 1, exponent 5 (bias 15), fraction 10.  Exponent 0 is
    subnormal (f * 2**-24); exponent 31 is Inf (f == 0) or NaN."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(f, -24), np.ldexp(1024.0 + f, (e - 25).astype(np.int64)))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def unpack_nibbles(packed) -> np.ndarray:
    """uint8 [..., K/2] -> uint8 [..., K]; element 2j is the low nibble of byte j."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_nibbles(codes) -> np.ndarray:
    """uint8 [..., K] (values < 16) -> uint8 [..., K/2], even element low."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------- encoders --

# Non-negative codes in increasing value order, with their values.  For these
# sign-magnitude formats the value grows with the code, so the grid is sorted.
_E2M1_POS_CODES = np.arange(0, 8, dtype=np.int64)
_E2M1_POS_VALUES = E2M1_TABLE[:8].copy()
_E4M3_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)          # 0x7F is NaN
_E4M3_POS_VALUES = E4M3_TABLE[:0x7F].copy()
assert np.all(np.diff(_E2M1_POS_VALUES) > 0) and np.all(np.diff(_E4M3_POS_VALUES) > 0)


def _round_to_grid(mag, values, codes) -> np.ndarray:
    """Nearest grid value to each non-negative ``mag``; ties -> even code;
    above the top of the grid -> the top (satfinite)."""
    mag = np.asarray(mag, dtype=np.float64)
    assert np.all(mag >= 0) and not np.any(np.isnan(mag)), "encoder takes finite magnitudes"
    hi = np.searchsorted(values, mag, side="left")        # values[hi-1] < mag <= values[hi]
    top = len(values) - 1
    hi_c = np.minimum(hi, top)
    lo_c = np.maximum(hi - 1, 0)
    d_lo = mag - values[lo_c]                            # exact: both are short binary fractions
    d_hi = values[hi_c] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi_c] & 1) == 0))
    out = np.where(pick_hi, codes[hi_c], codes[lo_c])
    out = np.where(hi == 0, codes[0], out)               # mag == 0 (or below grid)
    out = np.where(mag >= values[top], codes[top], out)  # saturate
    return out.astype(np.uint8)


def encode_e2m1_mag(mag) -> np.ndarray:
    """|q| -> 3-bit E2M1 magnitude code, RNE, saturating at 6."""
    return _round_to_grid(mag, _E2M1_POS_VALUES, _E2M1_POS_CODES)


def encode_e4m3_mag(mag) -> np.ndarray:
    """|s| -> 7-bit E4M3 magnitude code, RNE, saturating at 448 (0x7E)."""
    return _round_to_grid(mag, _E4M3_POS_VALUES, _E4M3_POS_CODES)


def signbit_u8(x) -> np.ndarray:
    return np.signbit(np.asarray(x)).astype(np.uint8)
