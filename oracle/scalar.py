"""Second, scalar implementation of the quantizers, in exact rational arithmetic.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Used only to cross-check ``oracle.quantize`` on small inputs.  It shares
nothing with it but the recipe: values are ``fractions.Fraction``; every FP32
operation is the exact rational result rounded by ``round_f32`` below (binary32,
round-to-nearest-even, subnormals kept); encoders scan every code and keep the
nearest value (ties to the even code, saturating), instead of a sorted search;
decoders are the field formulas evaluated in rationals.
"""

from fractions import Fraction

TWO = Fraction(2)


def round_f32(r: Fraction) -> Fraction:
    """Round an exact rational to the nearest IEEE binary32 value (RNE)."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    while TWO ** E > a:
        E -= 1
    while TWO ** (E + 1) <= a:
        E += 1
    E = max(E, -126)                       # below 2**-126 the quantum stays 2**-149
    quantum = TWO ** (E - 23)
    n = a / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    out = k * quantum
    assert out < TWO ** 128, "FP32 overflow is outside the recipe's range"
    return sign * out


def f32(x) -> Fraction:
    """Exact rational value of a Python float that holds an FP32 value."""
    fr = Fraction(x)
    assert round_f32(fr) == fr, "not an FP32 value"
    return fr


def e2m1_frac(code: int) -> Fraction:
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * TWO ** (e - 1)
    return -mag if s else mag


def e4m3_frac(code: int) -> Fraction:
    s, e, m = (code >> 7) & 1, (code >> 3) & 0xF, code & 7
    assert not (e == 15 and m == 7), "NaN code"
    mag = Fraction(m, 8) * TWO ** -6 if e == 0 else (1 + Fraction(m, 8)) * TWO ** (e - 7)
    return -mag if s else mag


def _nearest_code(mag: Fraction, codes, value_of) -> int:
    best, best_d = None, None
    top = max(codes, key=value_of)
    if mag >= value_of(top):
        return top
    for c in codes:
        d = abs(value_of(c) - mag)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def e2m1_encode_mag(mag: Fraction) -> int:
    return _nearest_code(mag, range(8), e2m1_frac)


def e4m3_encode_mag(mag: Fraction) -> int:
    return _nearest_code(mag, range(0x7F), e4m3_frac)


def _signbit(x: float) -> int:
    import math
    return 1 if math.copysign(1.0, x) < 0 else 0


def quantize_nvfp4_scalar(rows, tensor_scale=None):
    """rows: list of lists of FP32-valued floats, len % 16 == 0.
    Returns (codes as list of lists of 4-bit ints (unpacked), scale codes, s_t)."""
    amax = max((abs(f32(v)) for r in rows for v in r), default=Fraction(0))
    s_t = round_f32(amax / 2688) if tensor_scale is None else f32(tensor_scale)
    codes, scales = [], []
    for r in rows:
        rc, rs = [], []
        for b0 in range(0, len(r), 16):
            blk = [f32(v) for v in r[b0:b0 + 16]]
            signs = [_signbit(v) for v in r[b0:b0 + 16]]
            bamax = max(abs(v) for v in blk)
            if s_t == 0:
                sc = 0
            else:
                s_real = round_f32(round_f32(bamax / 6) / s_t)
                sc = e4m3_encode_mag(s_real)
            S = round_f32(e4m3_frac(sc) * s_t)
            rs.append(sc)
            for v, sg in zip(blk, signs):
                if S == 0:
                    rc.append(sg << 3)
                else:
                    q = round_f32(v / S)
                    rc.append((sg << 3) | e2m1_encode_mag(abs(q)))
        codes.append(rc)
        scales.append(rs)
    return codes, scales, s_t


def quantize_mxfp8_scalar(rows):
    """rows: list of lists of FP32-valued floats, len % 32 == 0.
    Returns (codes, scale codes) as lists of lists of ints."""
    codes, scales = [], []
    for r in rows:
        rc, rs = [], []
        for b0 in range(0, len(r), 32):
            blk = [f32(v) for v in r[b0:b0 + 32]]
            signs = [_signbit(v) for v in r[b0:b0 + 32]]
            bamax = max(abs(v) for v in blk)
            if bamax == 0:
                e = -127
            else:
                e = -127
                while 448 * TWO ** e < bamax:  # least e with 448 * 2**e >= bamax
                    e += 1
                e = min(e, 127)
            rs.append(e + 127)
            for v, sg in zip(blk, signs):
                q = v * TWO ** -e
                rc.append((sg << 7) | e4m3_encode_mag(abs(q)))
        codes.append(rc)
        scales.append(rs)
    return codes, scales


def quantize_mxfp4_scalar(rows):
    """rows: list of lists of FP32-valued floats, len % 32 == 0.
    Returns (element codes, scale codes) as lists of lists of ints; element
    codes are unpacked 4-bit values (sign << 3 | E2M1 magnitude)."""
    codes, scales = [], []
    for r in rows:
        rc, rs = [], []
        for b0 in range(0, len(r), 32):
            blk = [f32(v) for v in r[b0:b0 + 32]]
            signs = [_signbit(v) for v in r[b0:b0 + 32]]
            bamax = max(abs(v) for v in blk)
            e = -127
            while bamax != 0 and 6 * TWO ** e < bamax:  # least e with 6 * 2**e >= bamax
                e += 1
            e = min(e, 127)
            rs.append(e + 127)
            for v, sg in zip(blk, signs):
                rc.append((sg << 3) | e2m1_encode_mag(abs(v * TWO ** -e)))
        codes.append(rc)
        scales.append(rs)
    return codes, scales
