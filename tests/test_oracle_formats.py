"""Pins for the oracle's format decoders and encoders (CPU only).

Each check pins ``oracle.formats`` to something other than itself: torch's
independent float8 casts, a generic minifloat decoder written here from the
field widths alone, the format definitions' anchor values, and exact rational
comparisons at every rounding midpoint."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import scalar as S


def _generic_minifloat(code, ebits, mbits, bias):
    """Decode sign|exponent|mantissa by enumerating (1 + m / 2**mbits) * 2**(e - bias)
    (normal) and (m / 2**mbits) * 2**(1 - bias) (subnormal)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        v = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return -v if s else v


def test_e2m1_values_are_the_format_list():
    # E2M1 magnitudes fixed by its field widths (1 sign, 2 exponent, 1 mantissa, bias 1)
    assert list(F.E2M1_TABLE[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(F.E2M1_TABLE[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(F.E2M1_TABLE[8])
    for c in range(16):
        assert F.E2M1_TABLE[c] == float(_generic_minifloat(c, 2, 1, 1))


def test_e4m3_decode_matches_torch_and_generic():
    codes = torch.arange(256, dtype=torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.decode_e4m3(np.arange(256))
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(np.nonzero(nan)[0], [0x7F, 0xFF])
    assert np.array_equal(t[~nan], ours[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(ours[~nan]))
    for c in range(256):
        if c & 0x7F != 0x7F:
            assert ours[c] == float(_generic_minifloat(c, 4, 3, 7))


def test_e4m3_anchors():
    v = F.decode_e4m3
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6 and v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9
    assert v(0x38) == 1.0 and np.isnan(v(0x7F))


def test_e8m0_decode_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = F.decode_e8m0(np.arange(256))
    assert np.isnan(t[255]) and np.isnan(ours[255])
    assert np.array_equal(t[:255], ours[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = F.decode_bf16(bits)
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(t[~nan], ours[~nan])


def test_nibble_order_even_element_low():
    codes = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    packed = F.pack_nibbles(codes)
    assert packed.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(F.unpack_nibbles(packed), codes)


def _f32_neighbours(v):
    v = np.float32(v)
    return [np.nextafter(v, np.float32(-np.inf)), v, np.nextafter(v, np.float32(np.inf))]


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_encoder_rne_at_every_midpoint(fmt):
    """At each midpoint between consecutive representable magnitudes and at its
    float32 neighbours, the encoder returns the exactly nearest code, the even
    one on a tie -- decided here with rational arithmetic."""
    if fmt == "e2m1":
        vals, enc, ncodes = F.E2M1_TABLE[:8], F.encode_e2m1_mag, 8
    else:
        vals, enc, ncodes = F.E4M3_TABLE[:0x7F], F.encode_e4m3_mag, 0x7F
    for c in range(ncodes - 1):
        lo, hi = Fraction(float(vals[c])), Fraction(float(vals[c + 1]))
        mid = (lo + hi) / 2
        for x in _f32_neighbours(float(mid)):
            fx = Fraction(float(x))
            if fx == mid:
                want = c if c % 2 == 0 else c + 1
            elif fx < mid:
                want = c if fx >= lo else None
            else:
                want = c + 1 if fx <= hi else None
            if want is None:
                continue
            assert int(enc(np.array([x], np.float32))[0]) == want, (fmt, c, float(x))


def test_e4m3_encoder_matches_torch_below_overflow():
    r = np.random.Generator(np.random.PCG64(7))
    x = np.concatenate([
        r.uniform(0, 464, 200000).astype(np.float32),
        np.exp2(r.uniform(-12, 9, 200000)).astype(np.float32),
        (F.E4M3_TABLE[:0x7E] + F.E4M3_TABLE[1:0x7F]).astype(np.float32) / 2,  # ties
    ])
    x = x[x < 464]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.encode_e4m3_mag(x), t)


def test_encoders_saturate():
    assert F.encode_e4m3_mag(np.array([448.0, 449.0, 464.0, 1e30], np.float32)).tolist() == [0x7E] * 4
    assert F.encode_e2m1_mag(np.array([6.0, 6.5, 7.0, 1e30], np.float32)).tolist() == [7] * 4


def test_e2m1_ties_table():
    # ties go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2, 2.5->2, 3.5->4, 5->4
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    got = F.E2M1_TABLE[F.encode_e2m1_mag(x)]
    assert got.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


def test_encoders_agree_with_scalar_bruteforce():
    r = np.random.Generator(np.random.PCG64(11))
    x2 = np.abs(r.standard_normal(3000).astype(np.float32) * 3)
    x4 = np.exp2(r.uniform(-11, 9.2, 3000)).astype(np.float32)
    e2 = F.encode_e2m1_mag(x2)
    e4 = F.encode_e4m3_mag(x4)
    for i in range(0, 3000, 7):
        assert e2[i] == S.e2m1_encode_mag(Fraction(float(x2[i])))
        assert e4[i] == S.e4m3_encode_mag(Fraction(float(x4[i])))
