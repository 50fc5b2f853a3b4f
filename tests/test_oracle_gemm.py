"""Pins for the oracle's GEMM references and acceptance test (CPU only).

The float64 references are pinned against exact rational brute force on tiny
inputs (decoded with the scalar field formulas of ``oracle.scalar``), closed
forms (constant codes, one-hot rows), an invariance (a consistent permutation
of K blocks leaves C unchanged), and reductions between the variants.  Planted
mistakes (wrong nibble order, wrong scale index, dropped tensor scale, a
transposed operand) must make these pins fail: that is checked too."""

from fractions import Fraction

import numpy as np
import pytest

from block_scaled_precision_bsgemm_amd import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q
from oracle import scalar as S


def _exact_nvfp4(codes, scales, st):
    """Rational dequantisation from the scalar field formulas."""
    un = F.unpack_nibbles(codes)
    R, K = un.shape
    stf = Fraction(float(np.float32(st)))
    return [[S.e2m1_frac(int(un[r, k])) * S.e4m3_frac(int(scales[r, k // 16])) * stf
             for k in range(K)] for r in range(R)]


def _exact_mxfp8(codes, scales):
    R, K = codes.shape
    return [[S.e4m3_frac(int(codes[r, k])) * Fraction(2) ** (int(scales[r, k // 32]) - 127)
             for k in range(K)] for r in range(R)]


def _exact_mxfp4(codes, scales):
    un = F.unpack_nibbles(codes)
    R, K = un.shape
    return [[S.e2m1_frac(int(un[r, k])) * Fraction(2) ** (int(scales[r, k // 32]) - 127)
             for k in range(K)] for r in range(R)]


def _exact_gemm(a, b):
    return [[sum((x * y for x, y in zip(ra, rb)), Fraction(0)) for rb in b] for ra in a]


def _exact_mag(a, b):
    return [[sum((abs(x * y) for x, y in zip(ra, rb)), Fraction(0)) for rb in b] for ra in a]


def _nvfp4_tiny(seed, m=4, k=64):
    x = synth.normal_f32((m, k), seed)
    x[:, 16:32] *= np.float32(0.01)          # mixed block scales
    x[1, 40:48] *= np.float32(30.0)
    return Q.quantize_nvfp4(x)


def test_nvfp4_gemm_equals_exact_bruteforce():
    a = _nvfp4_tiny(31)
    b = _nvfp4_tiny(32)
    c, t = G.gemm_nvfp4(*a, *b)
    ea, eb = _exact_nvfp4(*a), _exact_nvfp4(*b)
    ce, te = _exact_gemm(ea, eb), _exact_mag(ea, eb)
    for i in range(4):
        for j in range(4):
            assert abs(Fraction(float(c[i, j])) - ce[i][j]) <= Fraction(1e-12) * te[i][j]
            assert abs(Fraction(float(t[i, j])) - te[i][j]) <= Fraction(1e-12) * te[i][j]


def test_mxfp8_gemm_equals_exact_bruteforce():
    xa = synth.normal_f32((4, 32), 41)
    xb = synth.normal_f32((4, 32), 42)
    xa[2] *= np.float32(1e3)
    a, b = Q.quantize_mxfp8(xa), Q.quantize_mxfp8(xb)
    c, t = G.gemm_mxfp8(*a, *b)
    ea, eb = _exact_mxfp8(*a), _exact_mxfp8(*b)
    ce, te = _exact_gemm(ea, eb), _exact_mag(ea, eb)
    for i in range(4):
        for j in range(4):
            assert abs(Fraction(float(c[i, j])) - ce[i][j]) <= Fraction(1e-12) * te[i][j]


def test_nvfp4_constant_codes_closed_form():
    M, N, K = 3, 5, 64
    va, vb = 0x3, 0xA                                   # 1.5 and -1.0
    sa, sb = 0x41, 0x2C                                 # e4m3: 2.25 and 0.375
    a = (np.full((M, K // 2), va | (va << 4), np.uint8), np.full((M, K // 16), sa, np.uint8), np.float32(0.5))
    b = (np.full((N, K // 2), vb | (vb << 4), np.uint8), np.full((N, K // 16), sb, np.uint8), np.float32(3.0))
    c, t = G.gemm_nvfp4(*a, *b)
    want = K * 1.5 * -1.0 * 2.25 * 0.375 * 0.5 * 3.0
    assert np.all(c == want) and np.all(t == abs(want))


def test_nvfp4_one_hot_rows_select_scaled_b():
    K = 64
    b = _nvfp4_tiny(5, m=6, k=K)
    bd = G.dequant_nvfp4(*b)
    codes = np.zeros((2, K), np.uint8)
    codes[0, 17] = 0x2                                   # 1.0 at k = 17
    codes[1, 50] = 0xC                                   # -2.0 at k = 50
    scales = np.full((2, K // 16), 0x38, np.uint8)       # 1.0
    c, _ = G.gemm_nvfp4(F.pack_nibbles(codes), scales, np.float32(1.0), *b)
    assert np.array_equal(c[0], bd[:, 17]) and np.array_equal(c[1], -2.0 * bd[:, 50])


def test_mxfp4_gemm_equals_exact_bruteforce():
    xa = synth.normal_f32((4, 96), 43)
    xb = synth.normal_f32((4, 96), 44)
    xa[2] *= np.float32(1e3)
    xb[:, 32:64] *= np.float32(1e-2)
    a, b = Q.quantize_mxfp4(xa), Q.quantize_mxfp4(xb)
    c, t = G.gemm_mxfp4(*a, *b)
    ea, eb = _exact_mxfp4(*a), _exact_mxfp4(*b)
    ce, te = _exact_gemm(ea, eb), _exact_mag(ea, eb)
    for i in range(4):
        for j in range(4):
            assert abs(Fraction(float(c[i, j])) - ce[i][j]) <= Fraction(1e-12) * te[i][j]
            assert abs(Fraction(float(t[i, j])) - te[i][j]) <= Fraction(1e-12) * te[i][j]


def test_mxfp4_constant_codes_and_one_hot_closed_forms():
    K = 128
    # constant codes: every A element 1.5 (code 3) at scale 2**2, every B element -0.5 (code 9) at 2**-3
    a = (F.pack_nibbles(np.full((2, K), 3, np.uint8)), np.full((2, K // 32), 129, np.uint8))
    b = (F.pack_nibbles(np.full((3, K), 9, np.uint8)), np.full((3, K // 32), 124, np.uint8))
    c, t = G.gemm_mxfp4(*a, *b)
    assert np.all(c == K * 1.5 * 4 * -0.5 / 8) and np.all(t == -c)
    # one-hot A rows pick one dequantised element of each B row
    xb = synth.normal_f32((5, K), 45)
    b = Q.quantize_mxfp4(xb)
    bd = G.dequant_mxfp4(*b)
    codes = np.zeros((2, K), np.uint8)
    codes[0, 70] = 2                                      # +1.0
    codes[1, 5] = 8 | 4                                   # -2.0
    a = (F.pack_nibbles(codes), np.full((2, K // 32), 127, np.uint8))
    c, _ = G.gemm_mxfp4(*a, *b)
    assert np.array_equal(c[0], bd[:, 70]) and np.array_equal(c[1], -2.0 * bd[:, 5])


def test_planted_mxfp4_scale_index_fails_the_bruteforce_pin(monkeypatch):
    xa, xb = synth.normal_f32((4, 96), 46), synth.normal_f32((4, 96), 47)
    xa[:, 32:64] *= np.float32(50.0)
    a, b = Q.quantize_mxfp4(xa), Q.quantize_mxfp4(xb)
    ea, eb = _exact_mxfp4(*a), _exact_mxfp4(*b)
    ce, te = _exact_gemm(ea, eb), _exact_mag(ea, eb)
    orig = G.dequant_mxfp4
    monkeypatch.setattr(G, "dequant_mxfp4", lambda codes, scales: orig(codes, np.roll(scales, 1, axis=1)))
    c, _ = G.gemm_mxfp4(*a, *b)
    worst = max(abs(Fraction(float(c[i, j])) - ce[i][j]) / te[i][j] for i in range(4) for j in range(4))
    assert worst > Fraction(1e-6)


def test_mxfp8_block_permutation_invariance():
    xa, xb = synth.normal_f32((8, 256), 51), synth.normal_f32((8, 256), 52)
    a, b = Q.quantize_mxfp8(xa), Q.quantize_mxfp8(xb)
    c, t = G.gemm_mxfp8(*a, *b)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(8)
    def pb(codes, scales):
        return (codes.reshape(8, 8, 32)[:, perm].reshape(8, 256), scales[:, perm])
    c2, t2 = G.gemm_mxfp8(*pb(*a), *pb(*b))
    assert np.allclose(c, c2, rtol=0, atol=1e-12 * t.max()) and np.allclose(t, t2, rtol=1e-14)


def test_grouped_reduces_to_per_group_products_and_handles_empty_groups():
    K, N = 64, 6
    counts = np.array([3, 0, 5, 0, 1])
    off = synth.offsets_from_counts(counts)
    x = synth.normal_f32((int(counts.sum()), K), 61)
    a = Q.quantize_nvfp4(x)
    w = synth.bf16_bits(synth.normal_f32((len(counts), N, K), 62, std=0.02))
    c, t = G.grouped_nvfp4_bf16(*a, off, w)
    ea = _exact_nvfp4(*a)
    for g in range(len(counts)):
        wg = [[Fraction(float(v)) for v in row] for row in F.decode_bf16(w[g])]
        for r in range(off[g], off[g + 1]):
            ce = _exact_gemm([ea[r]], wg)[0]
            for n in range(N):
                assert abs(Fraction(float(c[r, n])) - ce[n]) <= Fraction(1e-12) * (1 + abs(ce[n]))
    # restricting rows returns the same rows
    rows = np.array([8, 0, 4])
    c2, _ = G.grouped_nvfp4_bf16(*a, off, w, rows=rows)
    assert np.array_equal(c2, c[rows])


def _f16_frac(bits):
    """Exact value of a finite FP16 bit pattern, from its fields."""
    b = int(bits) & 0xFFFF
    sign = -1 if b >> 15 else 1
    e, f = (b >> 10) & 0x1F, b & 0x3FF
    assert e != 31
    return sign * (Fraction(f, 1 << 24) if e == 0 else Fraction(1024 + f, 1 << 10) * Fraction(2) ** (e - 15))


def test_decode_f16_matches_numpy_float16_on_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = F.decode_f16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.all((ours == ref) | (np.isnan(ours) & np.isnan(ref)))
    for b in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xC000, 0x8001):
        assert Fraction(float(ours[b])) == _f16_frac(b)


def _grouped_ex_case(seed, w_dtype):
    r = np.random.Generator(np.random.PCG64(seed))
    counts = np.array([3, 0, 4, 2])
    off = synth.offsets_from_counts(counts)
    M, K, N, a_rows = int(counts.sum()), 64, 5, 7
    x = synth.normal_f32((a_rows, K), seed + 1)
    x[2, 16:32] *= np.float32(0.01)
    a = Q.quantize_nvfp4(x)
    wf = synth.normal_f32((len(counts), N, K), seed + 2, std=0.5)
    w = synth.bf16_bits(wf) if w_dtype == "bf16" else wf.astype(np.float16).view(np.uint16)
    gather = r.integers(0, a_rows, M).astype(np.int32)
    scatter = r.permutation(M).astype(np.int32)
    bias = r.standard_normal((len(counts), N)).astype(np.float32)
    gamma = r.uniform(-2, 2, M).astype(np.float32)
    return a, off, w, gather, scatter, bias, gamma


def _grouped_ex_exact(a, off, w, w_dtype, gather, scatter, bias, gamma):
    """Element by element in rationals: y = (s_t sum a w + bias) gamma, stored
    at the scattered row."""
    ea = _exact_nvfp4(*a)
    M, N = int(off[-1]), w.shape[1]
    dec = (lambda v: Fraction(float(F.decode_bf16(v)))) if w_dtype == "bf16" else _f16_frac
    out = {}
    for g in range(len(off) - 1):
        for r in range(off[g], off[g + 1]):
            row = ea[int(gather[r])]
            vals = []
            for n in range(N):
                acc = sum((x * dec(w[g, n, k]) for k, x in enumerate(row)), Fraction(0))
                vals.append((acc + Fraction(float(bias[g, n]))) * Fraction(float(gamma[r])))
            out[int(scatter[r])] = vals
    assert sorted(out) == list(range(M))
    return out


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
def test_grouped_ex_equals_exact_bruteforce(w_dtype):
    a, off, w, gather, scatter, bias, gamma = _grouped_ex_case(91, w_dtype)
    c, t = G.grouped_nvfp4_ex(*a, off, w, w_dtype, bias, gamma, gather, scatter)
    ex = _grouped_ex_exact(a, off, w, w_dtype, gather, scatter, bias, gamma)
    for row, vals in ex.items():
        for n, v in enumerate(vals):
            assert abs(Fraction(float(c[row, n])) - v) <= Fraction(1e-12) * (1 + abs(v)), (row, n)
            assert t[row, n] >= abs(float(v)) * (1 - 1e-12)
    # planted mistakes: gamma taken by physical row, or bias of the wrong group
    cw, _ = G.grouped_nvfp4_ex(*a, off, w, w_dtype, bias, gamma[scatter], gather, scatter)
    assert not np.allclose(cw, c, rtol=1e-9, atol=1e-9)
    cb, _ = G.grouped_nvfp4_ex(*a, off, w, w_dtype, bias[::-1].copy(), gamma, gather, scatter)
    assert not np.allclose(cb, c, rtol=1e-9, atol=1e-9)


def test_grouped_ex_reductions():
    a, off, w, gather, scatter, bias, gamma = _grouped_ex_case(92, "bf16")
    M = int(off[-1])
    # no variants: the plain grouped reference on the same rows of A
    ident = np.arange(M)
    x = synth.normal_f32((M, 64), 93)
    aq = Q.quantize_nvfp4(x)
    c0, t0 = G.grouped_nvfp4_bf16(*aq, off, w)
    c1, t1 = G.grouped_nvfp4_ex(*aq, off, w, "bf16", gather=ident, scatter=ident)
    assert np.allclose(c0, c1, rtol=1e-14, atol=1e-14 * t0.max()) and np.allclose(t0, t1, rtol=1e-14)
    c2, _ = G.grouped_nvfp4_ex(*aq, off, w, "bf16", bias=np.zeros((len(off) - 1, w.shape[1]), np.float32),
                               gamma=np.ones(M, np.float32))
    assert np.allclose(c0, c2, rtol=1e-14, atol=1e-14 * t0.max())
    # gamma = 2^j scales rows exactly; scatter permutes rows
    gam = np.exp2(np.arange(M) % 5 - 2).astype(np.float32)
    c3, _ = G.grouped_nvfp4_ex(*aq, off, w, "bf16", gamma=gam)
    assert np.array_equal(c3, c0 * gam[:, None].astype(np.float64))
    perm = np.random.Generator(np.random.PCG64(94)).permutation(M)
    c4, _ = G.grouped_nvfp4_ex(*aq, off, w, "bf16", scatter=perm)
    assert np.array_equal(c4[perm], c0)
    # zero activations leave bias * gamma (closed form)
    z = (np.zeros_like(aq[0]), aq[1], aq[2])
    c5, _ = G.grouped_nvfp4_ex(*z, off, w, "bf16", bias=bias, gamma=gamma[:M])
    grp = np.searchsorted(off, np.arange(M), side="right") - 1
    assert np.array_equal(c5, bias[grp].astype(np.float64) * gamma[:M, None].astype(np.float64))
    # out_rows selects physical rows
    rows = np.array([5, 0, 8])
    c6, _ = G.grouped_nvfp4_ex(*a, off, w, "bf16", bias, gamma, gather, scatter, out_rows=rows)
    c7, _ = G.grouped_nvfp4_ex(*a, off, w, "bf16", bias, gamma, gather, scatter)
    assert np.array_equal(c6, c7[rows])


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
def test_grouped_kragged_bruteforce_and_invariants(w_dtype):
    M, N, K = 3, 4, 96
    off = np.array([0, 32, 32, 96])                  # an empty group in the middle
    x = synth.normal_f32((M, K), 95)
    x[:, 40:56] *= np.float32(0.01)
    a = Q.quantize_nvfp4(x)
    wf = synth.normal_f32((N, K), 96, std=0.5)
    w = synth.bf16_bits(wf) if w_dtype == "bf16" else wf.astype(np.float16).view(np.uint16)
    c, t = G.grouped_kragged(*a, off, w, w_dtype)
    assert c.shape == (3, M, N)
    ea = _exact_nvfp4(*a)
    dec = (lambda v: Fraction(float(F.decode_bf16(v)))) if w_dtype == "bf16" else _f16_frac
    for g in range(3):
        for m in range(M):
            for n in range(N):
                ex = sum((ea[m][k] * dec(w[n, k]) for k in range(off[g], off[g + 1])), Fraction(0))
                assert abs(Fraction(float(c[g, m, n])) - ex) <= Fraction(1e-12) * (1 + abs(ex))
    assert np.all(c[1] == 0) and np.all(t[1] == 0)
    # the groups partition K: their sum is the one-group product over all of K
    c1, t1 = G.grouped_kragged(*a, np.array([0, K]), w, w_dtype)
    assert np.allclose(c.sum(axis=0), c1[0], rtol=0, atol=1e-12 * t1.max())
    assert np.allclose(t.sum(axis=0), t1[0], rtol=1e-12)
    # planted mistake: slices taken from the wrong end of K
    cw, _ = G.grouped_kragged(*a, off, w[:, ::-1].copy(), w_dtype)
    assert not np.allclose(cw, c, rtol=1e-9, atol=1e-9)


def test_w4a16_equals_exact_bruteforce():
    M, N, K = 3, 4, 64
    x = synth.bf16_bits(synth.normal_f32((M, K), 71))
    wq = Q.quantize_nvfp4(synth.normal_f32((N, K), 72, std=0.02))
    c, t = G.w4a16(x, *wq)
    xe = [[Fraction(float(v)) for v in row] for row in F.decode_bf16(x)]
    ce = _exact_gemm(xe, _exact_nvfp4(*wq))
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(float(c[i, j])) - ce[i][j]) <= Fraction(1e-12) * (1 + abs(ce[i][j]))


def test_check_accepts_rounded_reference_and_rejects_errors():
    a, b = _nvfp4_tiny(81, m=8), _nvfp4_tiny(82, m=8)
    c, t = G.gemm_nvfp4(*a, *b)
    bits = synth.bf16_bits(c.astype(np.float32))
    assert G.check(bits, c, t)["ok"]
    bad = bits.copy()
    bad[0, 0] ^= 0x0040                                  # a large mantissa bit
    assert not G.check(bad, c, t)["ok"]
    nan = bits.copy()
    nan[1, 1] = 0x7FC0
    r = G.check(nan, c, t)
    assert not r["ok"] and r["n_nonfinite"] == 1


# ---------------------------------------------------- negative controls --

def _planted(monkeypatch, what):
    if what == "nibble_order":
        def wrong(p):
            p = np.asarray(p, np.uint8)
            out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
            out[..., 0::2], out[..., 1::2] = p >> 4, p & 0xF
            return out
        monkeypatch.setattr(G, "unpack_nibbles", wrong)
    elif what == "scale_index":
        orig = G.nvfp4_units
        def wrong(codes, scales):
            return orig(codes, np.roll(scales, 1, axis=1))
        monkeypatch.setattr(G, "nvfp4_units", wrong)
    elif what == "tensor_scale":
        orig = G.gemm_nvfp4
        monkeypatch.setattr(G, "gemm_nvfp4", lambda ac, asc, ats, bc, bs, bts, rows=None: orig(ac, asc, 1.0, bc, bs, bts, rows))
    elif what == "transpose":
        monkeypatch.setattr(G, "_matmul_and_mag", lambda a, b: ((a @ b.T).T, np.abs(a) @ np.abs(b).T))


@pytest.mark.parametrize("what", ["scale_index", "tensor_scale", "transpose"])
def test_planted_oracle_mistakes_fail_the_bruteforce_pin(monkeypatch, what):
    a = _nvfp4_tiny(91)
    b = _nvfp4_tiny(92)
    a = (a[0], a[1], np.float32(0.75) if what == "tensor_scale" else a[2])
    ea, eb = _exact_nvfp4(*a), _exact_nvfp4(*b)
    ce, te = _exact_gemm(ea, eb), _exact_mag(ea, eb)
    _planted(monkeypatch, what)
    c, _ = G.gemm_nvfp4(*a, *b)
    worst = max(abs(Fraction(float(c[i, j])) - ce[i][j]) / te[i][j] for i in range(4) for j in range(4))
    assert worst > Fraction(1e-6), what


def test_planted_nibble_swap_fails_the_one_sided_pins(monkeypatch):
    """Swapping the nibble order on BOTH operands of an NVFP4 x NVFP4 product is
    a consistent K permutation inside each 16-block, so C cannot see it; the
    elementwise dequantisation and the mixed NVFP4 x dense products can."""
    a = _nvfp4_tiny(93)
    ea = _exact_nvfp4(*a)
    x = synth.bf16_bits(synth.normal_f32((3, 64), 94))
    c0, _ = G.w4a16(x, *a)
    _planted(monkeypatch, "nibble_order")
    d = G.dequant_nvfp4(*a)
    assert any(Fraction(float(d[r, k])) != ea[r][k] for r in range(4) for k in range(64))
    c1, t1 = G.w4a16(x, *a)
    assert np.max(np.abs(c1 - c0) / t1) > 1e-6


def test_nvfp4_negative_tensor_scale():
    """T is the sum of the magnitudes of the summed terms, so a negative
    tensor scale flips C and leaves T as for its magnitude; T >= |C|."""
    r = np.random.Generator(np.random.PCG64(11))
    a = (r.integers(0, 256, (5, 16)).astype(np.uint8), r.integers(0, 0xFF, (5, 2)).astype(np.uint8) & 0xFE)
    b = (r.integers(0, 256, (7, 16)).astype(np.uint8), r.integers(0, 0x7F, (7, 2)).astype(np.uint8))
    cp, tp = G.gemm_nvfp4(a[0], a[1], np.float32(0.5), b[0], b[1], np.float32(3.0))
    cn, tn = G.gemm_nvfp4(a[0], a[1], np.float32(0.5), b[0], b[1], np.float32(-3.0))
    assert np.array_equal(cn, -cp) and np.array_equal(tn, tp)
    assert np.all(tn >= np.abs(cn)) and np.all(tn > 0)
