"""Block-scaled GEMM references and the per-element acceptance test.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The operation throughout is C[m, n] = sum_k deq(A)[m, k] * deq(B)[n, k]: A is
[M, K], B (or W) is [N, K], both K-contiguous, C is [M, N] ("Together AI Ports
ThunderKittens GEMM Kernels to NVIDIA Vera Rubin NVL72", section "Building the
GEMM": M x N output tiles over a K loop; "Triton #11171 ...", section "The
missing case was defined by shape, layout, and execution mode together":
M x N x K cases with BF16 output).  Every code is decoded exactly to float64
and the sums are float64 (numpy matmul); the FP32 accumulation and BF16
rounding of the library are covered by the tolerance in ``check``.

Besides C the references return T[m, n] = sum_k |deq(A)[m, k] * deq(B)[n, k]|,
the scale of the accumulation error.
"""

import numpy as np

from .formats import (decode_bf16, decode_e2m1, decode_e4m3, decode_e8m0,
                      decode_f16, unpack_nibbles)

# ------------------------------------------------------------ dequantizers --


def nvfp4_units(codes, scales) -> np.ndarray:
    """e2m1(code) * e4m3(scale of its 16-block), float64 [R, K], without s_t.

    The product of a 2-significant-bit and a 4-significant-bit value is exact
    in float64 (and in FP16/BF16, which is what lets the library stage it)."""
    c = unpack_nibbles(codes)
    R, K = c.shape
    s = decode_e4m3(scales)
    assert s.shape == (R, K // 16)
    return decode_e2m1(c) * np.repeat(s, 16, axis=1)


def dequant_nvfp4(codes, scales, tensor_scale) -> np.ndarray:
    """x_hat = e2m1(code) * e4m3(scale) * s_t, exactly, float64 [R, K]."""
    return nvfp4_units(codes, scales) * np.float64(np.float32(tensor_scale))


def dequant_mxfp8(codes, scales) -> np.ndarray:
    """x_hat = e4m3(code) * 2**(scale - 127), exactly, float64 [R, K]."""
    c = np.asarray(codes)
    R, K = c.shape
    s = decode_e8m0(scales)
    assert s.shape == (R, K // 32)
    return decode_e4m3(c) * np.repeat(s, 32, axis=1)


# ------------------------------------------------------------------- GEMMs --


def _matmul_and_mag(a, b):
    return a @ b.T, np.abs(a) @ np.abs(b).T


def gemm_nvfp4(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, rows=None):
    """NVFP4 x NVFP4: returns (C_ref, T), float64 [M or len(rows), N].

    The sum is taken over the per-block products (e2m1*e4m3)_A (e2m1*e4m3)_B
    and multiplied once by s_tA * s_tB (exact in float64)."""
    a_codes, a_scales = np.asarray(a_codes), np.asarray(a_scales)
    if rows is not None:
        a_codes, a_scales = a_codes[rows], a_scales[rows]
    ua, ub = nvfp4_units(a_codes, a_scales), nvfp4_units(b_codes, b_scales)
    st = np.float64(np.float32(a_ts)) * np.float64(np.float32(b_ts))
    c, t = _matmul_and_mag(ua, ub)
    return c * st, t * abs(st)     # T sums the terms' magnitudes


def dequant_mxfp4(codes, scales) -> np.ndarray:
    """x_hat = e2m1(code) * 2**(scale - 127), exactly, float64 [R, K]."""
    c = unpack_nibbles(codes)
    R, K = c.shape
    s = decode_e8m0(scales)
    assert s.shape == (R, K // 32)
    return decode_e2m1(c) * np.repeat(s, 32, axis=1)


def gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, rows=None):
    """MXFP4 x MXFP4: returns (C_ref, T)."""
    a_codes, a_scales = np.asarray(a_codes), np.asarray(a_scales)
    if rows is not None:
        a_codes, a_scales = a_codes[rows], a_scales[rows]
    return _matmul_and_mag(dequant_mxfp4(a_codes, a_scales), dequant_mxfp4(b_codes, b_scales))


def gemm_mxfp8(a_codes, a_scales, b_codes, b_scales, rows=None):
    """MXFP8 x MXFP8: returns (C_ref, T)."""
    a_codes, a_scales = np.asarray(a_codes), np.asarray(a_scales)
    if rows is not None:
        a_codes, a_scales = a_codes[rows], a_scales[rows]
    return _matmul_and_mag(dequant_mxfp8(a_codes, a_scales), dequant_mxfp8(b_codes, b_scales))


def grouped_nvfp4_bf16(a_codes, a_scales, a_ts, offsets, w_bf16, rows=None):
    """Ragged grouped NVFP4 activations x dense BF16 weights.

    Rows off[g] .. off[g+1]-1 of A belong to group g and meet W[g] ([N, K]):
    C[r, :] = x_hat_A[r, :] @ W[g]^T ("Triton #11171 ...", sections "Ragged
    mode added routing rather than a plain matrix" and "NVFP4 x dense matmul").
    One tensor scale covers the whole activation tensor.  Empty groups add no
    rows.  ``rows`` restricts the output to those row indices (in order)."""
    off = np.asarray(offsets, dtype=np.int64)
    G = len(off) - 1
    w = np.asarray(w_bf16)
    assert w.shape[0] == G and off[0] == 0 and np.all(np.diff(off) >= 0)
    M = int(off[-1])
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    group_of = np.searchsorted(off, rows, side="right") - 1
    a_codes, a_scales = np.asarray(a_codes), np.asarray(a_scales)
    N = w.shape[1]
    c = np.zeros((len(rows), N))
    t = np.zeros((len(rows), N))
    for g in np.unique(group_of):
        sel = np.nonzero(group_of == g)[0]
        xa = dequant_nvfp4(a_codes[rows[sel]], a_scales[rows[sel]], a_ts)
        cg, tg = _matmul_and_mag(xa, decode_bf16(w[g]))
        c[sel], t[sel] = cg, tg
    return c, t


def grouped_nvfp4_ex(a_codes, a_scales, a_ts, offsets, w_bits, w_dtype="bf16", bias=None,
                     gamma=None, gather=None, scatter=None, out_rows=None):
    """Ragged grouped NVFP4 x dense GEMM with the epilogue variants of "Triton
    #11171 ...", sections "Scatter changes where output rows are written",
    "Gamma adds a per-row scaling input", "The ordinary variants also exercise
    the shared bias route" (NVFP4 x dense matmul + bias + optional gamma +
    optional scatter), the gathered-activation variant named in "Filter 3:
    gather variants are excluded", and the FP16 dense operand of the
    rhs_dtype sweep.

    Logical row r (off[g] <= r < off[g+1] puts it in group g):
        src(r) = gather[r] if gather is given, else r      (row of A it reads)
        y[r, n] = (s_t * sum_k x_hat_A[src(r), k] * W[g][n, k] + bias[g, n]) * gamma[r]
        C[dst(r), n] = y[r, n],  dst(r) = scatter[r] if scatter is given, else r
    bias ([G, N]) and gamma ([M]) are optional (absent = 0 and 1).  W holds
    BF16 or FP16 bit patterns ([G, N, K] uint16), decoded exactly.  The
    order (bias added to the scaled product, gamma applied to the sum) is the
    order the page lists them in.

    Returns (C_ref, T) over physical output rows 0..M-1 (or ``out_rows`` of
    them, in order), with T[dst(r), n] = (s_t * sum_k |a w| + |bias|) * |gamma|.
    A physical row that no logical row maps to stays 0 in both (scatter must
    be a permutation for every row to be written)."""
    off = np.asarray(offsets, dtype=np.int64)
    G = len(off) - 1
    w = np.asarray(w_bits)
    assert w.shape[0] == G and off[0] == 0 and np.all(np.diff(off) >= 0)
    M = int(off[-1])
    N = w.shape[1]
    decode = {"bf16": decode_bf16, "f16": decode_f16}[w_dtype]
    a_codes, a_scales = np.asarray(a_codes), np.asarray(a_scales)
    src = np.arange(M) if gather is None else np.asarray(gather, dtype=np.int64)
    dst = np.arange(M) if scatter is None else np.asarray(scatter, dtype=np.int64)
    assert src.shape == (M,) and dst.shape == (M,)
    gam = np.ones(M) if gamma is None else np.asarray(gamma, dtype=np.float64)
    if out_rows is None:
        out_rows = np.arange(M)
    out_rows = np.asarray(out_rows, dtype=np.int64)
    logical_of = np.full(M, -1, dtype=np.int64)
    logical_of[dst] = np.arange(M)
    logical = logical_of[out_rows]
    c = np.zeros((len(out_rows), N))
    t = np.zeros((len(out_rows), N))
    group_of = np.searchsorted(off, np.maximum(logical, 0), side="right") - 1
    for g in np.unique(group_of[logical >= 0]):
        sel = np.nonzero((group_of == g) & (logical >= 0))[0]
        lr = logical[sel]
        xa = dequant_nvfp4(a_codes[src[lr]], a_scales[src[lr]], 1.0)
        cg, tg = _matmul_and_mag(xa, decode(w[g]))
        cg, tg = cg * float(a_ts), tg * abs(float(a_ts))
        if bias is not None:
            b = np.asarray(bias, dtype=np.float64)[g]
            cg, tg = cg + b[None, :], tg + np.abs(b)[None, :]
        c[sel] = cg * gam[lr][:, None]
        t[sel] = tg * np.abs(gam[lr])[:, None]
    return c, t


def grouped_kragged(a_codes, a_scales, a_ts, k_offsets, w_bits, w_dtype="bf16"):
    """Inner-expert (K-ragged) grouped NVFP4 x dense GEMM: the groups split the
    contraction dimension K instead of the rows ("Triton #11171 ...",
    sections "Why `pad_a` represents the K-ragged boundary" (the activation's
    ragged dimension is 1, i.e. K, with ragged padding on A) and "K-ragged
    variants").

        C[g][m, n] = s_t * sum_{off[g] <= k < off[g+1]} x_hat_A[m, k] * W[n, k]

    A is NVFP4 [M, K], W holds BF16 or FP16 bit patterns [N, K]; each group's
    K slice is padded in both (the padding elements take part in the sum like
    any other element, so zero padding contributes nothing).  Returns
    (C [G, M, N], T [G, M, N]), T the sum of |products| times |s_t|."""
    off = np.asarray(k_offsets, dtype=np.int64)
    G = len(off) - 1
    w = np.asarray(w_bits)
    decode = {"bf16": decode_bf16, "f16": decode_f16}[w_dtype]
    xa = dequant_nvfp4(a_codes, a_scales, 1.0)
    xw = decode(w)
    assert off[0] == 0 and off[-1] == xa.shape[1] == xw.shape[1] and np.all(np.diff(off) >= 0)
    M, N = xa.shape[0], xw.shape[0]
    c = np.zeros((G, M, N))
    t = np.zeros((G, M, N))
    for g in range(G):
        sl = slice(int(off[g]), int(off[g + 1]))
        if off[g + 1] > off[g]:
            cg, tg = _matmul_and_mag(xa[:, sl], xw[:, sl])
            c[g], t[g] = cg * float(a_ts), tg * abs(float(a_ts))
    return c, t


def w4a16(x_bf16, w_codes, w_scales, w_ts):
    """BF16 activations X[M, K] x NVFP4 weights W[N, K]: C = X_hat @ W_hat^T
    ("Add sm121 (GB10) tier to the 4-bit GEMM dispatch heuristic", section
    "Methodology": the fused path is compared with dequantise-then-linear,
    which is this product)."""
    x = decode_bf16(x_bf16)
    w = dequant_nvfp4(w_codes, w_scales, w_ts)
    return _matmul_and_mag(x, w)


# -------------------------------------------------------------- acceptance --

REL_TOL = 2.0 ** -8
SUM_TOL = 1e-5


def check(c_bf16_bits, c_ref, t_ref, rel=REL_TOL, sumtol=SUM_TOL):
    """Per-element acceptance of a BF16 result against (C_ref, T):

        |C_gpu - C_ref| <= rel * |C_ref| + sumtol * T,   no NaN / Inf.

    2**-8 covers BF16 output rounding (<= 2**-9 relative) with margin; 1e-5 * T
    covers FP32 accumulation in any summation order.  Returns a dict with
    ``ok``, the number of failing elements and the worst ratio
    |err| / bound (ratio <= 1 passes)."""
    c = decode_bf16(c_bf16_bits)
    assert c.shape == np.shape(c_ref) == np.shape(t_ref)
    bound = rel * np.abs(c_ref) + sumtol * t_ref
    err = np.abs(c - c_ref)
    finite = np.isfinite(c)
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err == 0, 0.0, np.inf))
    ratio = np.where(finite, ratio, np.inf)
    bad = ~(finite & (err <= bound))
    return {"ok": bool(not bad.any()), "n_fail": int(bad.sum()),
            "n": int(c.size), "worst_ratio": float(ratio.max()) if c.size else 0.0,
            "n_nonfinite": int((~finite).sum())}
