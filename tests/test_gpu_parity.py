"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Quantizers must be bit-exact.  GEMM outputs must satisfy, element by element,
|C_gpu - C_ref| <= 2^-8 |C_ref| + 1e-5 sum_k |a_k b_k|, with no NaN.  Every
output buffer is prefilled with a NaN sentinel, so an element the kernel never
writes fails.

Inputs come from the seeded generators.  Small and mid-size cases quantize
them with the oracle and feed the oracle's bytes to the GPU GEMMs.  The
full-size workloads (16k^3 NVFP4, the 32-group ragged GEMM, the 14336 x 4096
W4A16 weight) quantize on the GPU; the oracle then independently quantizes a
sample of rows (with the tensor scale of the whole tensor).  Those rows must
match bit for bit, and the outputs that depend only on them are compared.
"""

import os

import numpy as np
import pytest
import torch

from block_scaled_precision_bsgemm_amd import lib as L
from block_scaled_precision_bsgemm_amd import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC0   # BF16 quiet NaN


def say(*a):
    print("[case]", *a, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def u16(t):
    return t.cpu().numpy().view(np.uint16)


def out_bf16(m, n):
    return torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")


def assert_ok(res, what):
    assert res["ok"], f"{what}: {res}"


# ----------------------------------------------------------- quantizers --

def _edge_matrix(k=256):
    """Rows rich in special cases for both quantizers."""
    r = np.random.Generator(np.random.PCG64(123))
    rows = []
    rows.append(np.zeros(k, np.float32))
    z = np.zeros(k, np.float32); z[1::2] = -0.0; rows.append(z)
    rows.append((r.integers(-24, 25, k) * np.float32(0.25)).astype(np.float32))      # E2M1 ties
    rows.append(np.exp2(r.uniform(-30, 30, k)).astype(np.float32) * np.sign(r.standard_normal(k)).astype(np.float32))
    rows.append((r.standard_normal(k) * 1e-3).astype(np.float32))
    t = np.zeros(k, np.float32); t[::16] = 1.0; t[1::16] = 0.25; t[2::16] = -0.75; rows.append(t)
    big = r.standard_normal(k).astype(np.float32); big[5] = 3.0e38; rows.append(big)
    tiny = np.full(k, 1e-40, np.float32); tiny[::3] = -1e-41; rows.append(tiny)
    rows.append(r.standard_normal(k).astype(np.float32))
    # E4M3 midpoints scaled into an MXFP8 block with exponent 0 (block max 448)
    mids = ((F.E4M3_TABLE[:0x7E] + F.E4M3_TABLE[1:0x7F]) / 2).astype(np.float32)
    mrow = np.resize(mids, k).astype(np.float32); mrow[::32] = 448.0; rows.append(mrow)
    return np.stack(rows).astype(np.float32)


def oracle_rows(fn, x, chunk=1024, **kw):
    """The oracle quantizer `fn` over row chunks of x on a thread pool (numpy
    releases the GIL in its array kernels).  Each quantizer is per row once
    the tensor scale is fixed (NVFP4 callers pass the whole tensor's), so the
    chunks concatenate to the whole-tensor result."""
    from concurrent.futures import ThreadPoolExecutor
    parts = [x[i:i + chunk] for i in range(0, x.shape[0], chunk)]
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        outs = list(ex.map(lambda p: fn(p, **kw), parts))
    # arrays are stacked by rows; a scalar (the NVFP4 tensor scale) is the same in every chunk
    return tuple(np.concatenate([o[j] for o in outs]) if np.ndim(outs[0][j]) else outs[0][j]
                 for j in range(len(outs[0])))


def _check_nvfp4_quant(x, what, rows=None):
    say("quantize_nvfp4", what, x.shape)
    c, s, ts = L.bsgemm_quantize_nvfp4(dev(x))
    torch.cuda.synchronize()
    st = Q.nvfp4_tensor_scale(x)
    assert ts.cpu().numpy()[0].tobytes() == np.float32(st).tobytes(), (what, ts.item(), st)
    xs = x if rows is None else x[rows]
    oc, os_, _ = Q.quantize_nvfp4(xs, tensor_scale=st)
    gc, gs = c.cpu().numpy(), s.cpu().numpy()
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    assert np.array_equal(gs, os_), f"{what}: scale bytes differ at {np.argwhere(gs != os_)[:5]}"
    assert np.array_equal(gc, oc), f"{what}: code bytes differ at {np.argwhere(gc != oc)[:5]}"
    return c, s, ts


def _check_mxfp8_quant(x, what):
    say("quantize_mxfp8", what, x.shape)
    c, s = L.bsgemm_quantize_mxfp8(dev(x))
    oc, os_ = Q.quantize_mxfp8(x)
    gc, gs = c.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(gs, os_), f"{what}: scale bytes differ at {np.argwhere(gs != os_)[:5]}"
    assert np.array_equal(gc, oc), f"{what}: code bytes differ at {np.argwhere(gc != oc)[:5]}"
    return c, s


def _check_mxfp4_quant(x, what, rows=None):
    say("quantize_mxfp4", what, x.shape)
    c, s = L.bsgemm_quantize_mxfp4(dev(x))
    xs = x if rows is None else x[rows]
    oc, os_ = Q.quantize_mxfp4(xs)
    gc, gs = c.cpu().numpy(), s.cpu().numpy()
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    assert np.array_equal(gs, os_), f"{what}: scale bytes differ at {np.argwhere(gs != os_)[:5]}"
    assert np.array_equal(gc, oc), f"{what}: code bytes differ at {np.argwhere(gc != oc)[:5]}"
    return c, s


def _mxfp4_tie_rows(k=256):
    """Blocks whose maximum is 6 (exponent 0) filled with every E2M1 midpoint
    (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) and its neighbours, both signs, and
    the same blocks scaled by 2^-3 and 2^20 (exact, so the ties stay ties)."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(7))])
    row = np.resize(np.concatenate([vals, -vals]), k).astype(np.float32)
    row[::32] = 6.0
    return np.stack([row, row * np.float32(0.125), row * np.float32(2.0 ** 20)])


def test_quantize_nvfp4_small_config(gpu_lib):
    a, b = synth.nvfp4_small_inputs()
    _check_nvfp4_quant(a, "256x128 A")
    _check_nvfp4_quant(b, "256x128 B")


def test_quantize_nvfp4_edges(gpu_lib):
    x = _edge_matrix()
    _check_nvfp4_quant(x, "edge rows")
    _check_nvfp4_quant(x[[0, 1]], "all-zero tensor")
    _check_nvfp4_quant(x[:, :32], "k = 32")
    _check_nvfp4_quant(x[[7]], "one row of FP32 subnormals")
    _check_nvfp4_quant(_edge_matrix(96), "k = 96")
    # chosen tensor scale 1.0 (amax 2688) exercises subnormal and saturated block scales
    y = (np.exp2(np.random.Generator(np.random.PCG64(9)).uniform(-14, 9, (64, 256)))).astype(np.float32)
    y[0, 0] = 2688.0
    _check_nvfp4_quant(y, "wide block-scale range")


def test_quantize_mxfp8_4k_config(gpu_lib):
    a, b = synth.mxfp8_inputs()
    _check_mxfp8_quant(a, "4096^2 A")
    _check_mxfp8_quant(b, "4096^2 B")


def test_quantize_mxfp8_edges(gpu_lib):
    x = _edge_matrix()
    _check_mxfp8_quant(x, "edge rows")
    _check_mxfp8_quant(x[:, :32], "k = 32")
    _check_mxfp8_quant(_edge_matrix(96), "k = 96")


def test_quantize_mxfp4_4k_config(gpu_lib):
    a, b, _, _ = synth.mxfp4_inputs(4096, 4096, 4096)
    _check_mxfp4_quant(a, "4096^2 A")
    _check_mxfp4_quant(b, "4096^2 B")


def test_quantize_mxfp4_edges(gpu_lib):
    x = _edge_matrix()
    _check_mxfp4_quant(x, "edge rows")
    _check_mxfp4_quant(x[:, :32], "k = 32")
    _check_mxfp4_quant(_edge_matrix(96), "k = 96")
    _check_mxfp4_quant(_mxfp4_tie_rows(), "E2M1 ties")
    # block maxima at FLT_MAX and just above 6 * 2^125 (largest exponents)
    y = np.random.Generator(np.random.PCG64(21)).standard_normal((4, 64)).astype(np.float32)
    y[0, 0] = np.finfo(np.float32).max
    y[1, 3] = np.float32(6 * 2.0 ** 125)
    y[2, 40] = np.nextafter(np.float32(6 * 2.0 ** 125), np.float32(np.inf))
    _check_mxfp4_quant(y, "largest block exponents")


def test_quantize_empty(gpu_lib):
    say("quantize empty")
    x = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    c, s, ts = L.bsgemm_quantize_nvfp4(x)
    torch.cuda.synchronize()
    assert ts.item() == 0.0
    c8, s8 = L.bsgemm_quantize_mxfp8(x)
    assert c8.numel() == 0
    c4, s4 = L.bsgemm_quantize_mxfp4(x)
    assert c4.numel() == 0


# ---------------------------------------------------------------- GEMMs --

def _quant(fmt, x):
    return {L.BSGEMM_NVFP4: Q.quantize_nvfp4, L.BSGEMM_MXFP8: Q.quantize_mxfp8,
            L.BSGEMM_MXFP8_EXACT: Q.quantize_mxfp8, L.BSGEMM_MXFP4: Q.quantize_mxfp4}[fmt](x)


def _ref(fmt, qa, qb, rows=None):
    return {L.BSGEMM_NVFP4: G.gemm_nvfp4, L.BSGEMM_MXFP8: G.gemm_mxfp8,
            L.BSGEMM_MXFP8_EXACT: G.gemm_mxfp8, L.BSGEMM_MXFP4: G.gemm_mxfp4}[fmt](*qa, *qb, rows=rows)


def _gpu_gemm(fmt, qa, qb, k):
    m, n = qa[0].shape[0], qb[0].shape[0]
    c = out_bf16(m, n)
    if fmt == L.BSGEMM_NVFP4:
        ta, tb = dev(np.array([qa[2]], np.float32)), dev(np.array([qb[2]], np.float32))
        L.bsgemm_run(fmt, dev(qa[0]), dev(qa[1]), ta, dev(qb[0]), dev(qb[1]), tb, k, c=c)
    else:
        L.bsgemm_run(fmt, dev(qa[0]), dev(qa[1]), None, dev(qb[0]), dev(qb[1]), None, k, c=c)
    return u16(c)


FMTS = {"nvfp4": L.BSGEMM_NVFP4, "mxfp8": L.BSGEMM_MXFP8, "mxfp4": L.BSGEMM_MXFP4,
        "mxfp8_exact": L.BSGEMM_MXFP8_EXACT}


def test_gemm_nvfp4_small_config(gpu_lib):
    a, b = synth.nvfp4_small_inputs()
    qa, qb = Q.quantize_nvfp4(a), Q.quantize_nvfp4(b)
    say("gemm nvfp4 256x256x128")
    c = _gpu_gemm(L.BSGEMM_NVFP4, qa, qb, 128)
    assert_ok(G.check(c, *G.gemm_nvfp4(*qa, *qb)), "nvfp4 256x256x128")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8", "mxfp4", "mxfp8_exact"])
@pytest.mark.parametrize("m,n,k", [
    (1, 1, 32), (7, 17, 64), (17, 255, 96), (256, 256, 128), (257, 300, 160),
    (300, 257, 512), (64, 520, 1024), (513, 129, 288), (1, 700, 2048),
    (260, 513, 384), (512, 512, 640),
])
def test_gemm_shapes(gpu_lib, fmt, m, n, k):
    f = FMTS[fmt]
    r = np.random.Generator(np.random.PCG64(m * 7919 + n * 31 + k))
    xa = r.standard_normal((m, k)).astype(np.float32)
    xb = r.standard_normal((n, k)).astype(np.float32)
    xa[:: max(1, m // 3)] *= np.float32(50.0)          # mixed block scales
    qa, qb = _quant(f, xa), _quant(f, xb)
    say("gemm", fmt, m, n, k)
    c = _gpu_gemm(f, qa, qb, k)
    assert_ok(G.check(c, *_ref(f, qa, qb)), f"{fmt} {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1536, 1400, 512), (1536, 1400, 640), (1300, 1600, 544), (1300, 1600, 2048),
                                   (1300, 1601, 1024)])   # n % 8 != 0: the epilogue's 2-byte stores
def test_gemm_nvfp4_large_grid_paths(gpu_lib, m, n, k):
    """Grids of at least 32 tiles of 256 x 256 (below that the small-problem
    kernel runs): the ring kernel (K % 256 == 0) and the register-staged
    kernel with K % 128 == 0 and K % 128 != 0, with ragged edges in M and N."""
    r = np.random.Generator(np.random.PCG64(m * 7919 + n * 31 + k))
    xa = r.standard_normal((m, k)).astype(np.float32)
    xb = r.standard_normal((n, k)).astype(np.float32)
    xa[:: 97] *= np.float32(50.0)                      # mixed block scales
    qa, qb = _quant(L.BSGEMM_NVFP4, xa), _quant(L.BSGEMM_NVFP4, xb)
    say("gemm nvfp4 large grid", m, n, k)
    c = _gpu_gemm(L.BSGEMM_NVFP4, qa, qb, k)
    assert_ok(G.check(c, *_ref(L.BSGEMM_NVFP4, qa, qb)), f"nvfp4 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1536, 1400, 512), (1536, 1400, 640), (1300, 1600, 544), (2048, 1024, 1024 + 512),
                                   (1536, 1402, 1024)])   # n % 8 != 0
def test_gemm_mxfp8_exact_large_grid_paths(gpu_lib, m, n, k):
    """Exact MXFP8 on grids of at least 32 tiles of 256 x 256: the ring kernel
    with 16-byte (K % 512 == 0) and 4-byte (K % 128 == 0) scale batches, and
    the register-staged 64 x 64 kernel (K % 128 != 0), with ragged M and N."""
    r = np.random.Generator(np.random.PCG64(m * 7919 + n * 31 + k + 5))
    xa = r.standard_normal((m, k)).astype(np.float32)
    xb = r.standard_normal((n, k)).astype(np.float32)
    xa[:: 97] *= np.float32(50.0)
    qa, qb = Q.quantize_mxfp8(xa), Q.quantize_mxfp8(xb)
    say("gemm mxfp8 exact large grid", m, n, k)
    c = _gpu_gemm(L.BSGEMM_MXFP8_EXACT, qa, qb, k)
    assert_ok(G.check(c, *G.gemm_mxfp8(*qa, *qb)), f"mxfp8 exact {m}x{n}x{k}")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("m,n,k", [(1300, 1500, 2048), (1536, 1402, 1024), (1300, 1600, 1536), (1536, 1400, 640)])
def test_gemm_mx_large_grid_paths(gpu_lib, fmt, m, n, k):
    """Native MXFP8 / MXFP4 on grids of 30+ tiles of 256 x 256 with ragged M
    and N (n % 8 != 0 in one case): the pair ring with 32-byte scale batches
    (K % 1024 == 0), with 16-byte batches (K % 512 == 0 only), and the
    single-step ring (K % 128 == 0)."""
    f = FMTS[fmt]
    r = np.random.Generator(np.random.PCG64(m * 7919 + n * 31 + k + 11))
    xa = r.standard_normal((m, k)).astype(np.float32)
    xb = r.standard_normal((n, k)).astype(np.float32)
    xa[:: 97] *= np.float32(50.0)                      # mixed block scales
    qa, qb = _quant(f, xa), _quant(f, xb)
    say("gemm", fmt, "large grid", m, n, k)
    c = _gpu_gemm(f, qa, qb, k)
    assert_ok(G.check(c, *_ref(f, qa, qb)), f"{fmt} {m}x{n}x{k}")


def _random_shapes(count, seed):
    """Seeded shapes that cross every dispatch boundary: K a multiple of 1024,
    512, 256, 128, 64 or only 32; M and N from single rows to grids of 40+
    tiles of 256 x 256, mostly ragged."""
    r = np.random.Generator(np.random.PCG64(seed))
    ks = [1024, 2048, 512 * 3, 256 * 5, 128 * 7, 64 * 9, 32 * 11, 32 * 37]
    out = []
    for i in range(count):
        k = ks[i % len(ks)]
        big = i % 2 == 0
        m = int(r.integers(1300, 1800)) if big else int(r.integers(1, 700))
        n = int(r.integers(1300, 1800)) if big else int(r.integers(1, 700))
        out.append((m, n, k))
    return out


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8", "mxfp4", "mxfp8_exact"])
@pytest.mark.parametrize("m,n,k", _random_shapes(16, 20261202))
def test_gemm_random_shapes(gpu_lib, fmt, m, n, k):
    """Every format on seeded random shapes against the oracle (all elements)."""
    f = FMTS[fmt]
    r = np.random.Generator(np.random.PCG64(m * 104729 + n * 131 + k))
    xa = r.standard_normal((m, k)).astype(np.float32)
    xb = r.standard_normal((n, k)).astype(np.float32)
    xa[:: 53] *= np.float32(30.0)                      # mixed block scales
    qa, qb = _quant(f, xa), _quant(f, xb)
    say("gemm random", fmt, m, n, k)
    c = _gpu_gemm(f, qa, qb, k)
    assert_ok(G.check(c, *_ref(f, qa, qb)), f"{fmt} {m}x{n}x{k}")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8", "mxfp4", "mxfp8_exact"])
def test_gemm_zero_rows_and_k0(gpu_lib, fmt):
    f = FMTS[fmt]
    xa = synth.normal_f32((40, 128), 5)
    xa[3] = 0.0                                          # an all-zero row
    xb = synth.normal_f32((50, 128), 6)
    qa, qb = _quant(f, xa), _quant(f, xb)
    say("gemm zero row", fmt)
    c = _gpu_gemm(f, qa, qb, 128)
    assert_ok(G.check(c, *_ref(f, qa, qb)), f"{fmt} zero row")
    assert np.all(F.decode_bf16(c[3]) == 0)
    say("gemm k = 0", fmt)
    e = np.zeros((40, 0), np.uint8)
    qa0 = (e, e, np.float32(1)) if f == L.BSGEMM_NVFP4 else (e, e)
    qb0 = (np.zeros((50, 0), np.uint8), np.zeros((50, 0), np.uint8), np.float32(1)) if f == L.BSGEMM_NVFP4 \
        else (np.zeros((50, 0), np.uint8), np.zeros((50, 0), np.uint8))
    c0 = _gpu_gemm(f, qa0, qb0, 0)
    assert np.all(c0 == 0)


def test_gemm_mxfp8_4k_config(gpu_lib):
    a, b = synth.mxfp8_inputs()
    qa, qb = Q.quantize_mxfp8(a), Q.quantize_mxfp8(b)
    say("gemm mxfp8 4096^3")
    c = _gpu_gemm(L.BSGEMM_MXFP8, qa, qb, 4096)
    rows = np.random.Generator(np.random.PCG64(1)).choice(4096, 512, replace=False)
    rows = np.sort(np.concatenate([rows, [0, 4095]]))
    assert_ok(G.check(c[rows], *G.gemm_mxfp8(*qa, *qb, rows=rows)), "mxfp8 4096^3 (514 rows, all columns)")


def test_gemm_mxfp4_4k_config(gpu_lib):
    a, b, ia, _ = synth.mxfp4_inputs(4096, 4096, 4096)
    qa, qb = Q.quantize_mxfp4(a), Q.quantize_mxfp4(b)
    say("gemm mxfp4 4096^3")
    c = _gpu_gemm(L.BSGEMM_MXFP4, qa, qb, 4096)
    rows = _sample(4096, 512, 2, ia)
    assert_ok(G.check(c[rows], *G.gemm_mxfp4(*qa, *qb, rows=rows)), "mxfp4 4096^3 (sampled rows, all columns)")


def test_mxfp4_16k_config_sampled(gpu_lib):
    """16384^3 MXFP4 with 1% outlier rows: GPU quantize + GEMM (the launch
    configuration the benchmark times), checked on (163 outlier + 256 random
    rows) x (163 outlier + 256 random columns)."""
    a, b, ia, ib = synth.mxfp4_inputs()
    rows = _sample(16384, 256, 13, ia)
    cols = _sample(16384, 256, 14, ib)
    ca, sa = _check_mxfp4_quant(a, "16k A (sampled rows)", rows)
    cb, sb = _check_mxfp4_quant(b, "16k B (sampled rows)", cols)
    del a, b
    say("gemm mxfp4 16384^3")
    c = out_bf16(16384, 16384)
    L.bsgemm_run(L.BSGEMM_MXFP4, ca, sa, None, cb, sb, None, 16384, c=c)
    sub = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    got = u16(sub)
    qa = (ca.cpu().numpy()[rows], sa.cpu().numpy()[rows])
    qb = (cb.cpu().numpy()[cols], sb.cpu().numpy()[cols])
    assert_ok(G.check(got, *G.gemm_mxfp4(*qa, *qb)), "mxfp4 16384^3 sampled")
    assert not torch.isnan(c.view(torch.bfloat16)).any().item()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp8_exact"])
def test_mxfp8_16k_config_sampled(gpu_lib, fmt):
    """16384^3 MXFP8 on N(0, 1) operands (the benchmark's inputs and launch
    configuration): GPU quantize + GEMM; 512 random rows (and the first and
    last) x 512 random columns against the oracle, whose own quantization of
    those rows must match the GPU's byte for byte; no unwritten element."""
    f = FMTS[fmt]
    a = synth.normal_f32((16384, 16384), synth.SEEDS["mxfp8_4k.A"])
    b = synth.normal_f32((16384, 16384), synth.SEEDS["mxfp8_4k.B"])
    rows = _sample(16384, 512, 15)
    cols = _sample(16384, 512, 16)
    qa = Q.quantize_mxfp8(a[rows])
    qb = Q.quantize_mxfp8(b[cols])
    say("quantize_mxfp8 16k A, B on the GPU")
    ca, sa = L.bsgemm_quantize_mxfp8(dev(a))
    cb, sb = L.bsgemm_quantize_mxfp8(dev(b))
    del a, b
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    assert np.array_equal(ca[ri].cpu().numpy(), qa[0]) and np.array_equal(sa[ri].cpu().numpy(), qa[1])
    assert np.array_equal(cb[ci].cpu().numpy(), qb[0]) and np.array_equal(sb[ci].cpu().numpy(), qb[1])
    say("gemm", fmt, "16384^3")
    c = out_bf16(16384, 16384)
    L.bsgemm_run(f, ca, sa, None, cb, sb, None, 16384, c=c)
    got = u16(c[ri][:, ci])
    assert not torch.isnan(c.view(torch.bfloat16)).any().item()
    del c, ca, sa, cb, sb
    assert_ok(G.check(got, *G.gemm_mxfp8(*qa, *qb)), f"{fmt} 16384^3 sampled")


def test_gemm_deterministic(gpu_lib):
    a, b = synth.nvfp4_small_inputs()
    for f in (L.BSGEMM_NVFP4, L.BSGEMM_MXFP8, L.BSGEMM_MXFP4, L.BSGEMM_MXFP8_EXACT):
        qa, qb = _quant(f, np.tile(a, (3, 4))), _quant(f, np.tile(b, (2, 4)))
        say("determinism", f)
        c1 = _gpu_gemm(f, qa, qb, 512)
        c2 = _gpu_gemm(f, qa, qb, 512)
        assert np.array_equal(c1, c2)


def _sample(n, count, seed, must=()):
    idx = np.random.Generator(np.random.PCG64(seed)).choice(n, min(count, n), replace=False)
    return np.unique(np.concatenate([idx, np.asarray(must, dtype=np.int64), [0, n - 1]]))


def test_nvfp4_16k_config_sampled(gpu_lib):
    """16384^3 NVFP4 with 1% outlier rows: GPU quantize + GEMM.  The oracle
    quantizes the 163 outlier rows and 1024 random rows of A and every row of
    B (with each tensor's own scale); those bytes must equal the GPU's, and
    the sampled rows of C are checked over all 16384 columns."""
    a, b, ia, ib = synth.nvfp4_16k_inputs()
    rows = _sample(16384, 1024, 11, ia)
    sta, stb = Q.nvfp4_tensor_scale(a), Q.nvfp4_tensor_scale(b)
    qa = Q.quantize_nvfp4(a[rows], tensor_scale=sta)
    say("oracle quantize of B (16384 rows)")
    qb = oracle_rows(Q.quantize_nvfp4, b, tensor_scale=stb)
    say("quantize_nvfp4 16k A, B on the GPU")
    ca, sa, ta = L.bsgemm_quantize_nvfp4(dev(a))
    cb, sb, tb = L.bsgemm_quantize_nvfp4(dev(b))
    del a, b
    ri = torch.from_numpy(rows).cuda()
    assert ta.cpu().numpy().tobytes() == np.float32(sta).tobytes()
    assert tb.cpu().numpy().tobytes() == np.float32(stb).tobytes()
    assert np.array_equal(ca[ri].cpu().numpy(), qa[0]) and np.array_equal(sa[ri].cpu().numpy(), qa[1])
    assert np.array_equal(cb.cpu().numpy(), qb[0]) and np.array_equal(sb.cpu().numpy(), qb[1])
    say("gemm nvfp4 16384^3")
    c = out_bf16(16384, 16384)
    L.bsgemm_run(L.BSGEMM_NVFP4, ca, sa, ta, cb, sb, tb, 16384, c=c)
    got = u16(c[ri])
    # nothing unwritten anywhere: the sentinel is a NaN
    assert not torch.isnan(c.view(torch.bfloat16)).any().item()
    del c, ca, sa, cb, sb
    say(f"oracle: {len(rows)} rows x 16384 columns")
    assert_ok(G.check(got, *G.gemm_nvfp4(*qa, *qb)), "nvfp4 16384^3 sampled rows, all columns")


@pytest.mark.parametrize("size", [65536, 131072])
def test_nvfp4_big_square_sampled(gpu_lib, size):
    """64k^3 and 128k^3 NVFP4 GEMMs on operands drawn as NVFP4 on the device;
    256 sampled rows x 256 sampled columns (plus the first and last of each)
    against the oracle, and no unwritten element anywhere."""
    dev0 = torch.device("cuda:0")
    qa = synth.nvfp4_random_operand(size, size, synth.SEEDS["nvfp4_big.A"], dev0)
    qb = synth.nvfp4_random_operand(size, size, synth.SEEDS["nvfp4_big.B"], dev0)
    say("gemm nvfp4", f"{size}^3")
    c = out_bf16(size, size)
    L.bsgemm_run(L.BSGEMM_NVFP4, *qa, *qb, size, c=c)
    rows = _sample(size, 256, 31)
    cols = _sample(size, 256, 32)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    got = u16(c[ri][:, ci])
    nan_free = not torch.isnan(c.view(torch.bfloat16)).any().item()
    ha = (qa[0][ri].cpu().numpy(), qa[1][ri].cpu().numpy(), np.float32(1))
    hb = (qb[0][ci].cpu().numpy(), qb[1][ci].cpu().numpy(), np.float32(1))
    del qa, qb, c
    torch.cuda.empty_cache()
    assert nan_free
    assert_ok(G.check(got, *G.gemm_nvfp4(*ha, *hb)), f"nvfp4 {size}^3 sampled")


# -------------------------------------------------------------- grouped --

def _grouped_case(counts, n, k, seed):
    off = synth.offsets_from_counts(np.asarray(counts))
    m = int(off[-1])
    x = synth.normal_f32((m, k), seed)
    qa = Q.quantize_nvfp4(x) if m else (np.zeros((0, k // 2), np.uint8), np.zeros((0, k // 16), np.uint8), np.float32(0))
    w = synth.bf16_bits(synth.normal_f32((len(counts), n, k), seed + 1, std=0.02))
    return qa, off, w


def _gpu_grouped(qa, off, w, k):
    m, n = qa[0].shape[0], w.shape[1]
    c = out_bf16(m, n)
    L.bsgemm_grouped_run(dev(qa[0]), dev(qa[1]), dev(np.array([qa[2]], np.float32)), dev(off),
                         dev(w), k, c=c)
    return u16(c)


@pytest.mark.parametrize("counts,n,k", [
    ([5], 64, 64),
    ([0, 3, 0, 0, 300, 1, 0], 96, 128),
    ([257, 0, 256, 255], 260, 96),
    ([1] * 40, 33, 32),
    ([600, 0, 0, 900], 512, 256),
    ([77, 256], 260, 320),                 # odd number of 64-element K steps
    ([512, 256, 0, 300], 512, 1280),       # whole 256-row tiles; 16-byte scale batches
    ([300, 0, 257], 258, 256),             # n % 4 != 0: 2-byte stores on the ping-pong path
    ([77, 256], 262, 320),                 # n % 4 != 0 on the 4-byte-scale ring
])
def test_grouped_shapes(gpu_lib, counts, n, k):
    qa, off, w = _grouped_case(counts, n, k, sum(counts) + n + k)
    say("grouped", counts, n, k)
    c = _gpu_grouped(qa, off, w, k)
    assert_ok(G.check(c, *G.grouped_nvfp4_bf16(*qa, off, w)), f"grouped {counts} n={n} k={k}")


def _random_grouped(count, seed):
    """Seeded grouped problems: 1-20 groups with empty ones, ragged N, and K
    on each kernel path (K % 256 == 0 ping-pong, K % 64 == 0 ring, K % 32 ==
    0 register-staged)."""
    r = np.random.Generator(np.random.PCG64(seed))
    ks = [256 * 3, 64 * 5, 32 * 7, 1024, 64 * 13, 32 * 33]
    out = []
    for i in range(count):
        g = int(r.integers(1, 21))
        counts = [int(c) if r.random() > 0.2 else 0 for c in r.integers(0, 700, g)]
        n = int(r.integers(1, 1200))
        out.append((counts, n, ks[i % len(ks)]))
    return out


@pytest.mark.parametrize("counts,n,k", _random_grouped(12, 20261203))
def test_grouped_random(gpu_lib, counts, n, k):
    """The grouped GEMM on seeded random group mixes against the oracle (every element)."""
    qa, off, w = _grouped_case(counts, n, k, sum(counts) * 7 + n + k)
    say("grouped random", len(counts), sum(counts), n, k)
    c = _gpu_grouped(qa, off, w, k)
    assert_ok(G.check(c, *G.grouped_nvfp4_bf16(*qa, off, w)), f"grouped random {counts} n={n} k={k}")


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
def test_grouped_tile_sizes(gpu_lib, w_dtype):
    """Group sizes around the ping-pong kernel's two tile sizes: remainders of
    0, 1, 127, 128 (one 128-row tile), 129, 255 (one more 256-row tile), with
    every routing and epilogue variant and without."""
    counts = [0, 1, 127, 128, 129, 255, 256, 257, 383, 384, 385, 640, 0, 513]
    n, k = 260, 512
    m = sum(counts)
    qa, off, w, v = _variant_case(counts, n, k, 900, w_dtype, a_rows=m)
    for use in ((), ALL):
        say("grouped tile sizes", w_dtype, use)
        c = _gpu_grouped_ex(qa, off, w, k, w_dtype, v, use, m)
        assert_ok(G.check(c, *_ref_ex(qa, off, w, w_dtype, v, use)), f"grouped tile sizes {w_dtype} {use}")
        assert not np.any(c == SENTINEL)


def test_grouped_config_sampled(gpu_lib):
    """32 groups, Dirichlet(0.5) counts over 16384 rows, K=7168, N=2048.
    GPU quantize + grouped GEMM; sampled rows: first/last row of every
    non-empty group plus 384 random rows, all 2048 columns."""
    x, off, w = synth.grouped_inputs()
    counts = np.diff(off.astype(np.int64))
    must = [r for g in range(32) if counts[g] for r in (off[g], off[g + 1] - 1)]
    rows = _sample(16384, 384, 21, must)
    ca, sa, ta = _check_nvfp4_quant(x, "grouped A (sampled rows)", rows)
    del x
    say("grouped 32 x (2048 x 7168), m=16384")
    c = out_bf16(16384, 2048)
    L.bsgemm_grouped_run(ca, sa, ta, dev(off), dev(w), 7168, c=c)
    got = u16(c)
    qa = (ca.cpu().numpy(), sa.cpu().numpy(), np.float32(ta.item()))
    assert_ok(G.check(got[rows], *G.grouped_nvfp4_bf16(*qa, off, w, rows=rows)), "grouped config sampled")
    assert not np.any(got == SENTINEL)


@pytest.mark.parametrize("k", [512, 320, 96])   # ping-pong, 4-byte-scale ring, register-staged
def test_grouped_malformed_offsets_stay_in_bounds(gpu_lib, k):
    """Group offsets are a documented precondition (non-decreasing, off[0] =
    0, off[G] = m_total).  The kernels clamp them, so malformed offsets
    (decreasing, negative, past m_total) still touch only A and C: the call
    succeeds and guard rows on both sides of C keep their sentinel."""
    m, n, guard = 800, 136, 8                        # 272-byte rows: the view stays 16-byte aligned
    qa, _, w = _grouped_case([160] * 5, n, k, 4242 + k)
    for off in ([0, 300, 100, 700, 650, 2000], [0, -50, 900, 400, 400, 800], [5, 5, 5, 5, 5, 5]):
        say("grouped malformed offsets", k, off)
        big = torch.full((m + 2 * guard, n), SENTINEL, dtype=torch.int16, device="cuda")
        c = big[guard:guard + m]
        L.bsgemm_grouped_run(dev(qa[0]), dev(qa[1]), dev(np.array([qa[2]], np.float32)),
                             dev(np.array(off, np.int32)), dev(w), k, c=c)
        torch.cuda.synchronize()
        g = u16(big)
        assert np.all(g[:guard] == SENTINEL) and np.all(g[guard + m:] == SENTINEL)


def test_grouped_kragged_malformed_offsets_stay_in_bounds(gpu_lib):
    """The K-ragged offsets are clamped to [0, K] and rounded down to 256:
    malformed ones (decreasing, negative, past K) still touch only A, W and
    C; guard groups on both sides of C keep their sentinel."""
    qa, _, w, k = _kragged_case([300, 200, 256], 300, 260, 77, "bf16")   # k = 1024
    for off in ([0, 512, 256, 2048], [-300, 1000, 9999, 512], [0, 0, 0, 0]):
        say("grouped K-ragged malformed offsets", off)
        big = torch.full((5, 300, 260), SENTINEL, dtype=torch.int16, device="cuda")
        c = big[1:4]
        L.bsgemm_grouped_kragged_run(dev(qa[0]), dev(qa[1]), dev(np.array([qa[2]], np.float32)),
                                     dev(np.array(off, np.int32)), dev(w), k, c=c)
        torch.cuda.synchronize()
        g = u16(big)
        assert np.all(g[0] == SENTINEL) and np.all(g[4] == SENTINEL)


# ------------------------------------------- grouped: routing / epilogue --

def _variant_case(counts, n, k, seed, w_dtype, a_rows=None):
    """Grouped inputs with every variant: gather from a_rows rows of A (with
    repeats), a scatter permutation, bias [G, n] and gamma [m]."""
    r = np.random.Generator(np.random.PCG64(seed))
    off = synth.offsets_from_counts(np.asarray(counts))
    m = int(off[-1])
    a_rows = m if a_rows is None else a_rows
    x = synth.normal_f32((a_rows, k), seed + 1)
    qa = Q.quantize_nvfp4(x)
    wf = synth.normal_f32((len(counts), n, k), seed + 2, std=0.02)
    w = synth.bf16_bits(wf) if w_dtype == "bf16" else wf.astype(np.float16).view(np.uint16)
    v = {"gather": r.integers(0, a_rows, m).astype(np.int32),
         "scatter": r.permutation(m).astype(np.int32),
         "bias": (r.standard_normal((len(counts), n)) * 0.1).astype(np.float32),
         "gamma": r.uniform(-2, 2, m).astype(np.float32)}
    return qa, off, w, v


def _gpu_grouped_ex(qa, off, w, k, w_dtype, v, use, m):
    c = out_bf16(m, w.shape[1])
    opt = {key: (dev(v[key]) if key in use else None) for key in ("bias", "gamma", "gather", "scatter")}
    L.bsgemm_grouped_run_ex(dev(qa[0]), dev(qa[1]), dev(np.array([qa[2]], np.float32)), dev(off), dev(w), k,
                            w_dtype=L.BSGEMM_W_F16 if w_dtype == "f16" else L.BSGEMM_W_BF16,
                            bias=opt["bias"], gamma=opt["gamma"], gather_idx=opt["gather"],
                            scatter_idx=opt["scatter"], m_total=m, c=c)
    return u16(c)


def _ref_ex(qa, off, w, w_dtype, v, use, rows=None):
    return G.grouped_nvfp4_ex(*qa, off, w, w_dtype, *(v[key] if key in use else None
                                                      for key in ("bias", "gamma", "gather", "scatter")),
                              out_rows=rows)


ALL = ("bias", "gamma", "gather", "scatter")


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("k,n", [(96, 260), (320, 260), (512, 260), (512, 254)])
def test_grouped_ex_all_variants(gpu_lib, w_dtype, k, n):
    """bias + gamma + gather (from fewer A rows than m, with repeats) + scatter,
    on the register-staged (K = 96), 4-byte-scale ring (K % 64) and
    ping-pong (K % 256) kernels, BF16 and FP16 weights; n = 254 takes the
    2-byte stores of the scattered epilogue."""
    counts = [77, 256, 0, 300]
    m = sum(counts)
    qa, off, w, v = _variant_case(counts, n, k, 700 + k, w_dtype, a_rows=500)
    say("grouped_ex all variants", w_dtype, counts, n, k)
    c = _gpu_grouped_ex(qa, off, w, k, w_dtype, v, ALL, m)
    assert_ok(G.check(c, *_ref_ex(qa, off, w, w_dtype, v, ALL)), f"grouped_ex {w_dtype} k={k} n={n}")
    assert not np.any(c == SENTINEL)


@pytest.mark.parametrize("use", [(), ("bias",), ("gamma",), ("gather",), ("scatter",), ("bias", "scatter")])
@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
def test_grouped_ex_single_variants(gpu_lib, use, w_dtype):
    counts, n, k = [300, 0, 5, 256], 136, 256
    m = sum(counts)
    qa, off, w, v = _variant_case(counts, n, k, 800 + len(use), w_dtype)
    say("grouped_ex", w_dtype, use)
    c = _gpu_grouped_ex(qa, off, w, k, w_dtype, v, use, m)
    assert_ok(G.check(c, *_ref_ex(qa, off, w, w_dtype, v, use)), f"grouped_ex {w_dtype} {use}")


def test_grouped_ex_plain_equals_grouped_run(gpu_lib):
    qa, off, w = _grouped_case([600, 0, 0, 900], 512, 256, 31)
    m = int(off[-1])
    say("grouped_ex plain vs grouped_run")
    c1 = _gpu_grouped(qa, off, w, 256)
    c2 = _gpu_grouped_ex(qa, off, w, 256, "bf16", {}, (), m)
    assert np.array_equal(c1, c2)


def test_grouped_ex_out_of_range_indices(gpu_lib):
    """A gather entry outside [0, a_rows) reads a zero row; a scatter entry
    outside [0, m) skips its store (that physical row keeps its old value)."""
    counts, n, k = [100, 60], 64, 128
    m = sum(counts)
    qa, off, w, v = _variant_case(counts, n, k, 901, "bf16", a_rows=90)
    v["gather"][7] = 90            # == a_rows: out of range
    v["gather"][130] = -3
    lost = int(v["scatter"][11])
    v["scatter"][11] = m + 5       # physical row `lost` is then never written
    say("grouped_ex out-of-range indices")
    c = _gpu_grouped_ex(qa, off, w, k, "bf16", v, ALL, m)
    # reference: the bad gather entries read an appended all-zero row of A
    za = (np.concatenate([qa[0], np.zeros((1, k // 2), np.uint8)]),
          np.concatenate([qa[1], np.zeros((1, k // 16), np.uint8)]), qa[2])
    g2 = v["gather"].copy()
    g2[[7, 130]] = 90
    s2 = v["scatter"].copy()
    s2[11] = lost
    cref, t = G.grouped_nvfp4_ex(*za, off, w, "bf16", v["bias"], v["gamma"], g2, s2)
    keep = np.arange(m) != lost
    assert_ok(G.check(c[keep], cref[keep], t[keep]), "grouped_ex out-of-range indices")
    assert np.all(c[lost] == SENTINEL)


def test_grouped_ex_config_sampled(gpu_lib):
    """The 32-group config (m = 16384, K = 7168, N = 2048) with FP16 weights and
    every variant (gather over all 16384 rows, random permutation scatter,
    bias, gamma); sampled physical rows, all columns."""
    x, off, w_bf = synth.grouped_inputs()
    del w_bf
    r = np.random.Generator(np.random.PCG64(4100))
    m, n, k, G_ = 16384, 2048, 7168, 32
    w = synth.normal_f32((G_, n, k), synth.SEEDS["grouped.W"], std=0.02).astype(np.float16).view(np.uint16)
    v = {"gather": r.integers(0, m, m).astype(np.int32), "scatter": r.permutation(m).astype(np.int32),
         "bias": (r.standard_normal((G_, n)) * 0.1).astype(np.float32),
         "gamma": r.uniform(-2, 2, m).astype(np.float32)}
    ca, sa, ta = L.bsgemm_quantize_nvfp4(dev(x))
    del x
    say("grouped_ex 32 x (2048 x 7168) f16, all variants")
    c = out_bf16(m, n)
    L.bsgemm_grouped_run_ex(ca, sa, ta, dev(off), dev(w), k, w_dtype=L.BSGEMM_W_F16, bias=dev(v["bias"]),
                            gamma=dev(v["gamma"]), gather_idx=dev(v["gather"]), scatter_idx=dev(v["scatter"]),
                            c=c)
    got = u16(c)
    rows = _sample(m, 384, 22)
    qa = (ca.cpu().numpy(), sa.cpu().numpy(), np.float32(ta.item()))
    assert_ok(G.check(got[rows], *_ref_ex(qa, off, w, "f16", v, ALL, rows=rows)), "grouped_ex config sampled")
    assert not np.any(got == SENTINEL)


# ------------------------------------------------ grouped: K-ragged mode --

def _kragged_case(counts, m, n, seed, w_dtype):
    """Groups split K: group g has counts[g] real K elements, padded with
    zeros to a multiple of 256 in A (before quantization) and in W."""
    pad = [-(-c // 256) * 256 for c in counts]
    off = np.concatenate([[0], np.cumsum(pad)]).astype(np.int32)
    k = int(off[-1])
    x = np.zeros((m, k), np.float32)
    wf = np.zeros((n, k), np.float32)
    r = np.random.Generator(np.random.PCG64(seed))
    for g, c in enumerate(counts):
        x[:, off[g]:off[g] + c] = r.standard_normal((m, c), dtype=np.float32)
        wf[:, off[g]:off[g] + c] = r.standard_normal((n, c), dtype=np.float32) * np.float32(0.02)
    qa = Q.quantize_nvfp4(x)
    w = synth.bf16_bits(wf) if w_dtype == "bf16" else wf.astype(np.float16).view(np.uint16)
    return qa, off, w, k


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("counts,m,n", [
    ([256], 256, 256),
    ([100, 0, 700, 256], 300, 260),        # an empty group, ragged m and n tails
    ([1, 255, 257, 1024], 64, 520),
    ([100, 300], 270, 258),                # n % 4 != 0: 2-byte stores
])
def test_grouped_kragged_shapes(gpu_lib, w_dtype, counts, m, n):
    qa, off, w, k = _kragged_case(counts, m, n, sum(counts) + m, w_dtype)
    say("grouped K-ragged", w_dtype, counts, m, n, k)
    c = torch.full((len(counts), m, n), SENTINEL, dtype=torch.int16, device="cuda")
    L.bsgemm_grouped_kragged_run(dev(qa[0]), dev(qa[1]), dev(np.array([qa[2]], np.float32)), dev(off), dev(w), k,
                                 w_dtype=L.BSGEMM_W_F16 if w_dtype == "f16" else L.BSGEMM_W_BF16, c=c)
    got = u16(c)
    cref, t = G.grouped_kragged(*qa, off, w, w_dtype)
    for g in range(len(counts)):
        assert_ok(G.check(got[g], cref[g], t[g]), f"K-ragged group {g} of {counts} {w_dtype}")


def _random_kragged(count, seed):
    """Seeded K-ragged problems: 1-12 experts with empty ones, ragged M and N."""
    r = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(count):
        g = int(r.integers(1, 13))
        counts = [int(c) if r.random() > 0.2 else 0 for c in r.integers(0, 900, g)]
        out.append((counts, int(r.integers(1, 800)), int(r.integers(1, 700)), "bf16" if i % 2 == 0 else "f16"))
    return out


@pytest.mark.parametrize("counts,m,n,w_dtype", _random_kragged(8, 20261204))
def test_grouped_kragged_random(gpu_lib, counts, m, n, w_dtype):
    """The K-ragged mode on seeded random expert mixes, every group against the oracle."""
    qa, off, w, k = _kragged_case(counts, m, n, sum(counts) * 3 + m + n, w_dtype)
    say("grouped K-ragged random", w_dtype, len(counts), m, n, k)
    c = torch.full((len(counts), m, n), SENTINEL, dtype=torch.int16, device="cuda")
    L.bsgemm_grouped_kragged_run(dev(qa[0]), dev(qa[1]), dev(np.array([qa[2]], np.float32)), dev(off), dev(w), k,
                                 w_dtype=L.BSGEMM_W_F16 if w_dtype == "f16" else L.BSGEMM_W_BF16, c=c)
    got = u16(c)
    cref, t = G.grouped_kragged(*qa, off, w, w_dtype)
    for g in range(len(counts)):
        assert_ok(G.check(got[g], cref[g], t[g]), f"K-ragged random group {g} of {counts} {w_dtype}")


def test_grouped_kragged_config_sampled(gpu_lib):
    """Weight-gradient shape of the grouped config: 32 experts' token counts
    (the Dirichlet draw over 16384 tokens) split K, each padded to 256;
    A = 7168 x K NVFP4, W = 2048 x K BF16, C = 32 x 7168 x 2048; sampled
    (group, row) pairs, all columns."""
    counts = synth.group_counts(32, 16384, 0.5, synth.SEEDS["grouped.counts"])
    m, n = 7168, 2048
    pad = [-(-int(c) // 256) * 256 for c in counts]
    off = np.concatenate([[0], np.cumsum(pad)]).astype(np.int32)
    k = int(off[-1])
    x = synth.normal_f32((m, k), 4301)
    wf = synth.normal_f32((n, k), 4302, std=0.02)
    for g, c in enumerate(counts):   # zero padding in both operands
        x[:, off[g] + int(c):off[g + 1]] = 0
        wf[:, off[g] + int(c):off[g + 1]] = 0
    w = synth.bf16_bits(wf)
    del wf
    rows = _sample(m, 24, 41)
    ca, sa, ta = _check_nvfp4_quant(x, "K-ragged A (sampled rows)", rows)
    del x
    say("grouped K-ragged 32 x (7168 x 2048), k =", k)
    c = out_bf16(32 * m, n).view(32, m, n)
    L.bsgemm_grouped_kragged_run(ca, sa, ta, dev(off), dev(w), k, c=c)
    assert not torch.isnan(c.view(torch.bfloat16)).any().item()
    got = u16(c[:, torch.from_numpy(rows).cuda()])
    qa = (ca.cpu().numpy()[rows], sa.cpu().numpy()[rows], np.float32(ta.item()))
    cref, t = G.grouped_kragged(*qa, off, w, "bf16")
    for g in range(32):
        assert_ok(G.check(got[g], cref[g], t[g]), f"K-ragged config group {g}")


# ---------------------------------------------------------------- W4A16 --

def _gpu_w4a16(x, qw, m):
    c = out_bf16(m, qw[0].shape[0])
    L.bsgemm_w4a16_run(dev(x), dev(qw[0]), dev(qw[1]), dev(np.array([qw[2]], np.float32)), c=c)
    return u16(c)


@pytest.mark.parametrize("m,n,k", [
    (1, 1, 32), (1, 33, 96), (1, 100, 4096), (1, 64, 8192 + 32), (2, 50, 64), (3, 16, 128),
    (16, 130, 256), (17, 64, 512), (64, 96, 4096), (65, 40, 160), (100, 33, 96), (256, 64, 1024),
    (5, 300, 1024), (16, 48, 8192 + 96), (32, 40, 4096 + 256), (33, 70, 2048 + 512),
])
def test_w4a16_shapes(gpu_lib, m, n, k):
    x = synth.bf16_bits(synth.normal_f32((m, k), m + n + k))
    qw = Q.quantize_nvfp4(synth.normal_f32((n, k), m * n + k, std=0.02))
    say("w4a16", m, n, k)
    c = _gpu_w4a16(x, qw, m)
    assert_ok(G.check(c, *G.w4a16(x, *qw)), f"w4a16 {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 16, 64, 256])
def test_w4a16_config_sampled(gpu_lib, m):
    """W 14336 x 4096 quantized on the GPU; all m rows x 1024 sampled columns."""
    x, wf = synth.w4a16_inputs(m)
    cols = _sample(14336, 1024, 31 + m)
    cw, sw, tw = _check_nvfp4_quant(wf, f"w4a16 W (sampled rows), m={m}", cols)
    say("w4a16 config m =", m)
    c = out_bf16(m, 14336)
    L.bsgemm_w4a16_run(dev(x), cw, sw, tw, c=c)
    got = u16(c)
    qw = (cw.cpu().numpy()[cols], sw.cpu().numpy()[cols], np.float32(tw.item()))
    assert_ok(G.check(got[:, cols], *G.w4a16(x, *qw)), f"w4a16 m={m} sampled")
    assert not np.any(got == SENTINEL)


@pytest.mark.parametrize("m,n,k,expect", [
    (128, 2048, 6144, "tile_m16_n64"),     # 16-row m tiles fit one wave
    (48, 2560, 5120, "tile_m16_n64"),
    (128, 6144, 4096, "tile_m64_n64"),     # 64-row m tiles fit one wave, n >= 6144
    (130, 7000, 1536, "tile_m64_n64"),     # ragged m and n
    (256, 8192, 2048, "tile_m64_n64"),     # past one wave, 64 x 64 tiles in fewer rounds
    (256, 10240, 2560, "tile_m128_n128"),  # past one wave, 128 x 128 tiles in fewer rounds
    (300, 9000, 1024, "tile_m128_n128"),
    (200, 6144, 4224, "mfma_m64_n64_t2"),  # K % 256 != 0: no tile kernel
])
def test_w4a16_selector_branches(gpu_lib, m, n, k, expect):
    """bsgemm_w4a16_run at shapes where the selector takes each of its
    tile-kernel branches (and one it must not): W quantized on the GPU, all
    m rows x 512 sampled columns against the oracle, no unwritten output."""
    assert L.w4a16_configs()[L.load().bsgemm_w4a16_select(m, n, k)] == expect
    x = synth.bf16_bits(synth.normal_f32((m, k), m + n + k))
    wf = synth.normal_f32((n, k), m * k + n, std=0.02)
    cols = _sample(n, 512, n + k)
    cw, sw, tw = _check_nvfp4_quant(wf, f"w4a16 W {n}x{k} (sampled rows)", cols)
    del wf
    say("w4a16 selector", expect, m, n, k)
    c = out_bf16(m, n)
    L.bsgemm_w4a16_run(dev(x), cw, sw, tw, c=c)
    got = u16(c)
    qw = (cw.cpu().numpy()[cols], sw.cpu().numpy()[cols], np.float32(tw.item()))
    assert_ok(G.check(got[:, cols], *G.w4a16(x, *qw)), f"w4a16 selector {expect} {m}x{n}x{k}")
    assert not np.any(got == SENTINEL)


def _w4_case(m, n, k, seed):
    x = synth.bf16_bits(synth.normal_f32((m, k), seed))
    qw = Q.quantize_nvfp4(synth.normal_f32((n, k), seed + 1, std=0.02))
    return x, qw


@pytest.mark.parametrize("config", range(34))
def test_w4a16_every_config(gpu_lib, config):
    """Each configuration, forced, on shapes it would never be chosen for:
    ragged m, n and K tails (K % 256 != 0 uses per-lane scale loads), and a
    K long enough to wrap the deepest W register ring (8 stages of 1024).
    The tile configurations need K % 512, 256 or 128 == 0 (their K per ring
    stage) and must refuse other K."""
    name = L.w4a16_configs()[config]
    for (m, n, k) in [(1, 300, 1024), (5, 72, 2048 + 96), (33, 129, 512), (70, 260, 4096 + 256),
                      (9, 40, 9216 + 32), (130, 258, 2048), (200, 131, 768), (17, 70, 1536 + 512)]:
        x, qw = _w4_case(m, n, k, 1000 * config + m)
        say("w4a16 forced", name, m, n, k)
        c = out_bf16(m, n)
        args = (config, dev(x.view(np.int16)), dev(qw[0]), dev(qw[1]), dev(np.array([qw[2]], np.float32)))
        if name.startswith("tile") and k % {"tile_m16_n64": 512, "tile_m64_n64": 256, "tile_m128_n128": 128}[name]:
            with pytest.raises(L.BsgemmError, match="UNSUPPORTED"):
                L.bsgemm_w4a16_run_config(*args, c=c)
            continue
        L.bsgemm_w4a16_run_config(*args, c=c)
        assert_ok(G.check(u16(c), *G.w4a16(x, *qw)), f"w4a16 {name} {m}x{n}x{k}")
        assert not np.any(u16(c) == SENTINEL)


def test_w4a16_environment_override(gpu_lib, monkeypatch):
    x, qw = _w4_case(3, 200, 1024, 77)
    args = (dev(x.view(np.int16)), dev(qw[0]), dev(qw[1]), dev(np.array([qw[2]], np.float32)))
    say("w4a16 environment override")
    forced = u16(L.bsgemm_w4a16_run_config("mfma_m64_n16", *args))
    monkeypatch.setenv("BSGEMM_W4A16_FORCE_CONFIG", "mfma_m64_n16")
    via_env = u16(L.bsgemm_w4a16_run(*args))
    monkeypatch.delenv("BSGEMM_W4A16_FORCE_CONFIG")
    auto = u16(L.bsgemm_w4a16_run(*args))
    assert np.array_equal(forced, via_env)
    assert_ok(G.check(auto, *G.w4a16(x, *qw)), "w4a16 selector")


# ------------------------------------------------- all codes, all scales --

@pytest.mark.parametrize("m,n,k", [(300, 260, 128), (300, 260, 256), (300, 260, 512), (300, 260, 1024),
                                   (300, 260, 2048 + 256), (1600, 1400, 256 + 128), (1600, 1400, 1024)])
def test_gemm_nvfp4_every_scale_code(gpu_lib, m, n, k):
    """Random E2M1 codes with E4M3 scale codes drawn uniformly from all 127
    finite non-negative codes (zero and subnormals included): 300 x 260 runs
    the small-problem kernel; 1600 x 1400 (42 tiles of 256 x 256) the
    register-staged (K % 256 != 0) and ring (K % 256 == 0) kernels."""
    r = np.random.Generator(np.random.PCG64(k + m))
    qa = (r.integers(0, 256, (m, k // 2)).astype(np.uint8),
          r.integers(0, 0x7F, (m, k // 16)).astype(np.uint8), np.float32(0.75))
    qb = (r.integers(0, 256, (n, k // 2)).astype(np.uint8),
          r.integers(0, 0x7F, (n, k // 16)).astype(np.uint8), np.float32(1.5))
    say("gemm nvfp4 every scale code, k =", k)
    c = _gpu_gemm(L.BSGEMM_NVFP4, qa, qb, k)
    assert_ok(G.check(c, *G.gemm_nvfp4(*qa, *qb)), f"nvfp4 every scale code k={k}")



# The block scale is a signed E4M3 value (the format's sign bit is part of
# e4m3(scale)); the quantizer only writes non-negative scales, so these cases
# set sign bits at random on its output.

def _signed(scales, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    return scales | (r.integers(0, 2, scales.shape).astype(np.uint8) << 7)


@pytest.mark.parametrize("m,n,k", [(300, 260, 256), (1600, 1400, 256 + 128), (1600, 1400, 1024)])
def test_gemm_nvfp4_signed_scale_codes(gpu_lib, m, n, k):
    """All 254 finite E4M3 scale codes, both signs: the small-problem,
    register-staged and ring kernels."""
    r = np.random.Generator(np.random.PCG64(7 * k + m))
    def scales(rows):
        c = r.integers(0, 254, (rows, k // 16))
        return (c + (c >= 0x7F)).astype(np.uint8)          # skip the NaN code 0x7F (and 0xFF)
    qa = (r.integers(0, 256, (m, k // 2)).astype(np.uint8), scales(m), np.float32(0.75))
    qb = (r.integers(0, 256, (n, k // 2)).astype(np.uint8), scales(n), np.float32(-1.5))
    say("gemm nvfp4 signed scale codes", m, n, k)
    c = _gpu_gemm(L.BSGEMM_NVFP4, qa, qb, k)
    assert_ok(G.check(c, *G.gemm_nvfp4(*qa, *qb)), f"nvfp4 signed scale codes {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(300, 260, 256), (1600, 1400, 256 + 128), (1600, 1400, 1024)])
def test_gemm_nvfp4_nan_scale_code(gpu_lib, m, n, k):
    """A NaN scale code (0x7F in A row 5, 0xFF in B row 7) makes every output
    its block feeds NaN, as the format defines; the rest is unaffected."""
    qa = Q.quantize_nvfp4(synth.normal_f32((m, k), m + k))
    qb = Q.quantize_nvfp4(synth.normal_f32((n, k), n + k + 1))
    qa = (qa[0], qa[1].copy(), qa[2])
    qb = (qb[0], qb[1].copy(), qb[2])
    qa[1][5, 0] = 0x7F
    qb[1][7, k // 16 - 1] = 0xFF
    say("gemm nvfp4 NaN scale code", m, n, k)
    c = _gpu_gemm(L.BSGEMM_NVFP4, qa, qb, k)
    nan = ((c & 0x7F80) == 0x7F80) & ((c & 0x7F) != 0)
    assert nan[5, :].all() and nan[:, 7].all()
    keep_r = np.setdiff1d(np.arange(m), [5])
    keep_c = np.setdiff1d(np.arange(n), [7])
    assert not nan[np.ix_(keep_r, keep_c)].any()
    cref, tref = G.gemm_nvfp4(*qa, *qb)
    assert_ok(G.check(c[np.ix_(keep_r, keep_c)], cref[np.ix_(keep_r, keep_c)], tref[np.ix_(keep_r, keep_c)]),
              f"nvfp4 NaN scale {m}x{n}x{k}")


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("counts,n,k", [([257, 0, 256, 255], 260, 96), ([77, 256], 260, 320),
                                        ([512, 256, 0, 300], 512, 1280)])
def test_grouped_signed_scale_codes(gpu_lib, w_dtype, counts, n, k):
    qa, off, w, v = _variant_case(counts, n, k, sum(counts) + k, w_dtype)
    qa = (qa[0], _signed(qa[1], k), qa[2])
    m = int(off[-1])
    say("grouped signed scale codes", w_dtype, counts, n, k)
    c = _gpu_grouped_ex(qa, off, w, k, w_dtype, v, (), m)
    assert_ok(G.check(c, *_ref_ex(qa, off, w, w_dtype, v, ())), f"grouped signed scales {counts} {w_dtype}")


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
def test_grouped_kragged_signed_scale_codes(gpu_lib, w_dtype):
    counts, m, n = [100, 0, 700, 256], 300, 260
    qa, off, w, k = _kragged_case(counts, m, n, 4242, w_dtype)
    qa = (qa[0], _signed(qa[1], 4243), qa[2])
    say("grouped K-ragged signed scale codes", w_dtype)
    c = torch.full((len(counts), m, n), SENTINEL, dtype=torch.int16, device="cuda")
    L.bsgemm_grouped_kragged_run(dev(qa[0]), dev(qa[1]), dev(np.array([qa[2]], np.float32)), dev(off), dev(w), k,
                                 w_dtype=L.BSGEMM_W_F16 if w_dtype == "f16" else L.BSGEMM_W_BF16, c=c)
    got = u16(c)
    cref, t = G.grouped_kragged(*qa, off, w, w_dtype)
    for g in range(len(counts)):
        assert_ok(G.check(got[g], cref[g], t[g]), f"K-ragged signed scales group {g} {w_dtype}")


def test_w4a16_signed_scale_codes(gpu_lib):
    """Every W4A16 configuration, forced, with signed weight scales."""
    for config, name in enumerate(L.w4a16_configs()):
        for (m, n, k) in [(1, 300, 1024), (33, 129, 2048)]:
            x, qw = _w4_case(m, n, k, 31 * config + m)
            qw = (qw[0], _signed(qw[1], config + k), qw[2])
            say("w4a16 signed scale codes", name, m, n, k)
            c = out_bf16(m, n)
            L.bsgemm_w4a16_run_config(config, dev(x.view(np.int16)), dev(qw[0]), dev(qw[1]),
                                      dev(np.array([qw[2]], np.float32)), c=c)
            assert_ok(G.check(u16(c), *G.w4a16(x, *qw)), f"w4a16 signed scales {name} {m}x{n}x{k}")



def _bf16_nan(c):
    return ((c & 0x7F80) == 0x7F80) & ((c & 0x7F) != 0)


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("counts,n,k", [([257, 0, 256, 255], 260, 96), ([512, 256, 0, 300], 512, 1280)])
def test_grouped_nan_scale_code(gpu_lib, w_dtype, counts, n, k):
    """A NaN scale code in A row 5 makes output row 5 NaN; the rest matches."""
    qa, off, w, v = _variant_case(counts, n, k, sum(counts) + n, w_dtype)
    qa = (qa[0], qa[1].copy(), qa[2])
    qa[1][5, 0] = 0x7F
    m = int(off[-1])
    say("grouped NaN scale code", w_dtype, counts, n, k)
    c = _gpu_grouped_ex(qa, off, w, k, w_dtype, v, (), m)
    nan = _bf16_nan(c)
    keep = np.setdiff1d(np.arange(m), [5])
    assert nan[5].all() and not nan[keep].any()
    cref, tref = _ref_ex(qa, off, w, w_dtype, v, ())
    assert_ok(G.check(c[keep], cref[keep], tref[keep]), f"grouped NaN scale {counts} {w_dtype}")


def test_w4a16_nan_scale_code(gpu_lib):
    """Every W4A16 configuration: a NaN scale code in W row 3 makes output
    column 3 NaN for every activation row; the rest matches."""
    for config, name in enumerate(L.w4a16_configs()):
        for (m, n, k) in [(1, 300, 1024), (33, 129, 2048)]:
            x, qw = _w4_case(m, n, k, 17 * config + m)
            qw = (qw[0], qw[1].copy(), qw[2])
            qw[1][3, 1] = 0xFF
            say("w4a16 NaN scale code", name, m, n, k)
            c = out_bf16(m, n)
            L.bsgemm_w4a16_run_config(config, dev(x.view(np.int16)), dev(qw[0]), dev(qw[1]),
                                      dev(np.array([qw[2]], np.float32)), c=c)
            got = u16(c)
            nan = _bf16_nan(got)
            keep = np.setdiff1d(np.arange(n), [3])
            assert nan[:, 3].all() and not nan[:, keep].any(), name
            cref, tref = G.w4a16(x, *qw)
            assert_ok(G.check(got[:, keep], cref[:, keep], tref[:, keep]), f"w4a16 NaN scale {name} {m}x{n}x{k}")


def _group_max_products(a, b, group=8):
    """G[m, n] = sum over aligned groups of `group` K elements of
    max_k |a[m, k] b[n, k]| (float64)."""
    m, k = a.shape
    out = np.zeros((m, b.shape[0]))
    for g0 in range(0, k, group):
        pa, pb = np.abs(a[:, g0:g0 + group]), np.abs(b[:, g0:g0 + group])
        out += np.max(pa[:, None, :] * pb[None, :, :], axis=2)
    return out


def _mx8_bound(fmt, qa, qb, cref, t):
    """The per-element bound each MXFP8 path documents at the C ABI: the plain
    2^-8 |C| + 1e-5 T for the exact path; for the native scaled FP8 MFMA also
    2^-10 G, G = sum over aligned groups of 8 K elements of the largest
    |product| (that MFMA sums a group to about 14 bits below its largest
    product; the groups are then combined in FP32)."""
    plain = 2.0 ** -8 * np.abs(cref) + 1e-5 * t
    if fmt == "mxfp8_exact":
        return plain
    return plain + 2.0 ** -10 * _group_max_products(G.dequant_mxfp8(*qa), G.dequant_mxfp8(*qb))


@pytest.mark.parametrize("fmt", ["mxfp8_exact", "mxfp8"])
@pytest.mark.parametrize("k", [128, 512, 1024, 2048 + 128])
def test_gemm_mxfp8_every_code(gpu_lib, fmt, k):
    """Random E4M3 codes (all finite codes, both signs) with E8M0 scales in
    [107, 147], on the 16-byte-scale ring (K % 512 == 0), the 4-byte-scale
    ring (K % 128 == 0) and the register-staged paths.

    Such codes put products spanning ~2^35 into one block.  The exact path
    must meet the plain bound; the native path the bound it documents (see
    _mx8_bound)."""
    r = np.random.Generator(np.random.PCG64(k + 1))
    m, n = 260, 300
    def codes(rows):
        c = r.integers(0, 256, (rows, k)).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x3C
        return c
    qa = (codes(m), r.integers(107, 148, (m, k // 32)).astype(np.uint8))
    qb = (codes(n), r.integers(107, 148, (n, k // 32)).astype(np.uint8))
    say("gemm", fmt, "every code, k =", k)
    c = _gpu_gemm(FMTS[fmt], qa, qb, k)
    cref, t = G.gemm_mxfp8(*qa, *qb)
    got = F.decode_bf16(c)
    bound = _mx8_bound(fmt, qa, qb, cref, t)
    assert np.all(np.isfinite(got)) and np.all(np.abs(got - cref) <= bound), \
        f"{fmt} every code k={k}: worst {np.max(np.abs(got - cref) / bound):.3g}"


@pytest.mark.parametrize("fmt", ["mxfp8_exact", "mxfp8"])
@pytest.mark.parametrize("k", [512, 2048])
def test_gemm_mxfp8_wide_range_encoder_output(gpu_lib, fmt, k):
    """MXFP8 encodings of data spanning 2^+-16 within each row (legal
    quantizer output: every block max lies in (224, 448] after scaling, yet
    one 32-block mixes products ~2^17 apart).  The exact path meets the plain
    bound; the native one the bound it documents (_mx8_bound)."""
    r = np.random.Generator(np.random.PCG64(k + 7))
    xa = (r.standard_normal((200, k)) * np.exp2(r.uniform(-16, 16, (200, k)))).astype(np.float32)
    xb = (r.standard_normal((180, k)) * np.exp2(r.uniform(-16, 16, (180, k)))).astype(np.float32)
    qa, qb = Q.quantize_mxfp8(xa), Q.quantize_mxfp8(xb)
    say("gemm", fmt, "wide-range encoder output, k =", k)
    c = _gpu_gemm(FMTS[fmt], qa, qb, k)
    cref, t = G.gemm_mxfp8(*qa, *qb)
    got = F.decode_bf16(c)
    bound = _mx8_bound(fmt, qa, qb, cref, t)
    assert np.all(np.isfinite(got)) and np.all(np.abs(got - cref) <= bound), \
        f"{fmt} wide range k={k}: worst {np.max(np.abs(got - cref) / bound):.3g}"


@pytest.mark.parametrize("k", [96, 128, 384, 512, 2048 + 512])
def test_gemm_mxfp4_every_code(gpu_lib, k):
    """Random bytes (every E2M1 code in both nibbles, both signs) with E8M0
    scales in [107, 147], on the 16-byte-scale ring (K % 512 == 0), the
    4-byte-scale ring (K % 128 == 0) and the register-staged path (K = 96),
    against the plain bound 2^-8 |C| + 1e-5 T.  (Two E2M1 products of one
    block are at most a factor 144 apart, so the FP4 MFMA loses nothing.)"""
    r = np.random.Generator(np.random.PCG64(k + 3))
    m, n = 260, 300
    qa = (r.integers(0, 256, (m, k // 2)).astype(np.uint8), r.integers(107, 148, (m, k // 32)).astype(np.uint8))
    qb = (r.integers(0, 256, (n, k // 2)).astype(np.uint8), r.integers(107, 148, (n, k // 32)).astype(np.uint8))
    say("gemm mxfp4 every code, k =", k)
    c = _gpu_gemm(L.BSGEMM_MXFP4, qa, qb, k)
    assert_ok(G.check(c, *G.gemm_mxfp4(*qa, *qb)), f"mxfp4 every code k={k}")


# ------------------------------------------------- graphs and streams --

def test_hot_path_graph_replays_and_two_streams(gpu_lib):
    """The whole hot path captured once in a HIP graph: the three quantizers
    (on the device, from FP32), the NVFP4, MXFP8, exact-MXFP8 and MXFP4 GEMMs,
    the grouped and K-ragged GEMMs and W4A16.  The graph is replayed three
    times with every output refilled between replays, eager library work and
    a synchronisation in between; every output of every replay must equal the
    eager run bit for bit (the kernels are deterministic, and nothing they
    launch is a memset node).  Then two GEMMs launched at once on two streams
    must equal their eager results too."""
    k = 1024
    xa, xb = dev(synth.normal_f32((512, k), 7001)), dev(synth.normal_f32((768, k), 7002))
    qa, qb = L.bsgemm_quantize_nvfp4(xa), L.bsgemm_quantize_nvfp4(xb)
    m8a, m8b = L.bsgemm_quantize_mxfp8(xa), L.bsgemm_quantize_mxfp8(xb)
    m4a, m4b = L.bsgemm_quantize_mxfp4(xa), L.bsgemm_quantize_mxfp4(xb)
    counts = [300, 0, 257, 1]
    gq, goff, gw = _grouped_case(counts, 260, 512, 7003)
    gq = (dev(gq[0]), dev(gq[1]), dev(np.array([gq[2]], np.float32)))
    goff, gw = dev(goff), dev(gw)
    kq, koff, kw, kk = _kragged_case([100, 0, 700, 256], 300, 260, 7004, "bf16")
    kq = (dev(kq[0]), dev(kq[1]), dev(np.array([kq[2]], np.float32)))
    koff, kw = dev(koff), dev(kw)
    wx = dev(synth.bf16_bits(synth.normal_f32((16, 4096), 7005)))
    wq = L.bsgemm_quantize_nvfp4(dev(synth.normal_f32((640, 4096), 7006, std=0.02)))
    outs = {"nv": out_bf16(512, 768), "mx8": out_bf16(512, 768), "mx8x": out_bf16(512, 768),
            "mx4": out_bf16(512, 768), "grouped": out_bf16(558, 260),
            "kragged": torch.full((4, 300, 260), SENTINEL, dtype=torch.int16, device="cuda"),
            "w4a16": out_bf16(16, 640)}
    quant_outs = {"qa": qa, "qb": qb, "m8a": m8a, "m8b": m8b, "m4a": m4a, "m4b": m4b}

    def run():
        L.bsgemm_quantize_nvfp4(xa, *qa)
        L.bsgemm_quantize_nvfp4(xb, *qb)
        L.bsgemm_run(L.BSGEMM_NVFP4, *qa, *qb, k, c=outs["nv"])
        L.bsgemm_quantize_mxfp8(xa, *m8a)
        L.bsgemm_quantize_mxfp8(xb, *m8b)
        L.bsgemm_run(L.BSGEMM_MXFP8, m8a[0], m8a[1], None, m8b[0], m8b[1], None, k, c=outs["mx8"])
        L.bsgemm_run(L.BSGEMM_MXFP8_EXACT, m8a[0], m8a[1], None, m8b[0], m8b[1], None, k, c=outs["mx8x"])
        L.bsgemm_quantize_mxfp4(xa, *m4a)
        L.bsgemm_quantize_mxfp4(xb, *m4b)
        L.bsgemm_run(L.BSGEMM_MXFP4, m4a[0], m4a[1], None, m4b[0], m4b[1], None, k, c=outs["mx4"])
        L.bsgemm_grouped_run(*gq, goff, gw, 512, c=outs["grouped"])
        L.bsgemm_grouped_kragged_run(*kq, koff, kw, kk, c=outs["kragged"])
        L.bsgemm_w4a16_run(wx, *wq, c=outs["w4a16"])

    def every_output():
        return dict(outs, **{f"{n}[{i}]": t for n, q in quant_outs.items() for i, t in enumerate(q)})

    def junk(t):
        return {torch.float32: float("nan"), torch.uint8: 0xAB}.get(t.dtype, SENTINEL)

    def clobber():
        for t in every_output().values():
            t.fill_(junk(t))

    say("graph: eager reference run")
    clobber()
    run()
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in every_output().items()}
    for n, t in eager.items():
        assert not torch.equal(t, torch.full_like(t, junk(t))), f"the eager run left {n} unwritten"
    assert_ok(G.check(u16(outs["nv"]), *G.gemm_nvfp4(*Q.quantize_nvfp4(xa.cpu().numpy()),
                                                   *Q.quantize_nvfp4(xb.cpu().numpy()))), "graph test eager NVFP4")

    say("graph: capture")
    clobber()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    scratch = out_bf16(512, 512)
    for rep in range(3):
        say("graph: replay", rep)
        clobber()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in every_output().items():
            assert torch.equal(t, eager[n]), f"replay {rep}: {n} differs from the eager run"
        # eager library work between replays, on the default stream
        L.bsgemm_run(L.BSGEMM_MXFP8, m8b[0][:512], m8b[1][:512], None, m8a[0], m8a[1], None, k, c=scratch)
        torch.cuda.synchronize()
    del g

    say("two streams")
    ya, yb = dev(synth.normal_f32((2048, 2048), 7007)), dev(synth.normal_f32((2048, 2048), 7008))
    na, nb = L.bsgemm_quantize_nvfp4(ya), L.bsgemm_quantize_nvfp4(yb)
    ea, eb = L.bsgemm_quantize_mxfp8(ya), L.bsgemm_quantize_mxfp8(yb)
    c1, c2 = out_bf16(2048, 2048), out_bf16(2048, 2048)
    L.bsgemm_run(L.BSGEMM_NVFP4, *na, *nb, 2048, c=c1)
    L.bsgemm_run(L.BSGEMM_MXFP8, ea[0], ea[1], None, eb[0], eb[1], None, 2048, c=c2)
    torch.cuda.synchronize()
    r1, r2 = c1.clone(), c2.clone()
    c1.fill_(SENTINEL)
    c2.fill_(SENTINEL)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            L.bsgemm_run(L.BSGEMM_NVFP4, *na, *nb, 2048, c=c1)
        with torch.cuda.stream(s2):
            L.bsgemm_run(L.BSGEMM_MXFP8, ea[0], ea[1], None, eb[0], eb[1], None, 2048, c=c2)
    torch.cuda.synchronize()
    assert torch.equal(c1, r1) and torch.equal(c2, r2)
