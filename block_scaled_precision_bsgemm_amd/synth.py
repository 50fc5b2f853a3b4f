"""Seeded synthetic inputs for block-scaled GEMM workloads.

This module only draws random numbers and lays them out; it holds none of the
quantization or GEMM arithmetic.  The tests (for both the CPU oracle and the HIP
library) and the benchmark take their inputs from here, so both sides always
see identical bytes.

Workloads (shapes and distributions; the pages give the shapes, the value
distributions are the library's stated synthetic recipe):

* ``nvfp4_small``   -- NVFP4 x NVFP4, M=N=256, K=128, A and B ~ N(0, 1)
  (the 256 x 256 x 128 case of "Triton #11171 ...", section "The missing case
  was defined by shape, layout, and execution mode together").
* ``mxfp8_4k``      -- MXFP8 x MXFP8, M=N=K=4096, ~ N(0, 1).
* ``nvfp4_big``     -- NVFP4 x NVFP4 at 65536^3 and 131072^3 ("Together AI Ports
  ThunderKittens ...", section "Building the GEMM": 64k and 128k square
  GEMMs).  FP32 sources would take 16-64 GiB per operand, so the operands are
  drawn directly as NVFP4 on the device: uniform random code bytes and E4M3
  scale codes uniform in [0x30, 0x40) (2^-1 .. 2^1), tensor scale 1
  (``nvfp4_random_operand``, torch's seeded device generator).
* ``mxfp4``         -- MXFP4 x MXFP4, M=N=K=4096 or 16384, ~ N(0, 1) with 1% of
  the rows of A and of B multiplied by 100 (the 16k-square recipe of
  ``nvfp4_16k``, own seeds).
* ``nvfp4_16k``     -- NVFP4 x NVFP4, M=N=K=16384 ("Together AI Ports
  ThunderKittens GEMM Kernels to NVIDIA Vera Rubin NVL72", section "Building
  the GEMM": 16k square GEMMs), ~ N(0, 1) with 1% of the rows of A and of B
  (163 distinct rows each, chosen without replacement) multiplied by 100.
* ``grouped``       -- 32 groups, row counts ~ Multinomial(16384,
  Dirichlet(0.5 * 1_32)) laid out in group order, K=7168, N=2048; activations
  ~ N(0, 1) (quantized to NVFP4), weights ~ N(0, 0.02) cast to BF16 (RNE).
* ``w4a16``         -- BF16 activations X[M, 4096] ~ N(0, 1), M in {1, 16, 64,
  256}, weights W[14336, 4096] ~ N(0, 0.02) quantized to NVFP4 (the Llama3-8B
  gate/up projection shape of "Add sm121 (GB10) tier to the 4-bit GEMM
  dispatch heuristic", section "Methodology").

Random numbers come from numpy ``Generator(PCG64(seed))``; every operand has
its own seed, listed in ``SEEDS``.
"""

import numpy as np

SEEDS = {
    "nvfp4_small.A": 1001, "nvfp4_small.B": 1002,
    "mxfp8_4k.A": 2001, "mxfp8_4k.B": 2002,
    "nvfp4_16k.A": 3001, "nvfp4_16k.B": 3002,
    "nvfp4_16k.A.rows": 3011, "nvfp4_16k.B.rows": 3012,
    "grouped.counts": 4000, "grouped.A": 4001, "grouped.W": 4002,
    "w4a16.X": 5001, "w4a16.W": 5002,
    "mxfp4.A": 6001, "mxfp4.B": 6002, "mxfp4.A.rows": 6011, "mxfp4.B.rows": 6012,
    "nvfp4_big.A": 7001, "nvfp4_big.B": 7002,
}

SHAPES = {
    "nvfp4_small": dict(M=256, N=256, K=128),
    "mxfp8_4k": dict(M=4096, N=4096, K=4096),
    "mxfp8_16k": dict(M=16384, N=16384, K=16384),
    "nvfp4_16k": dict(M=16384, N=16384, K=16384),
    "mxfp4_4k": dict(M=4096, N=4096, K=4096),
    "mxfp4_16k": dict(M=16384, N=16384, K=16384),
    "grouped": dict(G=32, M=16384, N=2048, K=7168, alpha=0.5),
    "w4a16": dict(Ms=(1, 16, 64, 256), N=14336, K=4096),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """float32 samples of N(0, std^2), row-major, drawn in float32 directly."""
    return rng(seed).standard_normal(size=shape, dtype=np.float32) * np.float32(std)


def with_outlier_rows(x: np.ndarray, seed: int, frac: float = 0.01, factor: float = 100.0):
    """Multiply floor(frac * rows) distinct rows (seeded choice) by ``factor``.
    Returns (x, sorted row indices).  The product is an FP32 multiply."""
    rows = x.shape[0]
    n = int(np.floor(frac * rows))
    idx = np.sort(rng(seed).choice(rows, size=n, replace=False))
    x[idx] *= np.float32(factor)
    return x, idx


def group_counts(G: int, M: int, alpha: float, seed: int) -> np.ndarray:
    """Row counts per group: p ~ Dirichlet(alpha * 1_G), counts ~ Multinomial(M, p).
    Empty groups are legal."""
    r = rng(seed)
    p = r.dirichlet(np.full(G, alpha))
    return r.multinomial(M, p).astype(np.int64)


def offsets_from_counts(counts) -> np.ndarray:
    """int32 offsets[G+1]: off[0] = 0, off[g+1] = off[g] + counts[g]."""
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    return off.astype(np.int32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even cast float32 -> BF16, returned as uint16 bits.
    (Uses torch's CPU cast; NaN inputs are not expected.)"""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# ------------------------------------------------------------- workloads --

def nvfp4_small_inputs():
    s = SHAPES["nvfp4_small"]
    return (normal_f32((s["M"], s["K"]), SEEDS["nvfp4_small.A"]),
            normal_f32((s["N"], s["K"]), SEEDS["nvfp4_small.B"]))


def mxfp8_inputs(M=4096, N=4096, K=4096):
    return (normal_f32((M, K), SEEDS["mxfp8_4k.A"]), normal_f32((N, K), SEEDS["mxfp8_4k.B"]))


def nvfp4_16k_inputs(M=16384, N=16384, K=16384):
    a, ia = with_outlier_rows(normal_f32((M, K), SEEDS["nvfp4_16k.A"]), SEEDS["nvfp4_16k.A.rows"])
    b, ib = with_outlier_rows(normal_f32((N, K), SEEDS["nvfp4_16k.B"]), SEEDS["nvfp4_16k.B.rows"])
    return a, b, ia, ib


def mxfp4_inputs(M=16384, N=16384, K=16384):
    """A [M, K], B [N, K] ~ N(0, 1) with 1% outlier rows (x100) in each."""
    a, ia = with_outlier_rows(normal_f32((M, K), SEEDS["mxfp4.A"]), SEEDS["mxfp4.A.rows"])
    b, ib = with_outlier_rows(normal_f32((N, K), SEEDS["mxfp4.B"]), SEEDS["mxfp4.B.rows"])
    return a, b, ia, ib


def nvfp4_random_operand(rows, k, seed, device):
    """NVFP4 operand drawn on `device`: (codes uint8 [rows, k/2] uniform
    bytes, scales uint8 [rows, k/16] uniform in [0x30, 0x40), tensor scale
    float32 [1] = 1), from torch's generator seeded with `seed`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    codes = torch.randint(0, 256, (rows, k // 2), dtype=torch.uint8, device=device, generator=g)
    scales = torch.randint(0x30, 0x40, (rows, k // 16), dtype=torch.uint8, device=device, generator=g)
    return codes, scales, torch.ones(1, dtype=torch.float32, device=device)


def grouped_inputs(G=32, M=16384, N=2048, K=7168, alpha=0.5):
    counts = group_counts(G, M, alpha, SEEDS["grouped.counts"])
    off = offsets_from_counts(counts)
    a = normal_f32((M, K), SEEDS["grouped.A"])
    w = bf16_bits(normal_f32((G, N, K), SEEDS["grouped.W"], std=0.02))
    return a, off, w


def w4a16_inputs(M, N=14336, K=4096):
    x = bf16_bits(normal_f32((M, K), SEEDS["w4a16.X"]))
    w = normal_f32((N, K), SEEDS["w4a16.W"], std=0.02)
    return x, w
