"""NVFP4, MXFP8 and MXFP4 quantizers (vectorised numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Both quantizers act on a row-major FP32 matrix X[R, K] whose rows are the GEMM
operand rows (A is [M, K], B and W are [N, K]) and whose blocks run along K --
the contraction dimension of the GEMMs on the pages ("Together AI Ports
ThunderKittens GEMM Kernels to NVIDIA Vera Rubin NVL72", section "Building the
GEMM": block-scaled MMAs whose scale factors travel with the K chunks).

Every FP32 step is an IEEE binary32 operation with round-to-nearest-even,
reproduced with numpy float32 arithmetic, in the order the recipe states it.
Readings taken where the statement is silent:

* division, not multiplication by a reciprocal, wherever the recipe says
  "over" or "/";
* encoders round to nearest, ties to even, and saturate (``formats``);
* the sign bit of every element code copies signbit(x), also for zero codes;
* an all-zero tensor (tensor scale 0) or a block whose scale code decodes to
  0 gets scale code 0 and sign-only element codes;
* subnormal E4M3 scales are kept; a block scale below 2**-10 rounds to 0;
* inputs are finite (asserted).
"""

import numpy as np

from .formats import (decode_e4m3, encode_e2m1_mag, encode_e4m3_mag,
                      pack_nibbles, signbit_u8)

F32 = np.float32
NVFP4_BLOCK = 16
MXFP8_BLOCK = 32
MXFP4_BLOCK = 32
E2M1_MAX = F32(6.0)
E4M3_MAX = F32(448.0)


def nvfp4_tensor_scale(x) -> np.float32:
    """s_t = fl32(amax / 2688), 2688 = 6 * 448: the FP32 per-tensor decode scale."""
    x = np.asarray(x, dtype=F32)
    amax = np.max(np.abs(x)) if x.size else F32(0)
    return F32(F32(amax) / F32(2688.0))


def quantize_nvfp4(x, tensor_scale=None):
    """NVFP4-quantize X[R, K] (K % 16 == 0).

    Returns (codes uint8 [R, K/2], scales uint8 [R, K/16], s_t float32):

    1. amax = max |x| over the whole tensor; s_t = fl32(amax / 2688).
    2. per 16-element block: bamax = max |x|;
       s_real = fl32(fl32(bamax / 6) / s_t); scale code = E4M3_RNE_sat(s_real).
    3. S = fl32(e4m3(scale code) * s_t); each element q = fl32(x / S),
       code = signbit(x) << 3 | E2M1_RNE_sat(|q|).
    4. byte j of a row holds element 2j in the low nibble, 2j+1 in the high.

    ``tensor_scale`` overrides step 1 (used only by tests that need a chosen s_t).
    """
    x = np.ascontiguousarray(x, dtype=F32)
    assert x.ndim == 2 and x.shape[1] % NVFP4_BLOCK == 0
    assert np.all(np.isfinite(x)), "inputs must be finite"
    R, K = x.shape
    s_t = nvfp4_tensor_scale(x) if tensor_scale is None else F32(tensor_scale)
    blocks = x.reshape(R, K // NVFP4_BLOCK, NVFP4_BLOCK)
    bamax = np.max(np.abs(blocks), axis=2) if x.size else np.zeros((R, 0), F32)
    if s_t == 0:
        scale_codes = np.zeros(bamax.shape, dtype=np.uint8)
    else:
        s_real = (bamax / E2M1_MAX).astype(F32) / s_t
        scale_codes = encode_e4m3_mag(s_real.astype(F32))
    S = (decode_e4m3(scale_codes).astype(F32) * s_t).astype(F32)
    sign = signbit_u8(blocks) << 3
    safe_S = np.where(S == 0, F32(1), S).astype(F32)
    q = (blocks / safe_S[:, :, None]).astype(F32)
    mag = encode_e2m1_mag(np.abs(q))
    mag = np.where((S == 0)[:, :, None], 0, mag).astype(np.uint8)
    codes = (sign | mag).reshape(R, K).astype(np.uint8)
    return pack_nibbles(codes), scale_codes.astype(np.uint8), F32(s_t)


def mx_block_exponent(bamax, top) -> np.ndarray:
    """e = min{ e in Z : top * 2**e >= bamax }, clamped to [-127, 127], where
    `top` is the element format's largest value (448 for E4M3, 6 for E2M1).

    This is the exact value of ceil(log2(bamax / top)).  The search starts
    below the answer (from the binary exponents of bamax and top) and walks up
    to the least e meeting the definition, checked in exact float64
    arithmetic.  bamax == 0 gives -127.
    """
    b = np.asarray(bamax, dtype=np.float64)
    _, E = np.frexp(b)
    _, Et = np.frexp(top)
    e = E.astype(np.int64) - int(Et) - 1
    for _ in range(3):  # walk up to the least e meeting the definition
        e = np.where(top * np.ldexp(1.0, e) >= b, e, e + 1)
    ok = top * np.ldexp(1.0, e) >= b
    minimal = ~(top * np.ldexp(1.0, e - 1) >= b)
    assert np.all(ok & (minimal | (b == 0)))
    e = np.where(b == 0, -127, e)
    return np.clip(e, -127, 127)


def mxfp8_block_exponent(bamax) -> np.ndarray:
    """e = min{ e in Z : 448 * 2**e >= bamax }, clamped to [-127, 127]."""
    return mx_block_exponent(bamax, 448.0)


def mxfp4_block_exponent(bamax) -> np.ndarray:
    """e = min{ e in Z : 6 * 2**e >= bamax }, clamped to [-127, 127]."""
    return mx_block_exponent(bamax, 6.0)


def quantize_mxfp8(x):
    """MXFP8-quantize X[R, K] (K % 32 == 0).

    Returns (codes uint8 [R, K], scales uint8 [R, K/32]):

    1. per 32-element block: bamax = max |x|; e = ceil(log2(bamax / 448))
       computed exactly (``mxfp8_block_exponent``); scale code = e + 127 (E8M0).
    2. q = x * 2**-e (exact: a power-of-two scaling of an FP32 value, done in
       float64); code = signbit(x) << 7 | E4M3_RNE_sat(|q|).  By construction
       |q| <= 448, so saturation never triggers.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    assert x.ndim == 2 and x.shape[1] % MXFP8_BLOCK == 0
    assert np.all(np.isfinite(x)), "inputs must be finite"
    R, K = x.shape
    blocks = x.reshape(R, K // MXFP8_BLOCK, MXFP8_BLOCK).astype(np.float64)
    bamax = np.max(np.abs(blocks), axis=2) if x.size else np.zeros((R, 0))
    e = mxfp8_block_exponent(bamax)
    q = blocks * np.ldexp(1.0, -e)[:, :, None]
    codes = (signbit_u8(blocks) << 7) | encode_e4m3_mag(np.abs(q))
    return codes.reshape(R, K).astype(np.uint8), (e + 127).astype(np.uint8)


def quantize_mxfp4(x):
    """MXFP4-quantize X[R, K] (K % 32 == 0).

    Returns (codes uint8 [R, K/2], scales uint8 [R, K/32]):

    1. per 32-element block: bamax = max |x|; e = ceil(log2(bamax / 6))
       computed exactly (``mxfp4_block_exponent``); scale code = e + 127
       (E8M0).  This is the MXFP8 rule with E2M1's largest value, 6, in place
       of 448, so no element saturates.
    2. q = x * 2**-e (exact: a power-of-two scaling of an FP32 value, done in
       float64); code = signbit(x) << 3 | E2M1_RNE(|q|).
    3. byte j of a row holds element 2j in the low nibble, 2j+1 in the high.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    assert x.ndim == 2 and x.shape[1] % MXFP4_BLOCK == 0
    assert np.all(np.isfinite(x)), "inputs must be finite"
    R, K = x.shape
    blocks = x.reshape(R, K // MXFP4_BLOCK, MXFP4_BLOCK).astype(np.float64)
    bamax = np.max(np.abs(blocks), axis=2) if x.size else np.zeros((R, 0))
    e = mxfp4_block_exponent(bamax)
    q = blocks * np.ldexp(1.0, -e)[:, :, None]
    codes = (signbit_u8(blocks) << 3) | encode_e2m1_mag(np.abs(q))
    return pack_nibbles(codes.reshape(R, K).astype(np.uint8)), (e + 127).astype(np.uint8)
