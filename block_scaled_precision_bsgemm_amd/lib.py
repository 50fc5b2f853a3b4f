"""ctypes binding of libbsgemm.so: the C ABI of include/bsgemm.h, same names.

Argument marshalling only: torch tensors are turned into raw device pointers
and the current HIP stream, output tensors are allocated when not given, and
a non-zero status raises ``BsgemmError``.  All computation runs in the HIP
library; there is no fallback of any kind.  If the library is missing the
calls raise.

Before any call, every tensor is checked against the layout the C ABI implies
(dtype, shape, contiguity, on the current device); a mismatch raises
``ValueError``, so a wrong-sized buffer never reaches a kernel.  BF16 and FP16
bit patterns may be passed as int16, uint16 or the floating dtype itself.
"""

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbsgemm.so")

BSGEMM_OK = 0
BSGEMM_ERR_INVALID_ARG = 1
BSGEMM_ERR_UNSUPPORTED = 2
BSGEMM_ERR_BAD_ALIGNMENT = 3
BSGEMM_ERR_DEVICE = 4
BSGEMM_ERR_RESOURCE = 5
BSGEMM_ERR_LAUNCH = 6
BSGEMM_NVFP4 = 1
BSGEMM_MXFP8 = 2
BSGEMM_MXFP4 = 3
BSGEMM_MXFP8_EXACT = 4
BSGEMM_W_BF16 = 1
BSGEMM_W_F16 = 2

# Symbols declared in include/bsgemm.h with their ctypes signatures.
_i64, _p, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
SIGNATURES = {
    "bsgemm_quantize_nvfp4": (_int, [_i64, _i64, _p, _p, _p, _p, _p]),
    "bsgemm_quantize_mxfp8": (_int, [_i64, _i64, _p, _p, _p, _p]),
    "bsgemm_quantize_mxfp4": (_int, [_i64, _i64, _p, _p, _p, _p]),
    "bsgemm_run": (_int, [_int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p]),
    "bsgemm_grouped_run": (_int, [_int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p]),
    "bsgemm_grouped_run_ex": (_int, [_int, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _int, _p, _p, _p, _p, _p,
                                     _p, _p]),
    "bsgemm_grouped_kragged_run": (_int, [_int, _i64, _i64, _i64, _p, _p, _p, _p, _int, _p, _p, _p]),
    "bsgemm_w4a16_run": (_int, [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p]),
    "bsgemm_w4a16_run_config": (_int, [_int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p]),
    "bsgemm_w4a16_num_configs": (_int, []),
    "bsgemm_w4a16_config_name": (ctypes.c_char_p, [_int]),
    "bsgemm_w4a16_select": (_int, [_i64, _i64, _i64]),
    "bsgemm_status_string": (ctypes.c_char_p, [_int]),
    "bsgemm_last_error": (ctypes.c_char_p, []),
    "bsgemm_version": (_int, []),
}

_lib = None


class BsgemmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} ({status})")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once and set every declared signature."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it with `python -m block_scaled_precision_bsgemm_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _lib = lib
    return _lib


def _check(status):
    if status != BSGEMM_OK:
        lib = load()
        raise BsgemmError(lib.bsgemm_status_string(status).decode(), lib.bsgemm_last_error().decode())


_U16 = tuple(d for d in (torch.int16, getattr(torch, "uint16", None)) if d is not None)
BF16_BITS = _U16 + (torch.bfloat16,)
F16_BITS = _U16 + (torch.float16,)
U8 = (torch.uint8,)
F32 = (torch.float32,)
I32 = (torch.int32,)


def _need(t, name, dtypes, shape=None, ndim=None):
    """Raise ValueError unless t is a tensor with one of `dtypes` and (when
    given) exactly `shape` or `ndim` dimensions.  Placement (on the current
    device, contiguous) is checked by _ptr, for every tensor, before the call."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected a {ndim}-D tensor, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(v) for v in shape)}")
    return t


def _need_scalar(t, name):
    """A device float32 slot holding one value (a tensor scale)."""
    _need(t, name, F32)
    if t.numel() != 1:
        raise ValueError(f"{name}: expected one float32 element, got {t.numel()}")
    return t


def _need_2d(t, name, dtypes):
    return _need(t, name, dtypes, ndim=2)


def _operand_shapes(fmt, rows, k):
    """(codes shape, scales shape) of an operand [rows][k] in format `fmt`."""
    if fmt == BSGEMM_NVFP4:
        return (rows, k // 2), (rows, k // 16)
    if fmt in (BSGEMM_MXFP8, BSGEMM_MXFP8_EXACT):
        return (rows, k), (rows, k // 32)
    if fmt == BSGEMM_MXFP4:
        return (rows, k // 2), (rows, k // 32)
    raise ValueError(f"unknown format {fmt}")


def _ptr(t):
    """Device address of t, after checking that it is contiguous and on the
    current device (the library takes every pointer on the current device)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"tensor of shape {tuple(t.shape)} must be a device tensor (got {t.device})")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"tensor of shape {tuple(t.shape)} must be contiguous")
    return t.data_ptr() or None


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def bsgemm_quantize_nvfp4(x, codes=None, scales=None, tensor_scale=None, stream=None):
    """x: float32 [rows, k] -> (codes uint8 [rows, k/2], scales uint8 [rows, k/16], tensor_scale float32 [1])."""
    rows, k = _need_2d(x, "x", F32).shape
    codes = _empty((rows, k // 2), torch.uint8, x) if codes is None else _need(codes, "codes", U8, (rows, k // 2))
    scales = _empty((rows, k // 16), torch.uint8, x) if scales is None else _need(scales, "scales", U8, (rows, k // 16))
    tensor_scale = _empty((1,), torch.float32, x) if tensor_scale is None else _need_scalar(tensor_scale, "tensor_scale")
    _check(load().bsgemm_quantize_nvfp4(rows, k, _ptr(x), _ptr(codes), _ptr(scales),
                                        _ptr(tensor_scale), _stream(stream)))
    return codes, scales, tensor_scale


def bsgemm_quantize_mxfp8(x, codes=None, scales=None, stream=None):
    """x: float32 [rows, k] -> (codes uint8 [rows, k], scales uint8 [rows, k/32])."""
    rows, k = _need_2d(x, "x", F32).shape
    codes = _empty((rows, k), torch.uint8, x) if codes is None else _need(codes, "codes", U8, (rows, k))
    scales = _empty((rows, k // 32), torch.uint8, x) if scales is None else _need(scales, "scales", U8, (rows, k // 32))
    _check(load().bsgemm_quantize_mxfp8(rows, k, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def bsgemm_quantize_mxfp4(x, codes=None, scales=None, stream=None):
    """x: float32 [rows, k] -> (codes uint8 [rows, k/2], scales uint8 [rows, k/32])."""
    rows, k = _need_2d(x, "x", F32).shape
    codes = _empty((rows, k // 2), torch.uint8, x) if codes is None else _need(codes, "codes", U8, (rows, k // 2))
    scales = _empty((rows, k // 32), torch.uint8, x) if scales is None else _need(scales, "scales", U8, (rows, k // 32))
    _check(load().bsgemm_quantize_mxfp4(rows, k, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def bsgemm_run(fmt, a, a_scales, a_tscale, b, b_scales, b_tscale, k, c=None, stream=None):
    """C[m, n] (BF16 bits as int16/uint16 tensor) = deq(A) @ deq(B)^T; k is the logical K.
    fmt: BSGEMM_NVFP4 (tensor scales required), BSGEMM_MXFP8, BSGEMM_MXFP8_EXACT or
    BSGEMM_MXFP4 (tensor scales None)."""
    m, n = _need_2d(a, "a", U8).shape[0], _need_2d(b, "b", U8).shape[0]
    (ca, sa), (cb, sb) = _operand_shapes(fmt, m, k), _operand_shapes(fmt, n, k)
    _need(a, "a", U8, ca)
    _need(a_scales, "a_scales", U8, sa)
    _need(b, "b", U8, cb)
    _need(b_scales, "b_scales", U8, sb)
    for t, name in ((a_tscale, "a_tscale"), (b_tscale, "b_tscale")):
        if t is not None:
            _need_scalar(t, name)
    c = _empty((m, n), torch.int16, a) if c is None else _need(c, "c", BF16_BITS, (m, n))
    _check(load().bsgemm_run(fmt, m, n, k, _ptr(a), _ptr(a_scales), _ptr(a_tscale), _ptr(b),
                             _ptr(b_scales), _ptr(b_tscale), _ptr(c), _stream(stream)))
    return c


def bsgemm_grouped_run(a, a_scales, a_tscale, group_offsets, w_bf16, k, c=None, stream=None):
    """Grouped NVFP4 A [m_total, k] x BF16 W [G, n, k] -> C [m_total, n] (BF16 bits)."""
    _need(w_bf16, "w_bf16", BF16_BITS)
    if w_bf16.dim() != 3 or w_bf16.shape[2] != k:
        raise ValueError(f"w_bf16: expected [G, n, {k}], got {tuple(w_bf16.shape)}")
    G, n = w_bf16.shape[0], w_bf16.shape[1]
    m_total = _need_2d(a, "a", U8).shape[0]
    _need(a, "a", U8, (m_total, k // 2))
    _need(a_scales, "a_scales", U8, (m_total, k // 16))
    _need_scalar(a_tscale, "a_tscale")
    _need(group_offsets, "group_offsets", I32, (G + 1,))
    c = _empty((m_total, n), torch.int16, a) if c is None else _need(c, "c", BF16_BITS, (m_total, n))
    _check(load().bsgemm_grouped_run(G, m_total, n, k, _ptr(a), _ptr(a_scales), _ptr(a_tscale),
                                     _ptr(group_offsets), _ptr(w_bf16), _ptr(c), _stream(stream)))
    return c


def bsgemm_grouped_run_ex(a, a_scales, a_tscale, group_offsets, w, k, w_dtype=BSGEMM_W_BF16, bias=None,
                          gamma=None, gather_idx=None, scatter_idx=None, m_total=None, c=None, stream=None):
    """Grouped NVFP4 A [a_rows, k] x dense W [G, n, k] (BF16 or FP16 bits) with optional
    bias [G, n], gamma [m_total], gather_idx [m_total] and scatter_idx [m_total] -> C
    [m_total, n] (BF16 bits).  m_total defaults to the gather length, else to a_rows."""
    _need(w, "w", BF16_BITS if w_dtype == BSGEMM_W_BF16 else F16_BITS)
    if w.dim() != 3 or w.shape[2] != k:
        raise ValueError(f"w: expected [G, n, {k}], got {tuple(w.shape)}")
    G, n = w.shape[0], w.shape[1]
    a_rows = _need_2d(a, "a", U8).shape[0]
    if m_total is None:
        m_total = gather_idx.shape[0] if gather_idx is not None else a_rows
    _need(a, "a", U8, (a_rows, k // 2))
    _need(a_scales, "a_scales", U8, (a_rows, k // 16))
    _need_scalar(a_tscale, "a_tscale")
    _need(group_offsets, "group_offsets", I32, (G + 1,))
    if bias is not None:
        _need(bias, "bias", F32, (G, n))
    if gamma is not None:
        _need(gamma, "gamma", F32, (m_total,))
    for t, name in ((gather_idx, "gather_idx"), (scatter_idx, "scatter_idx")):
        if t is not None:
            _need(t, name, I32, (m_total,))
    c = _empty((m_total, n), torch.int16, a) if c is None else _need(c, "c", BF16_BITS, (m_total, n))
    _check(load().bsgemm_grouped_run_ex(G, m_total, n, k, a_rows, _ptr(a), _ptr(a_scales), _ptr(a_tscale),
                                        _ptr(group_offsets), w_dtype, _ptr(w), _ptr(bias), _ptr(gamma),
                                        _ptr(gather_idx), _ptr(scatter_idx), _ptr(c), _stream(stream)))
    return c


def bsgemm_grouped_kragged_run(a, a_scales, a_tscale, k_offsets, w, k, w_dtype=BSGEMM_W_BF16, c=None,
                               stream=None):
    """K-ragged grouped NVFP4 A [m, k] x dense W [n, k] (BF16 or FP16 bits), groups split K at
    k_offsets [G + 1] -> C [G, m, n] (BF16 bits)."""
    G = _need(k_offsets, "k_offsets", I32).shape[0] - 1
    if k_offsets.dim() != 1 or G < 1:
        raise ValueError(f"k_offsets: expected [G + 1] with G >= 1, got {tuple(k_offsets.shape)}")
    m = _need_2d(a, "a", U8).shape[0]
    n = _need_2d(w, "w", BF16_BITS if w_dtype == BSGEMM_W_BF16 else F16_BITS).shape[0]
    _need(a, "a", U8, (m, k // 2))
    _need(a_scales, "a_scales", U8, (m, k // 16))
    _need_scalar(a_tscale, "a_tscale")
    _need(w, "w", (w.dtype,), (n, k))
    c = _empty((G, m, n), torch.int16, a) if c is None else _need(c, "c", BF16_BITS, (G, m, n))
    _check(load().bsgemm_grouped_kragged_run(G, m, n, k, _ptr(a), _ptr(a_scales), _ptr(a_tscale),
                                             _ptr(k_offsets), w_dtype, _ptr(w), _ptr(c), _stream(stream)))
    return c


def _w4a16_check(x_bf16, w, w_scales, w_tscale):
    m, k = _need_2d(x_bf16, "x_bf16", BF16_BITS).shape
    n = _need_2d(w, "w", U8).shape[0]
    _need(w, "w", U8, (n, k // 2))
    _need(w_scales, "w_scales", U8, (n, k // 16))
    _need_scalar(w_tscale, "w_tscale")
    return m, k, n


def bsgemm_w4a16_run(x_bf16, w, w_scales, w_tscale, c=None, stream=None):
    """BF16 X [m, k] x NVFP4 W [n, k] -> C [m, n] (BF16 bits)."""
    m, k, n = _w4a16_check(x_bf16, w, w_scales, w_tscale)
    c = _empty((m, n), torch.int16, x_bf16) if c is None else _need(c, "c", BF16_BITS, (m, n))
    _check(load().bsgemm_w4a16_run(m, n, k, _ptr(x_bf16), _ptr(w), _ptr(w_scales), _ptr(w_tscale),
                                   _ptr(c), _stream(stream)))
    return c


def bsgemm_w4a16_run_config(config, x_bf16, w, w_scales, w_tscale, c=None, stream=None):
    """bsgemm_w4a16_run with configuration `config` (id or name) forced."""
    if isinstance(config, str):
        config = w4a16_config_id(config)
    m, k, n = _w4a16_check(x_bf16, w, w_scales, w_tscale)
    c = _empty((m, n), torch.int16, x_bf16) if c is None else _need(c, "c", BF16_BITS, (m, n))
    _check(load().bsgemm_w4a16_run_config(config, m, n, k, _ptr(x_bf16), _ptr(w), _ptr(w_scales),
                                          _ptr(w_tscale), _ptr(c), _stream(stream)))
    return c


def w4a16_configs():
    """Names of the W4A16 configurations, indexed by id."""
    lib = load()
    return [lib.bsgemm_w4a16_config_name(i).decode() for i in range(lib.bsgemm_w4a16_num_configs())]


def w4a16_config_id(name):
    return w4a16_configs().index(name)


def bsgemm_w4a16_select(m, n, k):
    return load().bsgemm_w4a16_select(m, n, k)


def version() -> int:
    return load().bsgemm_version()
