"""ctypes binding of libbsgemm.so: the C ABI of include/bsgemm.h, same names.

Argument marshalling only: torch tensors are turned into raw device pointers
and the current HIP stream, output tensors are allocated when not given, and
a non-zero status raises ``BsgemmError``.  All computation runs in the HIP
library; there is no fallback of any kind.  If the library is missing the
calls raise.
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


def _ptr(t):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous CUDA tensors"
    return t.data_ptr() or None


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def bsgemm_quantize_nvfp4(x, codes=None, scales=None, tensor_scale=None, stream=None):
    """x: float32 [rows, k] -> (codes uint8 [rows, k/2], scales uint8 [rows, k/16], tensor_scale float32 [1])."""
    rows, k = x.shape
    codes = _empty((rows, k // 2), torch.uint8, x) if codes is None else codes
    scales = _empty((rows, k // 16), torch.uint8, x) if scales is None else scales
    tensor_scale = _empty((1,), torch.float32, x) if tensor_scale is None else tensor_scale
    _check(load().bsgemm_quantize_nvfp4(rows, k, _ptr(x), _ptr(codes), _ptr(scales),
                                        _ptr(tensor_scale), _stream(stream)))
    return codes, scales, tensor_scale


def bsgemm_quantize_mxfp8(x, codes=None, scales=None, stream=None):
    """x: float32 [rows, k] -> (codes uint8 [rows, k], scales uint8 [rows, k/32])."""
    rows, k = x.shape
    codes = _empty((rows, k), torch.uint8, x) if codes is None else codes
    scales = _empty((rows, k // 32), torch.uint8, x) if scales is None else scales
    _check(load().bsgemm_quantize_mxfp8(rows, k, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def bsgemm_quantize_mxfp4(x, codes=None, scales=None, stream=None):
    """x: float32 [rows, k] -> (codes uint8 [rows, k/2], scales uint8 [rows, k/32])."""
    rows, k = x.shape
    codes = _empty((rows, k // 2), torch.uint8, x) if codes is None else codes
    scales = _empty((rows, k // 32), torch.uint8, x) if scales is None else scales
    _check(load().bsgemm_quantize_mxfp4(rows, k, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def bsgemm_run(fmt, a, a_scales, a_tscale, b, b_scales, b_tscale, k, c=None, stream=None):
    """C[m, n] (BF16 bits as int16/uint16 tensor) = deq(A) @ deq(B)^T; k is the logical K."""
    m, n = a.shape[0], b.shape[0]
    c = _empty((m, n), torch.int16, a) if c is None else c
    _check(load().bsgemm_run(fmt, m, n, k, _ptr(a), _ptr(a_scales), _ptr(a_tscale), _ptr(b),
                             _ptr(b_scales), _ptr(b_tscale), _ptr(c), _stream(stream)))
    return c


def bsgemm_grouped_run(a, a_scales, a_tscale, group_offsets, w_bf16, k, c=None, stream=None):
    """Grouped NVFP4 A [m_total, k] x BF16 W [G, n, k] -> C [m_total, n] (BF16 bits)."""
    G, n = w_bf16.shape[0], w_bf16.shape[1]
    m_total = a.shape[0]
    c = _empty((m_total, n), torch.int16, a) if c is None else c
    _check(load().bsgemm_grouped_run(G, m_total, n, k, _ptr(a), _ptr(a_scales), _ptr(a_tscale),
                                     _ptr(group_offsets), _ptr(w_bf16), _ptr(c), _stream(stream)))
    return c


def bsgemm_grouped_run_ex(a, a_scales, a_tscale, group_offsets, w, k, w_dtype=BSGEMM_W_BF16, bias=None,
                          gamma=None, gather_idx=None, scatter_idx=None, m_total=None, c=None, stream=None):
    """Grouped NVFP4 A [a_rows, k] x dense W [G, n, k] (BF16 or FP16 bits) with optional
    bias [G, n], gamma [m_total], gather_idx [m_total] and scatter_idx [m_total] -> C
    [m_total, n] (BF16 bits).  m_total defaults to the gather length, else to a_rows."""
    G, n = w.shape[0], w.shape[1]
    a_rows = a.shape[0]
    if m_total is None:
        m_total = gather_idx.shape[0] if gather_idx is not None else a_rows
    c = _empty((m_total, n), torch.int16, a) if c is None else c
    _check(load().bsgemm_grouped_run_ex(G, m_total, n, k, a_rows, _ptr(a), _ptr(a_scales), _ptr(a_tscale),
                                        _ptr(group_offsets), w_dtype, _ptr(w), _ptr(bias), _ptr(gamma),
                                        _ptr(gather_idx), _ptr(scatter_idx), _ptr(c), _stream(stream)))
    return c


def bsgemm_grouped_kragged_run(a, a_scales, a_tscale, k_offsets, w, k, w_dtype=BSGEMM_W_BF16, c=None,
                               stream=None):
    """K-ragged grouped NVFP4 A [m, k] x dense W [n, k] (BF16 or FP16 bits), groups split K at
    k_offsets [G + 1] -> C [G, m, n] (BF16 bits)."""
    G = k_offsets.shape[0] - 1
    m, n = a.shape[0], w.shape[0]
    c = _empty((G, m, n), torch.int16, a) if c is None else c
    _check(load().bsgemm_grouped_kragged_run(G, m, n, k, _ptr(a), _ptr(a_scales), _ptr(a_tscale),
                                             _ptr(k_offsets), w_dtype, _ptr(w), _ptr(c), _stream(stream)))
    return c


def bsgemm_w4a16_run(x_bf16, w, w_scales, w_tscale, c=None, stream=None):
    """BF16 X [m, k] x NVFP4 W [n, k] -> C [m, n] (BF16 bits)."""
    m, k = x_bf16.shape
    n = w.shape[0]
    c = _empty((m, n), torch.int16, x_bf16) if c is None else c
    _check(load().bsgemm_w4a16_run(m, n, k, _ptr(x_bf16), _ptr(w), _ptr(w_scales), _ptr(w_tscale),
                                   _ptr(c), _stream(stream)))
    return c


def bsgemm_w4a16_run_config(config, x_bf16, w, w_scales, w_tscale, c=None, stream=None):
    """bsgemm_w4a16_run with configuration `config` (id or name) forced."""
    if isinstance(config, str):
        config = w4a16_config_id(config)
    m, k = x_bf16.shape
    n = w.shape[0]
    c = _empty((m, n), torch.int16, x_bf16) if c is None else c
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
