"""Host-side tests of the C ABI (CPU only, no GPU compute).

The library must load and export every entry point that include/bsgemm.h
declares.  Argument validation must return the documented status codes
before anything is launched; pointers in these tests are fake and are never
dereferenced.  The "no device" case runs only where no GPU is visible."""

import ctypes
import os
import re
import threading

import pytest

from block_scaled_precision_bsgemm_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 0x10000          # fake, 16-byte aligned "device" address
MIS = 0x10004        # fake, misaligned


@pytest.fixture(scope="module")
def so():
    return L.load()


def test_exports_every_declared_symbol(so):
    header = open(os.path.join(ROOT, "include", "bsgemm.h")).read()
    declared = set(re.findall(r"\b(bsgemm_\w+)\s*\(", header))
    assert declared == set(L.SIGNATURES), (declared, set(L.SIGNATURES))
    for name in declared:
        assert hasattr(so, name)
    nm = os.popen(f"nm -D --defined-only {L.LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}\b", nm), name


def test_status_strings_and_version(so):
    assert so.bsgemm_status_string(0) == b"BSGEMM_OK"
    for code, name in [(1, b"BSGEMM_ERR_INVALID_ARG"), (2, b"BSGEMM_ERR_UNSUPPORTED"),
                       (3, b"BSGEMM_ERR_BAD_ALIGNMENT"), (4, b"BSGEMM_ERR_DEVICE"),
                       (5, b"BSGEMM_ERR_RESOURCE"), (6, b"BSGEMM_ERR_LAUNCH")]:
        assert so.bsgemm_status_string(code) == name
    assert so.bsgemm_status_string(99) == b"unknown status"
    assert so.bsgemm_version() == 600


def run(so, fmt=L.BSGEMM_NVFP4, m=64, n=64, k=64, a=P, sa=P, ta=P, b=P, sb=P, tb=P, c=P):
    return so.bsgemm_run(fmt, m, n, k, a, sa, ta, b, sb, tb, c, None)


def test_run_validation(so):
    assert run(so, a=None) == L.BSGEMM_ERR_INVALID_ARG
    assert b"a is NULL" in so.bsgemm_last_error()
    assert run(so, c=None) == L.BSGEMM_ERR_INVALID_ARG
    assert run(so, m=-1) == L.BSGEMM_ERR_INVALID_ARG
    assert run(so, ta=None) == L.BSGEMM_ERR_INVALID_ARG
    assert run(so, k=48) == L.BSGEMM_ERR_UNSUPPORTED
    assert run(so, fmt=7) == L.BSGEMM_ERR_UNSUPPORTED
    assert run(so, fmt=L.BSGEMM_MXFP8) == L.BSGEMM_ERR_UNSUPPORTED      # tensor scales given
    assert run(so, fmt=L.BSGEMM_MXFP4) == L.BSGEMM_ERR_UNSUPPORTED
    assert b"MXFP4 takes no tensor scales" in so.bsgemm_last_error()
    assert run(so, fmt=L.BSGEMM_MXFP4, ta=None, tb=None, k=80) == L.BSGEMM_ERR_UNSUPPORTED
    assert run(so, fmt=L.BSGEMM_MXFP4, ta=None, tb=None, sb=MIS) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert run(so, fmt=L.BSGEMM_MXFP8_EXACT) == L.BSGEMM_ERR_UNSUPPORTED   # tensor scales given
    assert b"MXFP8 takes no tensor scales" in so.bsgemm_last_error()
    assert run(so, fmt=L.BSGEMM_MXFP8_EXACT, ta=None, tb=None, k=80) == L.BSGEMM_ERR_UNSUPPORTED
    assert run(so, fmt=L.BSGEMM_MXFP8_EXACT, ta=None, tb=None, a=MIS) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert run(so, fmt=5) == L.BSGEMM_ERR_UNSUPPORTED
    assert run(so, a=MIS) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert run(so, c=MIS) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert run(so, sa=MIS) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert b"a_scales is not 16-byte aligned" in so.bsgemm_last_error()
    assert run(so, sb=MIS) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert run(so, k=1 << 22) == L.BSGEMM_ERR_RESOURCE
    # an empty operand may be NULL; the error then comes from the next check
    assert run(so, m=0, a=None, sa=None, c=None, k=48) == L.BSGEMM_ERR_UNSUPPORTED


def test_quantize_validation(so):
    q4, q8, m4 = so.bsgemm_quantize_nvfp4, so.bsgemm_quantize_mxfp8, so.bsgemm_quantize_mxfp4
    assert m4(-1, 64, P, P, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert m4(4, 64, None, P, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert m4(4, 64, P, P, None, None) == L.BSGEMM_ERR_INVALID_ARG
    assert m4(4, 48, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED
    assert m4(4, 64, MIS, P, P, None) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert m4(4, 64, P, MIS, P, None) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert m4(4, 64, P, P, MIS, None) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert q4(4, 64, None, P, P, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert q4(4, 64, P, P, P, None, None) == L.BSGEMM_ERR_INVALID_ARG
    assert q4(4, 40, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED
    assert q4(4, 64, MIS, P, P, P, None) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert q4(4, 64, P, P, MIS, P, None) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert q8(-1, 64, P, P, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert q8(4, 64, P, None, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert q8(4, 16, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED
    assert q8(4, 64, P, MIS, P, None) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert q8(4, 64, P, P, MIS, None) == L.BSGEMM_ERR_BAD_ALIGNMENT


def test_grouped_and_w4a16_validation(so):
    g = so.bsgemm_grouped_run
    assert g(0, 64, 64, 64, P, P, P, P, P, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert g(2, 64, 64, 64, P, P, P, None, P, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert g(2, 64, 64, 64, P, P, None, P, P, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert g(2, 64, 64, 33, P, P, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED
    assert g(2, 64, 64, 64, P, P, P, P, MIS, P, None) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert g(2, 64, 64, 64, P, MIS, P, P, P, P, None) == L.BSGEMM_ERR_BAD_ALIGNMENT
    w = so.bsgemm_w4a16_run
    assert w(1, 64, 64, None, P, P, P, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert w(1, 64, 64, P, P, P, None, P, None) == L.BSGEMM_ERR_INVALID_ARG
    assert w(1, 64, 80, P, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED
    assert w(1, 64, 64, MIS, P, P, P, P, None) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert w(1, 64, 64, P, P, MIS, P, P, None) == L.BSGEMM_ERR_BAD_ALIGNMENT


def test_grouped_ex_validation(so):
    def gx(G=2, m=64, n=64, k=64, a_rows=64, a=P, sa=P, ta=P, off=P, wd=L.BSGEMM_W_BF16, w=P,
           bias=None, gamma=None, gather=None, scatter=None, c=P):
        return so.bsgemm_grouped_run_ex(G, m, n, k, a_rows, a, sa, ta, off, wd, w, bias, gamma, gather,
                                        scatter, c, None)
    assert gx(G=0) == L.BSGEMM_ERR_INVALID_ARG
    assert gx(a_rows=-1) == L.BSGEMM_ERR_INVALID_ARG
    assert gx(a_rows=32) == L.BSGEMM_ERR_INVALID_ARG          # a_rows != m without gather
    assert b"a_rows must equal m_total" in so.bsgemm_last_error()
    assert gx(ta=None) == L.BSGEMM_ERR_INVALID_ARG
    assert gx(off=None) == L.BSGEMM_ERR_INVALID_ARG
    assert gx(wd=7) == L.BSGEMM_ERR_UNSUPPORTED
    assert gx(k=48) == L.BSGEMM_ERR_UNSUPPORTED
    assert gx(w=MIS) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert gx(gamma=0x10002) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert gx(scatter=0x10001) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert gx(gather=P, a_rows=1 << 26, k=1024) == L.BSGEMM_ERR_RESOURCE   # A past 2^31 bytes
    import torch
    if not torch.cuda.is_available():
        assert gx(gather=P, a_rows=32, bias=P, gamma=P, scatter=P, wd=L.BSGEMM_W_F16) == L.BSGEMM_ERR_DEVICE


def test_w4a16_configs_and_exhaustive_selector(so):
    n_cfg = so.bsgemm_w4a16_num_configs()
    names = [so.bsgemm_w4a16_config_name(i).decode() for i in range(n_cfg)]
    assert n_cfg == 34 and len(set(names)) == n_cfg and names[0] == "valu_gemv"
    assert so.bsgemm_w4a16_config_name(n_cfg) is None and so.bsgemm_w4a16_config_name(-1) is None
    tile = {nm: (0 if nm.startswith("valu_gemv") else int(nm.split("_")[1][1:])) for nm in names}

    def mtile(nm):
        return int(nm.split("_")[1][1:])

    def grid(m, n, mt, nb):
        return -(-n // nb) * -(-m // mt)
    # Exhaustive over the grid, checking the selector's stated rule by its
    # properties: the vector ALU for m <= 2 or m <= 4 with n <= 2048; for
    # n >= 14273 the thin tile kernels (m <= 16 with k % 512 == 0, and
    # 48 < m <= 64 with k % 256 == 0 while the grid is one wave); (2 W
    # rows per wave where 4 would leave few waves); then 16-row W slabs with
    # an 8-way K split while that grid fits one wave of 256 workgroups (m
    # tile 16, else 32), or two waves with the 16-row tile at k >= 7168; then
    # the vector ALU for m <= 8 with m * n <= 24576; then the 128 x 128 tile
    # kernel for m > 64 once its grid fills a wave (224 tiles); then, with
    # the smallest m tile whose grid fits one wave with 64-row slabs: the
    # 16 x 64 tile kernel (16-row m tile, k % 512 == 0), the 64 x 64 one
    # (64-row m tile, n >= 6144, k % 256 == 0), or the four-tile kernel
    # (variant by m tile and K); otherwise no tile fits: the tile kernel's
    # 128 x 128 tiles (m > 128, where 2.5 x their rounds of 256 workgroups
    # are fewer than the 64 x 64 tiles' rounds) or 64 x 64 tiles, or a
    # four-tile pick with 64-row slabs.
    decisions = 0
    for n in (1, 64, 896, 1536, 3072, 4096, 4112, 5120, 7168, 8192, 10240, 14336, 65536):
        for k in (32, 4096, 7168, 8192, 14336):
            for m in list(range(0, 130)) + [192, 256, 384, 1024, 1 << 20]:
                c = so.bsgemm_w4a16_select(m, n, k)
                decisions += 1
                assert 0 <= c < n_cfg
                nm = names[c]
                if m > 2 and -(-n // 64) >= 224 and ((m <= 16 and k % 512 == 0) or
                                                      (48 < m <= 64 and k % 256 == 0 and -(-n // 64) <= 256)):
                    assert nm == ("tile_m16_n64" if m <= 16 else "tile_m64_n64"), (m, n, k, nm)
                    continue
                slabs = -(-n // 16)
                if m <= 2 or (m <= 4 and n <= 2048):
                    ks = None
                elif slabs * -(-m // 16) <= 256:
                    ks = "mfma_m16_n16_ks8_r4"
                elif slabs * -(-m // 32) <= 256:
                    ks = "mfma_m32_n16_ks8"
                elif k >= 7168 and slabs * -(-m // 16) <= 512:
                    ks = "mfma_m16_n16_ks8_r4"
                else:
                    ks = None
                valu = m <= 2 or (m <= 4 and n <= 2048) or (ks is None and m <= 8 and m * n <= 24576)
                assert nm.startswith("valu_gemv") == valu, (m, n, nm)
                if valu:
                    w2 = n <= 2560 or (m <= 1 and n <= 4096)
                    assert nm == ("valu_gemv_w2" if w2 else "valu_gemv"), (m, n, nm)
                    continue
                if ks:
                    assert nm == ks, (m, n, k, nm)
                    continue
                if m > 64 and k % 128 == 0 and -(-m // 128) * -(-n // 128) >= 224:
                    assert nm == "tile_m128_n128", (m, n, k, nm)
                    continue
                fits = [t for t in (16, 32, 64) if grid(m, n, t, 64) <= 256]
                if fits:
                    if fits[0] == 16 and k % 512 == 0:
                        assert nm == "tile_m16_n64", (m, n, k, nm)
                    elif fits[0] == 64 and n >= 6144 and k % 256 == 0:
                        assert nm == "tile_m64_n64", (m, n, k, nm)
                    else:
                        sfx = {16: "_b2" if k >= 7168 else "_r2", 32: "_b2" if k >= 4096 else "", 64: "_t2"}[fits[0]]
                        assert nm == f"mfma_m{fits[0]}_nfit" + sfx, (m, n, k, nm)
                elif nm in ("tile_m128_n128", "tile_m64_n64", "mfma_m64_n64_t2"):
                    # 64-row slabs over more than one wave
                    r128 = -(-(-(-m // 128) * -(-n // 128)) // 256)
                    r64 = -(-(-(-m // 64) * -(-n // 64)) // 256)
                    if m > 128 and k % 128 == 0 and 5 * r128 < 2 * r64:
                        assert nm == "tile_m128_n128", (m, n, k, nm)
                    else:
                        assert nm == ("tile_m64_n64" if k % 256 == 0 else "mfma_m64_n64_t2"), (m, n, k, nm)
                else:
                    assert nm.endswith("_n64"), (m, n, nm)
    assert decisions == 13 * 5 * 135
    assert so.bsgemm_w4a16_select(4, 64, 48) == -1 and so.bsgemm_w4a16_select(-1, 64, 64) == -1


def test_w4a16_forced_config_validation(so, monkeypatch):
    rc = so.bsgemm_w4a16_run_config
    assert rc(99, 1, 64, 64, P, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED
    assert rc(-1, 1, 64, 64, P, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED
    assert rc(0, 70000, 64, 64, P, P, P, P, P, None) == L.BSGEMM_ERR_RESOURCE     # vector ALU: m <= 65535
    assert b"valu_gemv" in so.bsgemm_last_error()
    assert rc(3, 1, 64, 80, P, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED      # k % 32
    monkeypatch.setenv("BSGEMM_W4A16_FORCE_CONFIG", "no_such_tile")
    assert so.bsgemm_w4a16_run(1, 64, 64, P, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED
    assert b"FORCE_CONFIG" in so.bsgemm_last_error()
    assert rc(31, 1, 64, 256, P, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED    # tile m16: k % 512
    assert b"k % 512" in so.bsgemm_last_error()
    assert rc(33, 1, 64, 96, P, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED     # tile m128: k % 128
    monkeypatch.setenv("BSGEMM_W4A16_FORCE_CONFIG", "34")
    assert so.bsgemm_w4a16_run(1, 64, 64, P, P, P, P, P, None) == L.BSGEMM_ERR_UNSUPPORTED
    import torch
    if not torch.cuda.is_available():
        monkeypatch.setenv("BSGEMM_W4A16_FORCE_CONFIG", "mfma_m32_n16")
        assert so.bsgemm_w4a16_run(1, 64, 64, P, P, P, P, P, None) == L.BSGEMM_ERR_DEVICE


def test_grouped_kragged_validation(so):
    def kr(G=2, m=64, n=64, k=512, a=P, sa=P, ta=P, off=P, wd=L.BSGEMM_W_BF16, w=P, c=P):
        return so.bsgemm_grouped_kragged_run(G, m, n, k, a, sa, ta, off, wd, w, c, None)
    assert kr(G=0) == L.BSGEMM_ERR_INVALID_ARG
    assert kr(off=None) == L.BSGEMM_ERR_INVALID_ARG
    assert kr(ta=None) == L.BSGEMM_ERR_INVALID_ARG
    assert kr(k=384) == L.BSGEMM_ERR_UNSUPPORTED                 # not a multiple of 256
    assert b"multiple of 256" in so.bsgemm_last_error()
    assert kr(wd=0) == L.BSGEMM_ERR_UNSUPPORTED
    assert kr(c=MIS) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert kr(off=0x10002) == L.BSGEMM_ERR_BAD_ALIGNMENT
    assert kr(m=0, a=None, sa=None, c=None) in (L.BSGEMM_OK, L.BSGEMM_ERR_DEVICE)


def test_last_error_is_per_thread(so):
    assert run(so, a=None) == L.BSGEMM_ERR_INVALID_ARG
    seen = {}

    def other():
        seen["msg"] = so.bsgemm_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == b""
    assert b"a is NULL" in so.bsgemm_last_error()


def test_no_device_is_reported_not_launched(so):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; this case checks the no-device path")
    assert run(so) == L.BSGEMM_ERR_DEVICE
    assert so.bsgemm_quantize_mxfp8(4, 64, P, P, P, None) == L.BSGEMM_ERR_DEVICE
    assert so.bsgemm_quantize_mxfp4(4, 64, P, P, P, None) == L.BSGEMM_ERR_DEVICE
    assert run(so, fmt=L.BSGEMM_MXFP4, ta=None, tb=None) == L.BSGEMM_ERR_DEVICE
    assert run(so, fmt=L.BSGEMM_MXFP8_EXACT, ta=None, tb=None) == L.BSGEMM_ERR_DEVICE


def test_binding_raises_on_error():
    import torch
    x = torch.zeros(4, 40)
    with pytest.raises(Exception):
        L.bsgemm_quantize_mxfp8(x)   # CPU tensor: rejected before any call


def test_binding_validates_before_calling():
    """The binding rejects wrong dtypes, shapes and layouts with ValueError
    before any call into the library (dtype and shape are checked before the
    device, so CPU tensors exercise them here)."""
    import torch
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)   # noqa: E731
    f32 = lambda *s: torch.zeros(*s, dtype=torch.float32)   # noqa: E731
    with pytest.raises(ValueError, match="dtype"):
        L.bsgemm_quantize_nvfp4(torch.zeros(4, 64, dtype=torch.float64))
    with pytest.raises(ValueError, match="2-D"):
        L.bsgemm_quantize_mxfp8(f32(256))
    with pytest.raises(ValueError, match="codes: shape"):
        L.bsgemm_quantize_nvfp4(f32(4, 64), codes=u8(4, 16))
    with pytest.raises(ValueError, match="tensor_scale"):
        L.bsgemm_quantize_nvfp4(f32(4, 64), codes=u8(4, 32), scales=u8(4, 4), tensor_scale=f32(2))
    ts = f32(1)
    # NVFP4 operand [rows, 64]: codes [rows, 32], scales [rows, 4]
    with pytest.raises(ValueError, match="a_scales: shape"):
        L.bsgemm_run(L.BSGEMM_NVFP4, u8(8, 32), u8(8, 2), ts, u8(4, 32), u8(4, 4), ts, 64)
    with pytest.raises(ValueError, match="a: shape"):          # k disagrees with the codes
        L.bsgemm_run(L.BSGEMM_NVFP4, u8(8, 32), u8(8, 4), ts, u8(4, 32), u8(4, 4), ts, 128)
    with pytest.raises(ValueError, match="b: shape"):          # MXFP8 codes are [rows, k]
        L.bsgemm_run(L.BSGEMM_MXFP8_EXACT, u8(8, 64), u8(8, 2), None, u8(4, 32), u8(4, 2), None, 64)
    with pytest.raises(ValueError, match="c: shape"):
        L.bsgemm_run(L.BSGEMM_MXFP4, u8(8, 32), u8(8, 2), None, u8(4, 32), u8(4, 2), None, 64,
                     c=torch.zeros(4, 8, dtype=torch.int16))
    with pytest.raises(ValueError, match="c: dtype"):
        L.bsgemm_run(L.BSGEMM_MXFP4, u8(8, 32), u8(8, 2), None, u8(4, 32), u8(4, 2), None, 64,
                     c=torch.zeros(8, 4, dtype=torch.float32))
    with pytest.raises(ValueError, match="group_offsets"):
        L.bsgemm_grouped_run(u8(8, 32), u8(8, 4), ts, torch.zeros(2, dtype=torch.int32),
                             torch.zeros(2, 16, 64, dtype=torch.int16), 64)
    with pytest.raises(ValueError, match="gamma"):
        L.bsgemm_grouped_run_ex(u8(8, 32), u8(8, 4), ts, torch.zeros(3, dtype=torch.int32),
                                torch.zeros(2, 16, 64, dtype=torch.int16), 64, gamma=f32(7))
    with pytest.raises(ValueError, match="w_scales: shape"):
        L.bsgemm_w4a16_run(torch.zeros(2, 64, dtype=torch.bfloat16), u8(16, 32), u8(16, 2), ts)
    with pytest.raises(ValueError, match="k_offsets"):
        L.bsgemm_grouped_kragged_run(u8(8, 128), u8(8, 16), ts, torch.zeros(3, dtype=torch.int64),
                                     torch.zeros(16, 256, dtype=torch.int16), 256)
    with pytest.raises(ValueError, match="w: shape"):
        L.bsgemm_grouped_kragged_run(u8(8, 128), u8(8, 16), ts, torch.zeros(3, dtype=torch.int32),
                                     torch.zeros(16, 512, dtype=torch.int16), 256)
    with pytest.raises(ValueError, match="c: shape"):
        L.bsgemm_grouped_kragged_run(u8(8, 128), u8(8, 16), ts, torch.zeros(3, dtype=torch.int32),
                                     torch.zeros(16, 256, dtype=torch.int16), 256,
                                     c=torch.zeros(2, 16, 8, dtype=torch.int16))
    # every check passes: only the placement check (CPU tensors) is left
    with pytest.raises(ValueError, match="device tensor"):
        L.bsgemm_grouped_kragged_run(u8(8, 128), u8(8, 16), ts, torch.zeros(3, dtype=torch.int32),
                                     torch.zeros(16, 256, dtype=torch.uint16), 256)
    with pytest.raises(ValueError, match="device tensor"):
        L.bsgemm_grouped_run_ex(u8(8, 32), u8(8, 4), ts, torch.zeros(3, dtype=torch.int32),
                                torch.zeros(2, 16, 64, dtype=torch.float16), 64, w_dtype=L.BSGEMM_W_F16,
                                bias=f32(2, 16), gamma=f32(8), gather_idx=torch.zeros(8, dtype=torch.int32),
                                scatter_idx=torch.zeros(8, dtype=torch.int32))
    with pytest.raises(ValueError, match="device tensor"):
        L.bsgemm_w4a16_run(torch.zeros(2, 64, dtype=torch.bfloat16), u8(16, 32), u8(16, 4), ts)
    with pytest.raises(ValueError, match="device tensor"):
        L.bsgemm_run(L.BSGEMM_MXFP8_EXACT, u8(8, 64), u8(8, 2), None, u8(4, 64), u8(4, 2), None, 64)
