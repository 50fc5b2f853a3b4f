"""Register and LDS budgets of the gfx950 kernels, and the memory
instructions they use (CPU only: hipcc's resource-usage remarks and its
assembly, no GPU).

A VGPR spill in a main loop goes to scratch memory and costs more than any
scheduling choice, and it appears silently when a change shifts the
compiler's register allocation.  Every kernel must fit the CU's LDS, and
none may spill except the ones listed, whose spills sit outside their main
loops (epilogue address registers) or in a fallback path; outside the
fallback paths, no scratch access may sit inside a loop that issues MFMAs.

Every global write must go through the vector memory path: the library
writes nothing through the scalar data cache (no scalar stores or atomics,
no scalar cache write-back or discard)."""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_scaled_precision_bsgemm_amd import build as B

LDS_BYTES = 160 * 1024
# kernel-name fragment -> most VGPR spills accepted
SPILL_ALLOWED = {
    "grouped_ring_kernel": 8,      # the row-chunk epilogue's addresses, after the main loop
    "nvfp4_gemm_ring_kernel": 1,   # likewise
    "mx_gemm_kernelILb1E": 40,     # register-staged MXFP4 fallback (K % 128 != 0)
}


def _hipcc():
    path = "/opt/rocm/bin/hipcc"
    return path if os.path.exists(path) else shutil.which("hipcc")


# scalar-memory writes: stores, atomics, cache write-back / discard
SCALAR_WRITE = re.compile(r"^\s*s_(store|atomic|dcache_wb|dcache_discard|buffer_store|buffer_atomic|scratch_store)\w*",
                          re.MULTILINE)


# kernels whose spills may sit inside an MFMA loop (fallback paths only)
LOOP_SPILL_ALLOWED = ("mx_gemm_kernelILb1E",)

LABEL = re.compile(r"^(\.LBB\d+_\d+):")
BACK_BRANCH = re.compile(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)")


def _scratch_in_mfma_loops(text):
    """Per kernel in an assembly listing: scratch accesses that lie inside a
    loop (a label and a later branch back to it) whose body issues MFMAs."""
    lines = text.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\S*:", l)]
    out = {}
    for a, b in zip(starts, starts[1:] + [len(lines)]):
        labels, hits = {}, 0
        for i in range(a, b):
            m = LABEL.match(lines[i])
            if m:
                labels[m.group(1)] = i
            m = BACK_BRANCH.search(lines[i])
            if m and m.group(1) in labels:
                body = lines[labels[m.group(1)]:i + 1]
                if any("v_mfma" in l for l in body):
                    hits += sum(1 for l in body if "scratch_" in l and not l.lstrip().startswith(";"))
        out[lines[a].split(":")[0]] = hits
    return out


def _resources(src, tmp):
    asm = os.path.join(tmp, src + ".s")
    cmd = [_hipcc()] + [f for f in B.COMMON_FLAGS if f != "-Wall"] + B.EXTRA_FLAGS.get(src, []) + \
        (["-x", "hip"] if src.endswith(".cpp") else []) + \
        ["--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", asm,
         "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    with open(asm) as f:
        text = f.read()
    bad = SCALAR_WRITE.findall(text)
    assert not bad, f"{src}: scalar-memory writes in the device code: {sorted(set(bad))}"
    for name, n in _scratch_in_mfma_loops(text).items():
        assert n == 0 or any(k in name for k in LOOP_SPILL_ALLOWED), \
            f"{src}: {name} has {n} scratch accesses inside a loop that issues MFMAs"
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs Spill|AGPRs|VGPRs|LDS Size \[bytes/block\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.skipif(_hipcc() is None, reason="hipcc is not installed")
def test_kernel_register_and_lds_budgets(tmp_path):
    srcs = [s for s in B.SOURCES if s.endswith(".hip")]
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        per_src = dict(zip(srcs, ex.map(lambda s: _resources(s, str(tmp_path)), srcs)))
    seen = 0
    for src, kernels in per_src.items():
        for name, res in kernels.items():
            seen += 1
            assert res.get("LDS Size [bytes/block]", 0) <= LDS_BYTES, (src, name, res)
            assert res.get("VGPRs", 0) + res.get("AGPRs", 0) <= 512, (src, name, res)
            cap = next((v for k, v in SPILL_ALLOWED.items() if k in name), 0)
            assert res.get("VGPRs Spill", 0) <= cap, f"{src}: {name} spills {res.get('VGPRs Spill')} VGPRs"
    assert seen >= 20   # every kernel of the library was reported


def test_scratch_in_mfma_loops_finder():
    listing = "\n".join([
        "_Zk1:", ".LBB0_1:", "\tv_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]",
        "\tscratch_load_dword v8, off, off", "\ts_cbranch_scc0 .LBB0_1", "\tscratch_store_dword off, v1, off",
        "_Zk2:", ".LBB1_1:", "\tv_add_u32 v0, v0, v1", "\tscratch_load_dword v8, off, off", "\ts_cbranch_scc0 .LBB1_1",
        "\tv_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]", "\tscratch_store_dword off, v1, off"])
    # k1: one access inside its MFMA loop (the one after the loop does not count);
    # k2: its loop issues no MFMA
    assert _scratch_in_mfma_loops(listing) == {"_Zk1": 1, "_Zk2": 0}


def test_scalar_write_pattern():
    # the pattern catches the scalar-memory write forms and nothing the kernels legitimately use
    for line in ("\ts_store_dword s4, s[0:1], 0x0", "  s_atomic_add s2, s[4:5], 0x10", "\ts_dcache_wb",
                 "\ts_buffer_store_dwordx2 s[2:3], s[8:11], 0x0"):
        assert SCALAR_WRITE.search(line), line
    for line in ("\ts_load_dwordx2 s[0:1], s[0:1], 0x0", "\tglobal_store_dword v0, v0, s[0:1]",
                 "\tbuffer_store_dwordx4 v[0:3], v4, s[8:11], 0 offen", "\ts_waitcnt lgkmcnt(0)",
                 "\tglobal_atomic_umax v0, v1, s[0:1]"):
        assert not SCALAR_WRITE.search(line), line
