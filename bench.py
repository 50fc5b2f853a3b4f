#!/usr/bin/env python3
"""Benchmark of the block-scaled GEMM library on one MI355X.

One step is one NVFP4 x NVFP4 GEMM at M = N = K = 16384 (BF16 output).  Its
operands are already quantized and resident in HBM.  This is the 16k-square
workload of "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA Vera
Rubin NVL72", section "Building the GEMM", with 1% outlier rows.  ``value`` is
its throughput in TFLOPS, from the wall clock around exactly ``--steps``
launches, synchronised on both sides.

Nothing is trusted before it is checked ("Add sm121 (GB10) tier to the 4-bit
GEMM dispatch heuristic", tile-selection follow-up: sentinel prefill and a
reference gate before any timing counts).  Every output buffer is prefilled
with a BF16 NaN; after timing, the outputs of the last launch are compared
with the CPU oracle, which quantizes the same FP32 inputs itself (its bytes
must equal the GPU's).  The headline is checked on every element of its
output; the other rows on samples.  ``parity`` in the JSON line holds
every verdict, and any failure makes the exit status non-zero.

The same JSON line carries:
  - ``roofline``: the GEMM kernel's average time from HIP events on its own
    stream over the timed region, against the dense peak of the MFMA it runs
    (FP16: the NVFP4 E4M3 scales force an exact FP16 path on gfx950);
    ``frac_of_fp4_peak`` gives the fraction of the FP4 peak too.
  - ``cpu_baseline``: the CPU oracle's GEMM on the whole headline problem
    (the parity reference), timed on the host's cores, with the CPU model.
  - ``rows``: every part of the hot path, each timed as 15 repeats of a HIP
    graph of 20 launches after 10 warm-up launches (median, min and max per
    launch; "TokenSpeed MLA 2", section "Benchmark results").  Graph output is
    compared bit for bit with an eager launch.  Inputs of the 4096^3 MXFP8
    and the W4A16 rows rotate through copies larger than the 256 MB Infinity
    Cache, so their operands are read cold.

``--only headline|mx|grouped|w4a16|big`` runs one group of rows (profiler
runs); all but ``big`` add a 1 GiB device copy that calibrates HBM byte
counters.  ``--no-parity`` skips the oracle checks.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOPS (and % of MFMA peak) for NVFP4/MXFP8 GEMM at 16384^3; W4A16 HBM GB/s"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK = {"f16": 2500.0, "bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0, "hbm_gbps": 8000.0}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "nvfp4_gemm_16384_hbm_counters.txt")
KERNEL_SOURCES = ["gemm_nvfp4.hip", "common.hpp"]
SENTINEL = 0x7FC0          # BF16 quiet NaN
REPS, ITERS, WARM = 15, 20, 10


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_scaled_precision_bsgemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_counters():
    """HBM bytes per launch of the headline kernel from the committed counter
    summary, or None when it is missing or was taken on other kernel source."""
    try:
        with open(COUNTERS_FILE) as fh:
            rec = json.loads("".join(l for l in fh if not l.startswith("#")))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- timing --

def graph_stats(fn, reps=REPS, iters=ITERS, warmup=WARM, out=None):
    """Per-launch ms of fn(i): `warmup` eager launches, then a HIP graph of
    `iters` launches fn(0..iters-1) replayed `reps` times, each replay timed
    with events.  Returns {median, min, max} and whether the graph's output
    (`out`, after the last replay) equals an eager launch's bit for bit."""
    import torch
    for i in range(warmup):
        fn(i)
    eager = None
    if out is not None:
        fn(iters - 1)
        torch.cuda.synchronize()
        eager = out.clone()
        out.fill_(SENTINEL)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) / iters)
    same = None if out is None else bool(torch.equal(out, eager))
    del g
    times.sort()
    return {"ms": times[len(times) // 2], "ms_min": times[0], "ms_max": times[-1], "graph_matches_eager": same}


def time_events(fn, steps, warmup):
    """Average ms per call from HIP events recorded on the current stream."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def flops_row(st, flops, peak_key, extra=None):
    tf = flops / (st["ms"] * 1e-3) / 1e12
    row = {"ms": round(st["ms"], 4), "ms_min": round(st["ms_min"], 4), "ms_max": round(st["ms_max"], 4),
           "tflops": round(tf, 2), f"frac_{peak_key}_peak": round(tf / PEAK[peak_key], 4),
           "graph_matches_eager": st["graph_matches_eager"], "timing": f"{REPS} x {ITERS} graph launches, median"}
    row.update(extra or {})
    return row


# ---------------------------------------------------------------- parity --

def oracle_rows(fn, x, chunk=1024, **kw):
    """Oracle quantizer `fn` over row chunks of x on a thread pool (numpy
    releases the GIL in its array kernels); each quantizer is per row once the
    tensor scale is fixed, so the chunks concatenate to the whole result."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    parts = [x[i:i + chunk] for i in range(0, x.shape[0], chunk)]
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        outs = list(ex.map(lambda p: fn(p, **kw), parts))
    return tuple(np.concatenate([o[j] for o in outs]) if np.ndim(outs[0][j]) else outs[0][j]
                 for j in range(len(outs[0])))


class Parity:
    """Collects per-row verdicts: quantized bytes equal to the oracle's, and
    GEMM outputs within the acceptance bound."""

    def __init__(self, enabled):
        self.enabled = enabled
        self.rows = {}

    def same_bytes(self, name, gpu, ref):
        import numpy as np
        ok = all(np.array_equal(np.asarray(g), np.asarray(r)) for g, r in zip(gpu, ref))
        rec = self.rows.setdefault(name, {"ok": True})
        rec["quantized_bytes_match"] = ok
        rec["ok"] = rec["ok"] and ok
        return ok

    def gemm(self, name, c_bits, cref, t, what):
        import numpy as np
        from oracle import gemm as G
        res = G.check(np.asarray(c_bits).view(np.uint16), cref, t)
        rec = self.rows.setdefault(name, {"ok": True})
        rec.update({"checked": what, "n": res["n"], "n_fail": res["n_fail"],
                    "worst_ratio": round(res["worst_ratio"], 4)})
        rec["ok"] = rec["ok"] and res["ok"]
        log(f"parity {name}: {what}: {'ok' if res['ok'] else 'FAIL'} (worst {res['worst_ratio']:.3g})")
        return res["ok"]

    def flag(self, name, ok, note):
        rec = self.rows.setdefault(name, {"ok": True})
        rec[note] = bool(ok)
        rec["ok"] = rec["ok"] and bool(ok)

    def ok(self):
        return all(r["ok"] for r in self.rows.values())


def sample(n, count, seed, must=()):
    import numpy as np
    idx = np.random.Generator(np.random.PCG64(seed)).choice(n, min(count, n), replace=False)
    return np.unique(np.concatenate([idx, np.asarray(must, dtype=np.int64), [0, n - 1]]))


def u16(t):
    import numpy as np
    return t.cpu().numpy().view(np.uint16)


def sentinel_out(shape, dev):
    import torch
    return torch.full(shape, SENTINEL, dtype=torch.int16, device=dev)


def no_nan(c):
    import torch
    return not torch.isnan(c.view(torch.bfloat16)).any().item()


# ------------------------------------------------------------------ rows --

def mx_rows(L, synth, dev, par, time_quantizers=False):
    """MXFP8 (native and exact), MXFP4 at 16384^3 on N(0, 1) inputs; MXFP8 at
    4096^3 with 8 operand copies rotated (and, with time_quantizers, the MXFP8
    and MXFP4 quantizers at 16384^2)."""
    import numpy as np
    import torch
    from oracle import gemm as G
    from oracle import quantize as Q
    rows = {}
    M = N = K = 16384
    n_el, flops = M * K, 2.0 * M * N * K
    log("generating MX 16k inputs")
    mx_a = synth.normal_f32((M, K), synth.SEEDS["mxfp8_4k.A"])
    mx_b = synth.normal_f32((N, K), synth.SEEDS["mxfp8_4k.B"])
    ri, ci = sample(M, 256, 41), sample(N, 256, 42)
    dma, dmb = torch.from_numpy(mx_a).to(dev), torch.from_numpy(mx_b).to(dev)
    c8a, s8a = L.bsgemm_quantize_mxfp8(dma)
    c8b, s8b = L.bsgemm_quantize_mxfp8(dmb)
    c4a, s4a = L.bsgemm_quantize_mxfp4(dma)
    c4b, s4b = L.bsgemm_quantize_mxfp4(dmb)
    if time_quantizers:
        st = graph_stats(lambda i: L.bsgemm_quantize_mxfp8(dma, c8a, s8a), iters=5)
        rows["quantize_mxfp8_16384x16384"] = {"ms": round(st["ms"], 4), "ms_min": round(st["ms_min"], 4),
                                              "gbps": round(n_el * (4 + 1.03125) / (st["ms"] * 1e-3) / 1e9, 1)}
        st = graph_stats(lambda i: L.bsgemm_quantize_mxfp4(dma, c4a, s4a), iters=5)
        rows["quantize_mxfp4_16384x16384"] = {"ms": round(st["ms"], 4), "ms_min": round(st["ms_min"], 4),
                                              "gbps": round(n_el * (4 + 0.53125) / (st["ms"] * 1e-3) / 1e9, 1)}
    del dma, dmb
    tri, tci = torch.from_numpy(ri).to(dev), torch.from_numpy(ci).to(dev)
    q8 = q4 = None
    if par.enabled:
        q8 = (Q.quantize_mxfp8(mx_a[ri]), Q.quantize_mxfp8(mx_b[ci]))
        q4 = (Q.quantize_mxfp4(mx_a[ri]), Q.quantize_mxfp4(mx_b[ci]))
        for name, q, ga, gb in (("mxfp8_gemm_16384", q8, (c8a, s8a), (c8b, s8b)),
                                ("mxfp4_gemm_16384", q4, (c4a, s4a), (c4b, s4b))):
            par.same_bytes(name, [t[tri].cpu().numpy() for t in ga] + [t[tci].cpu().numpy() for t in gb],
                           list(q[0]) + list(q[1]))
    del mx_a, mx_b
    c16 = sentinel_out((M, N), dev)
    for name, fmt, ops, peak in (("mxfp4_gemm_16384", L.BSGEMM_MXFP4, (c4a, s4a, c4b, s4b), "fp4"),
                                 ("mxfp8_gemm_16384", L.BSGEMM_MXFP8, (c8a, s8a, c8b, s8b), "fp8"),
                                 ("mxfp8_exact_gemm_16384", L.BSGEMM_MXFP8_EXACT, (c8a, s8a, c8b, s8b), "bf16")):
        log("timing", name)
        c16.fill_(SENTINEL)
        x, sx, y, sy = ops
        st = graph_stats(lambda i: L.bsgemm_run(fmt, x, sx, None, y, sy, None, K, c=c16), out=c16)
        extra = {"frac_fp8_peak": round(flops / (st["ms"] * 1e-3) / 1e12 / PEAK["fp8"], 4)} if peak == "bf16" else {}
        rows[name] = flops_row(st, flops, peak, extra)
        if par.enabled:
            par.flag(name, no_nan(c16), "no_unwritten_output")
            q = q4 if fmt == L.BSGEMM_MXFP4 else q8
            ref = (G.gemm_mxfp4 if fmt == L.BSGEMM_MXFP4 else G.gemm_mxfp8)(*q[0], *q[1])
            par.gemm(name, u16(c16[tri][:, tci]), *ref, f"{len(ri)} x {len(ci)} sampled outputs")
    del c4a, s4a, c4b, s4b, c8a, s8a, c8b, s8b, c16

    # 4096^3: 8 copies of the operands (8 x 34.6 MB > the 256 MB Infinity Cache)
    log("MXFP8 4096^3")
    a4, b4 = synth.mxfp8_inputs()
    q4a = L.bsgemm_quantize_mxfp8(torch.from_numpy(a4).to(dev))
    q4b = L.bsgemm_quantize_mxfp8(torch.from_numpy(b4).to(dev))
    copies = 8
    ops = [(q4a[0].clone(), q4a[1].clone(), q4b[0].clone(), q4b[1].clone()) for _ in range(copies)]
    c4 = sentinel_out((4096, 4096), dev)
    st = graph_stats(lambda i: L.bsgemm_run(L.BSGEMM_MXFP8, ops[i % copies][0], ops[i % copies][1], None,
                                            ops[i % copies][2], ops[i % copies][3], None, 4096, c=c4),
                     iters=2 * copies, out=c4)
    rows["mxfp8_gemm_4096"] = flops_row(st, 2.0 * 4096 ** 3, "fp8", {"operand_copies_rotated": copies})
    if par.enabled:
        r4 = sample(4096, 256, 43)
        qa = Q.quantize_mxfp8(a4[r4])
        qb = oracle_rows(Q.quantize_mxfp8, b4)
        par.same_bytes("mxfp8_gemm_4096", [q4a[0][torch.from_numpy(r4).to(dev)].cpu().numpy(),
                                           q4a[1][torch.from_numpy(r4).to(dev)].cpu().numpy(),
                                           q4b[0].cpu().numpy(), q4b[1].cpu().numpy()], list(qa) + list(qb))
        par.flag("mxfp8_gemm_4096", no_nan(c4), "no_unwritten_output")
        par.gemm("mxfp8_gemm_4096", u16(c4)[r4], *G.gemm_mxfp8(*qa, *qb), f"{len(r4)} rows x 4096 columns")
    return rows


def grouped_rows(L, synth, dev, par):
    """The 32-group NVFP4 x BF16 problem, the same problem with FP16 weights and
    every routing and epilogue variant, and its K-ragged weight-gradient form."""
    import numpy as np
    import torch
    from oracle import gemm as G
    from oracle import quantize as Q

    rows = {}
    log("generating grouped inputs")
    gx, off, gw = synth.grouped_inputs()
    qg = L.bsgemm_quantize_nvfp4(torch.from_numpy(gx).to(dev))
    dw = torch.from_numpy(gw.view(np.int16)).to(dev)
    doff = torch.from_numpy(off).to(dev)
    counts = np.diff(off.astype(np.int64))
    must = [r for g in range(32) if counts[g] for r in (off[g], off[g + 1] - 1)]
    srows = sample(16384, 64, 44, must)
    qa = None
    if par.enabled:
        sta = Q.nvfp4_tensor_scale(gx)
        qa = Q.quantize_nvfp4(gx[srows], tensor_scale=sta)
        tr = torch.from_numpy(srows).to(dev)
        par.same_bytes("grouped_nvfp4_bf16", [qg[0][tr].cpu().numpy(), qg[1][tr].cpu().numpy(),
                                              np.float32(qg[2].item())], list(qa))
    cg = sentinel_out((16384, 2048), dev)
    gflops = 2.0 * 16384 * 2048 * 7168
    gbytes = 16384 * 7168 * 0.5625 + int((counts > 0).sum()) * 2048 * 7168 * 2 + 16384 * 2048 * 2
    st = graph_stats(lambda i: L.bsgemm_grouped_run(*qg, doff, dw, 7168, c=cg), out=cg)
    rows["grouped_nvfp4_bf16"] = flops_row(st, gflops, "bf16", {
        "gbps_algorithmic": round(gbytes / (st["ms"] * 1e-3) / 1e9, 1),
        "groups_nonempty": int((counts > 0).sum()), "max_group_rows": int(counts.max())})
    if par.enabled:
        par.flag("grouped_nvfp4_bf16", no_nan(cg), "no_unwritten_output")
        # the oracle indexes A by row: place the sampled rows in a full-size A
        qfa = (np.zeros((16384, 3584), np.uint8), np.zeros((16384, 448), np.uint8), qa[2])
        qfa[0][srows], qfa[1][srows] = qa[0], qa[1]
        par.gemm("grouped_nvfp4_bf16", u16(cg)[srows], *G.grouped_nvfp4_bf16(*qfa, off, gw, rows=srows),
                 f"{len(srows)} rows (first/last of every group + random) x 2048 columns")

    # The same problem through the variant entry point: FP16 weights (the BF16
    # weights rounded to FP16 on the host), gather over all rows, a scatter
    # permutation, bias and gamma.
    rng = np.random.Generator(np.random.PCG64(4200))
    w16 = torch.from_numpy(gw.view(np.int16)).view(torch.bfloat16).to(torch.float16).view(torch.int16).numpy()
    w16 = w16.view(np.uint16)
    dw16 = torch.from_numpy(w16.view(np.int16)).to(dev)
    v = {"gather": rng.integers(0, 16384, 16384).astype(np.int32), "scatter": rng.permutation(16384).astype(np.int32),
         "bias": (rng.standard_normal((32, 2048)) * 0.1).astype(np.float32),
         "gamma": rng.uniform(-2, 2, 16384).astype(np.float32)}
    dv = {key: torch.from_numpy(val).to(dev) for key, val in v.items()}
    cg.fill_(SENTINEL)
    st = graph_stats(lambda i: L.bsgemm_grouped_run_ex(*qg, doff, dw16, 7168, w_dtype=L.BSGEMM_W_F16, bias=dv["bias"],
                                                       gamma=dv["gamma"], gather_idx=dv["gather"],
                                                       scatter_idx=dv["scatter"], c=cg), out=cg)
    rows["grouped_nvfp4_f16_all_variants"] = flops_row(st, gflops, "f16",
                                                       {"variants": "gather + scatter + bias + gamma, FP16 W"})
    if par.enabled:
        # physical output rows to check, and the A rows they read
        prow = sample(16384, 64, 45)
        logical = np.argsort(v["scatter"])[prow]
        need = np.unique(v["gather"][logical])
        qfull = (np.zeros((16384, 3584), np.uint8), np.zeros((16384, 448), np.uint8), qa[2])
        qn = Q.quantize_nvfp4(gx[need], tensor_scale=qa[2])
        qfull[0][need], qfull[1][need] = qn[0], qn[1]
        par.flag("grouped_nvfp4_f16_all_variants", no_nan(cg), "no_unwritten_output")
        par.gemm("grouped_nvfp4_f16_all_variants", u16(cg)[prow],
                 *G.grouped_nvfp4_ex(*qfull, off, w16, "f16", v["bias"], v["gamma"], v["gather"], v["scatter"],
                                     out_rows=prow), f"{len(prow)} physical rows x 2048 columns")
    del qg, dw, doff, cg, dw16, dv, gx

    # Inner-expert (K-ragged) grouped GEMM: the weight-gradient shape of the
    # same problem (the experts' token counts split K, each padded to 256),
    # operands drawn on the device.
    koff = np.concatenate([[0], np.cumsum([-(-int(c) // 256) * 256 for c in counts])]).astype(np.int32)
    kk = int(koff[-1])
    qk = synth.nvfp4_random_operand(7168, kk, synth.SEEDS["nvfp4_big.A"], dev)
    gk = torch.Generator(device=dev)
    gk.manual_seed(4400)
    wk = (torch.randn((2048, kk), generator=gk, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
    ck = sentinel_out((32, 7168, 2048), dev)
    dkoff = torch.from_numpy(koff).to(dev)
    st = graph_stats(lambda i: L.bsgemm_grouped_kragged_run(*qk, dkoff, wk, kk, c=ck), out=ck)
    real_k = int(counts.sum())
    rows["grouped_kragged_nvfp4_bf16"] = flops_row(st, 2.0 * 7168 * 2048 * real_k, "bf16", {
        "shape": f"32 groups, A 7168 x {kk} NVFP4, W 2048 x {kk} BF16, C 32 x 7168 x 2048",
        "flops_counted": f"2 * 7168 * 2048 * {real_k} (real K; the K-slices are padded to {kk})",
        "tflops_padded_k": round(2.0 * 7168 * 2048 * kk / (st["ms"] * 1e-3) / 1e12, 2)})
    if par.enabled:
        kr = sample(7168, 16, 46)
        tkr = torch.from_numpy(kr).to(dev)
        qkh = (qk[0][tkr].cpu().numpy(), qk[1][tkr].cpu().numpy(), np.float32(1))
        par.flag("grouped_kragged_nvfp4_bf16", no_nan(ck), "no_unwritten_output")
        cref, t = G.grouped_kragged(*qkh, koff, u16(wk), "bf16")
        par.gemm("grouped_kragged_nvfp4_bf16", u16(ck[:, tkr]), cref, t,
                 f"every group: {len(kr)} rows x 2048 columns")
    del qk, wk, ck, dkoff
    return rows


def w4a16_rows(L, synth, dev, par):
    """W4A16 at M = 1, 16, 64, 256 on the 14336 x 4096 NVFP4 weight, rotated
    through 16 copies (16 x 33 MB > the 256 MB Infinity Cache: every launch
    reads cold weights).  Kernel durations for these microsecond launches are
    in the rocprofv3 traces under profiles/."""
    import numpy as np
    import torch
    from oracle import gemm as G
    from oracle import quantize as Q
    rows = {}
    Nw, Kw = 14336, 4096
    _, wf = synth.w4a16_inputs(1)
    qw = L.bsgemm_quantize_nvfp4(torch.from_numpy(wf).to(dev))
    cols = sample(Nw, 1024, 47)
    qwr = None
    if par.enabled:
        stw = Q.nvfp4_tensor_scale(wf)
        qwr = Q.quantize_nvfp4(wf[cols], tensor_scale=stw)
        tc = torch.from_numpy(cols).to(dev)
        par.same_bytes("w4a16", [qw[0][tc].cpu().numpy(), qw[1][tc].cpu().numpy(), np.float32(qw[2].item())],
                       list(qwr))
    # the measured stream floor: a 1 GiB device-to-device copy (read + write
    # bytes over its event-timed duration), beside the 8 TB/s nameplate
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record()
    for _ in range(5):
        dst.copy_(src)
    e_ev.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * (1 << 30) / (s_ev.elapsed_time(e_ev) * 1e-3) / 1e9
    del src, dst
    copies = 16
    wc = [qw[0].clone() for _ in range(copies)]
    ws = [qw[1].clone() for _ in range(copies)]
    for m in (1, 16, 64, 256):
        x = synth.bf16_bits(synth.normal_f32((m, Kw), synth.SEEDS["w4a16.X"]))
        dx = torch.from_numpy(x.view(np.int16)).to(dev)
        cw = sentinel_out((m, Nw), dev)
        st = graph_stats(lambda i: L.bsgemm_w4a16_run(dx, wc[i % copies], ws[i % copies], qw[2], c=cw),
                         iters=2 * copies, out=cw)
        nbytes = Nw * Kw // 2 + Nw * Kw // 16 + 4 + 2 * m * Kw + 2 * m * Nw
        gbps = nbytes / (st["ms"] * 1e-3) / 1e9
        rows[f"w4a16_m{m}"] = {
            "config": L.w4a16_configs()[L.bsgemm_w4a16_select(m, Nw, Kw)],
            "us": round(st["ms"] * 1e3, 2), "us_min": round(st["ms_min"] * 1e3, 2), "us_max": round(st["ms_max"] * 1e3, 2),
            "gbps": round(gbps, 1), "frac_hbm": round(gbps / PEAK["hbm_gbps"], 4),
            "stream_copy_gbps": round(copy_gbps, 1), "frac_stream_copy": round(gbps / copy_gbps, 4),
            "tflops": round(2.0 * m * Nw * Kw / (st["ms"] * 1e-3) / 1e12, 2),
            "graph_matches_eager": st["graph_matches_eager"],
            "timing": f"{REPS} x {2 * copies} graph launches, median, weights rotated through {copies} copies"}
        if par.enabled:
            par.flag(f"w4a16_m{m}", no_nan(cw), "no_unwritten_output")
            par.gemm(f"w4a16_m{m}", u16(cw)[:, cols], *G.w4a16(x, *qwr), f"{m} rows x {len(cols)} columns")
    return rows


def headline(L, synth, dev, args, par):
    """NVFP4 16384^3: value (wall clock), roofline (events), graph stats,
    parity of rows 0..8191 over all columns, and the CPU oracle timing."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info
    from oracle import gemm as G
    from oracle import quantize as Q

    M = N = K = 16384
    log("generating NVFP4 16k inputs")
    a, b, _, _ = synth.nvfp4_16k_inputs(M, N, K)
    da = torch.from_numpy(a).to(dev)
    db = torch.from_numpy(b).to(dev)
    ca, sa, ta = L.bsgemm_quantize_nvfp4(da)
    cb, sb, tb = L.bsgemm_quantize_nvfp4(db)
    c = sentinel_out((M, N), dev)
    torch.cuda.synchronize()

    def step(_):
        L.bsgemm_run(L.BSGEMM_NVFP4, ca, sa, ta, cb, sb, tb, K, c=c)

    flops = 2.0 * M * N * K
    for _ in range(args.warmup):
        step(0)
    torch.cuda.synchronize()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s_ev.record()
    for i in range(args.steps):
        step(i)
    e_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    kernel_ms = s_ev.elapsed_time(e_ev) / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    log(f"nvfp4 16k: {ms_per_step:.3f} ms/step wall, {kernel_ms:.3f} ms kernel, {value:.1f} TFLOPS")
    alg_bytes = 2 * M * K * 0.5625 + 2 * M * N
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK["f16"], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK["f16"], 4), "traffic": traffic_from_counters(),
                "dtype_of_peak": "f16 (dense MFMA; the exact NVFP4 mapping on gfx950)",
                "frac_of_fp4_peak": round(achieved / PEAK["fp4"], 4),
                "algorithmic_bytes": int(alg_bytes), "flops_per_launch": flops,
                "timed_region": f"{args.steps} launches after {args.warmup} warm-up, HIP events on the launch stream"}
    res = {"value": value, "ms_per_step": ms_per_step, "kernel_ms": kernel_ms, "roofline": roofline}
    if args.only == "headline":
        return res

    res["parity_nan_free"] = no_nan(c)     # the sentinel: every element of the timed output written
    got = u16(c)                            # the whole timed output
    log("headline graph stats")
    st = graph_stats(step, out=c)
    res["row"] = flops_row(st, flops, "f16", {"frac_fp4_peak": round(flops / (st["ms"] * 1e-3) / 1e12 / PEAK["fp4"], 4)})

    # The oracle's own quantization of the same inputs (all of A and B), checked byte for byte against the GPU's; then
    # the oracle GEMM on those bytes, timed: the CPU baseline and the parity
    # reference of the timed output.
    if par.enabled or not args.no_cpu_baseline:
        log("oracle quantization of A and B")
        t0 = time.perf_counter()
        sta, stb = Q.nvfp4_tensor_scale(a), Q.nvfp4_tensor_scale(b)
        qa = oracle_rows(Q.quantize_nvfp4, a, tensor_scale=sta)
        qb = oracle_rows(Q.quantize_nvfp4, b, tensor_scale=stb)
        tq = time.perf_counter() - t0
        del a, b
        par.same_bytes("nvfp4_gemm_16384", [ca.cpu().numpy(), sa.cpu().numpy(),
                                            np.float32(ta.item()), cb.cpu().numpy(), sb.cpu().numpy(),
                                            np.float32(tb.item())], list(qa) + list(qb))
        log("oracle GEMM A x B")
        t0 = time.perf_counter()
        cref, tref = G.gemm_nvfp4(*qa, *qb)
        t = time.perf_counter() - t0
        # The parts of that time, measured again separately: the exact float64
        # decode of both operands and the two BLAS products (C_ref and the
        # magnitude sum T of the acceptance bound).
        t0 = time.perf_counter()
        ua, ub = G.nvfp4_units(qa[0], qa[1]), G.nvfp4_units(qb[0], qb[1])
        t_dec = time.perf_counter() - t0
        t0 = time.perf_counter()
        _ = ua @ ub.T
        t_c = time.perf_counter() - t0
        t0 = time.perf_counter()
        _ = np.abs(ua) @ np.abs(ub).T
        t_t = time.perf_counter() - t0
        del ua, ub, _
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        res["cpu_baseline"] = {
            "value": round(2.0 * M * N * K / t / 1e12, 4), "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "seconds": round(t, 2), "cpu_model": cpu_model(), "oracle_quantize_seconds": round(tq, 2),
            "parts_seconds": {"decode": round(t_dec, 2), "c_ref_matmul": round(t_c, 2), "t_matmul": round(t_t, 2)},
            "c_ref_gflops": round(2.0 * M * N * K / t_c / 1e9, 1),
            "sample": f"oracle.gemm.gemm_nvfp4 on the whole {M} x {N} x {K} problem "
                      "(float64 decode of every code, C and sum|ab| matmuls); the same result is the parity "
                      "reference of the timed output"}
        if par.enabled:
            par.flag("nvfp4_gemm_16384", res["parity_nan_free"], "no_unwritten_output")
            par.gemm("nvfp4_gemm_16384", got, cref, tref, f"all {M} x {N} outputs of the timed launch")
        del cref, tref
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "headline", "big", "w4a16", "mx", "grouped"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path, so every "
              "figure it reports is one GPU's; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_scaled_precision_bsgemm_amd import lib as L
    from block_scaled_precision_bsgemm_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    L.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    par = Parity(not args.no_parity and args.only not in ("headline", "big"))

    def copy_calibration(out):
        # HBM counter calibration: a plain 1 GiB device-to-device copy.
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_bytes"] = 1 << 30

    def finish(out):
        if par.enabled:
            out["parity"] = {"ok": par.ok(), "rows": par.rows}
        print(json.dumps(out))
        if par.enabled and not par.ok():
            log("PARITY FAILURE: see the parity field")
            sys.exit(1)

    if args.only == "w4a16":
        out = w4a16_rows(L, synth, dev, par)
        copy_calibration(out)
        finish(out)
        return
    if args.only == "grouped":
        out = grouped_rows(L, synth, dev, par)
        copy_calibration(out)
        finish(out)
        return
    if args.only == "mx":
        out = mx_rows(L, synth, dev, par)
        copy_calibration(out)
        finish(out)
        return
    if args.only == "big":
        # 64k^3 and 128k^3 NVFP4 GEMMs (operands drawn as NVFP4 on the device),
        # and 16k^3 on the same kind of operands as the control
        out = {}
        for size in (16384, 65536, 131072):
            qa = synth.nvfp4_random_operand(size, size, synth.SEEDS["nvfp4_big.A"], dev)
            qb = synth.nvfp4_random_operand(size, size, synth.SEEDS["nvfp4_big.B"], dev)
            cbig = torch.empty((size, size), dtype=torch.int16, device=dev)
            ms = time_events(lambda i: L.bsgemm_run(L.BSGEMM_NVFP4, *qa, *qb, size, c=cbig),
                             {16384: 10, 65536: 3}.get(size, 2), 1)
            tf = 2.0 * size ** 3 / (ms * 1e-3) / 1e12
            out[f"nvfp4_gemm_{size}"] = {"ms": round(ms, 2), "tflops": round(tf, 1), "frac_f16_peak": round(tf / PEAK["f16"], 4)}
            log(f"nvfp4 {size}^3: {ms:.1f} ms, {tf:.1f} TFLOPS")
            del qa, qb, cbig
            torch.cuda.empty_cache()
        print(json.dumps(out))
        return

    hl = headline(L, synth, dev, args, par)
    if args.only == "headline":
        out = {"headline_tflops": round(hl["value"], 2), "kernel_ms": round(hl["kernel_ms"], 4),
               "source_sha": kernel_source_sha()}
        copy_calibration(out)
        print(json.dumps(out))
        return
    rows = {"nvfp4_gemm_16384": hl["row"]}
    torch.cuda.empty_cache()

    # ------------------------------------------------ quantizers at 16384^2
    from oracle import quantize as Q
    xq = synth.normal_f32((16384, 16384), synth.SEEDS["nvfp4_16k.A"])
    dxq = torch.from_numpy(xq).to(dev)
    qn = L.bsgemm_quantize_nvfp4(dxq)
    st = graph_stats(lambda i: L.bsgemm_quantize_nvfp4(dxq, *qn), iters=5)
    rows["quantize_nvfp4_16384x16384"] = {"ms": round(st["ms"], 4), "ms_min": round(st["ms_min"], 4),
                                          "gbps": round(16384 * 16384 * (8 + 0.5625) / (st["ms"] * 1e-3) / 1e9, 1),
                                          "bytes_model": "2 reads of FP32 + codes + scales"}
    if par.enabled:
        rq = sample(16384, 256, 48)
        trq = torch.from_numpy(rq).to(dev)
        ref = Q.quantize_nvfp4(xq[rq], tensor_scale=Q.nvfp4_tensor_scale(xq))
        par.same_bytes("quantize_nvfp4_16384x16384", [qn[0][trq].cpu().numpy(), qn[1][trq].cpu().numpy(),
                                                      np.float32(qn[2].item())], list(ref))
    del xq, dxq, qn
    rows.update(mx_rows(L, synth, dev, par, time_quantizers=True))
    torch.cuda.empty_cache()

    # --------------------------------------------------- NVFP4 256x256x128
    from oracle import gemm as G
    sa0, sb0 = synth.nvfp4_small_inputs()
    qa0 = L.bsgemm_quantize_nvfp4(torch.from_numpy(sa0).to(dev))
    qb0 = L.bsgemm_quantize_nvfp4(torch.from_numpy(sb0).to(dev))
    c0 = sentinel_out((256, 256), dev)
    small = lambda i: L.bsgemm_run(L.BSGEMM_NVFP4, *qa0, *qb0, 128, c=c0)  # noqa: E731
    ms_eager = time_events(small, 200, 20)
    st = graph_stats(small, iters=64, out=c0)
    rows["nvfp4_gemm_256x256x128"] = {"us": round(st["ms"] * 1e3, 2), "us_min": round(st["ms_min"] * 1e3, 2),
                                      "us_max": round(st["ms_max"] * 1e3, 2), "us_eager": round(ms_eager * 1e3, 2),
                                      "graph_matches_eager": st["graph_matches_eager"],
                                      "note": "graph replay gives the GPU time per launch; eager launches through "
                                              "the Python binding are bound by the host"}
    if par.enabled:
        r0a, r0b = Q.quantize_nvfp4(sa0), Q.quantize_nvfp4(sb0)
        par.same_bytes("nvfp4_gemm_256x256x128", [t.cpu().numpy() if hasattr(t, "cpu") else t
                                                  for t in (qa0[0], qa0[1], np.float32(qa0[2].item()),
                                                            qb0[0], qb0[1], np.float32(qb0[2].item()))],
                       list(r0a) + list(r0b))
        par.gemm("nvfp4_gemm_256x256x128", u16(c0), *G.gemm_nvfp4(*r0a, *r0b), "all 256 x 256 outputs")

    rows.update(grouped_rows(L, synth, dev, par))
    torch.cuda.empty_cache()
    rows.update(w4a16_rows(L, synth, dev, par))

    out = {
        "metric": METRIC, "value": round(hl["value"], 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(hl["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "nvfp4_gemm_16384x16384x16384", "M": 16384, "N": 16384, "K": 16384,
                   "operands": "NVFP4 (E2M1 + E4M3/16 + FP32 tensor scale), N(0,1), 1% rows x100",
                   "output": "bf16"},
        "roofline": hl["roofline"], "cpu_baseline": hl.get("cpu_baseline"), "rows": rows,
    }
    finish(out)


if __name__ == "__main__":
    main()
