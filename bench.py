#!/usr/bin/env python3
"""Benchmark of the block-scaled GEMM library on one MI355X.

One step is one NVFP4 x NVFP4 GEMM at M = N = K = 16384 (BF16 output).  Its
operands are already quantized and resident in HBM.  This is the 16k-square
workload of "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA Vera
Rubin NVL72", section "Building the GEMM", with 1% outlier rows.  ``value`` is
its throughput in TFLOPS, from the wall clock around exactly ``--steps``
launches, synchronised on both sides.

The same JSON line carries:
  - ``roofline``: the GEMM kernel's time from HIP events on its own stream,
    against the MFMA peak of the arithmetic it runs (FP16).  The NVFP4 E4M3
    scales force an exact FP16 path on gfx950; ``frac_of_fp4_peak`` gives the
    fraction of the FP4 peak too.
  - ``cpu_baseline``: the CPU oracle's GEMM timed on a bounded sample.
  - ``rows``: the other parts of the hot path, each timed with HIP events:
    the MXFP8 GEMM at 16384^3 and 4096^3, the MXFP4 GEMM at 16384^3 (on
    the MXFP8 row's N(0, 1) inputs), the ragged grouped NVFP4 x BF16
    GEMM (and the same problem with FP16 weights and every routing and
    epilogue variant, and its K-ragged weight-gradient form), the W4A16
    GEMM at M = 1, 16, 64, 256 with weights rotated through 16 copies (cold
    cache; back-to-back launches, and the same launches replayed from a HIP
    graph), the three quantizers at 16384^2, and the 256 x 256 x 128 NVFP4
    GEMM latency.

``--only w4a16`` runs just the W4A16 rows (for profiler runs).
``--only mx`` runs just the MX GEMM rows and a 1 GiB device copy (for profiler
runs: kernel traces and HBM byte counters of the MX GEMMs).
``--only grouped`` runs just the grouped rows and the same 1 GiB device copy (for
profiler runs).
``--only big`` times the 64k^3 and 128k^3 NVFP4 GEMMs (about 60 GB of device
memory, operands drawn as NVFP4 on the device; 16k^3 on the same kind of
operands as the control) and prints their rows.
``--only headline`` runs just the headline GEMM (for profiler runs).  It adds
a 1 GiB device copy (read 1 GiB, write 1 GiB) that calibrates HBM byte
counters.
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


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_scaled_precision_bsgemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_counters(launches_per_step=1):
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


def grouped_rows(L, synth, dev):
    """The grouped rows: the 32-group NVFP4 x BF16 problem, the same problem with FP16 weights
    and every routing and epilogue variant, and its K-ragged weight-gradient form."""
    import numpy as np
    import torch

    rows = {}
    # ------------------------------------------------------------- grouped
    log("generating grouped inputs")
    gx, off, gw = synth.grouped_inputs()
    qg = L.bsgemm_quantize_nvfp4(torch.from_numpy(gx).to(dev))
    dw = torch.from_numpy(gw.view(np.int16)).to(dev)
    doff = torch.from_numpy(off).to(dev)
    del gx, gw
    cg = torch.empty((16384, 2048), dtype=torch.int16, device=dev)
    ms = time_events(lambda i: L.bsgemm_grouped_run(*qg, doff, dw, 7168, c=cg), 10, 3)
    gflops = 2.0 * 16384 * 2048 * 7168
    counts = np.diff(off.astype(np.int64))
    gbytes = 16384 * 7168 * 0.5625 + int((counts > 0).sum()) * 2048 * 7168 * 2 + 16384 * 2048 * 2
    tf = gflops / (ms * 1e-3) / 1e12
    rows["grouped_nvfp4_bf16"] = {"ms": round(ms, 4), "tflops": round(tf, 2), "frac_bf16_peak": round(tf / PEAK["bf16"], 4),
                                  "gbps_algorithmic": round(gbytes / (ms * 1e-3) / 1e9, 1),
                                  "groups_nonempty": int((counts > 0).sum()), "max_group_rows": int(counts.max())}
    # the same problem through the variant entry point: FP16 weights (the BF16
    # weights converted to FP16 on the device), gather over all rows, a
    # scatter permutation, bias and gamma
    rng = np.random.Generator(np.random.PCG64(4200))
    dw16 = dw.view(torch.bfloat16).to(torch.float16).view(torch.int16)
    vg = torch.from_numpy(rng.integers(0, 16384, 16384).astype(np.int32)).to(dev)
    vs = torch.from_numpy(rng.permutation(16384).astype(np.int32)).to(dev)
    vb = torch.from_numpy((rng.standard_normal((32, 2048)) * 0.1).astype(np.float32)).to(dev)
    vgm = torch.from_numpy(rng.uniform(-2, 2, 16384).astype(np.float32)).to(dev)
    ms = time_events(lambda i: L.bsgemm_grouped_run_ex(*qg, doff, dw16, 7168, w_dtype=L.BSGEMM_W_F16, bias=vb,
                                                       gamma=vgm, gather_idx=vg, scatter_idx=vs, c=cg), 10, 3)
    tf = gflops / (ms * 1e-3) / 1e12
    rows["grouped_nvfp4_f16_all_variants"] = {"ms": round(ms, 4), "tflops": round(tf, 2),
                                              "frac_f16_peak": round(tf / PEAK["f16"], 4),
                                              "variants": "gather + scatter + bias + gamma, FP16 W"}
    del qg, dw, doff, cg, dw16, vg, vs, vb, vgm

    # inner-expert (K-ragged) grouped GEMM: the weight-gradient shape of the
    # same problem (experts' token counts split K, each padded to 256),
    # operands drawn on the device
    kcounts = np.diff(off.astype(np.int64))
    koff = np.concatenate([[0], np.cumsum([-(-int(c) // 256) * 256 for c in kcounts])]).astype(np.int32)
    kk = int(koff[-1])
    qk = synth.nvfp4_random_operand(7168, kk, synth.SEEDS["nvfp4_big.A"], dev)
    gk = torch.Generator(device=dev)
    gk.manual_seed(4400)
    wk = (torch.randn((2048, kk), generator=gk, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
    ck = torch.empty((32, 7168, 2048), dtype=torch.int16, device=dev)
    dkoff = torch.from_numpy(koff).to(dev)
    ms = time_events(lambda i: L.bsgemm_grouped_kragged_run(*qk, dkoff, wk, kk, c=ck), 10, 3)
    kflops = 2.0 * 7168 * 2048 * kk
    tf = kflops / (ms * 1e-3) / 1e12
    rows["grouped_kragged_nvfp4_bf16"] = {"ms": round(ms, 4), "tflops": round(tf, 2), "frac_bf16_peak": round(tf / PEAK["bf16"], 4),
                                          "shape": f"32 groups, A 7168 x {kk} NVFP4, W 2048 x {kk} BF16, C 32 x 7168 x 2048",
                                          "flops_counted": "2 * 7168 * 2048 * padded K"}
    del qk, wk, ck, dkoff
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "headline", "big", "w4a16", "mx", "grouped"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(see the sharding notes in DESIGN.md); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_scaled_precision_bsgemm_amd import lib as L
    from block_scaled_precision_bsgemm_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    L.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only == "w4a16":
        print(json.dumps(w4a16_rows(L, synth, dev)))
        return

    if args.only == "grouped":
        out = grouped_rows(L, synth, dev)
        # HBM counter calibration: a plain 1 GiB device-to-device copy.
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_bytes"] = 1 << 30
        print(json.dumps(out))
        return

    if args.only == "mx":
        out = mx_rows(L, synth, dev, args.steps)
        # HBM counter calibration: a plain 1 GiB device-to-device copy.
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_bytes"] = 1 << 30
        print(json.dumps(out))
        return

    if args.only == "big":
        # 64k^3 and 128k^3 NVFP4 GEMMs (operands drawn as NVFP4 on the device),
        # and 16k^3 on the same kind of operands as the control
        out = {}
        for size in (16384, 65536, 131072):
            qa = synth.nvfp4_random_operand(size, size, synth.SEEDS["nvfp4_big.A"], dev)
            qb = synth.nvfp4_random_operand(size, size, synth.SEEDS["nvfp4_big.B"], dev)
            cbig = torch.empty((size, size), dtype=torch.int16, device=dev)
            ms = time_events(lambda i: L.bsgemm_run(L.BSGEMM_NVFP4, *qa, *qb, size, c=cbig), {16384: 10, 65536: 3}.get(size, 2), 1)
            tf = 2.0 * size ** 3 / (ms * 1e-3) / 1e12
            out[f"nvfp4_gemm_{size}"] = {"ms": round(ms, 2), "tflops": round(tf, 1), "frac_f16_peak": round(tf / PEAK["f16"], 4)}
            log(f"nvfp4 {size}^3: {ms:.1f} ms, {tf:.1f} TFLOPS")
            del qa, qb, cbig
            torch.cuda.empty_cache()
        print(json.dumps(out))
        return

    # ------------------------------------------------ headline: NVFP4 16k^3
    M = N = K = 16384
    log("generating NVFP4 16k inputs")
    a, b, _, _ = synth.nvfp4_16k_inputs(M, N, K)
    da = torch.from_numpy(a).to(dev)
    db = torch.from_numpy(b).to(dev)
    del a, b
    ca, sa, ta = L.bsgemm_quantize_nvfp4(da)
    cb, sb, tb = L.bsgemm_quantize_nvfp4(db)
    c = torch.empty((M, N), dtype=torch.int16, device=dev)
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
                "algorithmic_bytes": int(alg_bytes), "flops_per_launch": flops}

    if args.only == "headline":
        # HBM counter calibration: a plain 1 GiB device-to-device copy.
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"headline_tflops": round(value, 2), "kernel_ms": round(kernel_ms, 4),
                          "source_sha": kernel_source_sha(), "copy_bytes": 1 << 30}))
        return

    rows = {"nvfp4_gemm_16384": {"ms": round(kernel_ms, 4), "tflops": round(achieved, 2),
                                 "frac_f16_peak": round(achieved / PEAK["f16"], 4),
                                 "frac_fp4_peak": round(achieved / PEAK["fp4"], 4)}}

    # ---------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(ca, sa, ta, cb, sb, tb, K)
        log("cpu baseline", cpu)

    # ------------------------------------------------ quantizers at 16384^2
    n_el = M * K
    ms = time_events(lambda i: L.bsgemm_quantize_nvfp4(da, ca, sa, ta), 5, 2)
    rows["quantize_nvfp4_16384x16384"] = {"ms": round(ms, 4), "gbps": round(n_el * (8 + 0.5625) / (ms * 1e-3) / 1e9, 1),
                                          "bytes_model": "2 reads of FP32 + codes + scales"}
    del ca, sa, ta, cb, sb, tb, c, da, db
    rows.update(mx_rows(L, synth, dev, args.steps, time_quantizers=True))

    # --------------------------------------------------- NVFP4 256x256x128
    sa0, sb0 = synth.nvfp4_small_inputs()
    qa0 = L.bsgemm_quantize_nvfp4(torch.from_numpy(sa0).to(dev))
    qb0 = L.bsgemm_quantize_nvfp4(torch.from_numpy(sb0).to(dev))
    c0 = torch.empty((256, 256), dtype=torch.int16, device=dev)
    small = lambda i: L.bsgemm_run(L.BSGEMM_NVFP4, *qa0, *qb0, 128, c=c0)  # noqa: E731
    ms = time_events(small, 200, 20)
    ms_graph, graph = time_graph(small, 64, 8)
    del graph
    rows["nvfp4_gemm_256x256x128"] = {"us": round(ms * 1e3, 2), "us_graph": round(ms_graph * 1e3, 2),
                                      "note": "eager launches through the Python binding are bound by the "
                                              "host; the graph replay gives the GPU time per launch"}

    rows.update(grouped_rows(L, synth, dev))

    # --------------------------------------------------------------- W4A16
    rows.update(w4a16_rows(L, synth, dev))

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "nvfp4_gemm_16384x16384x16384", "M": M, "N": N, "K": K,
                   "operands": "NVFP4 (E2M1 + E4M3/16 + FP32 tensor scale), N(0,1), 1% rows x100",
                   "output": "bf16"},
        "roofline": roofline, "cpu_baseline": cpu, "rows": rows,
    }
    print(json.dumps(out))


def mx_rows(L, synth, dev, steps, time_quantizers=False):
    """MXFP4 and MXFP8 GEMMs at 16384^3 on N(0, 1) inputs, MXFP8 at 4096^3
    (and, with time_quantizers, the MXFP8 and MXFP4 quantizers at 16384^2)."""
    import torch
    rows = {}
    M = N = K = 16384
    n_el, flops = M * K, 2.0 * M * N * K
    mx_a = synth.normal_f32((M, K), synth.SEEDS["mxfp8_4k.A"])
    mx_b = synth.normal_f32((N, K), synth.SEEDS["mxfp8_4k.B"])
    dma, dmb = torch.from_numpy(mx_a).to(dev), torch.from_numpy(mx_b).to(dev)
    del mx_a, mx_b
    c8a, s8a = L.bsgemm_quantize_mxfp8(dma)
    c8b, s8b = L.bsgemm_quantize_mxfp8(dmb)
    if time_quantizers:
        ms = time_events(lambda i: L.bsgemm_quantize_mxfp8(dma, c8a, s8a), 5, 2)
        rows["quantize_mxfp8_16384x16384"] = {"ms": round(ms, 4), "gbps": round(n_el * (4 + 1.03125) / (ms * 1e-3) / 1e9, 1)}
    # MXFP4 from the same N(0, 1) 16k inputs
    c4a, s4a = L.bsgemm_quantize_mxfp4(dma)
    c4b, s4b = L.bsgemm_quantize_mxfp4(dmb)
    if time_quantizers:
        ms = time_events(lambda i: L.bsgemm_quantize_mxfp4(dma, c4a, s4a), 5, 2)
        rows["quantize_mxfp4_16384x16384"] = {"ms": round(ms, 4), "gbps": round(n_el * (4 + 0.53125) / (ms * 1e-3) / 1e9, 1)}
    del dma, dmb
    c16 = torch.empty((M, N), dtype=torch.int16, device=dev)
    ms = time_events(lambda i: L.bsgemm_run(L.BSGEMM_MXFP4, c4a, s4a, None, c4b, s4b, None, K, c=c16),
                     max(3, steps // 2), 2)
    tf = flops / (ms * 1e-3) / 1e12
    rows["mxfp4_gemm_16384"] = {"ms": round(ms, 4), "tflops": round(tf, 2), "frac_fp4_peak": round(tf / PEAK["fp4"], 4)}
    del c4a, s4a, c4b, s4b

    ms = time_events(lambda i: L.bsgemm_run(L.BSGEMM_MXFP8, c8a, s8a, None, c8b, s8b, None, K, c=c16),
                     max(3, steps // 2), 2)
    tf = flops / (ms * 1e-3) / 1e12
    rows["mxfp8_gemm_16384"] = {"ms": round(ms, 4), "tflops": round(tf, 2), "frac_fp8_peak": round(tf / PEAK["fp8"], 4)}
    del c8a, s8a, c8b, s8b, c16
    a4, b4 = synth.mxfp8_inputs()
    q4a = L.bsgemm_quantize_mxfp8(torch.from_numpy(a4).to(dev))
    q4b = L.bsgemm_quantize_mxfp8(torch.from_numpy(b4).to(dev))
    c4 = torch.empty((4096, 4096), dtype=torch.int16, device=dev)
    ms = time_events(lambda i: L.bsgemm_run(L.BSGEMM_MXFP8, q4a[0], q4a[1], None, q4b[0], q4b[1], None, 4096, c=c4), 50, 10)
    tf = 2.0 * 4096 ** 3 / (ms * 1e-3) / 1e12
    rows["mxfp8_gemm_4096"] = {"ms": round(ms, 4), "tflops": round(tf, 2), "frac_fp8_peak": round(tf / PEAK["fp8"], 4)}
    return rows


def time_graph(fn, launches, replays):
    """Average ms per call with `launches` calls captured in one HIP graph and
    the graph replayed `replays` times (launch overhead amortised)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (replays * launches), g


def w4a16_rows(L, synth, dev):
    """W4A16 at M = 1, 16, 64, 256 on the 14336 x 4096 NVFP4 weight, rotated
    through 16 copies (cold weights): back-to-back launches timed with events,
    and the same launches captured in a HIP graph (the graph's last output is
    checked bit for bit against an eager launch first)."""
    import numpy as np
    import torch
    rows = {}
    Nw, Kw = 14336, 4096
    _, wf = synth.w4a16_inputs(1)
    qw = L.bsgemm_quantize_nvfp4(torch.from_numpy(wf).to(dev))
    copies = 16   # 16 x 33 MB > 256 MB Infinity Cache: every launch reads cold weights
    wc = [qw[0].clone() for _ in range(copies)]
    ws = [qw[1].clone() for _ in range(copies)]
    for m in (1, 16, 64, 256):
        x = synth.bf16_bits(synth.normal_f32((m, Kw), synth.SEEDS["w4a16.X"]))
        dx = torch.from_numpy(x.view(np.int16)).to(dev)
        cw = torch.empty((m, Nw), dtype=torch.int16, device=dev)
        call = lambda i: L.bsgemm_w4a16_run(dx, wc[i % copies], ws[i % copies], qw[2], c=cw)  # noqa: E731
        ms = time_events(call, 64, 16)
        eager = L.bsgemm_w4a16_run(dx, wc[0], ws[0], qw[2]).clone()
        ms_graph, graph = time_graph(call, 64, 8)
        graph.replay()
        torch.cuda.synchronize()
        graph_ok = bool(torch.equal(cw, eager))
        del graph
        nbytes = Nw * Kw // 2 + Nw * Kw // 16 + 4 + 2 * m * Kw + 2 * m * Nw
        row = {"config": L.w4a16_configs()[L.bsgemm_w4a16_select(m, Nw, Kw)]}
        for tag, t in (("", ms), ("_graph", ms_graph)):
            gbps = nbytes / (t * 1e-3) / 1e9
            tf = 2.0 * m * Nw * Kw / (t * 1e-3) / 1e12
            row.update({f"us{tag}": round(t * 1e3, 2), f"gbps{tag}": round(gbps, 1),
                        f"frac_hbm{tag}": round(gbps / 8000.0, 4), f"tflops{tag}": round(tf, 2)})
        row["graph_output_matches_eager"] = graph_ok
        rows[f"w4a16_m{m}"] = row
    return rows


def cpu_baseline(ca, sa, ta, cb, sb, tb, K):
    """The CPU oracle's NVFP4 GEMM (float64 decode + BLAS matmul for C and
    sum |ab|) on A[0:8192] x B[0:16384] of the benchmark's operands, full K:
    about 10-20 s of host work, half the output of one step."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import gemm as G

    ms_, ns_ = 8192, 16384
    qa = (ca[:ms_].cpu().numpy(), sa[:ms_].cpu().numpy(), np.float32(ta.item()))
    qb = (cb[:ns_].cpu().numpy(), sb[:ns_].cpu().numpy(), np.float32(tb.item()))
    t0 = time.perf_counter()
    G.gemm_nvfp4(*qa, *qb)
    t = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(2.0 * ms_ * ns_ * K / t / 1e12, 4), "unit": "TFLOPS", "cores": threads,
            "kind": "oracle", "seconds": round(t, 2),
            "sample": f"oracle.gemm.gemm_nvfp4 on A[0:{ms_}] x B[0:{ns_}] of the 16384^3 operands, K={K} "
                      "(float64 decode of every code, C and sum|ab| matmuls)"}


if __name__ == "__main__":
    main()
