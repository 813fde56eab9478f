#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 hot path on one MI355X.

Timed step (the headline): forward + backward of all 7 linears of a
LLaMA-33B-shaped block (q, k, v, o 6656x6656; gate, up 6656->17920; down
17920->6656) for 8192 tokens (4 x 2048) with NF4 + DQ base weights drawn
from a Student-t distribution with 4 degrees of freedom (std 0.02), LoRA
rank 64 on every linear, s = 0.25. Per linear: qlora_linear_fwd (Y and T)
then qlora_linear_bwd (dX, dL1, dL2). The weights are quantised once before
timing (the base is frozen, as in QLoRA training). Inputs are synthetic and
already resident in HBM when timing starts. The K timed steps are repeated
in 5 trials; value is the median trial.

value = algorithmic fwd+bwd flops per step / time per step, with flops
4 M K N + 6 M r (K + N) per linear (3 forward and 5 backward products, no
weight gradient; dequantisation is not counted).

The same run also measures:
  * what the GPU attains on plain loops: the library's register-only bf16
    MFMA loop (with its shader clock) and a 1 GiB streaming read, reported
    beside the published peaks (roofline.attainable, attainable);
  * roofline of the dominant kernel, the bf16 MFMA GEMM (gemm_nt_kernel) that
    computes both Y = X Wd^T + (s X L1) L2 and dX = dY Wd + (s dY L2^T) L1^T,
    from HIP events that the library records around each of its launches on
    the call's stream, in a second pass of the same steps (the timed steps
    themselves run without those brackets); its HBM traffic comes from
    rocprofv3 FETCH_SIZE / WRITE_SIZE counters stored under profiles/
    (scaled by the same counters on a plain device copy, see --copy-probe),
    with the exact bytes of the request-size counters beside it
    (traffic_exact), both reported only while the kernel source still has
    the hash recorded with them;
  * the same step on the LLaMA-7B-shaped layer set (normal weights with 0.1 %
    outliers x10), with its own GEMM roofline;
  * the same headline step with LoRA dropout 0.05 (the pages' 33B setting);
  * the small-M dequant-GEMV (M in {1, 4, 16}; 4096->11008 and 11008->4096)
    in GB/s against 8 TB/s, cycling >= 24 distinct weight copies (> 512 MB)
    so the 256 MB last-level cache cannot serve the weights;
  * the LLaMA-65B-shaped quantisation pass: 80 layers x 7 tensors (560
    tensors, 64.76 B weights) quantised from fp32 and from bf16, drawn from
    a pool of 2 layers cycled 40 times into 80 distinct output sets;
  * the four 4-bit data types (NF4, Int4, FP4 E2M1, FP4 E3M0, all with DQ)
    and NF4 without DQ on a 4096 x 11008 weight: relative RMS error of the
    dequantised weight for normal (0.1 % outliers) and Student-t weights,
    storage bits per parameter and quantise GB/s;
  * the blockwise Int8 absmax codec: quantise and dequantise GB/s on the
    LLaMA-65B gate-shaped tensor, and the error by block size (64 .. 4096);
  * the batched-decode forward at M in {32, 64, 128};
  * the optimiser step (clip + Adam) at the size of all LLaMA-7B adapters,
    with 0-100 % of the Adam state paged out to pinned host memory;
  * the adapter merge (bf16 dequantised base + s L1 L2, r = 64) in GB/s on
    the LLaMA-7B linear shapes;
  * the CPU oracle on the headline step (all 7 linears, 8192 tokens) as a
    baseline, and on one layer of the 65B quantisation pass (x80).
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
GEMM_SOURCE = os.path.join(ROOT, "bit_nf4_quantized_amd", "csrc", "dense_gemm.hip")
HEADLINE = "llama33b-layer"


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"gemm_nt_{workload}_hbm-traffic.md")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def linear_flops(M, K, N, r):
    return 4 * M * K * N + 6 * M * r * (K + N)


def nf4_bytes(K, N, double_quant=True):
    numel = K * N
    nb = -(-numel // 64)
    ng = -(-nb // 256)
    return numel // 2 + (nb + 4 * ng + 4 if double_quant else 4 * nb)


def setup_layer(api, workloads, name, M=None):
    import torch

    cfg = workloads.WORKLOADS[name]
    layers = []
    host = []
    for idx, shp in enumerate(cfg["linears"]):
        _, inp = workloads.layer_linear(name, idx, M=M)
        W = torch.from_numpy(inp.W).cuda()
        q = api.qlora_quantize(W)
        torch.cuda.synchronize()
        del W
        Mx = inp.X.shape[0]
        r = inp.L1.shape[1]
        d = dict(shape=shp, q=q, s=inp.s, M=Mx, r=r,
                 X=api.to_device_bf16(inp.X), dY=api.to_device_bf16(inp.dY),
                 L1=api.to_device_bf16(inp.L1), L2=api.to_device_bf16(inp.L2))
        d["Y"] = torch.empty((Mx, shp.N), dtype=torch.bfloat16, device="cuda")
        d["T"] = torch.empty((Mx, r), dtype=torch.bfloat16, device="cuda")
        d["dX"] = torch.empty((Mx, shp.K), dtype=torch.bfloat16, device="cuda")
        d["dL1"] = torch.empty((shp.K, r), dtype=torch.float32, device="cuda")
        d["dL2"] = torch.empty((r, shp.N), dtype=torch.float32, device="cuda")
        layers.append(d)
        host.append((shp, inp))
        log(f"setup {shp.name} K={shp.K} N={shp.N} M={Mx}")
    ws_bytes = max(api.qlora_linear_workspace(d["M"], d["shape"].K, d["shape"].N, d["r"]) for d in layers)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    return layers, host, ws


def run_step(api, layers, ws):
    for d in layers:
        api.qlora_linear_fwd(d["q"], d["X"], d["L1"], d["L2"], d["s"], Y=d["Y"], T_out=d["T"], workspace=ws)
        api.qlora_linear_bwd(d["q"], d["X"], d["dY"], d["L1"], d["L2"], d["s"], T=d["T"], dX=d["dX"],
                             dL1=d["dL1"], dL2=d["dL2"], workspace=ws)


def bench_dropout_step(api, layers, flops_step, plain_ms, steps=5, warmup=2, p=0.1, seed=2024):
    """The same fwd+bwd step with LoRA dropout p on every adapter (the
    pages' Guanaco settings: 0.1 for 7B/13B, 0.05 for 33B/65B): ms per step
    and the cost over the plain step."""
    import torch

    ws_bytes = max(api.qlora_linear_workspace_dropout(d["M"], d["shape"].K, d["shape"].N, d["r"]) for d in layers)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def step(i):
        for d in layers:
            api.qlora_linear_fwd(d["q"], d["X"], d["L1"], d["L2"], d["s"], Y=d["Y"], T_out=d["T"], workspace=ws,
                                 dropout=(p, seed + i))
            api.qlora_linear_bwd(d["q"], d["X"], d["dY"], d["L1"], d["L2"], d["s"], T=d["T"], dX=d["dX"],
                                 dL1=d["dL1"], dL2=d["dL2"], workspace=ws, dropout=(p, seed + i))

    for i in range(warmup):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    log(f"dropout step (p = {p}): {ms:.3f} ms, {flops_step / (ms * 1e-3) / 1e12:.1f} TFLOP/s, "
        f"{100 * (ms / plain_ms - 1):.1f} % over the plain step")
    del ws
    return {"p": p, "ms_per_step": ms, "tflops": flops_step / (ms * 1e-3) / 1e12, "overhead_vs_plain": ms / plain_ms - 1}


def gemm_traffic(workload):
    """HBM bytes per gemm_nt_kernel launch from the stored counter summary of
    this workload: (FETCH_SIZE + WRITE_SIZE scaled by a plain copy's, exact
    bytes from the request-size counters), each None when absent or when the
    summary was taken on a different kernel source."""
    import hashlib

    try:
        text = open(traffic_file(workload)).read()
    except OSError:
        return None, None
    src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel source sha256") != src:
        return None, None
    out = []
    for key in ("bytes per launch (scaled)", "bytes per launch (exact, request counters)"):
        try:
            out.append(float(fields[key]))
        except (KeyError, ValueError):
            out.append(None)
    return tuple(out)


def attainable_peaks(api, iters=20000, read_bytes=1 << 30, reps=5):
    """What this GPU delivers on plain loops, for context beside the
    published peaks: the library's register-only bf16 MFMA loop (one
    8-wave workgroup per CU) with its shader clock, and a streaming read of
    1 GiB (4x the 256 MB last-level cache) with 16-byte loads. Median of
    ``reps`` launches each, timed with HIP events on the launch stream."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    flops = cus * 8 * iters * 8 * 32768
    api.qlora_probe_mfma(cus, 1000, sink, clocks)
    mf, clk = [], []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        api.qlora_probe_mfma(cus, iters, sink, clocks)
        e1.record()
        torch.cuda.synchronize()
        mf.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        c = clocks.cpu().tolist()
        clk.append(c[0] / (c[1] * 10.0))          # shader clocks per ns = GHz
    buf = torch.full((read_bytes // 4,), 0x01010101, dtype=torch.int32, device="cuda")
    rsink = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.qlora_probe_read(buf, 0xFFFFFFFF, rsink)  # words XOR to 0: never 0xFFFFFFFF
    rd = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        api.qlora_probe_read(buf, 0xFFFFFFFF, rsink)
        e1.record()
        torch.cuda.synchronize()
        rd.append(read_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    med = lambda v: sorted(v)[len(v) // 2]
    out = {"mfma_bf16_tflops": med(mf), "mfma_clock_ghz": med(clk), "hbm_read_GBps": med(rd),
           "mfma_loop": f"{cus} workgroups x 8 waves x {iters} rounds of 8 independent v_mfma_f32_32x32x16_bf16",
           "read": f"{read_bytes} bytes once, 16-byte loads, 16 per thread issued before use"}
    log(f"attainable: MFMA loop {out['mfma_bf16_tflops']:.0f} TFLOP/s at {out['mfma_clock_ghz']:.2f} GHz, "
        f"streaming read {out['hbm_read_GBps']:.0f} GB/s")
    return out


def copy_probe(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (run it under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import torch

    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def kernel_summary(durs_ms, flops):
    tot_ms = sum(durs_ms)
    tot_f = sum(flops)
    return {"launches": len(durs_ms), "avg_ms": tot_ms / max(len(durs_ms), 1),
            "tflops": tot_f / (tot_ms * 1e-3) / 1e12 if tot_ms > 0 else None, "total_ms": tot_ms}


def bench_gemv(api, workloads, reps=4, oracle=False):
    """Decode-style forward, M in {1, 4, 16}, weights cycled over distinct copies.
    With ``oracle``, the float64 oracle's dequant + forward of the same call
    is timed on the host beside each GPU figure."""
    import torch

    out = []
    for K, N in ((4096, 11008), (11008, 4096)):
        inp = workloads.gemv_inputs(K, N, 16)
        q0 = api.qlora_quantize(torch.from_numpy(inp.W).cuda())
        wbytes = nf4_bytes(K, N)
        copies = max(24, -(-600 * 2 ** 20 // wbytes))
        qs = [api.NF4Tensor(q0.rows, q0.cols, q0.codes.clone(), q0.absmax8.clone(), q0.scale2.clone(),
                            q0.mean.clone()) for _ in range(copies)]
        Xall = api.to_device_bf16(inp.X)
        L1, L2 = api.to_device_bf16(inp.L1), api.to_device_bf16(inp.L2)
        r = L1.shape[1]
        for M in (1, 4, 16):
            X = Xall[:M].contiguous()
            Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(api.qlora_linear_workspace(M, K, N, r), dtype=torch.uint8, device="cuda")
            for i in range(copies):   # warm-up pass over every copy
                api.qlora_linear_fwd(qs[i], X, L1, L2, inp.s, Y=Y, workspace=ws)
            n = copies * reps
            timer = api.KernelTimer(api.QLORA_TIMING_GEMV, capacity=n)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            with timer:
                e0.record()
                for i in range(n):
                    api.qlora_linear_fwd(qs[i % copies], X, L1, L2, inp.s, Y=Y, workspace=ws)
                e1.record()
            torch.cuda.synchronize()
            durs = timer.durations_ms()
            avg = sum(durs) / len(durs)
            kbytes = wbytes + 2 * M * K + 2 * M * r + 2 * r * N + 2 * M * N   # kernel's own stream
            cbytes = wbytes + 2 * r * (K + N) + 2 * M * K + 2 * M * N          # whole call
            call_ms = e0.elapsed_time(e1) / n
            # The same calls replayed from a captured HIP graph: the GPU time of
            # a whole call without the host's per-call cost (which bounds the
            # eager loop above). The replayed result must equal the eager one.
            api.qlora_linear_fwd(qs[copies - 1], X, L1, L2, inp.s, Y=Y, workspace=ws)
            torch.cuda.synchronize()
            y_eager = Y.clone()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(copies):
                    api.qlora_linear_fwd(qs[i], X, L1, L2, inp.s, Y=Y, workspace=ws)
            graph.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            graph_ms = e0.elapsed_time(e1) / (reps * copies)
            same = bool(torch.equal(Y.view(torch.int16), y_eager.view(torch.int16)))
            del graph
            out.append({"K": K, "N": N, "M": M, "kernel_us": avg * 1e3,
                        "kernel_GBps": kbytes / (avg * 1e-3) / 1e9,
                        "kernel_frac_of_hbm_peak": kbytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                        "call_us": call_ms * 1e3, "call_GBps": cbytes / (call_ms * 1e-3) / 1e9,
                        "graph_call_us": graph_ms * 1e3, "graph_call_GBps": cbytes / (graph_ms * 1e-3) / 1e9,
                        "graph_call_frac_of_hbm_peak": cbytes / (graph_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                        "graph_result_equal": same, "weight_copies": copies})
            if oracle:
                from oracle import linear, nf4

                qt = nf4.quantize(inp.W)                 # the frozen base: outside the timed call
                t0 = time.perf_counter()
                Wd = nf4.dequantize(qt, inp.W.shape)
                linear.linear_fwd(inp.X[:M], Wd, inp.L1, inp.L2, inp.s)
                dt = time.perf_counter() - t0
                out[-1]["cpu_oracle"] = {"call_us": dt * 1e6, "GBps": cbytes / dt / 1e9, "kind": "oracle",
                                         "sample": "one call: float64 NumPy dequant (single-threaded) + forward"}
                log(f"gemv K={K} N={N} M={M}: oracle call {dt*1e3:.1f} ms")
            log(f"gemv K={K} N={N} M={M}: kernel {avg*1e3:.2f} us "
                f"{out[-1]['kernel_GBps']:.0f} GB/s, call {call_ms*1e3:.2f} us, "
                f"graph-replayed call {graph_ms*1e3:.2f} us ({out[-1]['graph_call_GBps']:.0f} GB/s, "
                f"{'same bits' if same else 'DIFFERENT bits'})")
        del qs
        torch.cuda.empty_cache()
    return out


def bench_quantize(api, workloads, reps=5):
    """NF4 + DQ quantisation of a LLaMA-65B gate-shaped weight (22016 x 8192), from
    fp32 and from bf16, and the standalone doubleDequant of it back to bf16."""
    import torch

    shp = workloads.LLAMA65B[4]
    W32 = torch.from_numpy(workloads.quantize_weight(shp, 4, 4)).cuda()
    res = {}
    for dt, W in (("f32", W32), ("bf16", W32.to(torch.bfloat16))):
        q = api.qlora_quantize(W)
        ws = torch.empty(api.qlora_quant_sizes(shp.N, shp.K)["workspace"], dtype=torch.uint8, device="cuda")
        timer = api.KernelTimer(api.QLORA_TIMING_QUANT, capacity=reps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with timer:
            e0.record()
            for _ in range(reps):
                api.qlora_quantize(W, out=q, workspace=ws)
            e1.record()
        torch.cuda.synchronize()
        numel = shp.N * shp.K
        nbytes = numel * (4 if dt == "f32" else 2) + nf4_bytes(shp.K, shp.N)
        call_ms = e0.elapsed_time(e1) / reps
        k_ms = sum(timer.durations_ms()) / reps
        res[dt] = {"shape": [shp.N, shp.K], "call_ms": call_ms, "GBps": nbytes / (call_ms * 1e-3) / 1e9,
                   "frac_of_hbm_peak": nbytes / (call_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                   "pass1_kernel_ms": k_ms}
        log(f"quantize {dt} {shp.N}x{shp.K}: {call_ms:.3f} ms, {res[dt]['GBps']:.0f} GB/s")
    # the standalone doubleDequant of the same weight to bf16
    y = torch.empty(shp.N, shp.K, dtype=torch.bfloat16, device="cuda")
    api.qlora_dequantize(q, out=y)
    timer = api.KernelTimer(api.QLORA_TIMING_DEQUANT, capacity=reps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with timer:
        e0.record()
        for _ in range(reps):
            api.qlora_dequantize(q, out=y)
        e1.record()
    torch.cuda.synchronize()
    numel = shp.N * shp.K
    nbytes = nf4_bytes(shp.K, shp.N) + 2 * numel
    call_ms = e0.elapsed_time(e1) / reps
    k_ms = sum(timer.durations_ms()) / reps
    res["dequantize"] = {"shape": [shp.N, shp.K], "call_ms": call_ms, "GBps": nbytes / (call_ms * 1e-3) / 1e9,
                         "frac_of_hbm_peak": nbytes / (call_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                         "kernel_ms_bracketed": k_ms}
    log(f"dequantize {shp.N}x{shp.K} to bf16: {call_ms:.3f} ms, {res['dequantize']['GBps']:.0f} GB/s")
    return res


def bench_int8(api, workloads, reps=5):
    """Blockwise Int8 absmax codec: quantise (fp32 in) and dequantise (fp32 and
    bf16 out) throughput on a LLaMA-65B gate-shaped tensor (22016 x 8192,
    block 64), and the relative RMS error by block size on a 4096 x 11008
    normal weight with 0.1 % outliers x10 (std 0.02)."""
    import numpy as np
    import torch

    shp = workloads.LLAMA65B[4]
    numel = shp.N * shp.K
    X = torch.from_numpy(workloads.quantize_weight(shp, 4, 4)).cuda().reshape(-1)
    res = {"shape": [shp.N, shp.K], "block": 64}

    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    codes, absmax = api.qlora_int8_quantize(X, 64)
    y32 = torch.empty(numel, dtype=torch.float32, device="cuda")
    y16 = torch.empty(numel, dtype=torch.bfloat16, device="cuda")
    cb = numel + 4 * (numel // 64)
    for name, fn, nbytes in (
            ("quantize_f32", lambda: api.qlora_int8_quantize(X, 64, codes=codes, absmax=absmax), 4 * numel + cb),
            ("dequantize_f32", lambda: api.qlora_int8_dequantize(codes, absmax, 64, out=y32), cb + 4 * numel),
            ("dequantize_bf16", lambda: api.qlora_int8_dequantize(codes, absmax, 64, dtype=torch.bfloat16, out=y16),
             cb + 2 * numel)):
        ms = timed(fn)
        res[name] = {"call_ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9,
                     "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        log(f"int8 {name}: {ms:.3f} ms, {res[name]['GBps']:.0f} GB/s")
    del X, codes, absmax, y32, y16
    rng = np.random.default_rng(2024)
    W = torch.from_numpy(workloads.draw_weight(rng, 11008, 4096, "normal+outliers", 0.02)).cuda().reshape(-1)
    err = {}
    for block in api.INT8_BLOCKS:
        c, a = api.qlora_int8_quantize(W, block)
        d = api.qlora_int8_dequantize(c, a, block)
        err[str(block)] = ((d - W).double().pow(2).mean() / W.double().pow(2).mean()).sqrt().item()
    res["rel_rms_err_by_block"] = err
    log("int8 rel RMS err by block: " + ", ".join(f"{b}: {e:.5f}" for b, e in err.items()))
    return res


def bench_merge(api, workloads, reps=10):
    """Adapter merge (bf16 dequantised base + s L1 L2) for the LLaMA-7B
    linear shapes at r = 64: GB/s of the weight's algorithmic bytes (the
    quantised weight read once, the bf16 result written once, the adapters
    read once) against 8 TB/s; distinct weight copies so the caches cannot
    hold them."""
    import numpy as np
    import torch

    out = []
    for K, N in ((4096, 4096), (4096, 11008), (11008, 4096)):
        rng = np.random.default_rng(K + N)
        q0 = api.qlora_quantize(torch.from_numpy(workloads.draw_weight(rng, N, K, "normal", 0.02)).cuda())
        copies = 8
        qs = [api.NF4Tensor(q0.rows, q0.cols, q0.codes.clone(), q0.absmax8.clone(), q0.scale2.clone(),
                            q0.mean.clone()) for _ in range(copies)]
        L1 = (0.01 * torch.randn(K, 64, device="cuda")).to(torch.bfloat16)
        L2 = (0.01 * torch.randn(64, N, device="cuda")).to(torch.bfloat16)
        outs = [torch.empty((N, K), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        for i in range(copies):
            api.qlora_merge_adapters(qs[i], L1, L2, 0.25, out=outs[i % 2])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps * copies):
            api.qlora_merge_adapters(qs[i % copies], L1, L2, 0.25, out=outs[i % 2])
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * copies)
        nbytes = nf4_bytes(K, N) + 2 * N * K + 2 * 64 * (K + N)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out.append({"K": K, "N": N, "r": 64, "call_us": ms * 1e3, "GBps": gbps, "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS})
        log(f"merge {K}->{N} r=64: {ms * 1e3:.1f} us, {gbps:.0f} GB/s")
        del qs, outs
    return out


def bench_mid_m(api, workloads, reps=5):
    """Batched decode forward, M in {32, 64, 128}, on the LLaMA-7B linear
    shapes (r = 64): whole call and the fused dequant-GEMM + reduction
    (HIP events on the call's stream), weights cycled over 8 copies."""
    import numpy as np
    import torch

    out = []
    for K, N in ((4096, 4096), (4096, 11008), (11008, 4096)):
        rng = np.random.default_rng(K + 2 * N)
        q0 = api.qlora_quantize(torch.from_numpy(workloads.draw_weight(rng, N, K, "normal", 0.02)).cuda())
        copies = 8
        qs = [api.NF4Tensor(q0.rows, q0.cols, q0.codes.clone(), q0.absmax8.clone(), q0.scale2.clone(),
                            q0.mean.clone()) for _ in range(copies)]
        L1 = (0.01 * torch.randn(K, 64, device="cuda")).to(torch.bfloat16)
        L2 = (0.01 * torch.randn(64, N, device="cuda")).to(torch.bfloat16)
        for M in (32, 64, 128):
            X = torch.randn(M, K, device="cuda").to(torch.bfloat16)
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(api.qlora_linear_workspace(M, K, N, 64), dtype=torch.uint8, device="cuda")
            for i in range(copies):
                api.qlora_linear_fwd(qs[i], X, L1, L2, 0.25, Y=Y, workspace=ws)
            n = copies * reps
            timer = api.KernelTimer(api.QLORA_TIMING_MID_GEMM, capacity=n)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            with timer:
                e0.record()
                for i in range(n):
                    api.qlora_linear_fwd(qs[i % copies], X, L1, L2, 0.25, Y=Y, workspace=ws)
                e1.record()
            torch.cuda.synchronize()
            call_us = e0.elapsed_time(e1) / n * 1e3
            d = timer.durations_ms()
            k_us = sum(d) / len(d) * 1e3
            flops = 2 * M * N * K + 2 * M * 64 * (K + N)
            out.append({"K": K, "N": N, "M": M, "call_us": call_us, "kernel_us": k_us,
                        "kernel_weight_GBps": nf4_bytes(K, N) / (k_us * 1e-6) / 1e9,
                        "call_tflops": flops / (call_us * 1e-6) / 1e12})
            log(f"mid-M {K}->{N} M={M}: call {call_us:.1f} us, fused kernel + reduce {k_us:.1f} us")
        del qs
    return out


def bench_optim(api, reps=3):
    """The adapters' optimiser step at the size of all LLaMA-7B adapters
    (r = 64 on the 7 linears of 32 layers, 159.9 M fp32 values): the clip
    norm, and Adam with the first (1 - f) of the state (m, v) in HBM and the
    last f in pinned host memory, for f in {0, 0.25, 0.5, 0.75, 1} (one call
    per placement). The difference to f = 0 is the cost of paged-out state."""
    import torch

    n = 32 * 64 * (4 * (4096 + 4096) + 2 * (4096 + 11008) + (11008 + 4096))
    gen = torch.Generator(device="cuda").manual_seed(1)
    theta = 0.02 * torch.randn(n, device="cuda", generator=gen)
    g = 1e-4 * torch.randn(n, device="cuda", generator=gen)
    tb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    m_d = torch.zeros(n, device="cuda")
    v_d = torch.zeros(n, device="cuda")
    m_h = torch.zeros(n, dtype=torch.float32).pin_memory()
    v_h = torch.zeros(n, dtype=torch.float32).pin_memory()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    coef, _ = api.qlora_clip_grad_norm(g, 0.3)
    clip_ms = timed(lambda: api.qlora_clip_grad_norm(g, 0.3, coef=coef))
    out = {"params": n, "clip_ms": clip_ms, "clip_GBps": 4 * n / (clip_ms * 1e-3) / 1e9, "adam": []}
    log(f"optimiser: clip norm over {n} values {clip_ms:.3f} ms")
    state = [0]

    def step(frac):
        split = (int(n * (1 - frac)) // 4) * 4
        state[0] += 1
        t = state[0]
        if split > 0:
            api.qlora_adam_step(theta[:split], g[:split], m_d[:split], v_d[:split], t, lr=2e-4, coef=coef,
                                theta_bf16=tb[:split])
        if split < n:
            api.qlora_adam_step(theta[split:], g[split:], m_h[split:], v_h[split:], t, lr=2e-4, coef=coef,
                                theta_bf16=tb[split:])

    base = None
    for frac in (0.0, 0.25, 0.5, 0.75, 1.0):
        ms = timed(lambda: step(frac))
        base = ms if base is None else base
        host_bytes = 16 * (n - (int(n * (1 - frac)) // 4) * 4)
        row = {"host_fraction": frac, "ms": ms, "hbm_GBps_equiv": 30 * n / (ms * 1e-3) / 1e9,
               "host_link_GBps": host_bytes / (ms * 1e-3) / 1e9 if host_bytes else None, "vs_hbm_state": ms / base}
        out["adam"].append(row)
        log(f"optimiser: Adam with {int(100 * frac)} % of the state in host memory: {ms:.2f} ms "
            f"({ms / base:.1f}x the HBM-resident step)")
    del theta, g, tb, m_d, v_d, m_h, v_h
    return out


def bench_qtypes(api, workloads, reps=5):
    """The four 4-bit data types (with double quantisation) and NF4 without it
    on a 4096 x 11008 weight: relative RMS error of the dequantised weight
    (normal with 0.1 % outliers x10, and Student-t df = 4, both std 0.02),
    storage bits per parameter and quantise throughput (fp32 input)."""
    import numpy as np
    import torch

    out = {}
    rng = np.random.default_rng(2024)
    weights = {"normal+outliers": workloads.draw_weight(rng, 11008, 4096, "normal+outliers", 0.02),
               "student-t4": workloads.draw_weight(rng, 11008, 4096, "student-t4", 0.02)}
    variants = [(name, name, True) for name in api.QTYPES] + [("nf4_no_dq", "nf4", False)]
    for label, name, dq in variants:
        res = {"bits_per_param": 8 * nf4_bytes(4096, 11008, dq) / (4096 * 11008)}
        for kind, Wh in weights.items():
            W = torch.from_numpy(Wh).cuda()
            q = api.qlora_quantize(W, qtype=name, double_quant=dq)
            d = api.qlora_dequantize(q).float()
            err = ((d - W).double().pow(2).mean() / W.double().pow(2).mean()).sqrt().item()
            res[f"rel_rms_err_{kind}"] = err
            if kind == "normal+outliers":
                ws = torch.empty(api.qlora_quant_sizes(11008, 4096)["workspace"], dtype=torch.uint8, device="cuda")
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(reps):
                    api.qlora_quantize(W, out=q, workspace=ws)
                e1.record()
                torch.cuda.synchronize()
                call_ms = e0.elapsed_time(e1) / reps
                res["quantize_call_ms"] = call_ms
                res["quantize_GBps"] = (W.numel() * 4 + nf4_bytes(4096, 11008, dq)) / (call_ms * 1e-3) / 1e9
        out[label] = res
        log(f"qtype {label}: rel RMS err normal+outliers {res['rel_rms_err_normal+outliers']:.4f}, "
            f"student-t4 {res['rel_rms_err_student-t4']:.4f}; quantize {res['quantize_GBps']:.0f} GB/s")
    return out


def host_info():
    """Host cores, CPU model and BLAS library of this machine (for the
    oracle baselines)."""
    import subprocess

    import numpy as np

    info = {"os_cpu_count": os.cpu_count()}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info

        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = max(int(p.get("num_threads", 1)) for p in blas)
    except Exception:  # pragma: no cover
        pass
    if "blas" not in info:
        cfg = np.show_config(mode="dicts") if hasattr(np, "show_config") else {}
        try:
            info["blas"] = cfg["Build Dependencies"]["blas"]["name"]
        except Exception:  # pragma: no cover
            info["blas"] = "unknown"
    return info


def cpu_baseline(host, tokens=8192):
    """The oracle (dequant + forward + backward) on all 7 linears of the
    timed step, on the host cores; reported in the same unit."""
    from oracle import linear, nf4

    hi = host_info()
    cores = hi.get("blas_threads", os.cpu_count() or 1)
    qts = [(shp, inp, nf4.quantize(inp.W)) for shp, inp in host]   # outside the timed region
    flops = 0
    t0 = time.perf_counter()
    for shp, inp, qt in qts:
        Wd = nf4.dequantize(qt, inp.W.shape)
        X, dY = inp.X[:tokens], inp.dY[:tokens]
        linear.linear_fwd(X, Wd, inp.L1, inp.L2, inp.s)
        linear.linear_bwd(X, Wd, inp.L1, inp.L2, inp.s, dY)
        flops += linear_flops(tokens, shp.K, shp.N, inp.L1.shape[1])
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "seconds": dt, "host": hi,
            "sample": f"the whole timed step: all 7 linears, {tokens} tokens; float64 NumPy dequant + fwd + bwd. "
                      f"The matmuls run on {cores} BLAS threads; the dequantisation is single-threaded NumPy."}


def setup_and_time(api, workloads, name, steps, warmup, trials):
    """Quantise the 7 linears of a layer set, run warmup steps, then time
    ``trials`` runs of ``steps`` steps each (HIP events around each run,
    synchronised on both sides), and one more pass of the same steps with
    event brackets around every GEMM launch for the kernel's roofline."""
    import torch

    layers, host, ws = setup_layer(api, workloads, name)
    flops_step = sum(linear_flops(d["M"], d["shape"].K, d["shape"].N, d["r"]) for d in layers)
    fwd_flops = [2 * d["M"] * d["shape"].K * d["shape"].N + 2 * d["M"] * d["r"] * d["shape"].N for d in layers]
    dx_flops = [2 * d["M"] * d["shape"].K * d["shape"].N + 2 * d["M"] * d["r"] * d["shape"].K for d in layers]
    for _ in range(warmup):
        run_step(api, layers, ws)
    torch.cuda.synchronize()
    trial_ms = []
    wall = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            run_step(api, layers, ws)
        e1.record()
        torch.cuda.synchronize()
        wall.append((time.perf_counter() - w0) / steps * 1e3)
        trial_ms.append(e0.elapsed_time(e1) / steps)
    ms_step = sorted(trial_ms)[len(trial_ms) // 2]
    value = flops_step / (ms_step * 1e-3) / 1e12
    log(f"{name}: step {ms_step:.3f} ms (median of {trials} trials of {steps} steps: "
        f"{', '.join(f'{t:.3f}' for t in trial_ms)}), {value:.1f} TFLOP/s")
    n_l = len(layers)
    t_fwd = api.KernelTimer(api.QLORA_TIMING_FWD_GEMM, capacity=n_l * steps)
    t_dx = api.KernelTimer(api.QLORA_TIMING_DX_GEMM, capacity=n_l * steps)
    torch.cuda.synchronize()
    with t_fwd, t_dx:
        for _ in range(steps):
            run_step(api, layers, ws)
    torch.cuda.synchronize()
    dfwd, ddx = t_fwd.durations_ms(), t_dx.durations_ms()
    kf = kernel_summary(dfwd, fwd_flops * steps)
    kd = kernel_summary(ddx, dx_flops * steps)
    kg = kernel_summary(dfwd + ddx, fwd_flops * steps + dx_flops * steps)
    log(f"{name}: fwd GEMM {kf['tflops']:.1f} TFLOP/s avg {kf['avg_ms']:.3f} ms; "
        f"dX GEMM {kd['tflops']:.1f} TFLOP/s avg {kd['avg_ms']:.3f} ms")
    # gemm_nt_kernel runs both products (one launch each per linear): its
    # algorithmic flops per launch averaged over the 14 launches of a step,
    # over its average launch duration.
    traffic, traffic_exact = gemm_traffic(name)
    roofline = {"bound": "mfma", "achieved": kg["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": kg["tflops"] / PEAK_BF16_TFLOPS, "traffic": traffic, "traffic_exact": traffic_exact,
                "kernel": "gemm_nt_kernel", "avg_launch_ms": kg["avg_ms"], "launches": kg["launches"],
                "flops_per_launch": (sum(fwd_flops) + sum(dx_flops)) / (2 * n_l)}
    shp_desc = ", ".join(f"{d['shape'].name} {d['shape'].K}->{d['shape'].N}" for d in layers)
    cfg = workloads.WORKLOADS[name]
    config = {"workload": f"{name}: 7 linears ({shp_desc}), {layers[0]['M']} tokens, NF4+DQ base "
                          f"(block 64, DQ block 256, {cfg['w_kind']} weights std {cfg['w_std']}), "
                          f"LoRA r={layers[0]['r']} s={layers[0]['s']} on all 7, fwd+bwd per step",
              "tokens": layers[0]["M"], "rank": layers[0]["r"], "lora_scale": layers[0]["s"],
              "flops_per_step": flops_step}
    res = {"ms_per_step": ms_step, "value": value, "trials_ms_per_step": trial_ms,
           "wall_ms_per_step": wall, "roofline": roofline, "kernels": {"fwd_gemm": kf, "dx_gemm": kd},
           "config": config, "flops_per_step": flops_step}
    return res, layers, host, ws


def bench_quantize_pass(api, workloads, layers=80, pool=2, oracle_layer=True):
    """The LLaMA-65B-shaped quantisation pass: ``layers`` x 7 tensors (q, k,
    v, o 8192x8192; gate, up 8192->22016; down 22016->8192) quantised to NF4
    + DQ from fp32 and from bf16. The inputs are a pool of ``pool`` distinct
    layers (host-drawn, N(0, 0.015)), cycled so that every layer writes its
    own output set (codes, absmax8, scale2, mean); the whole pass is timed
    with HIP events, once with one qlora_quantize_batch call per layer (the
    reported figure) and once with one qlora_quantize call per tensor.
    GB/s = (input + output bytes) / time. The oracle
    quantises one layer (fp32 input) on the host cores; the pass estimate is
    that time x 80."""
    import torch

    shapes = workloads.LLAMA65B
    res = {"layers": layers, "tensors": layers * len(shapes), "pool_layers": pool}
    outs = []
    for _ in range(layers):
        outs.append([api.NF4Tensor.empty(sh.N, sh.K) for sh in shapes])
    ws = torch.empty(max(api.qlora_quant_sizes(sh.N, sh.K)["workspace"] for sh in shapes), dtype=torch.uint8,
                     device="cuda")
    numel = sum(sh.N * sh.K for sh in shapes) * layers
    out_bytes = sum(nf4_bytes(sh.K, sh.N) for sh in shapes) * layers
    res["weights"] = numel
    res["output_bytes"] = out_bytes
    pool32 = []
    for li in range(pool):
        pool32.append([torch.from_numpy(workloads.quantize_weight(sh, 4, 7 * li + i)).cuda()
                       for i, sh in enumerate(shapes)])
        log(f"65B pass: pool layer {li} drawn")
    ws_b = torch.empty(api.qlora_quant_batch_workspace([(sh.N, sh.K) for sh in shapes]), dtype=torch.uint8,
                       device="cuda")

    def timed_pass(src, batched):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for layer in range(layers):
            if batched:     # one call per layer: its 7 tensors share the launches
                api.qlora_quantize_batch(src[layer % pool], outs=outs[layer], workspace=ws_b)
            else:
                for i, w in enumerate(src[layer % pool]):
                    api.qlora_quantize(w, out=outs[layer][i], workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    for dt in ("f32", "bf16"):
        src = pool32 if dt == "f32" else [[w.to(torch.bfloat16) for w in lay] for lay in pool32]
        for i, w in enumerate(src[0]):      # warm-up of every shape, both call forms
            api.qlora_quantize(w, out=outs[0][i], workspace=ws)
        api.qlora_quantize_batch(src[0], outs=outs[0], workspace=ws_b)
        ms_single = timed_pass(src, False)
        ms = timed_pass(src, True)
        in_bytes = numel * (4 if dt == "f32" else 2)
        gbps = (in_bytes + out_bytes) / (ms * 1e-3) / 1e9
        gbps_single = (in_bytes + out_bytes) / (ms_single * 1e-3) / 1e9
        res[dt] = {"ms": ms, "input_bytes": in_bytes, "GBps": gbps, "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS,
                   "roofline_ms": (in_bytes + out_bytes) / (PEAK_HBM_GBPS * 1e9) * 1e3,
                   "calls": "qlora_quantize_batch, one per layer (7 tensors)",
                   "per_tensor_calls": {"ms": ms_single, "GBps": gbps_single,
                                        "frac_of_hbm_peak": gbps_single / PEAK_HBM_GBPS}}
        log(f"65B pass from {dt}: {ms:.1f} ms for {layers * len(shapes)} tensors, {gbps:.0f} GB/s "
            f"(one call per layer; one call per tensor: {ms_single:.1f} ms, {gbps_single:.0f} GB/s)")
        if dt == "bf16":
            del src
    del outs, ws, ws_b
    if oracle_layer:
        from oracle import nf4

        host = [workloads.quantize_weight(sh, 4, i) for i, sh in enumerate(shapes)]
        t0 = time.perf_counter()
        for w in host:
            nf4.quantize(w)
        dt = time.perf_counter() - t0
        res["cpu_oracle"] = {"seconds_one_layer": dt, "seconds_pass_estimate": dt * layers,
                             "GBps_estimate": (numel * 4 + out_bytes) / (dt * layers) / 1e9,
                             "sample": "one layer (7 tensors, 809.5M weights, fp32 input) through the NumPy "
                                       "oracle, single-threaded; the pass estimate is x80"}
        log(f"65B pass: oracle one layer {dt:.1f} s (x80 = {dt * layers:.0f} s)")
    del pool32
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=["llama7b-layer", "llama33b-layer"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline step")
    ap.add_argument("--only", choices=["gemv", "mid_m", "merge", "quantize", "quantize_pass", "attainable"],
                    help="run one extra section alone and print its JSON (for profiling)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (calibration of the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_nf4_quantized_amd import api, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe()
        return
    api.library()
    if args.only:
        fn = {"gemv": lambda: bench_gemv(api, workloads), "mid_m": lambda: bench_mid_m(api, workloads),
              "merge": lambda: bench_merge(api, workloads), "quantize": lambda: bench_quantize(api, workloads),
              "quantize_pass": lambda: bench_quantize_pass(api, workloads, oracle_layer=False),
              "attainable": lambda: attainable_peaks(api)}[args.only]
        print(json.dumps({args.only: fn()}), flush=True)
        return
    name = args.workload
    peaks = attainable_peaks(api)
    head, layers, host, ws = setup_and_time(api, workloads, name, args.steps, args.warmup, args.trials)
    head["roofline"]["attainable"] = peaks["mfma_bf16_tflops"]
    head["roofline"]["frac_of_attainable"] = head["roofline"]["achieved"] / peaks["mfma_bf16_tflops"]
    result = {
        "metric": "QLoRA NF4 linear fwd+bwd TFLOP/s; NF4 GEMV weight GB/s (% of peak)",
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "trials_ms_per_step": head["trials_ms_per_step"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "attainable": peaks,
    }
    if not args.no_extras:
        del ws
        torch.cuda.empty_cache()
        p_drop = 0.05 if name == "llama33b-layer" else 0.1
        result["dropout_step"] = bench_dropout_step(api, layers, head["flops_per_step"], head["ms_per_step"],
                                                    p=p_drop)
    del layers
    torch.cuda.empty_cache()
    if not args.no_extras:
        other = "llama7b-layer" if name == "llama33b-layer" else "llama33b-layer"
        sec, l2, host2, ws2 = setup_and_time(api, workloads, other, max(args.steps // 2, 5), 3, 1)
        del l2, ws2
        torch.cuda.empty_cache()
        result[other.replace("-", "_") + "_step"] = {k: sec[k] for k in ("value", "ms_per_step", "roofline",
                                                                          "kernels", "config")}
        if not args.no_cpu_baseline:   # the oracle on this step too (a context figure, like cpu_baseline)
            result[other.replace("-", "_") + "_step"]["cpu_oracle"] = cpu_baseline(host2)
            log(f"{other}: oracle step {result[other.replace('-', '_') + '_step']['cpu_oracle']['seconds']:.1f} s")
        del host2
        result["gemv"] = bench_gemv(api, workloads, oracle=not args.no_cpu_baseline)
        for g in result["gemv"]:
            g["graph_call_frac_of_attainable_read"] = g["graph_call_GBps"] / peaks["hbm_read_GBps"]
        result["quantize"] = bench_quantize(api, workloads)
        result["quantize_65b_pass"] = bench_quantize_pass(api, workloads, oracle_layer=not args.no_cpu_baseline)
        result["qtypes"] = bench_qtypes(api, workloads)
        result["int8"] = bench_int8(api, workloads)
        result["merge"] = bench_merge(api, workloads)
        result["mid_m"] = bench_mid_m(api, workloads)
        result["optimiser"] = bench_optim(api)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(host)
        log(f"cpu baseline {result['cpu_baseline']['value']:.4f} TFLOP/s in {result['cpu_baseline']['seconds']:.1f} s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
