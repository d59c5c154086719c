#!/usr/bin/env python3
"""Throughput of exact attention forward + backward on one MI355X, through the C ABI.

One step is one pass of the whole path over one batch: fa_fwd, then the backward's two phases as
fa_bwd runs them (fa_bwd_delta_dq: D = dO·O and dQ; fa_bwd_dkdv: dK and dV), with every input
already resident in device memory.
FLOPs follow the usual convention: forward 4·B·H·N²·d (halved when causal), backward 2.5× the
forward.  W untimed warm-up steps, then exactly K timed steps between two device
synchronisations; HIP events on the launch stream give each kernel's own duration.

Prints one JSON line on stdout (progress goes to stderr).  Only one GPU is used: --gpus above 1 is
refused.  The ``cpu_baseline`` leg times the fp64 CPU oracle on a bounded sample of the same
workload's heads; it is a reported baseline, not a target.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s fwd+bwd (bf16, d=128, N=4096 causal) and % of MFMA peak"
# MI355X published dense peaks: 256 CUs × 2.4 GHz; bf16 matrix cores 4096 FLOP/clk/CU.
BF16_PEAK_TFLOPS = 256 * 2.4e9 * 4096 / 1e12     # 2516.6
FP8_PEAK_TFLOPS = 2 * BF16_PEAK_TFLOPS            # 5033.2 (dense e4m3 matrix cores)
HBM_PEAK_GBS = 8000.0
# Published figures of the method on other hardware, for workloads the source does not state
# ("Anatomy of a FlashAttention Kernel", section "What changed between FlashAttention 1, 2, and 3?").
# Context only: none is for this metric and workload, so vs_baseline stays null.
PAGES_FIGURES = {
    "flashattention2_a100_fraction_of_peak": [0.50, 0.73],
    "flashattention3_h100_fp16_tflops": 740.0,
    "flashattention3_h100_fp16_fraction_of_peak": 0.75,
    "flashattention3_h100_fp8_tflops_about": 1200.0,
    "workloads": "not stated",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_text(path):
    """A source file's code without comments and blank lines: edits to comments leave it unchanged."""
    with open(path, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_sha(name):
    """sha256 prefix over the code (not the comments) of a kernel's source file and of the device
    headers every kernel includes."""
    h = hashlib.sha256()
    for part in (name, "fa_common.h", "fa_launch.h"):
        h.update(_code_text(os.path.join(ROOT, "io_aware_exact_18_amd", "csrc", part)).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, src):
    """HBM bytes per launch from the committed counter summary, if it was taken on this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("src_sha") != source_sha(src):
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, inp, budget_s):
    """Time the oracle's forward + backward on whole heads of the workload, up to ~budget_s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the visible core count
        threads = os.cpu_count()
    B, H, N, d = w.shape()
    flat = {k: inp[k].reshape(B * H, N, d) for k in ("q", "k", "v", "do")}
    heads, t_total = 0, 0.0
    while heads < B * H and t_total < budget_s:
        h = heads
        q, k, v, do = (flat[x][h].double().numpy() for x in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        oracle.attention_head_fwd64(q, k, v, w.causal, w.scale)
        oracle.attention_head_bwd64(q, k, v, do, w.causal, w.scale)
        t_total += time.perf_counter() - t0
        heads += 1
    per_head_flops = (w.fwd_flops() + w.bwd_flops()) / (B * H)
    tflops = heads * per_head_flops / t_total / 1e12
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle, forward+backward of {heads} of {B * H} heads "
                  f"(N={N}, d={d}, causal={w.causal}) in {t_total:.1f} s; whole-job time "
                  f"extrapolated as {B * H / heads:.1f}x (heads are independent and equal in cost)",
        "seconds_for_sample": t_total,
        "extrapolated_job_seconds": t_total * B * H / heads,
    }


def sclk_sysfs_path(torch):
    """The pp_dpm_sclk file of the device torch calls cuda:0, found by its PCI address, or None."""
    import glob
    pr = torch.cuda.get_device_properties(0)
    want = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}."
    for card in glob.glob("/sys/class/drm/card*/device"):
        try:
            if os.path.basename(os.path.realpath(card)).startswith(want):
                path = os.path.join(card, "pp_dpm_sclk")
                return path if os.access(path, os.R_OK) else None
        except OSError:
            continue
    return None


def sample_sclk(path, busy, seconds=1.0, period=0.01):
    """Mean shader clock (MHz) read from the driver's current-level line of pp_dpm_sclk while
    `busy()` keeps the GPU loaded for about `seconds`; None if the file cannot be read."""
    import threading
    samples, stop = [], threading.Event()

    def reader():
        while not stop.is_set():
            try:
                with open(path) as f:
                    for line in f:
                        if "*" in line:
                            mhz = "".join(ch for ch in line.split(":", 1)[1] if ch.isdigit())
                            if mhz:
                                samples.append(int(mhz))
            except OSError:
                return
            time.sleep(period)

    th = threading.Thread(target=reader, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        busy()
    stop.set()
    th.join()
    if not samples:
        return None
    return {"mean_mhz": sum(samples) / len(samples), "min_mhz": min(samples),
            "max_mhz": max(samples), "samples": len(samples), "source": path}


def device_block(fa, torch, busy):
    """Device facts reported beside the measurement: the bf16 peak recomputed from the device's
    compute units × peak clock × 4096 FLOP/clk/CU, and the shader clock seen under this load."""
    cus, khz = fa.device_info(0)
    path = sclk_sysfs_path(torch)
    return {
        "name": torch.cuda.get_device_properties(0).name,
        "arch": torch.cuda.get_device_properties(0).gcnArchName,
        "compute_units": cus,
        "peak_clock_mhz": khz / 1e3,
        "bf16_peak_from_device_tflops": cus * khz * 1e3 * 4096 / 1e12,
        "sclk_under_load": sample_sclk(path, busy) if path else None,
    }


def cpu_full_runs(workloads):
    """The oracle over every head of the two small workloads (forward, and backward where the
    workload has one), timed in full."""
    import oracle
    out = {}
    for name in ("fwd_small", "d64_2k"):
        w = workloads.WORKLOADS[name]
        B, H, N, d = w.shape()
        inp = workloads.make_inputs(name)
        flat = {k: inp[k].reshape(B * H, N, d) for k in inp}
        t0 = time.perf_counter()
        for h in range(B * H):
            q, k, v = (flat[x][h].double().numpy() for x in ("q", "k", "v"))
            oracle.attention_head_fwd64(q, k, v, w.causal, w.scale)
            if w.backward:
                oracle.attention_head_bwd64(q, k, v, flat["do"][h].double().numpy(), w.causal,
                                            w.scale)
        t = time.perf_counter() - t0
        flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0)
        out[name] = {"seconds": t, "heads": B * H, "tflops": flops / t / 1e12,
                     "passes": "forward+backward" if w.backward else "forward"}
    return out


def traffic_sweep(fa, torch, steps):
    """Forward at N = 1k..16k (B=1, H=32, d=128, causal), `steps` launches each, for HBM byte
    counters: measured bytes should grow linearly in N while S and P, had they been materialised in
    bf16 (written and read once each), would grow as N²."""
    B, H, d = 1, 32, 128
    g = torch.Generator().manual_seed(77)
    for N in (1024, 2048, 4096, 8192, 16384):
        q, k, v = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to("cuda:0")
                   for _ in range(3))
        for _ in range(steps):
            o, lse = fa.fwd(q, k, v, True, 1.0 / math.sqrt(d))
        torch.cuda.synchronize()
        print(json.dumps({"N": N, "B": B, "H": H, "d": d, "launches": steps,
                          "grid_workgroups": B * H * ((N + 127) // 128),
                          "algorithmic_bytes": 4 * B * H * N * d * 2 + B * H * N * 4,
                          "materialised_s_p_bytes": 4 * B * H * N * N * 2}), flush=True)
        del q, k, v, o, lse


# The secondary legs each start after idle host work (building their inputs). After such a pause the
# shader clock starts low and climbs over the first tens of milliseconds of load (kernel traces of
# causal_4k: steps of 3.0 ms falling to 2.24 ms over the first ~20). A secondary leg therefore warms
# up for at least `warmup` calls and at least SETTLE_S seconds of load before its timed calls, so
# that it is timed at the settled clock. The headline leg runs exactly the warm-up steps it is given.
SETTLE_S = 0.25


def settle(run, warmup, min_s=SETTLE_S):
    """Call run() at least `warmup` times and until min_s seconds of wall time have passed,
    synchronising every fourth call so that wall time follows the device's work."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < min_s:
        run()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    return n


def decode_measure(fa, workloads, lib, steps, warmup):
    """Secondary measurement: decoding against a key/value cache (both decoding workloads), timed
    with events around fa_decode (split and merge kernels).  HBM-bound: priced against 8 TB/s with
    the algorithmic bytes (cache read once, Q read, O and LSE written).  The inputs are N(0,1) bf16
    drawn on the device from a seeded generator (timing does not depend on the values; the parity
    tests use the CPU-drawn workload inputs)."""
    import torch
    out = {}
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for name in ("decode_32k", "specdec_32k"):
        w = workloads.DECODE_WORKLOADS[name]
        log(f"[bench] secondary: {name} decode B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d}")
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 * w.number)
        q = torch.randn(w.q_shape(), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn(w.kv_shape(), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn(w.kv_shape(), generator=gen, device=dev).to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty(w.q_shape()[:3], dtype=torch.float32, device=dev)
        ws_bytes = fa.decode_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def run():
            code = lib.fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), ws.data_ptr(), ws_bytes, w.B, w.H, w.Nq, w.Nk, w.d,
                                 int(w.causal), w.scale, stream.cuda_stream)
            if code != 0:
                raise fa.FaError("fa_decode", code, fa.status_str(code))

        settle(run, warmup)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(steps):
            run()
        ev[1].record(stream)
        torch.cuda.synchronize(dev)
        ms = ev[0].elapsed_time(ev[1]) / steps
        algo = w.kv_bytes() + 2 * q.numel() * 2 + lse.numel() * 4
        gbs = algo / (ms * 1e-3) / 1e9
        out[name + "_decode"] = {"workload": name, "kernels": ["decode_split_kernel", "decode_merge_kernel"],
                                 "ms": ms, "achieved_gbs": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": gbs / HBM_PEAK_GBS, "bound": "hbm",
                                 "algorithmic_bytes": algo, "workspace_bytes": ws_bytes}
        del q, k, v, o, lse, ws
        torch.cuda.empty_cache()
    return out


def fp8_forward(fa, workloads, lib, steps, warmup, name="fp8_8k"):
    """Secondary measurement: the FP8 forward on an fp8 workload (fp8_8k; fp8_d64_8k, fp8_d96_8k and
    fp8_d256_8k at the other head dimensions), timed with events."""
    import torch
    w = workloads.WORKLOADS[name]
    B, H, N, d = w.shape()
    log(f"[bench] secondary: {w.name} fp8 forward B={B} H={H} N={N} d={d} causal={w.causal}")
    inp = workloads.make_inputs(w.name)
    dev = torch.device("cuda:0")
    q8, k8, v8 = (inp[x].to(dev) for x in ("q8", "k8", "v8"))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run():
        code = lib.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), inp["sq"], inp["sk"],
                              inp["sv"], o.data_ptr(), lse.data_ptr(), B, H, N, d, int(w.causal),
                              w.scale, stream.cuda_stream)
        if code != 0:
            raise fa.FaError("fa_fwd_fp8", code, fa.status_str(code))

    settle(run, warmup)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        run()
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    ms = ev[0].elapsed_time(ev[1]) / steps
    tflops = w.fwd_flops() / (ms * 1e-3) / 1e12
    return {"workload": w.name, "kernel": "fwd_fp8_kernel", "ms": ms, "tflops": tflops,
            "peak": FP8_PEAK_TFLOPS, "frac": tflops / FP8_PEAK_TFLOPS, "bound": "mfma",
            "flops": w.fwd_flops()}


def fp8_backward(fa, workloads, lib, steps, warmup):
    """Secondary measurement: the FP8 backward (fa_bwd_fp8: widening of the e4m3 codes, D, dK/dV,
    dQ) on fp8bwd_8k with O and LSE from the FP8 forward, timed with events; FLOPs 2.5× the forward
    by the usual convention.  The FP8 forward is timed as well, for the whole fp8 step."""
    import torch
    w = workloads.WORKLOADS["fp8bwd_8k"]
    B, H, N, d = w.shape()
    log(f"[bench] secondary: {w.name} fp8 backward B={B} H={H} N={N} d={d} causal={w.causal}")
    inp = workloads.make_inputs(w.name)
    dev = torch.device("cuda:0")
    q8, k8, v8, do = (inp[x].to(dev) for x in ("q8", "k8", "v8", "do"))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(o) for _ in range(3))
    ws_bytes = fa.bwd_fp8_workspace_bytes(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    c = int(w.causal)

    def fwd():
        code = lib.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), inp["sq"], inp["sk"],
                              inp["sv"], o.data_ptr(), lse.data_ptr(), B, H, N, d, c, w.scale, sp)
        if code != 0:
            raise fa.FaError("fa_fwd_fp8", code, fa.status_str(code))

    def bwd():
        code = lib.fa_bwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), inp["sq"], inp["sk"],
                              inp["sv"], o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws_bytes, B, H, N, d, c,
                              w.scale, sp)
        if code != 0:
            raise fa.FaError("fa_bwd_fp8", code, fa.status_str(code))

    settle(lambda: (fwd(), bwd()), warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
    torch.cuda.synchronize(dev)
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    out = {"workload": w.name, "kernels": ["e4m3_to_bf16_kernel", "bwd_dq_kernel",
                                           "bwd_dkdv_kernel"],
           "bwd_ms": bwd_ms, "bwd_tflops": bwd_f / (bwd_ms * 1e-3) / 1e12, "fwd_ms": fwd_ms,
           "step_tflops": (fwd_f + bwd_f) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12,
           "bound": "mfma", "peak": BF16_PEAK_TFLOPS, "flops": bwd_f,
           "workspace_bytes": ws_bytes}
    out["frac"] = out["bwd_tflops"] / BF16_PEAK_TFLOPS
    del q8, k8, v8, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return out


def fwd_bwd_secondary(fa, workloads, lib, name, steps, warmup):
    """Secondary measurement: forward + backward of another bf16 workload (d256_4k, d96_4k: head
    dimensions 256 and 96; d64_2k, long_16k: the other forward + backward workloads), each phase
    bracketed by events; TFLOP/s by the same FLOP convention as the headline."""
    import torch
    w = workloads.WORKLOADS[name]
    B, H, N, d = w.shape()
    log(f"[bench] secondary: {name} forward+backward B={B} H={H} N={N} d={d} causal={w.causal}")
    inp = workloads.make_inputs(name)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    del inp
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws_bytes = fa.bwd_workspace_bytes(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    c = int(w.causal)

    def check(fn, code):
        if code != 0:
            raise fa.FaError(fn, code, fa.status_str(code))

    def step(ev):
        ev[0].record(stream)
        check("fa_fwd", lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), B, H, N, d, c, w.scale, sp))
        ev[1].record(stream)
        check("fa_bwd_delta_dq", lib.fa_bwd_delta_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                     o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                                     dq.data_ptr(), ws.data_ptr(), ws_bytes, B, H,
                                                     N, d, c, w.scale, sp))
        ev[2].record(stream)
        check("fa_bwd_dkdv", lib.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             lse.data_ptr(), do.data_ptr(), dk.data_ptr(),
                                             dv.data_ptr(), ws.data_ptr(), ws_bytes, B, H, N, d, c,
                                             w.scale, sp))
        ev[3].record(stream)

    spare = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    settle(lambda: step(spare), warmup)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize(dev)
    ph = [sum(e[i].elapsed_time(e[i + 1]) for e in events) / steps for i in range(3)]
    step_ms = sum(e[0].elapsed_time(e[3]) for e in events) / steps
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    out = {"workload": name, "ms": step_ms, "tflops": (fwd_f + bwd_f) / (step_ms * 1e-3) / 1e12,
           "peak": BF16_PEAK_TFLOPS, "bound": "mfma", "flops": fwd_f + bwd_f,
           "phases_ms": {"fwd": ph[0], "bwd_delta_dq": ph[1], "bwd_dkdv": ph[2]},
           "fwd_tflops": fwd_f / (ph[0] * 1e-3) / 1e12,
           "bwd_tflops": bwd_f / ((ph[1] + ph[2]) * 1e-3) / 1e12}
    out["frac"] = out["tflops"] / BF16_PEAK_TFLOPS
    del q, k, v, do, o, dq, dk, dv, lse, ws
    torch.cuda.empty_cache()
    return out


def split_secondary(fa, workloads, lib, name, steps, warmup):
    """Secondary measurement: forward + backward of a workload with too few query tiles to fill the
    device, once through fa_fwd + fa_bwd and once through the key-range split entry points
    (fa_fwd_split + fa_bwd_split) on the same inputs; each step bracketed by events."""
    import torch
    w = workloads.WORKLOADS[name]
    B, H, N, d = w.shape()
    log(f"[bench] secondary: {name} forward+backward, unsplit and split, B={B} H={H} N={N} d={d}")
    inp = workloads.make_inputs(name)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    del inp
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    c = int(w.causal)
    ws_f = fa.fwd_split_workspace_bytes(B, H, N, d, c)
    ws_b = fa.bwd_split_workspace_bytes(B, H, N, d, c)
    ws = torch.empty(max(ws_f, ws_b, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ptrs = [x.data_ptr() for x in (q, k, v, o, lse, do, dq, dk, dv)]

    def check(fn, code):
        if code != 0:
            raise fa.FaError(fn, code, fa.status_str(code))

    def plain(ev):
        ev[0].record(stream)
        check("fa_fwd", lib.fa_fwd(*ptrs[:5], B, H, N, d, c, w.scale, sp))
        ev[1].record(stream)
        check("fa_bwd", lib.fa_bwd(*ptrs, ws.data_ptr(), ws.numel(), B, H, N, d, c, w.scale, sp))
        ev[2].record(stream)

    def split(ev):
        ev[0].record(stream)
        check("fa_fwd_split", lib.fa_fwd_split(*ptrs[:5], ws.data_ptr(), ws.numel(), B, H, N, d, c,
                                               w.scale, sp))
        ev[1].record(stream)
        check("fa_bwd_split", lib.fa_bwd_split(*ptrs, ws.data_ptr(), ws.numel(), B, H, N, d, c,
                                               w.scale, sp))
        ev[2].record(stream)

    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    out = {"workload": name, "peak": BF16_PEAK_TFLOPS, "bound": "mfma", "flops": fwd_f + bwd_f,
           "fwd_split_workspace_bytes": ws_f, "bwd_split_workspace_bytes": ws_b}
    for label, fn in (("unsplit", plain), ("split", split)):
        spare = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        settle(lambda: fn(spare), warmup)
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            fn(events[i])
        torch.cuda.synchronize(dev)
        f_ms = sum(e[0].elapsed_time(e[1]) for e in events) / steps
        b_ms = sum(e[1].elapsed_time(e[2]) for e in events) / steps
        out[label] = {"ms": f_ms + b_ms, "fwd_ms": f_ms, "bwd_ms": b_ms,
                      "tflops": (fwd_f + bwd_f) / ((f_ms + b_ms) * 1e-3) / 1e12,
                      "fwd_tflops": fwd_f / (f_ms * 1e-3) / 1e12,
                      "bwd_tflops": bwd_f / (b_ms * 1e-3) / 1e12}
    del q, k, v, do, o, dq, dk, dv, lse, ws
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="causal_4k",
                    help="bf16 forward+backward workload (default: the throughput workload)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the cpu_baseline leg (0 skips it)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the secondary FP8 measurements (fp8_8k forward, fp8bwd_8k backward)")
    ap.add_argument("--no-fp8-bwd", action="store_true",
                    help="skip only the secondary FP8 backward measurement (fp8bwd_8k), whose "
                         "kernels are the causal d=128 backward instantiations")
    ap.add_argument("--no-head-dims", action="store_true",
                    help="skip the secondary measurements at head dimensions 256 and 96 "
                         "(d256_4k, d96_4k workloads)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the secondary measurements of the d64_2k, long_16k and "
                         "onehead_32k workloads (long_16k runs the causal d=128 kernel "
                         "instantiations, onehead_32k their split forms)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the secondary decoding measurements (decode_32k, specdec_32k)")
    ap.add_argument("--traffic-sweep", action="store_true",
                    help="instead of the bench, run the forward at N = 1k..16k (B=1, H=32, d=128, "
                         "causal) `--steps` times each, for HBM byte counters")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the bench, run a plain device copy of MIB MiB `--steps` times "
                         "(the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "attention over heads shards with no communication, so multi-GPU figures are not "
              "produced here", file=sys.stderr)
        sys.exit(2)

    import torch
    import io_aware_exact_18_amd as fa
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a ROCm device"
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}))
        return
    if args.traffic_sweep:
        traffic_sweep(fa, torch, args.steps)
        return
    w = workloads.WORKLOADS[args.workload]
    if w.fp8 or not w.backward:
        raise SystemExit("choose a bf16 forward+backward workload")
    B, H, N, d = w.shape()
    log(f"[bench] workload {w.name}: B={B} H={H} N={N} d={d} causal={w.causal}")
    inp = workloads.make_inputs(w.name)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws_bytes = fa.bwd_workspace_bytes(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    lib = fa.library()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    causal = int(w.causal)
    scale = w.scale

    def check(name, code):
        if code != 0:
            raise fa.FaError(name, code, fa.status_str(code))

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        check("fa_fwd", lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), B, H, N, d, causal, scale, sp))
        if ev is not None:
            ev[1].record(stream)
        check("fa_bwd_delta_dq", lib.fa_bwd_delta_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                     o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                                     dq.data_ptr(), ws.data_ptr(), ws_bytes, B, H,
                                                     N, d, causal, scale, sp))
        if ev is not None:
            ev[2].record(stream)
        check("fa_bwd_dkdv", lib.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             lse.data_ptr(), do.data_ptr(), dk.data_ptr(),
                                             dv.data_ptr(), ws.data_ptr(), ws_bytes, B, H, N, d,
                                             causal, scale, sp))
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    log(f"[bench] warm-up done ({args.warmup} steps)")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    def durations(a, b):
        return sorted(e[a].elapsed_time(e[b]) for e in events)

    def avg(a, b):
        return sum(durations(a, b)) / len(events)

    fwd_ms, dq_ms, dkdv_ms = avg(0, 1), avg(1, 2), avg(2, 3)
    spans = {"fwd_bf16_kernel": (0, 1), "bwd_dq_kernel": (1, 2), "bwd_dkdv_kernel": (2, 3)}
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    value = (fwd_f + bwd_f) / (ms_per_step * 1e-3) / 1e12

    ok = all(bool(torch.isfinite(t).all()) for t in (o, lse, dq, dk, dv))
    if not ok:
        raise SystemExit("non-finite output")

    # Algorithmic FLOPs per launch: the forward's 2 products; the backward's 5 counted products split
    # as dK/dV kernel = S, dP, dV, dK (4 of 5) and dQ kernel = dQ (1 of 5) — the dQ kernel's two
    # recomputed products (S, dP) are extra work, not counted, and so is its D = dO·O per query.
    kernels = {
        "fwd_bf16_kernel": {"ms": fwd_ms, "flops": fwd_f, "src": "fa_fwd.hip"},
        "bwd_dkdv_kernel": {"ms": dkdv_ms, "flops": bwd_f * 4 / 5, "src": "fa_bwd.hip"},
        "bwd_dq_kernel": {"ms": dq_ms, "flops": bwd_f * 1 / 5, "src": "fa_bwd.hip"},
    }
    for name, kk in kernels.items():
        dd = durations(*spans[name])
        kk["median_ms"] = dd[len(dd) // 2] if len(dd) % 2 else (dd[len(dd) // 2 - 1] + dd[len(dd) // 2]) / 2
        kk["min_ms"] = dd[0]
        if "flops" in kk:
            kk["tflops"] = kk["flops"] / (kk["ms"] * 1e-3) / 1e12
    dom = max(("fwd_bf16_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"),
              key=lambda n: kernels[n]["ms"])
    dom_k = kernels[dom]
    roofline = {
        "kernel": dom,
        "bound": "mfma",
        "achieved": dom_k["tflops"],
        "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": dom_k["tflops"] / BF16_PEAK_TFLOPS,
        "traffic": measured_traffic(dom, dom_k["src"]),
        "launch_ms": dom_k["ms"],
    }

    log("[bench] sampling the shader clock under the same load for ~1 s")
    device = device_block(fa, torch, lambda: (step(), torch.cuda.synchronize(dev)))

    secondary = {}
    if not args.no_fp8:
        secondary["fp8_8k_fwd"] = fp8_forward(fa, workloads, lib, args.steps, args.warmup)
        if not args.no_fp8_bwd:
            secondary["fp8bwd_8k_bwd"] = fp8_backward(fa, workloads, lib, args.steps, args.warmup)
    if not args.no_head_dims:
        for name in ("d256_4k", "d96_4k"):
            secondary[name + "_fwd_bwd"] = fwd_bwd_secondary(fa, workloads, lib, name, args.steps,
                                                             args.warmup)
        if not args.no_fp8:
            for name in ("fp8_d64_8k", "fp8_d96_8k", "fp8_d256_8k"):
                secondary[name + "_fwd"] = fp8_forward(fa, workloads, lib, args.steps, args.warmup,
                                                       name)
    if not args.no_configs:
        for name in ("d64_2k", "long_16k"):
            secondary[name + "_fwd_bwd"] = fwd_bwd_secondary(fa, workloads, lib, name, args.steps,
                                                             args.warmup)
        secondary["onehead_32k_fwd_bwd"] = split_secondary(fa, workloads, lib, "onehead_32k",
                                                           args.steps, args.warmup)
    if not args.no_decode:
        secondary.update(decode_measure(fa, workloads, lib, args.steps, args.warmup))

    cpu = None
    if args.cpu_budget > 0:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_budget:.0f} s")
        cpu = cpu_baseline(w, inp, args.cpu_budget)
        log(f"[bench] oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")
        log("[bench] timing the oracle over the two small workloads in full")
        cpu["full_runs"] = cpu_full_runs(workloads)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "softmax_scale": scale, "flops_per_step": fwd_f + bwd_f},
        "mfma_peak_frac": value / BF16_PEAK_TFLOPS,
        "phases_ms": {"fwd": fwd_ms, "bwd_delta_dq": dq_ms, "bwd_dkdv": dkdv_ms},
        "fwd_tflops": fwd_f / (fwd_ms * 1e-3) / 1e12,
        "bwd_tflops": bwd_f / ((dkdv_ms + dq_ms) * 1e-3) / 1e12,
        "kernels": {n: {k2: v2 for k2, v2 in kk.items() if k2 != "src"} for n, kk in kernels.items()},
        "roofline": roofline,
        "device": device,
        "secondary": secondary,
        "cpu_baseline": cpu,
        "context": PAGES_FIGURES,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
