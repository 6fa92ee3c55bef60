#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

Headline step: the DiT FFN pair, the largest single-GPU configuration
(seeded synthetic data, inputs resident in HBM before timing):

  X bf16 [8192, 3072] ~ N(0,1) with 0.1 % of entries x50,
  W_up [14336, 3072] and W_down [3072, 14336] ~ N(0, 0.02), quantised once
  to NVFP4 before timing (weights are materialised once in 4 bits).

  1. nvfp4_linear_q  quantise X per call -> W4A4 GEMM with the GELU-tanh
                     epilogue -> H [8192, 14336] handed on in NVFP4 (the
                     encoder folds the GEMM's per-tile output maxima, H is
                     read once)
  2. nvfp4_gemm      H (NVFP4) x W_down -> Y bf16 [8192, 3072]

`value` = 2 * (2*M*N*K) per step / step time (TFLOP/s): the step is captured
once in a HIP graph, W replays untimed, then exactly K replays between two
device synchronisations.  The same step is also run eagerly K times with an
event after every kernel (the library's launch-event testing hook), which
gives the per-kernel breakdown and the dominant kernel's roofline (the up
GEMM).  Further entries in `kernels` time the other configurations' kernels
(QKV and long-context GEMMs and quantisers, an 880-token frame step of QKV
projection + KV append with the append fused into the projection or not, the
65536-token KV append sequence and its read-back, the same cache in 8-frame chunks with adaptive
scales, with and without K-smoothing, attention of an 880-token query chunk over that
cache read in NVFP4 (plain and K-smoothed) against the same kernel on bf16 K/V, the FFN up
projection's weight gradient with Hadamard-transformed operands, a 1 GiB
device copy) with p10/p50/p90 over repetitions; the HBM-bound ones after a
1 GiB cache flush ("cold").
`cpu_baseline` is the CPU oracle on a bounded sample of the FFN step.

Other modes: --copy-only (1 GiB copy, for rocprofv3 counter calibration),
--gemm-clock (QKV GEMM on benchmark vs constant operands), --wgrad-only (the
weight-gradient configuration alone), --kv-smooth-only (the K-smoothed cache alone).
"""

from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A4 NVFP4 GEMM TFLOPS (% MFMA peak) + quantize GB/s (% HBM), 1×MI355X"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PEAK_F16_TFLOPS = 2500.0         # dense fp16/bf16 MFMA (the instruction the exact decode feeds)
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0
Q_BYTES_PER_ELEM = 2.5625        # 2 B bf16 read + 0.5 B codes + 1/16 B scale
PROFILE_PMC = os.path.join(ROOT, "profiles", "gemm_ffn_up_8192x14336x3072_pmc.txt")
# the GEMM kernel and its host dispatch (the traffic counters hold for these sources only)
GEMM_SRC = [os.path.join(ROOT, "bit_block_scaled_amd", "csrc", f) for f in ("gemm_kernel.h", "gemm.hip")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sha256_file(paths):
    """SHA-256 over the concatenated contents of one file or a list of files."""
    h = hashlib.sha256()
    for p in ([paths] if isinstance(paths, str) else paths):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline step (no other configurations)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle time")
    ap.add_argument("--copy-only", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--wgrad-only", action="store_true",
                    help="run only the FFN weight-gradient configuration (Hadamard-transformed operands and "
                         "their GEMM) and print its timings (for rocprofv3)")
    ap.add_argument("--kv-smooth-only", action="store_true",
                    help="run only the K-smoothed KV legs (8-frame adaptive appends, 880-token appends, "
                         "attention over the smoothed cache) and print their timings (for rocprofv3)")
    ap.add_argument("--gemm-clock", action="store_true",
                    help="run only the QKV GEMM, 20 launches on the benchmark's operands, then 20 on "
                         "constant-byte operands (for rocprofv3 --pmc GRBM_GUI_ACTIVE)")
    return ap.parse_args()


def pct(samples):
    """p10 / p50 / p90 / mean of a list of microsecond samples."""
    import numpy as np
    a = np.asarray(samples, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2), "p50": round(float(np.percentile(a, 50)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "mean": round(float(a.mean()), 2), "n": int(a.size)}


def roof_gemm(flops, us):
    t = flops / us / 1e6
    return {"bound": "mfma", "achieved": round(t, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(t / PEAK_F16_TFLOPS, 4), "frac_fp8_peak": round(t / PEAK_FP8_TFLOPS, 4),
            "frac_fp4_peak": round(t / PEAK_FP4_TFLOPS, 4)}


def roof_hbm(nbytes, us, copy_gbs=None):
    g = nbytes / us / 1e3
    r = {"bound": "hbm", "achieved": round(g, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": round(g / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes}
    if copy_gbs:
        r["frac_of_copy"] = round(g / copy_gbs, 4)
    return r


class CacheFlush:
    """Evicts L2 and the MALL by reading a 1 GiB buffer (written once here).

    A read leaves only clean lines behind; a written buffer would leave 1 GiB
    of dirty lines whose write-back competes with the timed kernel's reads."""

    def __init__(self, torch, dev):
        self.buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(7).view(torch.int64)
        torch.cuda.synchronize()

    def __call__(self):
        self.buf.max()


def time_us(torch, fn, reps, warmup=10, flush=None):
    """Microseconds of fn() per repetition, from HIP events on the current
    stream around each call (after a cache flush when `flush` is given)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3)
    return out


def cpu_baseline(w, qu, qd, seconds):
    """The oracle as it stands, on a sample of the FFN step's rows."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:      # threadpoolctl missing: numpy's BLAS default
        threads = os.cpu_count() or 1
    S = 32
    M, D = w.x.shape
    HID = w.w.shape[0]
    reps, t_total = 0, 0.0
    while reps == 0 or t_total < seconds:
        t0 = time.perf_counter()
        A = np.abs(oracle.bf16_bits_to_f32(w.x)).max()                   # tensor amax over all of X
        qa = oracle.quantize(w.x[:S], amax=A)
        _, h = oracle.gemm_ref(*qa, *qu, gelu=True)                      # up GEMM + GELU, bf16 H rows
        qh = oracle.quantize(h)                                          # H's amax over the sampled rows
        oracle.gemm_ref(*qh, *qd)                                        # down GEMM
        t_total += time.perf_counter() - t0
        reps += 1
        if reps >= 20:
            break
    tflops = 4.0 * S * HID * D * reps / t_total / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{S} of {M} rows of the FFN step, {reps} reps in {t_total:.1f} s: tensor amax over "
                       f"all of X, NVFP4 quantise of the sampled rows, FP64 up GEMM against the full "
                       f"pre-quantised W_up with GELU and bf16 rounding, NVFP4 quantise of those H rows "
                       f"(their own amax), FP64 down GEMM against the full pre-quantised W_down; host has "
                       f"{os.cpu_count()} logical CPUs, BLAS threads {threads}")}


def pmc_traffic():
    """HBM bytes per up-GEMM launch from the committed rocprofv3 counter summary
    (its `key: value` lines), or None when absent or taken on another GEMM
    source."""
    if not os.path.exists(PROFILE_PMC):
        return None
    d = {}
    for line in open(PROFILE_PMC):
        k, sep, v = line.partition(":")
        if sep and k.strip() and " " not in k.strip():
            d[k.strip()] = v.strip()
    if d.get("gemm_source_sha256") != sha256_file(GEMM_SRC):
        return None
    try:
        return int(d["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (the path runs on one "
              f"GPU; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import bit_block_scaled_amd as nv
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = nv.lib()

    if a.copy_only:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "dispatches": 3}))
        return

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if a.gemm_clock:
        gemm_clock(a, nv, torch, np, workloads, dev, up)
        return
    if a.wgrad_only:
        kernels = {}
        wgrad_leg(kernels, nv, torch, np, workloads, dev, up, CacheFlush(torch, dev))
        print(json.dumps({"kernels": kernels}))
        return
    if a.kv_smooth_only:
        kernels = {}
        kv_smooth_leg(kernels, nv, torch, np, workloads, dev, up, CacheFlush(torch, dev))
        print(json.dumps({"kernels": kernels}))
        return

    # ------------------------------------------------------------------ FFN step
    log("generating the FFN workload (seed 2)")
    w = workloads.ffn()
    M, D = w.x.shape
    HID = w.w.shape[0]
    x = up(w.x)
    Wu, Wd = up(w.w), up(w.w2)
    qu, qd = nv.quantize(Wu), nv.quantize(Wd)              # offline weight quantisation
    del Wu, Wd
    hq = torch.empty((M, HID // 2), dtype=torch.uint8, device=dev)
    hs = torch.empty((M, HID // 16), dtype=torch.uint8, device=dev)
    hg = torch.empty((1,), dtype=torch.float32, device=dev)
    Y = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    lq_ws = nv.workspace(nv.linear_q_workspace_bytes(M, HID, D), dev)
    torch.cuda.synchronize()

    def step():
        nv.linear_q(x, *qu, gelu=True, out=(hq, hs, hg), ws=lq_ws)
        nv.gemm(hq, hs, hg, *qd, out=Y)

    log(f"warmup {a.warmup} steps")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # eager steps: an event before the step and one after each of its four
    # kernels (quantise X, up GEMM, encode H, down GEMM)
    log(f"timing {a.steps} eager steps (per-kernel events)")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(a.steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    handles = [(C.c_void_p * 4)(*[C.c_void_p(e.cuda_event) for e in row[1:]]) for row in evs]
    t0 = time.perf_counter()
    for s in range(a.steps):
        evs[s][0].record()
        nv.check(L.nvfp4_testing_set_launch_events(handles[s], 4))
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    nv.check(L.nvfp4_testing_set_launch_events(None, 0))
    ms_eager = (t1 - t0) * 1e3 / a.steps
    names = ["quantize_x", "gemm_up", "encode_h", "gemm_down"]
    parts = {n: [evs[s][j].elapsed_time(evs[s][j + 1]) * 1e3 for s in range(a.steps)]
             for j, n in enumerate(names)}
    us = {n: float(np.mean(v)) for n, v in parts.items()}

    # the headline: the same step captured once in a HIP graph and replayed
    launch = "hip_graph"
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(a.warmup):
            graph.replay()
        torch.cuda.synchronize()
        log(f"timing {a.steps} graph-replayed steps")
        t0 = time.perf_counter()
        for _ in range(a.steps):
            graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1e3 / a.steps
    except Exception as exc:                     # capture unsupported: report the eager step
        log(f"graph capture failed ({exc}); reporting eager launches")
        launch, ms_per_step = "eager", ms_eager
    flops_gemm = 2.0 * M * HID * D
    flops = 2 * flops_gemm
    value = flops / (ms_per_step * 1e-3) / 1e12

    up_roof = roof_gemm(flops_gemm, us["gemm_up"])
    up_roof.update({"kernel": "up GEMM + GELU-tanh epilogue + per-tile output maxima (k_gemm, 256x256 tiles)",
                    "traffic": pmc_traffic(),
                    "algorithmic_per_launch": f"2*M*N*K = {flops_gemm:.4e} flop (M=8192, N=14336, K=3072)",
                    "avg_launch_us": round(us["gemm_up"], 2)})
    h_bytes = M * HID * Q_BYTES_PER_ELEM                  # encode H: 2 B read + 0.5625 B written
    x_bytes = M * D * Q_BYTES_PER_ELEM
    kernels = {
        "ffn_gemm_up": {"shape": [M, HID, D], "gelu": True, "us": pct(parts["gemm_up"]),
                        "roofline": roof_gemm(flops_gemm, us["gemm_up"])},
        "ffn_gemm_down": {"shape": [M, D, HID], "us": pct(parts["gemm_down"]),
                          "roofline": roof_gemm(flops_gemm, us["gemm_down"])},
        "ffn_quantize_x": {"shape": [M, D], "us": pct(parts["quantize_x"]),
                           "roofline": roof_hbm(x_bytes, us["quantize_x"])},
        "ffn_encode_h": {"shape": [M, HID], "us": pct(parts["encode_h"]),
                         "roofline": roof_hbm(h_bytes, us["encode_h"])},
    }
    del graph
    torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "launch": launch,
        "ms_per_step_eager": round(ms_eager, 5),
        "value_eager": round(flops / (ms_eager * 1e-3) / 1e12, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands (E2M1 + E4M3/16 + fp32), fp16 MFMA on exactly decoded products, fp32 accumulate",
        "data": "synthetic (seeded numpy draws, bf16)",
        "config": {"workload": "DiT FFN pair: X[8192,3072] (0.1% x50 outliers) -> NVFP4 W4A4 up-projection "
                               "to 14336 with GELU-tanh, H handed on in NVFP4 -> W4A4 down-projection to 3072",
                   "M": M, "D": D, "hidden": HID,
                   "gemm_tiles": {"up": list(nv.gemm_tile(M, HID, D)), "down": list(nv.gemm_tile(M, D, HID))}},
        "roofline": up_roof,
        "breakdown_us": {k: round(v, 2) for k, v in us.items()},
        "kernels": kernels,
        "inputs_sha256": {"x": workloads.sha256(w.x)[:16], "w_up": workloads.sha256(w.w)[:16],
                          "w_down": workloads.sha256(w.w2)[:16]},
    }

    if not a.no_extras:
        flush = CacheFlush(torch, dev)
        copy_gbs = extras(kernels, nv, torch, np, workloads, dev, up, flush, x, lq_ws, qu)
        out["copy_gbs"] = copy_gbs
        for k in kernels.values():
            r = k.get("roofline", {})
            if r.get("bound") == "hbm" and "frac_of_copy" not in r:
                r["frac_of_copy"] = round(r["achieved"] / copy_gbs, 4)
        del flush
    del x, hq, hs, hg, Y, lq_ws
    torch.cuda.empty_cache()

    if not a.no_cpu_baseline:
        import oracle
        log("CPU oracle baseline")
        qu_o, qd_o = oracle.quantize(w.w), oracle.quantize(w.w2)      # offline, outside the timed sample
        out["cpu_baseline"] = cpu_baseline(w, qu_o, qd_o, a.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def extras(kernels, nv, torch, np, workloads, dev, up, flush, x_ffn, lq_ws, qu):
    """Per-kernel timings of the other configurations (added to `kernels`);
    returns the measured 1 GiB device-copy rate in GB/s (read + write bytes)."""
    # 1 GiB device copy: the practical HBM rate
    log("extras: 1 GiB copy")
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    tc = time_us(torch, lambda: dst.copy_(src), 30, 5)
    copy_gbs = 2 * (1 << 30) / np.percentile(tc, 50) / 1e3
    kernels["copy_1gib"] = {"us": pct(tc), "gbs": round(copy_gbs, 1), "frac_hbm_peak": round(copy_gbs / PEAK_HBM_GBS, 4)}
    del src, dst

    # FFN: the hidden activation H quantised by itself (cold), and the X quantiser cold
    log("extras: FFN quantisers (cold)")
    M, D = x_ffn.shape
    H = nv.linear(x_ffn, *qu, gelu=True)
    HID = H.shape[1]
    hws = nv.workspace(nv.quantize_workspace_bytes(M, HID), dev)
    hq = torch.empty((M, HID // 2), dtype=torch.uint8, device=dev)
    hs = torch.empty((M, HID // 16), dtype=torch.uint8, device=dev)
    hg = torch.empty((1,), dtype=torch.float32, device=dev)
    t = time_us(torch, lambda: nv.quantize_into(H, hq, hs, hg, hws), 100, 5, flush)
    kernels["ffn_quantize_h_cold"] = {"shape": [M, HID], "us": pct(t),
                                      "roofline": roof_hbm(M * HID * Q_BYTES_PER_ELEM + 4, float(np.median(t)))}
    xq = torch.empty((M, D // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, D // 16), dtype=torch.uint8, device=dev)
    xws = nv.workspace(nv.quantize_workspace_bytes(M, D), dev)
    t = time_us(torch, lambda: nv.quantize_into(x_ffn, xq, xs, hg, xws), 100, 5, flush)
    kernels["ffn_quantize_x_cold"] = {"shape": [M, D], "us": pct(t),
                                      "roofline": roof_hbm(M * D * Q_BYTES_PER_ELEM + 4, float(np.median(t)))}
    del H, hq, hs, hws, xq, xs, xws
    torch.cuda.empty_cache()

    # QKV projection and the long-context out-projection: GEMM (warm, back to
    # back) and the activation quantiser (cold); QKV's K/V column slices into
    # a KV cache and back (cold)
    for name, fn in (("qkv", workloads.qkv), ("long", workloads.long_ctx)):
        log(f"extras: {name}")
        wl = fn()
        Mx, K = wl.x.shape
        N = wl.w.shape[0]
        xd = up(wl.x)
        wq = nv.quantize(up(wl.w))
        bias = up(wl.bias) if wl.bias is not None else None
        aq, asc, ag = nv.quantize(xd)
        Cm = torch.empty((Mx, N), dtype=torch.bfloat16, device=dev)
        t = time_us(torch, lambda: nv.gemm(aq, asc, ag, *wq, bias=bias, out=Cm), 30, 10)
        kernels[f"{name}_gemm"] = {"shape": [Mx, N, K], "bias": bias is not None, "tile": list(nv.gemm_tile(Mx, N, K)),
                                   "us": pct(t), "roofline": roof_gemm(2.0 * Mx * N * K, float(np.median(t)))}
        qws = nv.workspace(nv.quantize_workspace_bytes(Mx, K), dev)
        t = time_us(torch, lambda: nv.quantize_into(xd, aq, asc, ag, qws), 100, 5, flush)
        kernels[f"{name}_quantize_x_cold"] = {"shape": [Mx, K], "us": pct(t),
                                              "roofline": roof_hbm(Mx * K * Q_BYTES_PER_ELEM + 4, float(np.median(t)))}
        if name == "qkv":
            kv = nv.KVCache(Mx, 24, 128, max_chunks=1, device=dev)
            Kv, Vv = Cm[:, 3072:6144], Cm[:, 6144:9216]
            ko = torch.empty((Mx, 24, 128), dtype=torch.bfloat16, device=dev)
            vo = torch.empty_like(ko)

            def app():
                kv.reset()
                kv.append(Kv, Vv)
            t = time_us(torch, app, 100, 5, flush)
            kvb = 2 * Mx * 3072 * Q_BYTES_PER_ELEM + 8
            kernels["qkv_kv_append_cold"] = {"tokens": Mx, "us": pct(t), "roofline": roof_hbm(kvb, float(np.median(t)))}
            t = time_us(torch, lambda: kv.dequant(0, Mx, ko, vo), 100, 5, flush)
            kernels["qkv_kv_dequant_cold"] = {"tokens": Mx, "us": pct(t),
                                              "roofline": roof_hbm(2 * Mx * 3072 * Q_BYTES_PER_ELEM, float(np.median(t)))}
            del kv, ko, vo
        del xd, wq, aq, asc, Cm, qws, wl
        torch.cuda.empty_cache()

    # one frame step of the DiT at 880 tokens, 75 frames back to back: the QKV
    # projection alone, then with its K/V appended to the NVFP4 cache by a
    # separate append, then by nvfp4_qkv_append (the append encoded from the
    # GEMM's tile maxima)
    log("extras: 880-token frame step (QKV projection + KV append)")
    qf = workloads.qkv(M=880)
    xf, wqf, bf = up(qf.x), nv.quantize(up(qf.w)), up(qf.bias)
    frames = 75
    cf = nv.KVCache(880 * frames, 24, 128, max_chunks=frames, device=dev)
    cp = nv.KVCache(880 * frames, 24, 128, max_chunks=frames, device=dev)
    of = torch.empty((880, 9216), dtype=torch.bfloat16, device=dev)
    lwsf = nv.workspace(nv.linear_workspace_bytes(880, 3072), dev)

    def seq_linear():
        for _ in range(frames):
            nv.linear(xf, *wqf, bias=bf, out=of, ws=lwsf)

    def seq_unfused():
        cp.reset()
        for _ in range(frames):
            nv.linear(xf, *wqf, bias=bf, out=of, ws=lwsf)
            cp.append(of[:, 3072:6144], of[:, 6144:])

    def seq_fused():
        cf.reset()
        for _ in range(frames):
            cf.qkv_append(xf, *wqf, bias=bf, out=of)
    per = {}
    for name, fn in (("linear_only", seq_linear), ("linear_then_append", seq_unfused), ("qkv_append", seq_fused)):
        t = [v / frames for v in time_us(torch, fn, 5, 1)]
        per[name] = float(np.median(t))
        kernels[f"qkv880_frame_{name}"] = {"frames": frames, "us_per_frame": pct(t)}
    kernels["qkv880_frame_append_cost"] = {
        "unfused_us": round(per["linear_then_append"] - per["linear_only"], 2),
        "fused_us": round(per["qkv_append"] - per["linear_only"], 2)}
    del qf, xf, wqf, bf, cf, cp, of, lwsf
    torch.cuda.empty_cache()

    # the 65536-token KV cache: 74 appends of 880 tokens + one of 416, then a
    # read-back of the whole cache
    log("extras: 65536-token KV sequence")
    Kb, Vb, sizes = workloads.kv()
    kd, vd = up(Kb), up(Vb)
    T = Kb.shape[0]
    del Kb, Vb
    cache = nv.KVCache(T, 24, 128, max_chunks=len(sizes), device=dev)
    starts = np.r_[0, np.cumsum(sizes)]

    def seq():
        cache.reset()
        for i in range(len(sizes)):
            cache.append(kd[starts[i]:starts[i + 1]], vd[starts[i]:starts[i + 1]])
    t = time_us(torch, seq, 10, 2, flush)
    kvb = 2 * T * 3072 * Q_BYTES_PER_ELEM + 8 * len(sizes)
    kernels["kv65536_append_sequence_cold"] = {"appends": len(sizes), "tokens": T, "us": pct(t),
                                               "roofline": roof_hbm(kvb, float(np.median(t)))}
    # the same cache filled in the pages' KV chunks of 8 frames (9 appends of
    # 7040 tokens and one of 2176)
    sizes8 = workloads.kv_chunk_sizes(T, 8 * workloads.KV_CHUNK)
    starts8 = np.r_[0, np.cumsum(sizes8)]
    cache8 = nv.KVCache(T, 24, 128, max_chunks=len(sizes8), device=dev)

    def seq8():
        cache8.reset()
        for i in range(len(sizes8)):
            cache8.append(kd[starts8[i]:starts8[i + 1]], vd[starts8[i]:starts8[i + 1]])
    t = time_us(torch, seq8, 10, 2, flush)
    kernels["kv65536_append_8frame_chunks_cold"] = {"appends": len(sizes8), "tokens": T, "us": pct(t),
                                                    "roofline": roof_hbm(2 * T * 3072 * Q_BYTES_PER_ELEM + 8 * len(sizes8),
                                                                         float(np.median(t)))}
    # the pages' KV configuration: 8-frame chunks with adaptive {4, 6} scales,
    # without and with K-smoothing (the smoothed append adds three passes:
    # channel sums, centres, smoothed keys; the roofline counts only the
    # append's own bytes, so it shows what smoothing costs)
    cache8s = nv.KVCache(T, 24, 128, max_chunks=len(sizes8), device=dev, smooth_k=True)
    for name, c8 in (("adaptive", cache8), ("smoothed_adaptive", cache8s)):
        def seq8a(c8=c8):
            c8.reset()
            for i in range(len(sizes8)):
                c8.append(kd[starts8[i]:starts8[i + 1]], vd[starts8[i]:starts8[i + 1]], adaptive46=True)
        t = time_us(torch, seq8a, 10, 2, flush)
        kernels[f"kv65536_append_8frame_chunks_{name}_cold"] = {
            "appends": len(sizes8), "tokens": T, "us": pct(t),
            "roofline": roof_hbm(2 * T * 3072 * Q_BYTES_PER_ELEM + 8 * len(sizes8), float(np.median(t)))}
    del cache8, cache8s
    # 880-token appends with K-smoothing (the frame-by-frame cache), kept for
    # the attention comparison below
    cache_s = nv.KVCache(T, 24, 128, max_chunks=len(sizes), device=dev, smooth_k=True)

    def seq_s():
        cache_s.reset()
        for i in range(len(sizes)):
            cache_s.append(kd[starts[i]:starts[i + 1]], vd[starts[i]:starts[i + 1]])
    t = time_us(torch, seq_s, 10, 2, flush)
    kernels["kv65536_append_sequence_smoothed_cold"] = {"appends": len(sizes), "tokens": T, "us": pct(t),
                                                        "roofline": roof_hbm(kvb, float(np.median(t)))}
    # each 880-token append inside the back-to-back sequence: an event after
    # every append, per-append time = the gap between consecutive events
    per = []
    for _ in range(4):
        flush()
        cache.reset()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sizes) + 1)]
        ev[0].record()
        for i in range(len(sizes)):
            cache.append(kd[starts[i]:starts[i + 1]], vd[starts[i]:starts[i + 1]])
            ev[i + 1].record()
        torch.cuda.synchronize()
        per += [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(1, len(sizes) - 1)]
    b880 = 2 * 880 * 3072 * Q_BYTES_PER_ELEM + 8
    kernels["kv880_append"] = {"tokens": 880, "us": pct(per), "roofline": roof_hbm(b880, float(np.median(per)))}
    ko = torch.empty((T, 24, 128), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    t = time_us(torch, lambda: cache.dequant(0, T, ko, vo), 100, 5, flush)
    kernels["kv65536_dequant_cold"] = {"tokens": T, "us": pct(t),
                                       "roofline": roof_hbm(2 * T * 3072 * Q_BYTES_PER_ELEM, float(np.median(t)))}
    # attention of one 880-token query chunk over the cache (24 heads of 128):
    # the NVFP4 cache read inside the kernel, against the bf16 twin on the
    # cache's bf16 read-back, and against the read-back followed by the twin
    log("extras: attention over the NVFP4 cache vs bf16 K/V")
    del kd, vd
    torch.cuda.empty_cache()
    cache.dequant(0, T, ko, vo)
    rng = np.random.default_rng(5)
    qa = up(workloads.to_bf16_bits(rng.standard_normal((880, 24, 128)).astype(np.float32)))
    oa = torch.empty_like(qa)
    for name, ranges in (("full", [(0, T)]), ("sink_window", [(0, 880), (T - 8800, T)])):
        Tk = sum(b - a for a, b in ranges)
        ws_a = nv._attention_ws(880, 24, Tk, dev)
        flops_a = 4.0 * 880 * Tk * 24 * 128
        tn = time_us(torch, lambda: cache.attention(qa, ranges, out=oa, ws=ws_a), 10, 3)
        ts = time_us(torch, lambda: cache_s.attention(qa, ranges, out=oa, ws=ws_a), 10, 3)
        if name == "full":
            kb, vb = ko, vo
        else:
            kb = torch.cat([ko[a:b] for a, b in ranges]).contiguous()
            vb = torch.cat([vo[a:b] for a, b in ranges]).contiguous()
        tb = time_us(torch, lambda: nv.attention_bf16(qa, kb, vb, out=oa, ws=ws_a), 10, 3)

        offs = np.r_[0, np.cumsum([b - a for a, b in ranges])]

        def unfused():                   # read the key ranges back to bf16, then the twin
            for i, (a, b) in enumerate(ranges):
                cache.dequant(a, b, kb[offs[i]:offs[i + 1]], vb[offs[i]:offs[i + 1]])
            nv.attention_bf16(qa, kb, vb, out=oa, ws=ws_a)
        tu = time_us(torch, unfused, 10, 3)

        def one(fn):                     # one timed call, events on the work stream
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            return e0.elapsed_time(e1) * 1e3
        # the same two kernels timed in alternating pairs, so both see the
        # same clock and cache state; the ratio of each pair
        pairs = [one(lambda: cache.attention(qa, ranges, out=oa, ws=ws_a)) /
                 one(lambda: nv.attention_bf16(qa, kb, vb, out=oa, ws=ws_a)) for _ in range(20)]
        pn, pb, pu = float(np.median(tn)), float(np.median(tb)), float(np.median(tu))
        kernels[f"attention_{name}_nvfp4"] = {"queries": 880, "keys": Tk, "heads": 24, "us": pct(tn),
                                             "roofline": roof_gemm(flops_a, pn)}
        kernels[f"attention_{name}_nvfp4_smoothed"] = {"queries": 880, "keys": Tk, "heads": 24, "us": pct(ts),
                                                      "time_ratio_vs_nvfp4": round(float(np.median(ts)) / pn, 4),
                                                      "roofline": roof_gemm(flops_a, float(np.median(ts)))}
        kernels[f"attention_{name}_bf16_twin"] = {"queries": 880, "keys": Tk, "heads": 24, "us": pct(tb),
                                                 "roofline": roof_gemm(flops_a, pb)}
        kernels[f"attention_{name}_dequant_then_bf16"] = {"us": pct(tu)}
        kernels[f"attention_{name}_nvfp4_vs_bf16"] = {"time_ratio": round(pn / pb, 4),
                                                       "time_ratio_interleaved": {
                                                           "p10": round(float(np.percentile(pairs, 10)), 4),
                                                           "p50": round(float(np.median(pairs)), 4),
                                                           "p90": round(float(np.percentile(pairs, 90)), 4),
                                                           "n": len(pairs)},
                                                       "dequant_then_bf16_ratio": round(pu / pb, 4)}
        del ws_a
    del cache, cache_s, ko, vo, qa, oa
    torch.cuda.empty_cache()

    wgrad_leg(kernels, nv, torch, np, workloads, dev, up, flush)
    return round(float(copy_gbs), 1)


def kv_smooth_leg(kernels, nv, torch, np, workloads, dev, up, flush):
    """The K-smoothed cache alone (a short program for rocprofv3): the
    65536-token workload in 8-frame chunks with adaptive scales and in
    880-token appends, then attention of 880 queries over the latter."""
    Kb, Vb, sizes = workloads.kv()
    kd, vd = up(Kb), up(Vb)
    T = Kb.shape[0]
    del Kb, Vb
    sizes8 = workloads.kv_chunk_sizes(T, 8 * workloads.KV_CHUNK)
    for name, sz, adapt in (("8frame_chunks_smoothed_adaptive", sizes8, True), ("sequence_smoothed", sizes, False)):
        st = np.r_[0, np.cumsum(sz)]
        cache = nv.KVCache(T, 24, 128, max_chunks=len(sz), device=dev, smooth_k=True)

        def seq(cache=cache, st=st, sz=sz, adapt=adapt):
            cache.reset()
            for i in range(len(sz)):
                cache.append(kd[st[i]:st[i + 1]], vd[st[i]:st[i + 1]], adaptive46=adapt)
        t = time_us(torch, seq, 3, 1, flush)
        kernels[f"kv65536_append_{name}_cold"] = {"appends": len(sz), "tokens": T, "us": pct(t)}
    rng = np.random.default_rng(5)
    qa = up(workloads.to_bf16_bits(rng.standard_normal((880, 24, 128)).astype(np.float32)))
    oa = torch.empty_like(qa)
    ws_a = nv._attention_ws(880, 24, T, dev)
    t = time_us(torch, lambda: cache.attention(qa, [(0, T)], out=oa, ws=ws_a), 3, 1)
    kernels["attention_full_nvfp4_smoothed"] = {"queries": 880, "keys": T, "heads": 24, "us": pct(t)}


def wgrad_leg(kernels, nv, torch, np, workloads, dev, up, flush):
    """The weight-gradient configuration (added to `kernels`)."""
    # weight gradient of the FFN up-projection over 8192 tokens: dY and X each
    # through the random Hadamard transform and the NVFP4 quantisation of
    # their transposes (cold; two launches that read the operand twice, since
    # the tensor amax of the transform precedes every block scale), then the
    # W4A4 GEMM dW = dYᵀ·X
    log("extras: FFN weight gradient with the Hadamard transform")
    wg = workloads.wgrad()
    T = wg.x.shape[0]
    ops = {"dy": up(wg.dy), "x": up(wg.x)}
    mask = wg.sign_mask
    del wg
    qops = {}
    for k, xt in ops.items():
        N = xt.shape[1]
        c = torch.empty((N, T // 2), dtype=torch.uint8, device=dev)
        s_ = torch.empty((N, T // 16), dtype=torch.uint8, device=dev)
        g = torch.empty((1,), dtype=torch.float32, device=dev)
        ws_r = torch.empty((nv.quantize_rht_workspace_bytes(T, N),), dtype=torch.uint8, device=dev)
        t = time_us(torch, lambda xt=xt, c=c, s_=s_, g=g, ws_r=ws_r: nv.quantize_rht(xt, mask, c, s_, g, ws_r),
                    30, 5, flush)
        kernels[f"wgrad_quantize_rht_{k}_cold"] = {
            "shape": [T, N], "us": pct(t), "hbm_bytes_moved": T * N * (2 * 2 + 0.5 + 1 / 16),
            "roofline": roof_hbm(T * N * Q_BYTES_PER_ELEM + 4, float(np.median(t)))}
        qops[k] = (c, s_, g)
    O, I = ops["dy"].shape[1], ops["x"].shape[1]
    dW = torch.empty((O, I), dtype=torch.bfloat16, device=dev)
    t = time_us(torch, lambda: nv.gemm(*qops["dy"], *qops["x"], out=dW), 30, 10)
    kernels["wgrad_gemm"] = {"shape": [O, I, T], "tile": list(nv.gemm_tile(O, I, T)), "us": pct(t),
                             "roofline": roof_gemm(2.0 * O * I * T, float(np.median(t)))}
    del ops, qops, dW
    torch.cuda.empty_cache()


def gemm_clock(a, nv, torch, np, workloads, dev, up):
    """The QKV GEMM launched 20 times on the benchmark's operands, then 20 times
    after filling the codes and scales with constant bytes."""
    w = workloads.qkv()
    M, K, N = w.M, w.K, w.N
    x, bias = up(w.x), up(w.bias)
    wq, wsc, wg = nv.quantize(up(w.w))
    aq, asc, ag = nv.quantize(x)
    Cm = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    res = {}
    for kind in ("benchmark", "constant"):
        if kind == "constant":              # fixed byte patterns, every element alike
            aq.fill_(0x35); wq.fill_(0x53); asc.fill_(0x38); wsc.fill_(0x30)
        t = time_us(torch, lambda: nv.gemm(aq, asc, ag, wq, wsc, wg, bias=bias, out=Cm), 20, 3)
        res[kind + "_us"] = float(np.mean(t))
    print(json.dumps({"gemm_clock": res, "launches_per_kind": 20, "warmup_per_kind": 3}))


if __name__ == "__main__":
    main()
