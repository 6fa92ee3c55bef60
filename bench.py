#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

One step is one pass of the whole path over one batch of the DiT QKV
projection workload (X bf16 [4096, 3072] ~ N(0,1) with 0.1 % ×50 outliers,
W [9216, 3072] ~ N(0, 0.02), bias [9216] ~ N(0, 0.01); seeded synthetic data):

  1. nvfp4_quantize   X → NVFP4 codes / E4M3 block scales / FP32 tensor scale
  2. nvfp4_gemm       W4A4 GEMM against the pre-quantised W, + bias → C bf16
                      [4096, 9216]  (= the linear layer, quantise + GEMM)
  3. nvfp4_kv_append  the K and V column slices of C (24 heads x 128) appended
                      to an NVFP4 KV cache (read in place, token stride 9216)
  4. nvfp4_kv_dequant those 4096 tokens read back as bf16 K and V

The weights are quantised once before timing (they are materialised once in
4 bits).  Inputs are resident in HBM before the timed region; the K timed
steps run back to back on one stream, bracketed by device synchronisation.

Printed: one JSON line.  `value` is 2·M·N·K per step over the step time
(TFLOP/s of the linear layer, with the quantiser and the KV append/dequant
inside the step time).  `roofline` is for the dominant kernel (the GEMM),
timed with HIP events on the stream it runs on.  `cpu_baseline` is the CPU
oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
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
PEAK_F16_TFLOPS = 2500.0         # dense fp16/bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0
PROFILE_PMC = os.path.join(ROOT, "profiles", "gemm_qkv_4096x9216x3072_pmc_traffic.txt")
# the GEMM kernel and its host dispatch (the traffic counters are valid for these sources only)
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
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle time")
    ap.add_argument("--extended", metavar="PATH", default=None,
                    help="also measure the other DiT shapes and the 65536-token KV sequence; "
                         "write JSON lines to PATH")
    ap.add_argument("--copy-only", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--gemm-clock", action="store_true",
                    help="run only the QKV GEMM, 20 launches on the benchmark's operands, then 20 on "
                         "constant-byte operands (for rocprofv3 --pmc GRBM_GUI_ACTIVE: the clock "
                         "under load depends on the operand bits)")
    return ap.parse_args()


class Timer:
    """HIP events recorded on the current (work) stream."""

    def __init__(self, torch, n):
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.i = 0

    def mark(self):
        self.ev[self.i].record()
        self.i += 1


def cpu_baseline(w, qw_oracle, seconds):
    """The oracle as it stands, on a sample of the step's rows."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:      # threadpoolctl missing: numpy's BLAS default
        threads = os.cpu_count() or 1
    S = 256
    H, D = 24, 128
    N, K = w.N, w.K
    reps, t_total = 0, 0.0
    while reps == 0 or t_total < seconds:
        t0 = time.perf_counter()
        A = np.abs(oracle.bf16_bits_to_f32(w.x)).max()                   # tensor amax over all of X
        qa = oracle.quantize(w.x[:S], amax=A)
        _, cref = oracle.gemm_ref(*qa, *qw_oracle, bias_bits=w.bias)
        kv = oracle.KVCacheRef(S, H, D)
        kv.append(np.ascontiguousarray(cref[:, 3072:6144]).reshape(S, H, D),
                  np.ascontiguousarray(cref[:, 6144:9216]).reshape(S, H, D))
        kv.dequant(0, S)
        t_total += time.perf_counter() - t0
        reps += 1
        if reps >= 50:
            break
    tflops = 2.0 * S * N * K * reps / t_total / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{S} of {w.M} rows of the QKV step, {reps} reps in {t_total:.1f} s: tensor amax "
                       f"over all of X, NVFP4 quantise of the sampled rows, FP64 GEMM against the full "
                       f"pre-quantised W + bias with bf16 rounding, KV append + dequant of their K/V; "
                       f"host has {os.cpu_count()} logical CPUs, BLAS threads {threads}")}


def pmc_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary
    (its `key: value` lines), or None when absent or taken on a different GEMM
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
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (this build has "
              f"no multi-GPU path; run with --gpus 1)", file=sys.stderr)
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

    log("generating the QKV workload (seed 1)")
    w = workloads.qkv()
    M, K, N = w.M, w.K, w.N
    HD = 3072
    x, W, bias = up(w.x), up(w.w), up(w.bias)
    wq, wsc, wg = nv.quantize(W)                           # offline weight quantisation
    aq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    asc = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    ag = torch.empty((1,), dtype=torch.float32, device=dev)
    qws = nv.workspace(nv.quantize_workspace_bytes(M, K), dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    kv = nv.KVCache(M, 24, 128, max_chunks=1, device=dev)
    k_out = torch.empty((M, 24, 128), dtype=torch.bfloat16, device=dev)
    v_out = torch.empty_like(k_out)
    Kv, Vv = C[:, HD:2 * HD], C[:, 2 * HD:3 * HD]
    torch.cuda.synchronize()

    if a.gemm_clock:
        nv.quantize_into(x, aq, asc, ag, qws)
        res = {}
        for kind in ("benchmark", "constant"):
            if kind == "constant":              # fixed byte patterns, every element alike
                aq.fill_(0x35); wq.fill_(0x53); asc.fill_(0x38); wsc.fill_(0x30)
            for _ in range(3):
                nv.gemm(aq, asc, ag, wq, wsc, wg, bias=bias, out=C)
            ts = Timer(torch, 21)
            for _ in range(20):
                ts.mark()
                nv.gemm(aq, asc, ag, wq, wsc, wg, bias=bias, out=C)
            ts.mark()
            torch.cuda.synchronize()
            res[kind + "_us"] = float(np.mean([ts.ev[i].elapsed_time(ts.ev[i + 1]) * 1e3 for i in range(20)]))
        print(json.dumps({"gemm_clock": res, "launches_per_kind": 20, "warmup_per_kind": 3}))
        return

    def step(t=None):
        if t: t.mark()
        nv.quantize_into(x, aq, asc, ag, qws)
        if t: t.mark()
        nv.gemm(aq, asc, ag, wq, wsc, wg, bias=bias, out=C)
        if t: t.mark()
        kv.reset()
        kv.append(Kv, Vv)
        if t: t.mark()
        kv.dequant(0, M, k_out, v_out)
        if t: t.mark()

    log(f"warmup {a.warmup} steps")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # --- eager launches, K steps with events between the calls of every step
    #     (per-call breakdown and the GEMM's roofline)
    timer = Timer(torch, 5 * a.steps)
    log(f"timing {a.steps} eager steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step(timer)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_eager = (t1 - t0) * 1e3 / a.steps
    parts = {"quantize": [], "gemm": [], "kv_append": [], "kv_dequant": []}
    names = list(parts)
    for s in range(a.steps):
        for j, nm in enumerate(names):
            parts[nm].append(timer.ev[5 * s + j].elapsed_time(timer.ev[5 * s + j + 1]) * 1e3)  # µs
    us = {k: float(np.mean(v)) for k, v in parts.items()}
    flops = 2.0 * M * N * K
    q_bytes = M * K * 2.5625 + 4
    kv_bytes = 2 * M * HD * 2.5625
    gemm_tflops = flops / us["gemm"] / 1e6
    q_gbs = q_bytes / us["quantize"] / 1e3

    # --- the headline: the same step captured once in a HIP graph, W replays
    #     untimed, then exactly K replays timed (every call is replay-safe: the
    #     quantiser's call counter lives in its workspace; the KV append writes
    #     the same token range each replay, which the eager step gets from its
    #     reset)
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
    value = flops / (ms_per_step * 1e-3) / 1e12

    # --- cold (MALL and L2 flushed) timings of the HBM-bound kernels
    flush = CacheFlush(torch, dev)
    cold = {"quantize": [], "kv_append": [], "kv_dequant": []}
    for _ in range(10):
        for nm in cold:
            flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if nm == "quantize":
                e0.record(); nv.quantize_into(x, aq, asc, ag, qws); e1.record()
            elif nm == "kv_append":
                kv.reset()
                e0.record(); kv.append(Kv, Vv); e1.record()
            else:
                e0.record(); kv.dequant(0, M, k_out, v_out); e1.record()
            torch.cuda.synchronize()
            cold[nm].append(e0.elapsed_time(e1) * 1e3)
    del flush
    cold_us = {k: float(np.median(v)) for k, v in cold.items()}

    # --- back-to-back repetitions (one event pair around 50 calls): per-call
    #     throughput without the event and launch gap of a single call
    def batch_us(fn, reps=50):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def kv_once():
        kv.reset()
        kv.append(Kv, Vv)
    batch = {"quantize": batch_us(lambda: nv.quantize_into(x, aq, asc, ag, qws)),
             "kv_append": batch_us(kv_once),
             "kv_dequant": batch_us(lambda: kv.dequant(0, M, k_out, v_out))}

    traffic = pmc_traffic()
    bm, bn = nv.gemm_tile(M, N, K)
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
        "dtype": "nvfp4 operands, f16 MFMA, f32 accumulate",
        "data": "synthetic (seeded numpy draws, bf16)",
        "config": {"workload": "DiT QKV projection: X[4096,3072] (0.1% x50 outliers) x W[9216,3072]^T "
                               "+ bias, NVFP4 W4A4, then K/V (24x128) NVFP4 KV append + dequant",
                   "M": M, "N": N, "K": K, "kv_heads": 24, "head_dim": 128, "gemm_tile": [bm, bn]},
        "roofline": {"bound": "mfma", "kernel": "nvfp4 gemm (k_gemm)",
                     "achieved": round(gemm_tflops, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_F16_TFLOPS, 4),
                     "traffic": traffic,
                     "algorithmic_per_launch": f"2*M*N*K = {flops:.4e} flop",
                     "avg_launch_us": round(us["gemm"], 2)},
        "breakdown_us": {k: round(v, 2) for k, v in us.items()},
        "gemm": {"tflops": round(gemm_tflops, 1), "frac_f16_peak": round(gemm_tflops / PEAK_F16_TFLOPS, 4),
                 "frac_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                 "frac_fp4_peak": round(gemm_tflops / PEAK_FP4_TFLOPS, 4)},
        # gbs_step: events around the call inside the timed steps; gbs_cold: one
        # call after a 1 GiB cache flush (both include one launch gap);
        # gbs_batch: 50 back-to-back calls, inputs warm in the MALL
        "quantize": {"gbs_step": round(q_gbs, 1), "frac_hbm_step": round(q_gbs / PEAK_HBM_GBS, 4),
                     "gbs_cold": round(q_bytes / cold_us["quantize"] / 1e3, 1),
                     "frac_hbm_cold": round(q_bytes / cold_us["quantize"] / 1e3 / PEAK_HBM_GBS, 4),
                     "gbs_batch": round(q_bytes / batch["quantize"] / 1e3, 1),
                     "frac_hbm_batch": round(q_bytes / batch["quantize"] / 1e3 / PEAK_HBM_GBS, 4),
                     "bytes_per_call": q_bytes},
        "kv_append": {"gbs_step": round(kv_bytes / us["kv_append"] / 1e3, 1),
                      "gbs_cold": round(kv_bytes / cold_us["kv_append"] / 1e3, 1),
                      "frac_hbm_cold": round(kv_bytes / cold_us["kv_append"] / 1e3 / PEAK_HBM_GBS, 4),
                      "gbs_batch": round(kv_bytes / batch["kv_append"] / 1e3, 1),
                      "frac_hbm_batch": round(kv_bytes / batch["kv_append"] / 1e3 / PEAK_HBM_GBS, 4)},
        "kv_dequant": {"gbs_step": round(kv_bytes / us["kv_dequant"] / 1e3, 1),
                       "gbs_cold": round(kv_bytes / cold_us["kv_dequant"] / 1e3, 1),
                       "frac_hbm_cold": round(kv_bytes / cold_us["kv_dequant"] / 1e3 / PEAK_HBM_GBS, 4),
                       "gbs_batch": round(kv_bytes / batch["kv_dequant"] / 1e3, 1),
                       "frac_hbm_batch": round(kv_bytes / batch["kv_dequant"] / 1e3 / PEAK_HBM_GBS, 4)},
        "inputs_sha256": {"x": workloads.sha256(w.x)[:16], "w": workloads.sha256(w.w)[:16],
                          "bias": workloads.sha256(w.bias)[:16]},
    }

    if a.extended:
        extended(a.extended, nv, torch, np, workloads, dev, up)

    if not a.no_cpu_baseline:
        import oracle
        log("CPU oracle baseline")
        qw_oracle = oracle.quantize(w.w)                # offline, outside the timed sample
        out["cpu_baseline"] = cpu_baseline(w, qw_oracle, a.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


class CacheFlush:
    """Evicts L2 and the MALL by reading a 1 GiB buffer (written once here).

    A read leaves only clean lines behind.  Writing the buffer instead would
    leave 1 GiB of dirty lines whose write-back then competes with the timed
    kernel's reads (the long-context X quantiser took 113 us after a write
    flush, 76 us after a read flush)."""

    def __init__(self, torch, dev):
        self.buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(7).view(torch.int64)
        torch.cuda.synchronize()

    def __call__(self):
        self.buf.max()


def _time_events(torch, fn, reps, flush=None):
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return ts


def _dequant_rel_err(torch, x, codes, scales, g):
    """‖x − Dequant(q)‖ / ‖x‖ in fp32 (a reported statistic, computed with torch)."""
    e2m1 = torch.tensor([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6],
                        dtype=torch.float32, device=x.device)
    lo, hi = (codes & 15).long(), (codes >> 4).long()
    vals = torch.stack((e2m1[lo], e2m1[hi]), dim=-1).reshape(codes.shape[0], -1)
    s = scales.view(torch.float8_e4m3fn).float().repeat_interleave(16, dim=1)
    d = vals * s * g.float()
    xf = x.float()
    return float(torch.linalg.vector_norm(xf - d) / torch.linalg.vector_norm(xf))


def extended(path, nv, torch, np, workloads, dev, up):
    """Per-kernel numbers on the other DiT shapes and the full KV sequence."""
    lines = []
    flush = CacheFlush(torch, dev)
    shapes = [("qkv", workloads.qkv, False), ("ffn_up", workloads.ffn, True), ("long", workloads.long_ctx, False)]
    for name, fn, gelu in shapes:
        log(f"extended: {name}")
        w = fn()
        x, W = up(w.x), up(w.w)
        M, K, N = w.M, w.K, w.N
        wq, wsc, wg = nv.quantize(W)
        aq, asc, ag = nv.quantize(x)
        bias = up(w.bias) if w.bias is not None else None
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        g = lambda: nv.gemm(aq, asc, ag, wq, wsc, wg, bias=bias, gelu=gelu, out=C)
        g(); torch.cuda.synchronize()
        tg = float(np.median(_time_events(torch, g, 20)))
        qws = nv.workspace(nv.quantize_workspace_bytes(M, K), dev)
        q = lambda: nv.quantize_into(x, aq, asc, ag, qws)
        tq = float(np.median(_time_events(torch, q, 20, flush)))
        qb = M * K * 2.5625
        lines.append({"shape": name, "M": M, "N": N, "K": K, "gemm_us": tg,
                      "gemm_tflops": 2 * M * N * K / tg / 1e6, "tile": nv.gemm_tile(M, N, K),
                      "quantize_us_cold": tq, "quantize_gbs_cold": qb / tq / 1e3})
        if name == "qkv":
            # adaptive {4, 6} block scales: time (cold) and normwise dequant error
            # against the standard amax→6 encoding, for X and for the weights
            for tname, t, rows in (("X", x, M), ("W", W, N)):
                ws_t = nv.workspace(nv.quantize_workspace_bytes(rows, K), dev)
                oc = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
                os_ = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev)
                og = torch.empty((1,), dtype=torch.float32, device=dev)
                rec = {"shape": f"qkv_{tname}_adaptive46", "rows": rows, "K": K}
                for mode, ad in (("std", False), ("adaptive", True)):
                    f = lambda: nv.quantize_into(t, oc, os_, og, ws_t, adaptive46=ad)
                    tt = float(np.median(_time_events(torch, f, 10, flush)))
                    f(); torch.cuda.synchronize()
                    rec[f"{mode}_us_cold"] = tt
                    rec[f"{mode}_gbs_cold"] = rows * K * 2.5625 / tt / 1e3
                    rec[f"{mode}_rel_err"] = _dequant_rel_err(torch, t, oc, os_, og)
                lines.append(rec)
            # two-dimensional 16x16 weight blocks (offline weight quantisation):
            # time (cold) and normwise dequant error against the 1-D blocks
            ws_w = nv.workspace(nv.quantize_workspace_bytes(N, K), dev)
            oc = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
            os_ = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
            og = torch.empty((1,), dtype=torch.float32, device=dev)
            rec = {"shape": "qkv_W_blocks2d", "rows": N, "K": K}
            for mode, b2 in (("1d", False), ("2d", True)):
                f = lambda: nv.quantize_into(W, oc, os_, og, ws_w, blocks2d=b2)
                tt = float(np.median(_time_events(torch, f, 10, flush)))
                f(); torch.cuda.synchronize()
                rec[f"{mode}_us_cold"] = tt
                rec[f"{mode}_gbs_cold"] = N * K * 2.5625 / tt / 1e3
                rec[f"{mode}_rel_err"] = _dequant_rel_err(torch, W, oc, os_, og)
            lines.append(rec)
        if name == "ffn_up":
            # down projection: H = GELU output (bf16 [8192, 14336]) quantised, times W_down
            Wd = up(w.w2)
            dq, dsc, dg = nv.quantize(Wd)
            hq, hsc, hg = nv.quantize(C)
            Cd = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
            gd = lambda: nv.gemm(hq, hsc, hg, dq, dsc, dg, out=Cd)
            gd(); torch.cuda.synchronize()
            td = float(np.median(_time_events(torch, gd, 20)))
            hws = nv.workspace(nv.quantize_workspace_bytes(M, N), dev)
            qh = lambda: nv.quantize_into(C, hq, hsc, hg, hws)
            tqh = float(np.median(_time_events(torch, qh, 20, flush)))
            lines.append({"shape": "ffn_down", "M": M, "N": K, "K": N, "gemm_us": td,
                          "gemm_tflops": 2 * M * N * K / td / 1e6, "tile": nv.gemm_tile(M, K, N),
                          "quantize_us_cold": tqh, "quantize_gbs_cold": M * N * 2.5625 / tqh / 1e3})
            # the whole FFN: linear(up, GELU) → quantise H → down GEMM, against
            # linear_q (H's maxima from the up GEMM's epilogue, H read once)
            lws = nv.workspace(nv.linear_workspace_bytes(M, K), dev)
            qws_ = nv.workspace(nv.linear_q_workspace_bytes(M, N, K), dev)

            def chain():
                nv.linear(x, wq, wsc, wg, gelu=True, out=C, ws=lws)
                nv.quantize_into(C, hq, hsc, hg, hws)
                nv.gemm(hq, hsc, hg, dq, dsc, dg, out=Cd)

            def chain_q():
                nv.linear_q(x, wq, wsc, wg, gelu=True, out=(hq, hsc, hg), ws=qws_)
                nv.gemm(hq, hsc, hg, dq, dsc, dg, out=Cd)
            chain(); chain_q(); torch.cuda.synchronize()
            tc = float(np.median(_time_events(torch, chain, 10, flush)))
            tcq = float(np.median(_time_events(torch, chain_q, 10, flush)))
            flops_ffn = 4.0 * M * N * K
            lines.append({"shape": "ffn_chain", "M": M, "D": K, "hidden": N,
                          "linear_quantize_gemm_us": tc, "linear_q_gemm_us": tcq,
                          "tflops_unfused": flops_ffn / tc / 1e6, "tflops_linear_q": flops_ffn / tcq / 1e6})
            del qws_, lws
        del x, W, C
        torch.cuda.empty_cache()
    # the 65536-token KV sequence: 74 appends of 880 tokens + one of 416, then a full dequant
    log("extended: kv sequence")
    Kb, Vb, sizes = workloads.kv()
    kd, vd = up(Kb), up(Vb)
    T = Kb.shape[0]
    cache = nv.KVCache(T, 24, 128, max_chunks=len(sizes), device=dev)
    starts = np.r_[0, np.cumsum(sizes)]

    def seq():
        cache.reset()
        for i in range(len(sizes)):
            cache.append(kd[starts[i]:starts[i + 1]], vd[starts[i]:starts[i + 1]])

    seq(); torch.cuda.synchronize()
    tseq = float(np.median(_time_events(torch, seq, 5, flush)))

    def seq46():
        cache.reset()
        for i in range(len(sizes)):
            cache.append(kd[starts[i]:starts[i + 1]], vd[starts[i]:starts[i + 1]], adaptive46=True)

    seq46(); torch.cuda.synchronize()
    tseq46 = float(np.median(_time_events(torch, seq46, 5, flush)))
    # the same 75 appends captured once in a HIP graph (each replay writes the
    # token ranges and chunk slots fixed at capture time)
    seq_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(seq_graph):
        seq()
    seq_graph.replay(); torch.cuda.synchronize()
    tseq_graph = float(np.median(_time_events(torch, seq_graph.replay, 5, flush)))
    seq(); torch.cuda.synchronize()
    ko = torch.empty((T, 24, 128), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    deq = lambda: cache.dequant(0, T, ko, vo)
    tdq = float(np.median(_time_events(torch, deq, 10, flush)))
    kvb = 2 * T * 3072 * 2.5625
    lines.append({"shape": "kv_65536", "appends": len(sizes), "append_seq_us": tseq,
                  "append_seq_gbs": kvb / tseq / 1e3, "append_us_per_chunk": tseq / len(sizes),
                  "append_seq_adaptive46_us": tseq46, "append_seq_graph_us": tseq_graph,
                  "append_seq_graph_gbs": kvb / tseq_graph / 1e3,
                  "dequant_us": tdq, "dequant_gbs": kvb / tdq / 1e3})
    with open(path, "w") as f:
        for l in lines:
            f.write(json.dumps(l) + "\n")
    log(f"extended results written to {path}")


if __name__ == "__main__":
    main()
