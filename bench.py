#!/usr/bin/env python3
"""Benchmark: ms per calibration Hessian on one MI355X.

A step is one whole Hessian: reset, every calibration batch through
hess_add_batch, then hess_materialize (scale 2/N, neutralize, 1% damping).
The headline workload is width 2,560 with 360 batches of 1..2,000 tokens,
bf16 activations N(0,1) x lognormal(0, 0.5) column scales, pre-staged in one
device buffer (inputs resident in HBM before the timed region starts).

Other workloads (width 4,096 ragged and a single 32K-token batch in bf16 and
fp32, 64 routed-expert Hessians in one grouped launch, 16x16 local blocks)
are timed after the headline and reported under "extra".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

P_BF16 = 2.5e15        # MI355X dense bf16 matrix peak, FLOP/s
P_F32_MFMA = 157.3e12  # MI355X fp32 matrix peak, FLOP/s
P_F64 = 78.6e12        # MI355X fp64 peak (matrix and vector), FLOP/s
HBM = 8.0e12           # MI355X HBM3E peak, bytes/s
METRIC = "ms per Hessian & TFLOP/s (MFMA util %) at d=2560/4096, ragged batches"
PAGES_MS = {2560: 11.0, 4096: 15.0}  # the pages' GB300 bf16-in numbers for ~360 ragged batches


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_hessian(torch, hs, d, views, steps, warmup, dtype, kernel_timing=False):
    """Whole-Hessian timing with per-step HIP events on the library's stream.

    With kernel_timing, the library also brackets each SYRK launch with HIP
    events (on the stream the kernel runs on) during the timed steps.
    Returns (mean ms, per-step ms array, host wall ms, (launches, tokens, syrk ms) or None).
    """
    h = hs.Hessian(d, dtype)
    out = torch.empty((d, d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def one():
        h.reset()
        for x in views:
            h.add_batch(x)
        h.materialize(0.01, out=out)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    if kernel_timing:
        h.set_timing(True)
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        one()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    ms = ev[0].elapsed_time(ev[steps]) / steps
    kt = None
    if kernel_timing:
        kt = h.timing()
        h.set_timing(False)
    h.close()
    return ms, per, wall, kt


KERNEL_SOURCES = ("syrk.hip", "hess_device.hpp", "hess_internal.hpp", "hess_api.hip")
BIG_KERNEL_SOURCES = ("syrk_big.hip", "hess_device.hpp", "hess_internal.hpp", "hess_api.hip")


def kernel_source_sha256(sources=KERNEL_SOURCES):
    """sha256 over a kernel's sources and its launch planning, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "gptq_hessian_accumulation_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(summary, sources=KERNEL_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None.

    None when the summary is missing or was taken on a different version of
    the kernel sources (their sha256 no longer matches).
    """
    try:
        with open(summary) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
        sha = kernel_source_sha256(sources)
        if kv.get("source_sha256", "").strip() != sha:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def syrk_flops(d, n):
    return float(n) * d * (d + 1)          # upper triangle incl. diagonal, 2 flops per MAC


def syrk_bytes(d, n, esize):
    return 4.0 * d * (d + 1) + float(n) * d * esize   # upper S read + write, X read


def _blas_info():
    """(vendor, threads) of the BLAS numpy calls, from threadpoolctl when it is there."""
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                return f"{p.get('internal_api', '?')} {p.get('version', '')}".strip(), int(p.get("num_threads", 1))
    except Exception:
        pass
    return "unknown", len(os.sched_getaffinity(0))


def cpu_baseline(W, O, torch, views, d, budget_s=45.0):
    """The float64 oracle on the host over the whole timed unit: every batch of the same
    workload (host copies of the device batches) and the materialize.  If the first batches
    show that the whole unit would take longer than budget_s, the rest is scaled by algorithmic
    flops (and said so).  The tiny configuration (d=256, 100/37/0 fp32 tokens) is also timed
    with one BLAS thread."""
    host = [W.host_copy(v, "bf16") for v in views]
    acc = O.GramAccumulator(d)
    t_used, flops_done, nb = 0.0, 0.0, 0
    total_flops = sum(syrk_flops(d, x.shape[0]) for x in host)
    for x in host:
        t0 = time.perf_counter()
        acc.add_batch(x, "bf16")
        t_used += time.perf_counter() - t0
        flops_done += syrk_flops(d, x.shape[0])
        nb += 1
        if nb >= 20 and t_used * total_flops / flops_done > budget_s:
            break
    t0 = time.perf_counter()
    acc.materialize(0.01)
    t_mat = time.perf_counter() - t0
    whole = nb == len(host)
    ms = (t_used * (1.0 if whole else total_flops / flops_done) + t_mat) * 1e3
    vendor, threads = _blas_info()
    cores = len(os.sched_getaffinity(0))
    tiny = W.tiny_case()
    tiny_ms = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            reps = 20
            t0 = time.perf_counter()
            for _ in range(reps):
                a = O.GramAccumulator(tiny.d)
                for b in tiny.batches:
                    a.add_batch(b, tiny.dtype)
                a.materialize(0.01)
            tiny_ms = (time.perf_counter() - t0) * 1e3 / reps
    except Exception:
        pass
    sample = (f"float64 NumPy oracle over the whole timed unit: all {len(host)} batches ({t_used:.1f} s) plus "
              f"materialize" if whole else
              f"float64 NumPy oracle on the first {nb} of {len(host)} batches ({t_used:.1f} s), scaled by "
              f"algorithmic flops to the whole Hessian, plus materialize")
    return {"value": round(ms, 1), "unit": "ms/Hessian", "cores": threads, "kind": "oracle", "sample": sample,
            "affinity_cores": cores, "blas": vendor, "blas_threads": threads,
            "tiny_d256_single_thread_ms": None if tiny_ms is None else round(tiny_ms, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--extras", default="all",
                    help="comma-separated subset of d4096_ragged,d4096_single,moe,local,imatrix,f16_staging,chol,quant,"
                         "thin,graph "
                         "(default all; imatrix runs with local)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--print-kernel-sha", action="store_true",
                    help="print the sha256 of the SYRK kernel sources and exit")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 256 MiB device copy (the byte-counter calibration kernel)")
    args = ap.parse_args()
    if args.print_kernel_sha:
        print("syrk", kernel_source_sha256())
        print("syrk_big", kernel_source_sha256(BIG_KERNEL_SOURCES))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the Hessian path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    import gptq_hessian_accumulation_amd as hs
    import workloads as W

    torch.cuda.set_device(0)
    d = 2560
    log("staging d=2560 ragged workload")
    buf, views, sizes, _ = W.torch_ragged(d, seed=1)
    N = int(sizes.sum())
    torch.cuda.synchronize()
    log(f"timing {args.steps} Hessians after {args.warmup} warm-ups")
    ms, per, wall, _ = time_hessian(torch, hs, d, views, args.steps, args.warmup, torch.bfloat16)
    log(f"headline: {ms:.3f} ms per Hessian (median {np.median(per):.3f}, host wall {wall:.3f} ms)")
    # Second pass of the same K steps with each SYRK launch bracketed by HIP
    # events on its stream (kept out of the headline pass: the extra event
    # packets between kernels cost time of their own).
    _, _, _, kt = time_hessian(torch, hs, d, views, args.steps, 1, torch.bfloat16, kernel_timing=True)
    flops = syrk_flops(d, N)
    tflops = flops / (ms * 1e-3) / 1e12
    # Roofline of the dominant kernel, the SYRK pass of each staging flush (a
    # dense bf16 contraction, on 256-tiles at this width and flush length):
    # algorithmic flops of the tokens each launch processed, N d (d + 1), over
    # the launches' HIP-event durations (main kernel), against the dense bf16
    # MFMA peak.
    launches, ktok, kms = kt
    achieved = syrk_flops(d, ktok) / (kms * 1e-3)
    traffic = read_traffic(os.path.join(ROOT, "profiles", "syrk_big_bf16_d2560_ragged_traffic.txt"),
                           BIG_KERNEL_SOURCES)
    result = {
        "metric": METRIC,
        "value": round(ms, 4),
        "unit": "ms/Hessian",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_median": round(float(np.median(per)), 4),
        "ms_min": round(float(per.min()), 4),
        "ms_p90": round(float(np.percentile(per, 90)), 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(ms / PAGES_MS[d], 4),
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "d=2560, 360 ragged calibration batches of U[1,2000] tokens, bf16 N(0,1) x "
                               "lognormal(0,0.5) column scales, one fp32 Hessian scaled 2/N, damp 1%",
                   "d": d, "batches": len(sizes), "tokens": N, "seed": 1},
        "tflops": round(tflops, 2),
        "mfma_util": round(flops / (ms * 1e-3) / P_BF16, 4),
        "pages_gb300_ms": PAGES_MS[d],
        "roofline": {"bound": "mfma", "achieved": round(achieved / 1e12, 1), "peak": P_BF16 / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / P_BF16, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": "syrk_big_bf16_t8 (256-tile SYRK main kernel of each staging flush, transposed staging)",
                     "launches_per_hessian": round(launches / args.steps, 2),
                     "mean_launch_us": round(kms * 1e3 / launches, 2),
                     "tokens_per_launch": round(ktok / launches, 1)},
    }
    del buf, views
    torch.cuda.empty_cache()

    if args.copy_calib:
        # A plain copy of known size: 256 MiB read and 256 MiB written per
        # dispatch.  Hardware byte counters read on this kernel give the factor
        # that turns the same counters on the SYRK into bytes.
        src = torch.empty(128 << 20, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 256 MiB device copies")
        del src, dst

    extra = {}
    if not args.no_extras:
        extra = run_extras(torch, hs, W, args)
        result["extra"] = extra

    if not args.no_cpu:
        import oracle as O
        log("cpu baseline (oracle)")
        buf, views, sizes, _ = W.torch_ragged(d, seed=1)
        result["cpu_baseline"] = cpu_baseline(W, O, torch, views, d)
        del buf, views
    print(json.dumps(result), flush=True)


def run_extras(torch, hs, W, args):
    extra = {}
    steps = max(3, args.steps // 2)
    want = set(args.extras.split(",")) if args.extras != "all" else {"d4096_ragged", "d4096_single", "moe", "local",
                                                                    "imatrix", "f16_staging", "chol", "quant",
                                                                    "thin", "graph"}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if "quant" in want:
        # error-propagating 4-bit quantization of a 4096 x 4096 layer (groups of 128), float64
        # inside: the propagation is rows * cols^2 flops (one multiply-add per remaining column)
        log("block quantize 4096 x 4096")
        dq = 4096
        gen = W.torch_generator(6, "cuda")
        sc = W.torch_column_scales(gen, dq, "cuda")
        x = W.torch_rows(gen, 2 * dq, dq, sc, "f32", "cuda")
        H = (x.T @ x) * (2.0 / (2 * dq))
        H += 0.01 * H.diagonal().mean() * torch.eye(dq, device="cuda")
        U = hs.chol_inverse_upper(H)
        Wq = torch.randn((dq, dq), generator=gen, device="cuda", dtype=torch.float32) * 0.02
        ws = torch.empty(hs._load().hess_gptq_quantize_workspace(dq, dq), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(Wq)
        for _ in range(2):
            hs.gptq_quantize(Wq, U, group_size=128, out=out, workspace=ws)
        torch.cuda.synchronize()
        reps = max(3, steps)
        e0.record()
        for _ in range(reps):
            hs.gptq_quantize(Wq, U, group_size=128, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        fl = float(dq) * dq * dq
        extra["gptq_quantize_4096x4096_g128"] = {"ms": round(ms, 4), "tflops_f64": round(fl / ms / 1e9, 2),
                                                 "f64_util": round(fl / (ms * 1e-3) / P_F64, 4)}
        del x, H, U, Wq, ws, out
    if "chol" in want:
        # upper Cholesky factor of the inverse damped Hessian, float64 inside:
        # 2 d^3 / 3 flops (factor d^3 / 3 + triangular inverse d^3 / 3)
        for dc in (2560, 4096):
            log(f"Cholesky of the inverse, d={dc}")
            gen = W.torch_generator(5, "cuda")
            sc = W.torch_column_scales(gen, dc, "cuda")
            x = W.torch_rows(gen, 2 * dc, dc, sc, "f32", "cuda")
            H = (x.T @ x) * (2.0 / (2 * dc))
            H += 0.01 * H.diagonal().mean() * torch.eye(dc, device="cuda")
            U = torch.empty_like(H)
            ws = torch.empty(hs._load().hess_chol_inverse_workspace(dc), dtype=torch.uint8, device="cuda")
            for _ in range(2):
                hs.chol_inverse_upper(H, out=U, workspace=ws, check=False)
            torch.cuda.synchronize()
            reps = max(3, steps)
            e0.record()
            for _ in range(reps):
                hs.chol_inverse_upper(H, out=U, workspace=ws, check=False)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            fl = 2.0 * dc ** 3 / 3.0
            extra[f"chol_inverse_upper_d{dc}"] = {"ms": round(ms, 4), "tflops_f64": round(fl / ms / 1e9, 2),
                                                  "f64_util": round(fl / (ms * 1e-3) / P_F64, 4)}
            del x, H, U, ws
    if "f16_staging" in want:
        # the d=2560 ragged workload with fp16 activations, staged in bf16:
        # each batch is rounded to bf16 by the staging copy
        log("d=2560 ragged, fp16 activations staged in bf16")
        buf, views, sizes, _ = W.torch_ragged(2560, seed=1, dtype="f16")
        N = int(sizes.sum())
        ms, _, _, _ = time_hessian(torch, hs, 2560, views, steps, 1, torch.bfloat16)
        fl = syrk_flops(2560, N)
        extra["d2560_ragged_f16_in_bf16_staging"] = {"ms": round(ms, 3), "tflops": round(fl / ms / 1e9, 1),
                                                     "mfma_util": round(fl / (ms * 1e-3) / P_BF16, 4),
                                                     "tokens": N}
        del buf, views
    # d=4096 ragged (bf16 and fp32), dead columns 1%
    for dt, tdt in (() if "d4096_ragged" not in want else (("bf16", torch.bfloat16), ("f32", torch.float32))):
        log(f"d=4096 ragged {dt}")
        buf, views, sizes, _ = W.torch_ragged(4096, seed=2, dtype=dt, dead_frac=0.01)
        N = int(sizes.sum())
        ms, _, _, _ = time_hessian(torch, hs, 4096, views, steps, 1, tdt)
        fl = syrk_flops(4096, N)
        extra[f"d4096_ragged_{dt}"] = {"ms": round(ms, 3), "tflops": round(fl / ms / 1e9, 1),
                                       "mfma_util": round(fl / (ms * 1e-3) / P_BF16, 4), "tokens": N,
                                       "pages_gb300_ms": PAGES_MS[4096] if dt == "bf16" else 244.0}
        del buf, views
    # d=4096, one 32768-token batch
    for dt, tdt in (() if "d4096_single" not in want else (("bf16", torch.bfloat16), ("f32", torch.float32))):
        log(f"d=4096 single 32K batch {dt}")
        x, _ = W.torch_single(4096, 32768, seed=2, dtype=dt, dead_frac=0.01)   # 41 zeroed columns
        ms, _, _, (nl, _, kms) = time_hessian(torch, hs, 4096, [x], steps, 1, tdt, kernel_timing=True)
        kern = kms / nl
        fl = syrk_flops(4096, 32768)
        peak = P_BF16 if dt == "bf16" else P_F32_MFMA
        extra[f"d4096_n32768_{dt}"] = {"ms": round(ms, 4), "syrk_ms": round(kern, 4),
                                       "syrk_tflops": round(fl / kern / 1e9, 1),
                                       "syrk_util": round(fl / (kern * 1e-3) / peak, 4),
                                       "peak_tflops": peak / 1e12}
        if dt == "bf16":
            # roofline of this launch's main kernel (the 256-tile SYRK): algorithmic
            # flops N d (d + 1) over its event-timed duration; counter traffic per launch
            traffic = read_traffic(os.path.join(ROOT, "profiles", "syrk_big_bf16_d4096_n32768_traffic.txt"),
                                   BIG_KERNEL_SOURCES)
            extra["d4096_n32768_bf16"]["roofline"] = {
                "bound": "mfma", "achieved": round(fl / kern / 1e9, 1), "peak": P_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": round(fl / (kern * 1e-3) / P_BF16, 4), "traffic": None if traffic is None else round(traffic),
                "kernel": "syrk_big_bf16 (256-tile SYRK main kernel, row-major batch; its fixup follows)"}
        del x
    if "moe" in want:
        # MoE: 64 routed experts, d=2048, 32768 tokens top-8, Zipf(1.1)
        log("MoE grouped")
        rng = np.random.default_rng(3)
        row_idx, offsets = W.moe_routing(rng, 32768, experts=64, topk=8)
        gen = W.torch_generator(3, "cuda")
        sc = W.torch_column_scales(gen, 2048, "cuda")
        x = W.torch_rows(gen, 32768, 2048, sc, "bf16", "cuda")
        ridx = torch.from_numpy(row_idx).cuda()
        hsx = [hs.Hessian(2048, torch.bfloat16, staging_bytes=0) for _ in range(64)]  # grouped updates only
        outs = [torch.empty((2048, 2048), dtype=torch.float32, device="cuda") for _ in range(64)]

        def moe_once():
            hs.reset_grouped(hsx)
            hs.add_batch_grouped(hsx, x, offsets, ridx)
            hs.materialize_grouped(hsx, 0.01, outs=outs)

        moe_once()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e2 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            hs.reset_grouped(hsx)
            hs.add_batch_grouped(hsx, x, offsets, ridx)
        e1.record()
        torch.cuda.synchronize()
        grouped_ms = e0.elapsed_time(e1) / steps
        e0.record()
        for _ in range(steps):
            hs.materialize_grouped(hsx, 0.01, outs=outs)
        e1.record()
        torch.cuda.synchronize()
        mat_ms = e0.elapsed_time(e1) / steps
        e0.record()
        for _ in range(steps):
            moe_once()
        e2.record()
        torch.cuda.synchronize()
        total_ms = e0.elapsed_time(e2) / steps
        fl = sum(syrk_flops(2048, int(offsets[e + 1] - offsets[e])) for e in range(64))
        # materialize bytes: each expert's upper triangle read (d (d + 1) / 2 floats), H written (d^2 floats)
        mat_bytes = 64 * (2.0 * 2048 * 2049 + 4.0 * 2048 * 2048)
        extra["moe_64x2048_grouped"] = {"ms_total": round(total_ms, 3), "ms_reset_plus_grouped": round(grouped_ms, 3),
                                        "tflops_grouped": round(fl / grouped_ms / 1e9, 1),
                                        "ms_materialize_64": round(mat_ms, 4),
                                        "materialize_hbm_frac": round(mat_bytes / (mat_ms * 1e-3) / HBM, 4),
                                        "rows": int(offsets[-1])}
        for h in hsx:
            h.close()
        del x, ridx
    if "local" in want:
        # local 16x16 blocks: 32768 x 4096 bf16, 16 distinct buffers cycled
        log("local blocks")
        gen = W.torch_generator(4, "cuda")
        sc = W.torch_column_scales(gen, 4096, "cuda")
        xs = [W.torch_rows(gen, 32768, 4096, sc, "bf16", "cuda") for _ in range(16)]
        out = torch.zeros((256, 16, 16), dtype=torch.float32, device="cuda")
        for xx in xs[:2]:
            hs.local_blocks(xx, out=out)
        torch.cuda.synchronize()
        e0.record()
        reps = 4
        for _ in range(reps):
            for xx in xs:
                hs.local_blocks(xx, out=out)
        e1.record()
        torch.cuda.synchronize()
        per = e0.elapsed_time(e1) / (reps * 16)
        byts = 32768 * 4096 * 2 + 256 * 256 * 4 * 2
        extra["local_32768x4096"] = {"ms_per_update": round(per, 4), "GBps": round(byts / per / 1e6, 1),
                                     "hbm_frac": round(byts / (per * 1e-3) / HBM, 4), "pages_rtx_pro_6000_ms": 0.40}
        if "imatrix" in want:
            # imatrix per-column sums of squares over the same 16 cold buffers
            log("imatrix")
            m = hs.ImatrixStat(4096, torch.bfloat16)
            for xx in xs[:2]:
                m.add_batch(xx)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                for xx in xs:
                    m.add_batch(xx)
            e1.record()
            torch.cuda.synchronize()
            per = e0.elapsed_time(e1) / (reps * 16)
            byts = 32768 * 4096 * 2 + 4096 * 4 * 2
            extra["imatrix_32768x4096"] = {"ms_per_update": round(per, 4), "GBps": round(byts / per / 1e6, 1),
                                           "hbm_frac": round(byts / (per * 1e-3) / HBM, 4)}
            m.close()
        del xs
    if "graph" in want:
        # the headline Hessian (reset, 360 add_batch calls, materialize) captured once in a HIP graph
        # and replayed: the same kernels without the host's per-call launch path
        log("headline Hessian as a replayed graph")
        dg = 2560
        buf, views, _, _ = W.torch_ragged(dg, seed=1)
        outg = torch.empty((dg, dg), dtype=torch.float32, device="cuda")
        hg = hs.Hessian(dg, torch.bfloat16)

        def one_g():
            hg.reset()
            for x in views:
                hg.add_batch(x)
            hg.materialize(0.01, out=outg)

        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            one_g()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        ref = outg.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cs):
            one_g()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(outg, ref))
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(3, steps)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        extra["headline_graph_replay"] = {"ms": round(e0.elapsed_time(e1) / reps, 4), "equal_to_eager": same}
        del graph, hg, buf, views
    if "thin" in want:
        # thin batches added straight into S (a handle without staging): the 64-tile kernel, whose
        # time is the read-modify-write of S's upper triangle (4 d (d + 1) bytes) plus the batch
        # (2 n d bytes).  batch_us: 200 back-to-back calls between two events on the stream (the
        # host's per-call cost, about 5 us from Python, bounds it when the kernel is shorter);
        # kernel_us: the library's HIP events around each launch (their own cost included).
        for dt, xdt in ((4096, "bf16"), (2560, "bf16"), (4096, "f32")):
            log(f"thin batches straight into S, d={dt} {xdt}")
            gen = W.torch_generator(8, "cuda")
            sc = W.torch_column_scales(gen, dt, "cuda")
            xs = W.torch_rows(gen, 64 * 16, dt, sc, xdt, "cuda")
            h = hs.Hessian(dt, torch.bfloat16 if xdt == "bf16" else torch.float32, staging_bytes=0)
            res = {}
            for n in (1, 64):
                views = [xs[i * 64:i * 64 + n] for i in range(16)]
                for v in views[:4]:
                    h.add_batch(v)
                torch.cuda.synchronize()
                reps = 200
                e0.record()
                for i in range(reps):
                    h.add_batch(views[i % 16])
                e1.record()
                torch.cuda.synchronize()
                b_us = e0.elapsed_time(e1) * 1e3 / reps
                h.set_timing(True)
                for i in range(reps):
                    h.add_batch(views[i % 16])
                launches, _, kms = h.timing()
                h.set_timing(False)
                # the same 200 calls captured once in a HIP graph and replayed: the GPU's time per
                # batch without the host's per-call cost
                cs = torch.cuda.Stream()
                cs.wait_stream(torch.cuda.current_stream())
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    for i in range(reps):
                        h.add_batch(views[i % 16])
                g.replay()
                torch.cuda.synchronize()
                e0.record()
                for _ in range(3):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                g_us = e0.elapsed_time(e1) * 1e3 / (3 * reps)
                del g
                byts = 4.0 * dt * (dt + 1) + (2.0 if xdt == "bf16" else 4.0) * n * dt
                res[f"n{n}"] = {"batch_us": round(b_us, 2), "kernel_us": round(kms * 1e3 / launches, 2),
                                "GBps": round(byts / b_us / 1e3, 1), "hbm_frac": round(byts / (b_us * 1e-6) / HBM, 4),
                                "graph_batch_us": round(g_us, 2),
                                "graph_hbm_frac": round(byts / (g_us * 1e-6) / HBM, 4)}
            h.close()
            extra[f"thin_direct_d{dt}" + ("" if xdt == "bf16" else "_f32")] = res
            del xs
    torch.cuda.empty_cache()
    return extra


if __name__ == "__main__":
    main()
