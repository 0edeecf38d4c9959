"""Throughput of the any4 quantizer on one MI355X.

A step is one any4_quantize call over a whole synthetic Llama3-8B-like up_proj weight
(14336 x 4096 bf16, group 128, 16 clusters, 20 Lloyd rounds): scaling, k-means++,
Lloyd, final assignment and emission.  Inputs are resident in HBM before timing;
outputs are preallocated.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1]
  python bench.py --profile-steps 3          # short run for rocprofv3
  python bench.py --profile-steps 2 --iters 0   # same, without Lloyd rounds (counter deltas)
  python bench.py --copy-calibration         # plain copy of known size (counter scale)
  python bench.py --bookends-only --profile-steps 5   # only E|x| and dequantization
  python bench.py --sorted-only --profile-steps 5     # only the sorted-row Lloyd stage

The same line reports the two bookend kernels (E|x| of a calibration batch and the
Eq. 4 dequantization of the quantized matrix) against the HBM roofline under
"bookends", and the sorted-row Lloyd stage on the same matrix under "sorted_lloyd";
they run after the timed quantizer steps and are not part of `value`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

KERNEL_SRC = os.path.join(ROOT, "weight_only_bit_row_amd", "csrc", "any4_kernels.hip")
COUNTERS = os.path.join(ROOT, "profiles", "any4_rows_up_proj_counters.md")
BOOKENDS_SRC = os.path.join(ROOT, "weight_only_bit_row_amd", "csrc", "any4_bookends.hip")
BOOKENDS_COUNTERS = os.path.join(ROOT, "profiles", "any4_bookends_calib32x2048_up_proj.md")
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

PEAK_FP32_TFLOPS = 157.3       # MI355X FP32 vector (packed FMA counted as 2 flops x 2 lanes)
METRIC = "Lloyd elem-iters/sec and % FP32 VALU peak; ms per 14336x4096 matrix"


def credited_flops_per_element(k: int, iters: int) -> int:
    """Algorithmic work per weight element for the whole call: scaling (~6 flop),
    k-means++ (4 per centre), `iters` Lloyd rounds of 3k+1 (k subtractions, k squares,
    k-1 compares, 2 adds) and a final E-step plus objective (3k+2)."""
    return 6 + 4 * k + iters * (3 * k + 1) + (3 * k + 2)


def kernel_source_hash(path: str = KERNEL_SRC) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(counters: str = COUNTERS, src: str = KERNEL_SRC, key: str = "traffic_bytes_per_launch"):
    """HBM bytes per launch from a committed counter summary, if it was taken on the
    current kernel source; otherwise None."""
    if not os.path.exists(counters):
        return None
    text = open(counters).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash(src):
        return None
    return float(t.group(1))


def cpu_baseline(m, group, k, iters, n_rows_sample=14336):
    """The CPU oracle, as it is, on a bounded row sample of the same matrix, spread over
    the host's cores with threads (ctypes releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    cores = min(16, len(os.sched_getaffinity(0)))
    rows = min(n_rows_sample, m.w.shape[0])
    bounds = np.linspace(0, rows, cores + 1).astype(int)

    def work(c):
        lo, hi = bounds[c], bounds[c + 1]
        if hi > lo:
            oracle.quantize(m.w[lo:hi], m.dtype, m.act, group, k, iters, seed=0, row_offset=int(lo))

    oracle.lib()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        list(ex.map(work, range(cores)))
    dt = time.perf_counter() - t0
    K = m.w.shape[1]
    return {
        "value": rows * K * iters / dt,
        "unit": "elem-iters/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"first {rows} of {m.w.shape[0]} rows of the same matrix, full path "
                  f"(scale, k-means++, {iters} Lloyd rounds, final E-step, emission); "
                  f"{dt:.2f} s wall on {cores} threads",
    }


def copy_calibration():
    import torch
    n = 1 << 28  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))


def sorted_lloyd(any4, torch, np, w, act, g, k, iters, c_reg, stream, n_launches=10):
    """The sorted-row Lloyd stage on the same matrix: scaled rows, sample weights and
    k-means++ centres from the GPU stages, then `iters` rounds, and 0 rounds (sort and
    prefix sums only), each the mean over a batch of launches with HIP events on the
    launch stream.  `rows_identical` compares its centroids with the register path's."""
    ws_, _, _, a = any4.stage_scale(w, act, group=g, n_clusters=k)
    c0, _ = any4.stage_seed(w, act, group=g, n_clusters=k)
    res = {"kernel": "sorted_lloyd_kernel", "n_rows": int(w.shape[0]), "n_cols": int(w.shape[1])}
    for n_it in (0, iters):
        c = any4.stage_lloyd_sorted(ws_, a, c0, n_clusters=k, iters=n_it, group=g)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_launches):
            any4.stage_lloyd_sorted(ws_, a, c0, n_clusters=k, iters=n_it, group=g)
        e1.record(stream)
        torch.cuda.synchronize()
        res["ms_rounds_%d" % n_it] = e0.elapsed_time(e1) / n_launches
    res["rows_identical_with_register_path"] = float(
        (c.view(torch.int32) == c_reg.view(torch.int32)).all(dim=1).float().mean().item())
    return res


def bookends(any4, torch, np, q, N, K, g, k, dev, stream, profile_steps=0):
    """E|x| of a calibration batch, the Eq. 4 dequantization of the quantized matrix and
    its LUT matrix-vector product with one and eight tokens, each timed over a batch of
    launches with HIP events on the launch stream (torch's bf16 product with the
    dequantized matrix is timed beside the LUT product as a point of comparison)."""
    from workloads import CALIB, make_activations

    x_np = make_activations("calib_32x2048")
    T, Kx = x_np.shape
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    del x_np
    act_out = torch.empty((Kx,), dtype=torch.float32, device=dev)
    ws = torch.empty((any4.act_absmean_workspace_bytes(T, Kx),), dtype=torch.uint8, device=dev)
    w_hat = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    x1, x8 = x[:1].contiguous(), x[:8].contiguous()     # decode tokens from the same batch
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
    y8 = torch.empty((8, N), dtype=torch.float32, device=dev)

    def run_abs():
        any4.act_absmean(x, out=act_out, ws=ws)

    def run_dq():
        any4.dequantize(q, g, k, out=w_hat)

    def run_gv1():
        any4.lut_gemv(q, x1, g, k, out=y1)

    def run_gv8():
        any4.lut_gemv(q, x8, g, k, out=y8)

    # a Llama-70B down_proj-sized product (8192 x 28672): seeded random codes, LUTs and
    # group scales (the kernel's time does not depend on the values)
    N70, K70 = 8192, 28672
    gen = torch.Generator(device=dev)
    gen.manual_seed(70)
    q70 = any4.Quantized(
        codes=torch.randint(0, 256, (N70, K70 // 2), dtype=torch.uint8, device=dev, generator=gen),
        lut=torch.randn((N70, k), device=dev, generator=gen).half(),
        scale=(torch.rand((N70, K70 // g), device=dev, generator=gen) * 1e-2).half(),
        offset=(torch.randn((N70, K70 // g), device=dev, generator=gen) * 1e-2).half(),
        objective=None)
    x70 = torch.randn((1, K70), device=dev, generator=gen).bfloat16()
    y70 = torch.empty((1, N70), dtype=torch.float32, device=dev)

    def run_gv70():
        any4.lut_gemv(q70, x70, g, k, out=y70)

    if profile_steps:
        for _ in range(profile_steps):
            run_abs()
            run_dq()
            run_gv1()
            run_gv8()
            run_gv70()
        torch.cuda.synchronize()
        return None

    def per_launch_ms(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_abs = per_launch_ms(run_abs, 20)
    ms_dq = per_launch_ms(run_dq, 100)
    ms_gv1 = per_launch_ms(run_gv1, 200)
    ms_gv8 = per_launch_ms(run_gv8, 100)
    ms_gv70 = per_launch_ms(run_gv70, 100)
    w70 = any4.dequantize(q70, g, k)
    ms_mm70 = per_launch_ms(lambda: torch.nn.functional.linear(x70, w70), 50)
    del w70
    run_dq()
    ms_mm1 = per_launch_ms(lambda: torch.nn.functional.linear(x1, w_hat), 200)
    ms_mm8 = per_launch_ms(lambda: torch.nn.functional.linear(x8, w_hat), 100)
    bytes_abs = T * Kx * 2 + Kx * 4                      # read x once, write E|x|
    bytes_w = N * K // 2 + N * k * 2 + 2 * N * (K // g) * 2     # codes, LUT, alpha/beta
    bytes_dq = bytes_w + N * K * 2                                # + bf16 out

    def bytes_gv(M, n=N, kk=K):
        wb = n * kk // 2 + n * k * 2 + 2 * n * (kk // g) * 2
        return wb + M * kk * 2 + M * n * 4                        # + bf16 x, fp32 y

    def roof(nbytes, ms, key):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS,
                "traffic": load_traffic(BOOKENDS_COUNTERS, BOOKENDS_SRC, key),
                "algorithmic_bytes": nbytes}

    return [
        {"kernel": "any4_act_absmean (absmean_partial_kernel + absmean_finish_kernel)",
         "workload": f"E|x| of {T} calibration tokens x {Kx} channels, bf16 "
                     f"(32 sequences of 2048 tokens, seed {CALIB['calib_32x2048'][2]})",
         "ms_per_call": ms_abs, "roofline": roof(bytes_abs, ms_abs, "absmean_traffic_bytes_per_launch")},
        {"kernel": "any4_dequantize (dequant_vec_kernel, bf16 out)",
         "workload": f"Eq. 4 dequantization of the quantized {N}x{K} up_proj (group {g}, "
                     f"{k} clusters) to bf16",
         "ms_per_call": ms_dq, "roofline": roof(bytes_dq, ms_dq, "dequant_traffic_bytes_per_launch")},
        {"kernel": "any4_lut_gemv (gemv_kernel<1, bf16 x, 2 rows per wave>)",
         "workload": f"one calibration token times the quantized {N}x{K} up_proj, fp32 out",
         "ms_per_call": ms_gv1, "bf16_matmul_ms_per_call": ms_mm1,
         "roofline": roof(bytes_gv(1), ms_gv1, "gemv1_traffic_bytes_per_launch")},
        {"kernel": "any4_lut_gemv (gemv_kernel<8, bf16 x, 2 rows per wave>)",
         "workload": f"eight calibration tokens times the quantized {N}x{K} up_proj, fp32 out",
         "ms_per_call": ms_gv8, "bf16_matmul_ms_per_call": ms_mm8,
         "roofline": roof(bytes_gv(8), ms_gv8, "gemv8_traffic_bytes_per_launch")},
        {"kernel": "any4_lut_gemv (gemv_kernel<1, bf16 x, 4 rows per wave>)",
         "workload": f"one token times a {N70}x{K70} matrix of seeded random codes (Llama-70B "
                     f"down_proj size), fp32 out",
         "ms_per_call": ms_gv70, "bf16_matmul_ms_per_call": ms_mm70,
         "roofline": roof(bytes_gv(1, N70, K70), ms_gv70, "gemv70_traffic_bytes_per_launch")},
    ]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many quantize calls (for rocprofv3), no baseline")
    ap.add_argument("--iters", type=int, default=None,
                    help="Lloyd rounds for --profile-steps runs (default: the workload's 20)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bookends", action="store_true",
                    help="skip the E|x|, dequant and LUT matrix-vector kernels")
    ap.add_argument("--sorted-only", action="store_true",
                    help="only the sorted-row Lloyd stage (with --profile-steps: launches per size)")
    ap.add_argument("--bookends-only", action="store_true",
                    help="with --profile-steps: run only the E|x|, dequant and LUT matrix-vector kernels")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the quantizer's rows are independent and this "
              "build runs on a single MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import weight_only_bit_row_amd as any4
    from workloads import make

    wl = make("up_proj")
    m = wl.matrices[0]
    N, K = m.w.shape
    g, k, iters = wl.group, wl.n_clusters, wl.iters
    dev = torch.device("cuda:0")
    w = torch.from_numpy(m.w.view(np.int16)).to(dev).view(torch.bfloat16)
    act = torch.from_numpy(m.act).to(dev)
    out = any4.quantize(w, act, group=g, n_clusters=k, iters=iters)   # allocates outputs
    ws = any4.workspace(dev)
    torch.cuda.synchronize()

    if args.sorted_only:
        _, c_reg, _, _ = any4.stage_full(w, act, g, k, iters, seed=0)
        res = sorted_lloyd(any4, torch, np, w, act, g, k, iters, c_reg, torch.cuda.current_stream(dev),
                           n_launches=args.profile_steps or 10)
        print(json.dumps({"sorted_lloyd": res}))
        return

    if args.profile_steps and args.bookends_only:
        bookends(any4, torch, np, out, N, K, g, k, dev, torch.cuda.current_stream(dev),
                 profile_steps=args.profile_steps)
        print(json.dumps({"profile_steps": args.profile_steps, "bookends_only": True}))
        return

    if args.profile_steps:
        p_iters = iters if args.iters is None else args.iters
        for _ in range(args.profile_steps):
            any4.quantize(w, act, group=g, n_clusters=k, iters=p_iters, out=out, ws=ws)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "status": any4.read_status(ws)}))
        return

    stream = torch.cuda.current_stream(dev)   # the stream the kernels are launched on

    def timed(n_iters, steps, warmup):
        for _ in range(warmup):
            any4.quantize(w, act, group=g, n_clusters=k, iters=n_iters, out=out, ws=ws)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        t0 = time.perf_counter()
        for e0, e1 in evs:
            e0.record(stream)
            any4.quantize(w, act, group=g, n_clusters=k, iters=n_iters, out=out, ws=ws)
            e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        return wall, ms

    wall, ms = timed(iters, args.steps, args.warmup)
    status = any4.read_status(ws)
    _, ms0 = timed(0, max(5, args.steps // 2), 2)
    ms_step = wall * 1e3 / args.steps
    ms_kernel = float(np.mean(ms))
    t20, t0_ = float(np.median(ms)), float(np.median(ms0))
    elem_iters = N * K * iters
    flops = credited_flops_per_element(k, iters) * N * K
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    traffic = load_traffic()

    line = {
        "metric": METRIC,
        "value": elem_iters / (ms_step * 1e-3),
        "unit": "elem-iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Llama3-8B-like up_proj 14336x4096 bf16, group 128, 16 clusters, "
                               "20 Lloyd rounds, Philox seed 0",
                   "n_rows": N, "n_cols": K, "group": g, "n_clusters": k, "iters": iters},
        "ms_per_matrix": t20,
        "lloyd_ms": t20 - t0_,
        "lloyd_elem_iters_per_s": elem_iters / ((t20 - t0_) * 1e-3) if t20 > t0_ else None,
        "lloyd_pct_fp32_peak_credited": (elem_iters * (3 * k + 1) / ((t20 - t0_) * 1e-3) / 1e12
                                         / PEAK_FP32_TFLOPS * 100) if t20 > t0_ else None,
        "ms_iters0": t0_,
        "device_status": status,
        "roofline": {
            "bound": "alu",
            "achieved": achieved,
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_TFLOPS,
            "traffic": traffic,
            "kernel": "any4_rows_kernel<E=%d, waves/row=%d>" % any4.launch_geometry(K),
            "credited_flops_per_element": credited_flops_per_element(k, iters),
            "kernel_ms_mean_hip_events": ms_kernel,
        },
    }
    if not args.no_bookends:
        line["bookends"] = bookends(any4, torch, np, out, N, K, g, k, dev, stream)
        _, c_reg, _, _ = any4.stage_full(w, act, g, k, iters, seed=0)
        line["sorted_lloyd"] = sorted_lloyd(any4, torch, np, w, act, g, k, iters, c_reg, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(m, g, k, iters)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
