"""Benchmark of the W4A4 Hadamard-quantized linear path on one MI355X.

One step = every linear of the workload, each as the two library calls of the online path:
qv_hadamard_smooth_quant (rotate + smooth + int4 quantize, HBM-bound) then qv_w4a4_gemm (int4 GEMM
on int8 MFMA with the dequant/GELU epilogue).  Inputs (seeded VGGT-shaped activations, packed int4
weights, smoothing factors) are resident in HBM before the timed region; nothing is skipped inside it.

Prints one JSON line: the effective TOPS of the step (2*M*N*K summed over the linears, divided by
the step time), the GEMM kernel's fraction of the dense INT8 MFMA peak, the rotate-quantize kernel's
fraction of HBM bandwidth, a bf16 hipBLASLt baseline on the same shapes, and the CPU oracle timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 linear effective TOPS + % INT8 MFMA peak at VGGT shapes"
PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, TOP/s
PEAK_HBM_GBPS = 8000.0    # MI355X HBM3E, GB/s
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=50,
                   help="untimed steps first: the GPU clock needs tens of milliseconds of load to ramp up from idle")
    p.add_argument("--workload", default="block_32frames")
    p.add_argument("--no-w8a8", dest="w8a8", action="store_false", help="skip the W8A8 line")
    p.add_argument("--group", type=int, default=128,
                   help="group size of the group-wise line (128, 256 or 512; 0 to skip it)")
    p.add_argument("--secondary", default="qkv_8frames",
                   help="a second workload timed the same way after the main one ('' to skip)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (profiling runs)")
    p.add_argument("--no-bf16-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=384, help="rows per linear in the oracle sample (about 10 s of host work)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="before the timed steps, copy this many MiB device-to-device once (a plain copy "
                        "of known size that calibrates the HBM byte counters of a profiling run)")
    return p.parse_args()


def kernel_source_hash(names):
    """Hash of the kernel sources' code: comments and whitespace are dropped first, so that a
    counter summary stays matched to its kernels until their code changes."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_ptq_reconstruction_amd", "csrc", n), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag, src_hash):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if taken on this source."""
    path = os.path.join(PROFILE_DIR, f"{kernel_tag}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != src_hash:
        return None
    return d.get("bytes_per_launch")


def sample_clock(step, torch):
    """Graphics clock while the steps keep running (after the timed region, so the sampling does
    not share it): the median of a few reads of the current DPM level's frequency in sysfs
    (pp_dpm_sclk, the line marked '*'); None where that file is not readable."""
    import glob
    import threading

    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not files:
        return None

    def read_mhz():
        for f in files:
            try:
                for line in open(f):
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
            except (OSError, ValueError, IndexError):
                continue
        return None

    samples = []

    def sampler():
        time.sleep(0.2)  # let the steps reach their steady clock
        for _ in range(5):
            v = read_mhz()
            if v is not None:
                samples.append(v)
            time.sleep(0.05)

    th = threading.Thread(target=sampler)
    th.start()
    while th.is_alive():
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    th.join()
    return float(sorted(samples)[len(samples) // 2]) if samples else None


def main():
    args = parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark times the path on one GPU (token rows shard across GPUs "
                                   "with no exchange); --gpus must be 1", "requested_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import bit_ptq_reconstruction_amd as qv
    from bit_ptq_reconstruction_amd import synth
    from bit_ptq_reconstruction_amd import workload
    from bit_ptq_reconstruction_amd.configs import EPI_GELU, WORKLOADS

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qv.lib()
    M = wl.M
    stream = torch.cuda.current_stream()

    # ---------------------------------------------------------------- resident inputs and weights
    # A multi-block stack shares the per-shape code/scale/output buffers across blocks (each step
    # overwrites them in order); activations and packed weights are per layer.
    layers = workload.build(qv, wl, dev, share_outputs=wl.blocks > 1)

    if args.copy_probe_mib > 0:
        nbytes = args.copy_probe_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        for L in layers:
            workload.run_linear(qv, L, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps

    ops_per_step = sum(2.0 * M * L.lin.N * L.lin.K for L in layers)
    value = ops_per_step / (wall / args.steps) / 1e12
    sclk = sample_clock(step, torch)

    # ---------------------------------------------------------------- per-kernel times (HIP events)
    # Events on the library's stream bracket back-to-back launches with no event between them (an
    # event between two kernels adds a dispatch gap of a few microseconds to the pair it separates).
    #   * kernel averages: every layer's launch of that kernel in step order, repeated, so the
    #     rotate-quantize inputs are as cold as in a step (the layers' inputs exceed the MALL);
    #   * per-layer GEMM: repeated launches of that layer's GEMM (compute-bound, cache-insensitive);
    #   * per-layer rotate-quantize: an event pair around each launch of the step-order loop, so
    #     these include the dispatch gap (reported, not used for the roofline).
    reps = max(3, args.steps // (10 * wl.blocks))
    launch_k1 = lambda L: qv.qv_hadamard_smooth_quant(L.X, L.inv, L.Xq, L.xs, stream)
    launch_k2 = lambda L: qv.qv_w4a4_gemm(L.Xq, L.xs, L.Wq, L.ws, None, L.Y, L.lin.epi, stream)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    def all_layers(launch):
        for _ in range(reps):
            for L in layers:
                launch(L)

    step()
    k1_t = timed(lambda: all_layers(launch_k1)) / (reps * len(layers))
    k2_t = timed(lambda: all_layers(launch_k2)) / (reps * len(layers))
    k1_bytes = sum(M * L.lin.K * L.X.element_size() + M * (L.lin.K // 2) + 4 * M for L in layers) / len(layers)
    k2_ops = ops_per_step / len(layers)
    k2_tops = k2_ops / k2_t / 1e12
    k1_gbps = k1_bytes / k1_t / 1e9

    pairs = []
    for _ in range(reps):
        for L in layers[:len(wl.linears)]:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            launch_k1(L)
            e[1].record(stream)
            launch_k2(L)
            pairs.append((L.lin.name, e))
    torch.cuda.synchronize()
    k1_layer = {}
    for name, e in pairs:
        k1_layer.setdefault(name, []).append(e[0].elapsed_time(e[1]) * 1e-3)

    def pct(ts):
        q = np.percentile(np.asarray(ts) * 1e6, [10, 50, 90])
        return [round(float(v), 2) for v in q]

    kernels = {}
    for L in layers[:len(wl.linears)]:
        lin = L.lin
        g = []
        for _ in range(reps):
            g.append(timed(lambda: launch_k2(L)))
        b1 = M * lin.K * L.X.element_size() + M * (lin.K // 2) + 4 * M
        t1 = sum(k1_layer[lin.name]) / len(k1_layer[lin.name])
        kernels[lin.name] = {"K": lin.K, "N": lin.N,
                             "rotate_quant_us_with_event_gap": round(1e6 * t1, 2),
                             "rotate_quant_us_p10_p50_p90": pct(k1_layer[lin.name]),
                             "rotate_quant_GBps_with_event_gap": round(b1 / t1 / 1e9, 1),
                             "gemm_us": round(1e6 * sum(g) / len(g), 2), "gemm_us_p10_p50_p90": pct(g),
                             "gemm_TOPS": round(2.0 * M * lin.N * lin.K / (sum(g) / len(g)) / 1e12, 1)}
    wq_bytes = sum(L.Wq.numel() + 4 * L.ws.numel() for L in layers)
    bf16_w_bytes = sum(2 * L.lin.N * L.lin.K for L in layers)

    gemm_hash = kernel_source_hash(["w4a4_gemm.hip"])
    rq_hash = kernel_source_hash(["rotate_quant.hip", "fwht_regs.h"])
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int4", "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "M": M, "blocks": wl.blocks,
                   "linears": [f"{l.name} {l.K}->{l.N}{' +GELU' if l.epi == EPI_GELU else ''}" for l in wl.linears],
                   "in_dtype": wl.in_dtype, "out_dtype": wl.out_dtype, "hadamard": "K (1024 or 4096)",
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "w4a4_gemm", "bound": "mfma", "achieved": round(k2_tops, 2),
                     "peak": PEAK_INT8_TOPS, "unit": "TOP/s", "frac": round(k2_tops / PEAK_INT8_TOPS, 4),
                     "traffic": read_traffic("w4a4_gemm", gemm_hash),
                     "avg_launch_us": round(1e6 * k2_t, 3), "ops_per_launch": k2_ops,
                     "frac_at_sampled_clock": (round(k2_tops / (PEAK_INT8_TOPS * sclk / 2400.0), 4)
                                               if sclk else None)},
        "rotate_quant_roofline": {"kernel": "rotate_quant", "bound": "hbm", "achieved": round(k1_gbps, 1),
                                  "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(k1_gbps / PEAK_HBM_GBPS, 4),
                                  "traffic": read_traffic("rotate_quant", rq_hash),
                                  "avg_launch_us": round(1e6 * k1_t, 3),
                                  "bytes_per_launch": k1_bytes},
        "kernels": kernels,
        "rotate_quant_share_of_linear_time": round(k1_t / (k1_t + k2_t), 4),
        "kernel_timing": f"HIP events around {reps} back-to-back repetitions of every layer's launch of the kernel",
        "gfx_clock_MHz_under_load": sclk,
        "weights_resident": {"int4_bytes_with_scales": wq_bytes, "bf16_bytes": bf16_w_bytes,
                             "ratio": round(bf16_w_bytes / wq_bytes, 3)},
        "gemm_only_TOPS": round(k2_tops, 2),
        "source_hash": {"w4a4_gemm": gemm_hash, "rotate_quant": rq_hash},
    }

    # ---------------------------------------------------------------- bf16 baseline (hipBLASLt)
    if not args.no_bf16_baseline:
        base = []
        for L in layers[:len(wl.linears)]:
            lin = L.lin
            Xb = synth.vggt_activations_torch(M, lin.K, 0, torch.bfloat16, dev)
            Wb = synth.weights_torch(lin.N, lin.K, 1, dev).to(torch.bfloat16)
            base.append((Xb, Wb, lin.epi))

        def bstep():
            for Xb, Wb, epi in base:
                y = torch.nn.functional.linear(Xb, Wb)
                if epi == EPI_GELU:
                    y = torch.nn.functional.gelu(y)
        for _ in range(args.warmup):
            bstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            for _ in range(wl.blocks):
                bstep()
        torch.cuda.synchronize()
        bt = (time.perf_counter() - t0) / args.steps
        result["bf16_baseline"] = {"what": "torch.nn.functional.linear (+gelu) in bf16, same shapes",
                                   "ms_per_step": round(1e3 * bt, 4), "TFLOPS": round(ops_per_step / bt / 1e12, 2),
                                   "w4a4_speedup": round(bt / (wall / args.steps), 3)}
        del base

        # hipBLASLt's int8 GEMM on the same shapes (int8 operands, int32 output, no scales): the
        # vendor library's contraction alone, against this GEMM with its unpack and epilogue.
        i8 = []
        for L in layers[:len(wl.linears)]:
            lin = L.lin
            g = torch.Generator(device=dev).manual_seed(lin.x_seed)
            A = torch.randint(-8, 8, (M, lin.K), dtype=torch.int8, device=dev, generator=g)
            Bt = torch.randint(-8, 8, (lin.N, lin.K), dtype=torch.int8, device=dev, generator=g)
            i8.append((A, Bt.t()))

        def istep():
            for A, B in i8:
                torch._int_mm(A, B)
        try:
            for _ in range(args.warmup):
                istep()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                for _ in range(wl.blocks):
                    istep()
            torch.cuda.synchronize()
            it = (time.perf_counter() - t0) / args.steps
            result["int8_baseline"] = {"what": "torch._int_mm (hipBLASLt int8 x int8 -> int32, no scales), same shapes",
                                       "TOPS": round(ops_per_step / it / 1e12, 2),
                                       "w4a4_gemm_speedup": round(k2_tops / (ops_per_step / it / 1e12), 3)}
        except RuntimeError as e:  # an int8 GEMM the installed torch does not offer on this device
            result["int8_baseline"] = {"what": "torch._int_mm", "error": str(e)[:200]}
        del i8

    # ---------------------------------------------------------------- CPU oracle on a bounded sample
    if not args.no_cpu_baseline:
        import oracle

        S = min(args.cpu_rows, M)
        t_cpu, ops_cpu = 0.0, 0.0
        packed = []
        for lin in wl.linears:
            X = synth.vggt_activations(S, lin.K, lin.x_seed, dtype=wl.in_dtype)
            W = synth.weights(lin.N, lin.K, lin.w_seed)
            Xh, Wh = oracle.rotate(X, oracle.ROT_FWHT), oracle.rotate(W, oracle.ROT_FWHT)
            s, inv = oracle.smoothing(Xh, Wh, 0.5)
            Wq, ws = oracle.pack_weights(W, s, oracle.ROT_FWHT)  # offline step: outside the timing
            packed.append((inv, Wq, ws))
            t0 = time.perf_counter()
            oracle.w4a4_linear(X, inv, Wq, ws, None, lin.epi, oracle.ROT_EXPLICIT)
            t_cpu += time.perf_counter() - t0
            ops_cpu += 2.0 * S * lin.N * lin.K
        result["cpu_baseline"] = {
            "value": round(ops_cpu / t_cpu / 1e12, 6), "unit": "TOPS", "cores": 1, "kind": "oracle",
            "sample": f"{S} rows of each of the {len(wl.linears)} linears of one block (online step only: "
                      f"explicit-matrix fp64 rotation, fp32 quantization, int64 triple-loop GEMM, fp64 "
                      f"dequant/GELU), single thread, {t_cpu:.1f} s",
            "host_cpus": os.cpu_count()}

        # The same oracle on the host cores this process may use (at most 16, one GPU's share of
        # the host): one slice of S rows per thread.  Each slice is a single call into the oracle's
        # C library, which runs with Python's lock released, so the threads compute in parallel.
        from concurrent.futures import ThreadPoolExecutor

        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        t_all, ops_all = 0.0, 0.0
        with ThreadPoolExecutor(threads) as pool:
            for lin, (inv, Wq, ws) in zip(wl.linears, packed):
                X = synth.vggt_activations(S * threads, lin.K, lin.x_seed, dtype=wl.in_dtype)
                slices = [X[i * S:(i + 1) * S] for i in range(threads)]
                t0 = time.perf_counter()
                list(pool.map(lambda x: oracle.w4a4_linear(x, inv, Wq, ws, None, lin.epi, oracle.ROT_EXPLICIT),
                              slices))
                t_all += time.perf_counter() - t0
                ops_all += 2.0 * S * threads * lin.N * lin.K
        result["cpu_baseline"]["all_cores"] = {
            "value": round(ops_all / t_all / 1e12, 6), "unit": "TOPS", "cores": threads,
            "sample": f"{S * threads} rows of each linear, {S} per thread, {t_all:.1f} s"}

    # ---------------------------------------------------------------- secondary workload
    if args.secondary and args.secondary != wl.name:
        del layers
        torch.cuda.empty_cache()
        wl2 = WORKLOADS[args.secondary]
        layers2 = workload.build(qv, wl2, dev, share_outputs=wl2.blocks > 1)

        def step2():
            for L in layers2:
                workload.run_linear(qv, L, stream)

        for _ in range(args.warmup):
            step2()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step2()
        torch.cuda.synchronize()
        w2 = (time.perf_counter() - t0) / args.steps
        ops2 = sum(2.0 * wl2.M * L.lin.N * L.lin.K for L in layers2)
        result["secondary"] = {"workload": wl2.name, "description": wl2.description,
                               "value": round(ops2 / w2 / 1e12, 2), "unit": "TOPS", "ms_per_step": round(1e3 * w2, 4)}
        del layers2

    # ---------------------------------------------------------------- W8A8 on the same workload
    if args.w8a8:
        torch.cuda.empty_cache()
        layers8 = workload.build(qv, wl, dev, share_outputs=wl.blocks > 1, bits=8)

        def step8():
            for L in layers8:
                workload.run_linear(qv, L, stream)

        for _ in range(args.warmup):
            step8()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step8()
        torch.cuda.synchronize()
        w8 = (time.perf_counter() - t0) / args.steps
        g8 = timed(lambda: [qv.qv_w8a8_gemm(L.Xq, L.xs, L.Wq, L.ws, None, L.Y, L.lin.epi, stream)
                            for _ in range(reps) for L in layers8]) / (reps * len(layers8))
        q8 = timed(lambda: [qv.qv_hadamard_smooth_quant8(L.X, L.inv, L.Xq, L.xs, stream)
                            for _ in range(reps) for L in layers8]) / (reps * len(layers8))
        b8 = sum(M * L.lin.K * L.X.element_size() + M * L.lin.K + 4 * M for L in layers8) / len(layers8)
        result["w8a8"] = {"what": "the same workload with 8-bit codes (scale absmax/127, int8 MFMA without unpacking)",
                          "value": round(ops_per_step / w8 / 1e12, 2), "unit": "TOPS", "ms_per_step": round(1e3 * w8, 4),
                          "gemm_TOPS": round(k2_ops / g8 / 1e12, 2), "gemm_frac": round(k2_ops / g8 / 1e12 / PEAK_INT8_TOPS, 4),
                          "rotate_quant_GBps": round(b8 / q8 / 1e9, 1)}
        del layers8

    # ---------------------------------------------------------------- group-wise scales, same workload
    if args.group:
        torch.cuda.empty_cache()
        G = args.group
        layersg = workload.build(qv, wl, dev, share_outputs=wl.blocks > 1, group=G)

        def stepg():
            for L in layersg:
                workload.run_linear(qv, L, stream)

        for _ in range(args.warmup):
            stepg()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            stepg()
        torch.cuda.synchronize()
        wg = (time.perf_counter() - t0) / args.steps
        gg = timed(lambda: [qv.qv_w4a4_gemm_grouped(L.Xq, L.xs, L.Wq, L.ws, None, L.Y, G, L.lin.epi, stream)
                            for _ in range(reps) for L in layersg]) / (reps * len(layersg))
        qg = timed(lambda: [qv.qv_hadamard_smooth_quant_grouped(L.X, L.inv, G, L.Xq, L.xs, stream)
                            for _ in range(reps) for L in layersg]) / (reps * len(layersg))
        bg = sum(M * L.lin.K * L.X.element_size() + M * (L.lin.K // 2) + 4 * M * (L.lin.K // G)
                 for L in layersg) / len(layersg)
        result["grouped"] = {"what": f"the same workload with one scale per row and group of {G} channels "
                                     "(group-wise dequantization in the GEMM's K loop)",
                             "group": G, "value": round(ops_per_step / wg / 1e12, 2), "unit": "TOPS",
                             "ms_per_step": round(1e3 * wg, 4), "gemm_TOPS": round(k2_ops / gg / 1e12, 2),
                             "gemm_frac": round(k2_ops / gg / 1e12 / PEAK_INT8_TOPS, 4),
                             "rotate_quant_GBps": round(bg / qg / 1e9, 1)}
        del layersg

    print(json.dumps(result))


if __name__ == "__main__":
    main()
