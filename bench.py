"""Benchmark of the W4A4 Hadamard-quantized linear path on one MI355X.

One step = every linear of the workload, each as the two library calls of the online path:
qv_hadamard_smooth_quant (rotate + smooth + int4 quantize, HBM-bound) then qv_w4a4_gemm (int4 GEMM
on int8 MFMA with the dequant/GELU epilogue).  The default workload is the 48-block linear stack at
100 frames (M = 137400 token rows, 192 linears per step).  Inputs (seeded VGGT-shaped activations,
packed int4 weights, smoothing factors) are resident in HBM before the timed region; nothing is
skipped inside it.

Prints one JSON line: the effective TOPS of the step (2*M*N*K summed over the linears, divided by
the step time), the GEMM kernel's fraction of the dense INT8 MFMA peak, the rotate-quantize kernel's
fraction of HBM bandwidth, bf16 and int8 hipBLASLt baselines on the same shapes, the CPU oracle
timed per stage on a bounded sample of the same workload, and the W8A8, group-wise and fused-MLP
variants.
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
sys.path.insert(0, ROOT)

METRIC = "W4A4 linear effective TOPS + % INT8 MFMA peak at VGGT shapes"
PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, TOP/s
PEAK_HBM_GBPS = 8000.0    # MI355X HBM3E, GB/s
PROFILE_DIR = os.path.join(ROOT, "profiles")
FLUSH_BYTES = 1 << 30     # scratch written between cold-cache timings (> 256 MB MALL + 8 x 4 MB L2)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10,
                   help="untimed steps first: the GPU clock needs tens of milliseconds of load to ramp up from idle")
    p.add_argument("--workload", default="stack48_100frames")
    p.add_argument("--no-w8a8", dest="w8a8", action="store_false", help="skip the W8A8 line")
    p.add_argument("--group", type=int, default=128,
                   help="group size of the group-wise line (128, 256 or 512; 0 to skip it)")
    p.add_argument("--secondary", default="qkv_8frames",
                   help="a second workload timed the same way after the main one ('' to skip)")
    p.add_argument("--no-mlp", dest="mlp", action="store_false",
                   help="skip the MLP chain line (mlp_24frames, unfused and fused)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (profiling runs)")
    p.add_argument("--no-bf16-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=256,
                   help="rows per linear in the oracle sample (per thread in the all-cores run)")
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


def read_traffic(kernel_tag, src_hash, workload):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if taken on this source and
    this workload."""
    path = os.path.join(PROFILE_DIR, f"{workload}_{kernel_tag}_traffic.json")
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
        step()
        torch.cuda.synchronize()
    th.join()
    return float(sorted(samples)[len(samples) // 2]) if samples else None


def time_steps(step, steps, warmup, torch):
    """Wall time per step of ``steps`` steps after ``warmup`` untimed ones, bracketed by device
    synchronizations (no event inside the timed region)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


class Timer:
    """HIP events on the library's stream around a group of launches; a 1 GiB scratch fill before
    each cold group evicts the L2s and the MALL (it runs before the first event, so it is not
    timed)."""

    def __init__(self, torch, stream, dev):
        self.torch, self.stream = torch, stream
        self.scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.n = 0

    def flush(self):
        self.n += 1
        with self.torch.cuda.stream(self.stream):
            self.scratch.fill_(self.n & 0xFF)

    def __call__(self, fn, cold=False):
        torch = self.torch
        if cold:
            self.flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        fn()
        e1.record(self.stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3


def pct(ts):
    import numpy as np

    q = np.percentile(np.asarray(ts) * 1e6, [10, 50, 90])
    return [round(float(v), 2) for v in q]


def rq_bytes(L, code_bytes_per_row=None):
    """Algorithmic bytes of one rotate-quantize launch: read the rows, write codes and scales."""
    M, K = L.X.shape
    codes = code_bytes_per_row if code_bytes_per_row is not None else K // 2
    scales = 4 * (L.xs.numel() // M)
    return M * K * L.X.element_size() + M * codes + M * scales


def cpu_oracle_baseline(wl, rows, torch):
    """The oracle (plain C, gcc -O2) on a bounded sample of the workload: each stage of the online
    step timed on its own, on one thread and on the host cores this process may use (one slice of
    ``rows`` rows per thread, each slice one call into the C library, which releases Python's lock).
    Per-row rates are scaled to whole workloads (labelled extrapolated)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from bit_ptq_reconstruction_amd import synth
    from bit_ptq_reconstruction_amd.configs import WORKLOADS

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    stage_names = ("rotate_explicit", "rotate_fwht", "quantize_pack", "int_gemm", "dequant_epilogue")
    shapes = {}
    for lin in wl.linears:
        shapes.setdefault((lin.K, lin.N, lin.epi), lin)
    per_row = {}  # (K, N, epi) -> {stage: (s/row at 1 thread, s/row at all threads)}
    total = {"1": 0.0, "all": 0.0}
    ops = {"1": 0.0, "all": 0.0}
    t_start = time.perf_counter()
    with ThreadPoolExecutor(threads) as pool:
        for (K, N, epi), lin in shapes.items():
            X = synth.vggt_activations(rows * threads, K, lin.x_seed, dtype=wl.in_dtype)
            W = synth.weights(N, K, lin.w_seed)
            Xh_all, Wh = oracle.rotate(X, oracle.ROT_FWHT), oracle.rotate(W, oracle.ROT_FWHT)
            s, inv = oracle.smoothing(Xh_all[:rows], Wh, 0.5)
            Wq, ws = oracle.pack_weights(W, s, oracle.ROT_FWHT)  # offline step: not timed
            qw = oracle.unpack_int4(Wq)
            slices = [X[i * rows:(i + 1) * rows] for i in range(threads)]

            def stages(x):
                t = {}
                t0 = time.perf_counter()
                xh = oracle.rotate(x, oracle.ROT_EXPLICIT)
                t["rotate_explicit"] = time.perf_counter() - t0
                t0 = time.perf_counter()
                oracle.rotate(x, oracle.ROT_FWHT)
                t["rotate_fwht"] = time.perf_counter() - t0
                t0 = time.perf_counter()
                q, sa = oracle.quantize_rows(xh, inv, 4)
                xq = oracle.pack_int4(q)
                t["quantize_pack"] = time.perf_counter() - t0
                t0 = time.perf_counter()
                acc = oracle.gemm_int(oracle.unpack_int4(xq), qw)
                t["int_gemm"] = time.perf_counter() - t0
                t0 = time.perf_counter()
                oracle.dequant(acc, sa, ws, None, epi)
                t["dequant_epilogue"] = time.perf_counter() - t0
                return t

            one = stages(slices[0])
            # all threads at once, stage by stage (a barrier per stage keeps the stages apart)
            many = {k: 0.0 for k in stage_names}
            xh_s = [None] * threads
            q_s = [None] * threads
            acc_s = [None] * threads

            def run_stage(name, fn):
                t0 = time.perf_counter()
                list(pool.map(fn, range(threads)))
                many[name] = time.perf_counter() - t0

            def st_rot(i):
                xh_s[i] = oracle.rotate(slices[i], oracle.ROT_EXPLICIT)

            def st_fwht(i):
                oracle.rotate(slices[i], oracle.ROT_FWHT)

            def st_quant(i):
                q, sa = oracle.quantize_rows(xh_s[i], inv, 4)
                q_s[i] = (oracle.pack_int4(q), sa)

            def st_gemm(i):
                acc_s[i] = oracle.gemm_int(oracle.unpack_int4(q_s[i][0]), qw)

            def st_deq(i):
                oracle.dequant(acc_s[i], q_s[i][1], ws, None, epi)

            for name, fn in zip(stage_names, (st_rot, st_fwht, st_quant, st_gemm, st_deq)):
                run_stage(name, fn)
            per_row[(K, N, epi)] = {k: (one[k] / rows, many[k] / (rows * threads)) for k in stage_names}
            n_lin = sum(1 for l in wl.linears if (l.K, l.N, l.epi) == (K, N, epi))
            online = ("rotate_explicit", "quantize_pack", "int_gemm", "dequant_epilogue")
            total["1"] += n_lin * sum(one[k] for k in online)
            total["all"] += n_lin * sum(many[k] for k in online)
            ops["1"] += n_lin * 2.0 * rows * N * K
            ops["all"] += n_lin * 2.0 * rows * threads * N * K
            del X, Xh_all, Wh
    wall = time.perf_counter() - t_start

    def linear_seconds(lin, M, which):
        r = per_row[(lin.K, lin.N, lin.epi)]
        return {k: M * r[k][which] for k in stage_names}

    extrap = {}
    for name in ("mlp_24frames", "block_32frames", "stack48_100frames"):
        w = WORKLOADS[name]
        if not all((l.K, l.N, l.epi) in per_row for l in w.linears):
            continue
        out = {}
        for which, label in ((0, "1_thread_s"), (1, f"{threads}_threads_s")):
            st = {k: 0.0 for k in stage_names}
            for lin in w.linears:
                for k, v in linear_seconds(lin, w.M, which).items():
                    st[k] += v * w.blocks
            out[label] = {k: round(v, 2) for k, v in st.items()}
            out[label]["online_step_explicit_rotation"] = round(
                sum(st[k] for k in ("rotate_explicit", "quantize_pack", "int_gemm", "dequant_epilogue")), 2)
        extrap[name] = out

    return {
        "value": round(ops["1"] / total["1"] / 1e12, 7), "unit": "TOPS", "cores": 1, "kind": "oracle",
        "sample": (f"{rows} rows of each distinct linear shape of {wl.name} (online step: explicit-matrix fp64 "
                   f"rotation, fp32 quantization + packing, int64 triple-loop GEMM, fp64 dequant/GELU), single "
                   f"thread, {total['1']:.1f} s of oracle time"),
        "all_cores": {"value": round(ops["all"] / total["all"] / 1e12, 7), "unit": "TOPS", "cores": threads,
                      "sample": f"{rows} rows per thread, {rows * threads} rows per shape, {total['all']:.1f} s"},
        "stages_us_per_row": {f"K{K}_N{N}{'_gelu' if epi else ''}": {
            k: {"1_thread": round(1e6 * v[0], 3), f"{threads}_threads": round(1e6 * v[1], 3)} for k, v in st.items()}
            for (K, N, epi), st in per_row.items()},
        "extrapolated_seconds": extrap,
        "extrapolation": "per-row stage times of the sample scaled by the workload's rows x blocks (not measured)",
        "host_cpus": os.cpu_count(), "wall_s": round(wall, 1),
    }


def main():
    args = parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark times the path on one GPU (token rows shard across GPUs "
                                   "with no exchange); --gpus must be 1", "requested_gpus": args.gpus}))
        sys.exit(2)

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
    print(f"bench: building {wl.name} (M={M}, {wl.blocks} block(s))", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- resident inputs and weights
    # A multi-block stack shares the per-shape code/scale/output buffers across blocks (each step
    # overwrites them in order); activations and packed weights are per layer.
    layers = workload.build(qv, wl, dev, share_outputs=wl.blocks > 1)
    timer = Timer(torch, stream, dev)

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

    print("bench: timed steps", file=sys.stderr, flush=True)
    t_step = time_steps(step, args.steps, args.warmup, torch)
    ms_per_step = 1e3 * t_step
    ops_per_step = sum(2.0 * M * L.lin.N * L.lin.K for L in layers)
    value = ops_per_step / t_step / 1e12
    sclk = sample_clock(step, torch)

    # ---------------------------------------------------------------- per-kernel times (HIP events)
    # Kernel durations in the context of the step: instrumented steps, after the timed ones, record
    # an event before and after every launch on the library's stream, so each rotate-quantize runs
    # after the previous layer's GEMM (its input cold in HBM, its codes read by the next GEMM) exactly
    # as inside a timed step.  An event adds a dispatch latency of a few microseconds to the interval
    # it opens, so these durations are slight upper bounds; the rocprofv3 kernel trace of the same
    # command gives the kernels' own durations.  The per-linear GEMM figures also time back-to-back
    # launches of one linear across the blocks, with no event in between.
    print("bench: per-kernel timing", file=sys.stderr, flush=True)
    reps = max(3, 60 // wl.blocks)
    launch_k1 = lambda L: qv.qv_hadamard_smooth_quant(L.X, L.inv, L.Xq, L.xs, stream)
    launch_k2 = lambda L: qv.qv_w4a4_gemm(L.Xq, L.xs, L.Wq, L.ws, None, L.Y, L.lin.epi, stream)

    inst_steps = max(2, 96 // len(layers))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(inst_steps * len(layers))]
    step()
    for i, e in enumerate(evs):
        L = layers[i % len(layers)]
        e[0].record(stream)
        launch_k1(L)
        e[1].record(stream)
        launch_k2(L)
        e[2].record(stream)
    torch.cuda.synchronize()
    k1_ts, k2_ts = {}, {}
    for i, e in enumerate(evs):
        name = layers[i % len(layers)].lin.name
        k1_ts.setdefault(name, []).append(e[0].elapsed_time(e[1]) * 1e-3)
        k2_ts.setdefault(name, []).append(e[1].elapsed_time(e[2]) * 1e-3)
    n_launch = len(evs)
    k1_t = sum(sum(v) for v in k1_ts.values()) / n_launch
    k2_t = sum(sum(v) for v in k2_ts.values()) / n_launch
    k1_bytes = sum(rq_bytes(L) for L in layers) / len(layers)
    k2_ops = ops_per_step / len(layers)
    k2_tops = k2_ops / k2_t / 1e12
    k1_gbps = k1_bytes / k1_t / 1e9

    kernels = {}
    for lin in wl.linears:
        group = [L for L in layers if L.lin.name == lin.name]
        g = [timer(lambda: [launch_k2(L) for L in group]) / len(group) for _ in range(reps)]
        r1, r2 = k1_ts[lin.name], k2_ts[lin.name]
        rs, gs = sum(r1) / len(r1), sum(r2) / len(r2)
        gb = sum(g) / len(g)
        b1 = rq_bytes(group[0])
        ops = 2.0 * M * lin.N * lin.K
        kernels[lin.name] = {"K": lin.K, "N": lin.N, "launches": len(r1),
                             "rotate_quant_us": round(1e6 * rs, 2), "rotate_quant_us_p10_p50_p90": pct(r1),
                             "rotate_quant_GBps": round(b1 / rs / 1e9, 1),
                             "rotate_quant_frac": round(b1 / rs / 1e9 / PEAK_HBM_GBPS, 4),
                             "gemm_us": round(1e6 * gs, 2), "gemm_us_p10_p50_p90": pct(r2),
                             "gemm_TOPS": round(ops / gs / 1e12, 1), "gemm_frac": round(ops / gs / 1e12 / PEAK_INT8_TOPS, 4),
                             "gemm_us_back_to_back": round(1e6 * gb, 2),
                             "gemm_TOPS_back_to_back": round(ops / gb / 1e12, 1)}
    wq_bytes = sum(L.Wq.numel() + 4 * L.ws.numel() for L in layers)
    bf16_w_bytes = sum(2 * L.lin.N * L.lin.K for L in layers)

    gemm_hash = kernel_source_hash(["w4a4_gemm.hip", "rq_mfma.h", "fwht_regs.h"])
    rq_hash = kernel_source_hash(["rotate_quant.hip", "rq_mfma.h", "fwht_regs.h"])
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int4", "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "M": M, "blocks": wl.blocks,
                   "linears_per_block": [f"{l.name} {l.K}->{l.N}{' +GELU' if l.epi == EPI_GELU else ''}"
                                         for l in wl.linears],
                   "in_dtype": wl.in_dtype, "out_dtype": wl.out_dtype, "hadamard": "K (1024 or 4096)",
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "w4a4_gemm", "bound": "mfma", "achieved": round(k2_tops, 2),
                     "peak": PEAK_INT8_TOPS, "unit": "TOP/s", "frac": round(k2_tops / PEAK_INT8_TOPS, 4),
                     "traffic": read_traffic("w4a4_gemm", gemm_hash, wl.name),
                     "avg_launch_us": round(1e6 * k2_t, 3), "ops_per_launch": k2_ops,
                     "frac_at_sampled_clock": (round(k2_tops / (PEAK_INT8_TOPS * sclk / 2400.0), 4)
                                               if sclk else None)},
        "rotate_quant_roofline": {"kernel": "rotate_quant", "bound": "hbm", "achieved": round(k1_gbps, 1),
                                  "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(k1_gbps / PEAK_HBM_GBPS, 4),
                                  "traffic": read_traffic("rotate_quant", rq_hash, wl.name),
                                  "avg_launch_us": round(1e6 * k1_t, 3), "bytes_per_launch": k1_bytes},
        "kernels": kernels,
        "rotate_quant_share_of_linear_time": round(k1_t / (k1_t + k2_t), 4),
        "kernel_timing": (f"HIP events before and after each launch of {inst_steps} instrumented steps "
                          f"({n_launch} launches of each kernel) after the timed ones; 'gemm_us_back_to_back': "
                          f"events around {reps} groups of one linear's launches across the blocks"),
        "gfx_clock_MHz_under_load": sclk,
        "weights_resident": {"int4_bytes_with_scales": wq_bytes, "bf16_bytes": bf16_w_bytes,
                             "ratio": round(bf16_w_bytes / wq_bytes, 3)},
        "gemm_only_TOPS": round(k2_tops, 2),
        "source_hash": {"w4a4_gemm": gemm_hash, "rotate_quant": rq_hash},
    }

    # ---------------------------------------------------------------- bf16 / int8 baselines (hipBLASLt)
    if not args.no_bf16_baseline:
        print("bench: hipBLASLt baselines", file=sys.stderr, flush=True)
        base = []
        for lin in wl.linears:
            Xb = synth.vggt_activations_torch(M, lin.K, 0, torch.bfloat16, dev)
            Wb = synth.weights_torch(lin.N, lin.K, 1, dev).to(torch.bfloat16)
            base.append((Xb, Wb, lin.epi))

        def bstep():
            for _ in range(wl.blocks):
                for Xb, Wb, epi in base:
                    y = torch.nn.functional.linear(Xb, Wb)
                    if epi == EPI_GELU:
                        y = torch.nn.functional.gelu(y)
        bt = time_steps(bstep, args.steps, args.warmup, torch)
        result["bf16_baseline"] = {"what": "torch.nn.functional.linear (+gelu) in bf16, same shapes",
                                   "ms_per_step": round(1e3 * bt, 4), "TFLOPS": round(ops_per_step / bt / 1e12, 2),
                                   "w4a4_speedup": round(bt / t_step, 3)}
        del base

        # hipBLASLt's int8 GEMM on the same shapes (int8 operands, int32 output, no scales): the
        # vendor library's contraction alone, against this GEMM with its unpack and epilogue.
        i8 = []
        for lin in wl.linears:
            g = torch.Generator(device=dev).manual_seed(lin.x_seed)
            A = torch.randint(-8, 8, (M, lin.K), dtype=torch.int8, device=dev, generator=g)
            Bt = torch.randint(-8, 8, (lin.N, lin.K), dtype=torch.int8, device=dev, generator=g)
            i8.append((A, Bt.t()))

        def istep():
            for _ in range(wl.blocks):
                for A, B in i8:
                    torch._int_mm(A, B)
        try:
            it = time_steps(istep, args.steps, args.warmup, torch)
            result["int8_baseline"] = {"what": "torch._int_mm (hipBLASLt int8 x int8 -> int32, no scales), same shapes",
                                       "TOPS": round(ops_per_step / it / 1e12, 2),
                                       "w4a4_gemm_speedup": round(k2_tops / (ops_per_step / it / 1e12), 3)}
        except RuntimeError as e:  # an int8 GEMM the installed torch does not offer on this device
            result["int8_baseline"] = {"what": "torch._int_mm", "error": str(e)[:200]}
        del i8
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- CPU oracle on a bounded sample
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_oracle_baseline(wl, args.cpu_rows, torch)

    # ---------------------------------------------------------------- W8A8 on the same workload
    # The variants reuse the activation tensors of the main workload (same seeded draws).
    if args.w8a8:
        print("bench: W8A8 line", file=sys.stderr, flush=True)
        layers8 = workload.build(qv, wl, dev, share_outputs=wl.blocks > 1, bits=8, inputs=layers)

        def step8():
            for L in layers8:
                workload.run_linear(qv, L, stream)

        w8 = time_steps(step8, args.steps, args.warmup, torch)
        g8 = sum(timer(lambda: [qv.qv_w8a8_gemm(L.Xq, L.xs, L.Wq, L.ws, None, L.Y, L.lin.epi, stream)
                                for L in layers8]) for _ in range(reps)) / (reps * len(layers8))
        q8 = sum(timer(lambda: [qv.qv_hadamard_smooth_quant8(L.X, L.inv, L.Xq, L.xs, stream) for L in layers8],
                       cold=True) for _ in range(reps)) / (reps * len(layers8))
        b8 = sum(rq_bytes(L, L.lin.K) for L in layers8) / len(layers8)
        result["w8a8"] = {"what": "the same workload with 8-bit codes (scale absmax/127, int8 MFMA without unpacking)",
                          "value": round(ops_per_step / w8 / 1e12, 2), "unit": "TOPS", "ms_per_step": round(1e3 * w8, 4),
                          "gemm_TOPS": round(k2_ops / g8 / 1e12, 2), "gemm_frac": round(k2_ops / g8 / 1e12 / PEAK_INT8_TOPS, 4),
                          "rotate_quant_GBps": round(b8 / q8 / 1e9, 1)}
        del layers8
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- group-wise scales, same workload
    if args.group:
        print("bench: group-wise line", file=sys.stderr, flush=True)
        G = args.group
        layersg = workload.build(qv, wl, dev, share_outputs=wl.blocks > 1, group=G, inputs=layers)

        def stepg():
            for L in layersg:
                workload.run_linear(qv, L, stream)

        wg = time_steps(stepg, args.steps, args.warmup, torch)
        gg = sum(timer(lambda: [qv.qv_w4a4_gemm_grouped(L.Xq, L.xs, L.Wq, L.ws, None, L.Y, G, L.lin.epi, stream)
                                for L in layersg]) for _ in range(reps)) / (reps * len(layersg))
        qg = sum(timer(lambda: [qv.qv_hadamard_smooth_quant_grouped(L.X, L.inv, G, L.Xq, L.xs, stream)
                                for L in layersg], cold=True) for _ in range(reps)) / (reps * len(layersg))
        bg = sum(rq_bytes(L) for L in layersg) / len(layersg)
        result["grouped"] = {"what": f"the same workload with one scale per row and group of {G} channels "
                                     "(group-wise dequantization in the GEMM's K loop)",
                             "group": G, "value": round(ops_per_step / wg / 1e12, 2), "unit": "TOPS",
                             "ms_per_step": round(1e3 * wg, 4), "gemm_TOPS": round(k2_ops / gg / 1e12, 2),
                             "gemm_frac": round(k2_ops / gg / 1e12 / PEAK_INT8_TOPS, 4),
                             "rotate_quant_GBps": round(bg / qg / 1e9, 1)}
        del layersg
        torch.cuda.empty_cache()

    del layers
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- secondary workload
    if args.secondary and args.secondary != wl.name:
        print(f"bench: secondary workload {args.secondary}", file=sys.stderr, flush=True)
        wl2 = WORKLOADS[args.secondary]
        layers2 = workload.build(qv, wl2, dev, share_outputs=wl2.blocks > 1)

        def step2():
            for L in layers2:
                workload.run_linear(qv, L, stream)

        w2 = time_steps(step2, max(args.steps, 50), max(args.warmup, 20), torch)
        ops2 = sum(2.0 * wl2.M * L.lin.N * L.lin.K for L in layers2)
        result["secondary"] = {"workload": wl2.name, "description": wl2.description,
                               "value": round(ops2 / w2 / 1e12, 2), "unit": "TOPS", "ms_per_step": round(1e3 * w2, 4)}
        del layers2
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- the MLP chain (fc1 -> GELU -> fc2)
    if args.mlp:
        print("bench: MLP chain mlp_24frames", file=sys.stderr, flush=True)
        wl3 = WORKLOADS["mlp_24frames"]
        layers3 = workload.build(qv, wl3, dev)

        def step3():
            for L in layers3:
                workload.run_linear(qv, L, stream)

        ops3 = sum(2.0 * wl3.M * L.lin.N * L.lin.K for L in layers3)
        L1, L2 = layers3
        work3 = torch.empty((qv.qv_w4a4_gemm_requant_workspace_size(wl3.M),), dtype=torch.uint8, device=dev)

        def step3_fused():
            qv.qv_hadamard_smooth_quant(L1.X, L1.inv, L1.Xq, L1.xs, stream)
            qv.qv_w4a4_gemm_requant(L1.Xq, L1.xs, L1.Wq, L1.ws, None, L1.Y, L2.inv, L2.Xq, L2.xs, work3,
                                    L1.lin.epi, stream)
            qv.qv_w4a4_gemm(L2.Xq, L2.xs, L2.Wq, L2.ws, None, L2.Y, L2.lin.epi, stream)

        # the two forms alternate, so that clock and thermal drift affect both alike
        w3u, w3f = [], []
        for _ in range(3):
            w3u.append(time_steps(step3, max(args.steps, 50), max(args.warmup, 20), torch))
            w3f.append(time_steps(step3_fused, max(args.steps, 50), max(args.warmup, 20), torch))
        w3, w3fm = min(w3u), min(w3f)
        g1 = sum(timer(lambda: qv.qv_w4a4_gemm(L1.Xq, L1.xs, L1.Wq, L1.ws, None, L1.Y, L1.lin.epi, stream))
                 for _ in range(reps)) / reps
        q2 = sum(timer(lambda: qv.qv_hadamard_smooth_quant(L1.Y, L2.inv, L2.Xq, L2.xs, stream), cold=True)
                 for _ in range(reps)) / reps
        gf = sum(timer(lambda: qv.qv_w4a4_gemm_requant(L1.Xq, L1.xs, L1.Wq, L1.ws, None, L1.Y, L2.inv, L2.Xq, L2.xs,
                                                        work3, L1.lin.epi, stream)) for _ in range(reps)) / reps
        result["mlp_chain"] = {
            "workload": wl3.name, "description": wl3.description,
            "unfused": {"value": round(ops3 / w3 / 1e12, 2), "unit": "TOPS", "ms_per_step": round(1e3 * w3, 4),
                        "what": "fc1 GEMM writes GELU(y) in bf16; fc2's rotate-quantize reads it back from HBM",
                        "fc1_gemm_us": round(1e6 * g1, 2), "fc2_rotate_quant_us": round(1e6 * q2, 2)},
            "fused": {"value": round(ops3 / w3fm / 1e12, 2), "unit": "TOPS", "ms_per_step": round(1e3 * w3fm, 4),
                      "what": "fc1 GEMM also rotates, smooths and quantizes each finished 128-row stripe of its "
                              "output for fc2 (qv_w4a4_gemm_requant)",
                      "fc1_gemm_requant_us": round(1e6 * gf, 2)},
            "timing": "best of 3 alternating runs of each form",
            "faster": "fused" if w3fm < w3 else "unfused"}
        del layers3, work3
        torch.cuda.empty_cache()

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
