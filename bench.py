#!/usr/bin/env python3
"""Benchmark of the masked, LDS-tiled fp32 GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--variant auto] [--workload square4096]

One step is one C = A @ B call through the C ABI on operands already resident
in device memory (4096 x 4096 x 4096, entries normal(0,1), seed 3, by default).
Prints ONE JSON line with the whole-job TFLOP/s (wall clock over K steps
bracketed by device synchronisation), the dominant kernel's roofline position
(its average duration from HIP events on the launch stream) and the fp64 CPU
oracle timed on a bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

PEAK_FP32_TFLOPS = 157.3  # MI355X dense fp32 (matrix and packed vector): 256 CUs x 256 flop/clk x 2.4 GHz
PEAK_16BIT_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak (no sparsity)
METRIC = "fp32 GEMM TFLOP/s at 4096³ on 1 MI355X; % of fp32 peak"
METRIC_16BIT = "{t}-input GEMM (fp32 accumulate) TFLOP/s on 1 MI355X; % of dense {t} peak"
KERNEL_SOURCES = ["gemm_kernels.hpp", "gemm_api.hip", "gemm_default.hip", "default_config.hpp", "launch.hpp",
                  "lds_layout.hpp", "pad_choice.hpp", "layout_gen.cpp",
                  "mfma_shapes.def", "mixed_kernels.hpp", "mixed_shapes.def"]


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update((ROOT / "dense_fp32_tiled_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(variant_name: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = ROOT / "profiles" / f"{variant_name}_{workload}_traffic.txt"
    if not path.exists():
        return None
    fields = {}
    for line in path.read_text().splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--variant", default="auto",
                    help="kernel variant by name (auto, mfma, mfma_direct, valu, ...; see VARIANT_NAMES); with "
                         "--splits, the kernel that computes the slices")
    ap.add_argument("--workload", default="square4096")
    ap.add_argument("--input", default="f32", choices=["f32", "bf16", "f16"],
                    help="element type of A and B: f32 (gemm_f32_ex) or 16-bit with fp32 accumulation "
                         "(gemm_mixed_f32; --variant then names a mixed variant: auto, 256x128, 256x256, ...)")
    ap.add_argument("--cpu-sample-rows", type=int, default=4096,
                    help="rows of C the CPU oracle computes for its baseline and parity check (0 = skip); "
                         "the default covers all of C at 4096^3 (about 2 s on 16 host threads)")
    ap.add_argument("--ablations", default="",
                    help="also time every variant and write one JSON line per variant to this file")
    ap.add_argument("--splits", type=int, default=-1,
                    help="run gemm_f32_splitk with this many K slices (0 = the library's choice) "
                         "instead of gemm_f32_ex; the workspace is allocated before timing")
    ap.add_argument("--cold-cache-mib", type=int, default=0,
                    help="after the timed region, time --steps more launches each preceded by a write of this "
                         "many MiB to a scratch buffer, which evicts A and B from L2 and the 256 MB MALL "
                         "(reported as cold_cache; 0 = skip, the default, so that a kernel trace of the default "
                         "command holds only the warm launches the roofline figure averages)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run one device-to-device copy of this many MiB (a "
                         "reference kernel of known traffic for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args(argv)


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the GEMM kernel is measured on "
              "one GPU's share; multi-GPU sharding is not built.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import dense_fp32_tiled_amd as dft
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    mixed = args.input != "f32"
    names = {v: k for k, v in (dft.MIXED_NAMES if mixed else dft.VARIANT_NAMES).items()}
    variant = names[args.variant]
    if mixed and args.splits >= 0:
        print("--splits applies to fp32 inputs only", file=sys.stderr)
        return 2
    cfg = workloads.CONFIG_BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    a_np, b_np = workloads.config_operands(cfg)
    if mixed:
        # the inputs are the 16-bit values; the oracle multiplies their exact widenings
        (a_bits, a_np), (b_bits, b_np) = workloads.to_16bit(a_np, args.input), workloads.to_16bit(b_np, args.input)
        a = torch.from_numpy(a_bits.view(np.int16)).to(dev)
        b = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    else:
        a = torch.from_numpy(a_np).to(dev)
        b = torch.from_numpy(b_np).to(dev)
    c = torch.empty((cfg.M, cfg.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream
    M, N, K = cfg.M, cfg.N, cfg.K
    pa, pb, pc = a.data_ptr(), b.data_ptr(), c.data_ptr()

    ws, ws_bytes = None, 0
    if args.splits >= 0:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        ws_bytes = dft.gemm_f32_splitk_workspace_bytes(M, N, K, args.splits, cus)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=dev)
        splits_used = args.splits or dft.gemm_f32_splitk_auto_splits(M, N, K, cus)

    input_type = {"bf16": dft.INPUT_BF16, "f16": dft.INPUT_F16}.get(args.input)

    def step(v=variant):
        if mixed:
            st = dft.gemm_mixed_f32(input_type, M, N, K, pa, K, pb, N, pc, N, handle, v)
        elif args.splits >= 0 and v == variant:
            st = dft.gemm_f32_splitk_ex(M, N, K, pa, K, pb, N, pc, N, ws.data_ptr(), ws_bytes, args.splits, handle,
                                        variant)
        else:
            st = dft.gemm_f32_ex(M, N, K, pa, K, pb, N, pc, N, handle, v)
        if st != dft.GEMM_OK:
            raise dft.GemmError(st, "gemm")

    def time_variant(v, steps, warmup):
        for _ in range(warmup):
            step(v)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step(v)
        torch.cuda.synchronize()
        wall_s = (time.perf_counter() - t0) / steps
        # per-launch durations from HIP events recorded on the launch stream
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in ev:
            e0.record(stream)
            step(v)
            e1.record(stream)
        torch.cuda.synchronize()
        durs = sorted(e0.elapsed_time(e1) / 1e3 for e0, e1 in ev)
        return wall_s, sum(durs) / len(durs), durs[len(durs) // 2], durs[0]

    wall_s, kern_avg_s, kern_med_s, kern_min_s = time_variant(variant, args.steps, args.warmup)

    # Cold caches: the timed region above re-reads A and B from L2 / MALL on
    # every launch after the first; here each launch follows a write of a
    # scratch buffer larger than the MALL (not timed; events bracket the GEMM).
    cold = None
    if args.cold_cache_mib > 0:
        scratch = torch.empty(args.cold_cache_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        durs = []
        for _ in range(args.steps):
            scratch.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(variant)
            e1.record(stream)
            torch.cuda.synchronize()
            durs.append(e0.elapsed_time(e1) / 1e3)
        del scratch
        durs.sort()
        cold = {"flush_mib": args.cold_cache_mib, "kernel_ms_avg": sum(durs) / len(durs) * 1e3,
                "kernel_ms_median": durs[len(durs) // 2] * 1e3,
                "tflops_kernel_avg": cfg.flops / (sum(durs) / len(durs)) / 1e12}
    tflops = cfg.flops / wall_s / 1e12
    achieved = cfg.flops / kern_avg_s / 1e12
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if mixed:
        resolved = dft.gemm_mixed_auto_variant(M, N, K, cus) if variant == dft.MIXED_AUTO else variant
        tile = dft.gemm_mixed_tile_config(resolved)
        run_name = f"mixed_{args.input}_{dft.MIXED_NAMES[resolved]}"
    else:
        if args.splits >= 0:
            resolved = dft.gemm_f32_splitk_auto_variant() if variant == dft.VARIANT_AUTO else variant
        elif variant == dft.VARIANT_AUTO:
            resolved = dft.gemm_f32_auto_variant(M, N, K, cus)
        else:
            resolved = variant
        tile = dft.gemm_f32_tile_config(resolved)
        run_name = dft.VARIANT_NAMES[resolved] + (f"+splitk{splits_used}" if args.splits >= 0 else "")
    peak = PEAK_16BIT_TFLOPS if mixed else PEAK_FP32_TFLOPS

    # correctness spot check and CPU baseline: the oracle on a bounded row sample
    cpu_baseline = None
    parity = None
    if args.cpu_sample_rows > 0:
        import oracle

        rows = workloads.sample_indices(cfg.M, min(args.cpu_sample_rows, cfg.M),
                                        cfg.seed + workloads.SAMPLE_SEED_OFFSET)
        threads = oracle.host_threads()
        t0 = time.perf_counter()
        cref, den = oracle.reference(a_np, b_np, rows=rows, threads=threads)
        cpu_s = time.perf_counter() - t0
        cpu_flops = 2.0 * len(rows) * cfg.N * cfg.K
        cpu_baseline = {
            "value": cpu_flops / cpu_s / 1e12,
            "unit": "TFLOP/s",
            "cores": threads,
            "kind": "oracle",
            "sample": (f"the whole product: all {cfg.M} rows of C (all {cfg.N} columns, K={cfg.K}); "
                       f"{cpu_s:.2f} s wall on {threads} threads" if len(rows) == cfg.M else
                       f"{len(rows)} of {cfg.M} rows of C (all {cfg.N} columns, K={cfg.K}), seeded sample; "
                       f"{cpu_s:.2f} s wall on {threads} threads; the whole product would take about "
                       f"{cpu_s * cfg.M / len(rows):.1f} s at this rate (projection)"),
        }
        c_rows = c[torch.from_numpy(rows).to(dev)].cpu().numpy()
        parity = {"rows_checked": int(len(rows)), "max_normalised_error": oracle.normalised_error(c_rows, cref, den)}

    result = {
        "metric": METRIC_16BIT.format(t=args.input) if mixed else METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.input,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: C[{M},{N}] = A[{M},{K}] @ B[{K},{N}], row-major "
                        + (f"{args.input} A and B (fp32 draws rounded to nearest even), fp32 accumulation and C, "
                           if mixed else "fp32, ")
                        + f"entries {'normal(0,1)' if cfg.dist == 'normal' else 'uniform[-1,1)'}, seed {cfg.seed}",
            "M": M, "N": N, "K": K,
            "variant": run_name,
            "tile": f"{tile['bm']}x{tile['bn']}x{tile['bk']}, {tile['threads']} threads, MFMA block "
                    f"{tile['mfma_block']}, {tile['stages']} LDS stages, LDS layout A pad {tile['a_pad']} "
                    f"swizzle {tile['a_swz_unit']}/{tile['a_swz_shift']}/{tile['a_swz_mask']}, B pad "
                    f"{tile['b_pad']} swizzle {tile['b_swz_unit']}/{tile['b_swz_shift']}/{tile['b_swz_mask']}",
            "fraction_of_peak": tflops / peak,
        },
        "roofline": {
            "bound": "mfma" if tile["mfma_block"] else "alu",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": measured_traffic(run_name, cfg.name),
            "kernel_ms": {"avg": kern_avg_s * 1e3, "median": kern_med_s * 1e3, "min": kern_min_s * 1e3},
            "flops_per_launch": cfg.flops,
        },
        "cpu_baseline": cpu_baseline,
        "cold_cache": cold,
        "parity_sample": parity,
    }

    if args.ablations:
        with open(args.ablations, "w") as f:
            for v in range(1, dft.MIXED_COUNT if mixed else dft.VARIANT_COUNT):
                w, kavg, kmed, kmin = time_variant(v, args.steps, args.warmup)
                vname = f"mixed_{args.input}_{dft.MIXED_NAMES[v]}" if mixed else dft.VARIANT_NAMES[v]
                f.write(json.dumps({"variant": vname, "workload": cfg.name,
                                    "tflops_wall": cfg.flops / w / 1e12, "tflops_kernel_avg": cfg.flops / kavg / 1e12,
                                    "kernel_ms_avg": kavg * 1e3, "kernel_ms_median": kmed * 1e3,
                                    "kernel_ms_min": kmin * 1e3}) + "\n")

    if args.copy_calibration_mib > 0:
        from dense_fp32_tiled_amd import lds_probe

        probe = lds_probe.load()
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        if probe.probe_copy_f32(src.data_ptr(), dst.data_ptr(), n, handle) != 0:
            raise RuntimeError("probe_copy_f32 failed")
        torch.cuda.synchronize()
        del src, dst

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
