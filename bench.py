#!/usr/bin/env python3
"""Benchmark of the masked, LDS-tiled fp32 GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--variant auto] [--workload square4096]

One step is one C = A @ B call through the C ABI on operands already resident
in device memory (4096 x 4096 x 4096, entries normal(0,1), seed 3, by default).
Prints ONE JSON line with the whole-job TFLOP/s (wall clock over K steps
bracketed by device synchronisation), the dominant kernel's roofline position
(its average duration from two HIP events on the launch stream around the
timed launches) and the fp64 CPU
oracle timed on a bounded sample of the same workload on the host cores.

Before the W warmup steps the step is repeated for --settle-ms of wall time
(untimed): an idle GPU raises its clock over the first tens of milliseconds
of work (a kernel trace of 20 steps after 5 warmups shows the 4096^3 kernel
taking 1.12 ms at first and 0.95 ms from about the 22nd launch on), so
without it a short timed region measures the ramp, not the kernel.

    python bench.py --sweep 1000x999x513,2048x256x16384 --sweep-variants auto,mfma_64_bk32_direct \
        --sweep-out FILE [--sweep-reps 5] [--input bf16]

instead times each listed variant on each shape (operands uniform[-1,1),
packed leading dimensions), interleaved over --sweep-reps rounds, and writes
one JSON line per shape and variant (median over the rounds of the kernel
TFLOP/s, from two HIP events around --steps back-to-back launches).
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
# The vector-ALU kernel's ceiling: the library is built without packed fp32, so
# it runs one-product v_fmac_f32; the probe (lds_probe --valu) and its
# SQ_INSTS_VALU / GRBM_GUI_ACTIVE counters measure 0.42 of them per cycle per
# SIMD with two or more waves alternating: 0.42 x 64 lanes x 2 flop x 1024
# SIMDs x 2.4 GHz.
PEAK_VALU_FMA_TFLOPS = 132.1
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


def host_cpu_model() -> str | None:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def sclk_mhz(props) -> float | None:
    """The GPU's current engine clock level (MHz) from its pp_dpm_sclk sysfs
    file (the line marked '*'), found by PCI address; None if unreadable."""
    import re

    candidates = []
    try:
        candidates.append(Path(f"/sys/bus/pci/devices/{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:"
                               f"{props.pci_device_id:02x}.0/pp_dpm_sclk"))
    except AttributeError:
        pass
    drm = sorted(Path("/sys/class/drm").glob("card*/device/pp_dpm_sclk"))
    if len(drm) == 1:
        candidates.append(drm[0])
    for path in candidates:
        try:
            for line in path.read_text().splitlines():
                m = re.search(r"(\d+)\s*Mhz\s*\*", line, re.IGNORECASE)
                if m:
                    return float(m.group(1))
        except OSError:
            continue
    return None


def run_metadata(torch, dev) -> dict:
    props = torch.cuda.get_device_properties(dev)
    return {"device": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count,
            "host_cpu": host_cpu_model()}


def settle(step, torch, ms: float) -> dict:
    """Repeat `step` (untimed) for at least `ms` of wall time, in batches
    ending with a device synchronisation."""
    launches = 0
    t0 = time.perf_counter()
    while ms > 0 and (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step()
        launches += 8
        torch.cuda.synchronize()
    return {"ms": (time.perf_counter() - t0) * 1e3, "launches": launches}


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
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="repeat the step for this long (wall ms, untimed) before the warmup steps, so that the "
                         "GPU clock has left its idle level when the timed region starts (0 = skip)")
    ap.add_argument("--sweep", default="",
                    help="comma-separated MxNxK shapes: time --sweep-variants on each (see the module docstring) "
                         "instead of the single-workload run")
    ap.add_argument("--sweep-variants", default="auto", help="comma-separated variant names for --sweep")
    ap.add_argument("--sweep-reps", type=int, default=5, help="interleaved rounds per shape for --sweep")
    ap.add_argument("--sweep-out", default="", help="output file (JSON lines) for --sweep")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run one device-to-device copy of this many MiB (a "
                         "reference kernel of known traffic for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args(argv)


def sweep(args, names: dict, mixed: bool) -> int:
    """Kernel TFLOP/s of several variants on several shapes, interleaved:
    each of --sweep-reps rounds times every variant once (--steps
    back-to-back launches between two HIP events, after --warmup), and each
    line reports the median round."""
    import numpy as np
    import torch

    import dense_fp32_tiled_amd as dft
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    variants = [names[v] for v in args.sweep_variants.split(",")]
    input_type = {"bf16": dft.INPUT_BF16, "f16": dft.INPUT_F16}.get(args.input)
    meta = run_metadata(torch, dev)
    out = open(args.sweep_out, "w") if args.sweep_out else sys.stdout
    for shape in args.sweep.split(","):
        M, N, K = (int(x) for x in shape.lower().split("x"))
        a_np, b_np = workloads.make_operands(M, N, K, "uniform", 7)
        if mixed:
            a = torch.from_numpy(workloads.to_16bit(a_np, args.input)[0].view(np.int16)).to(dev)
            b = torch.from_numpy(workloads.to_16bit(b_np, args.input)[0].view(np.int16)).to(dev)
            auto = dft.gemm_mixed_auto_variant(M, N, K, cus)
        else:
            a, b = torch.from_numpy(a_np).to(dev), torch.from_numpy(b_np).to(dev)
            auto = dft.gemm_f32_auto_variant_ex(M, N, K, cus, K % 4 == 0, N % 4 == 0)
        c = torch.empty((M, N), dtype=torch.float32, device=dev)

        def step(v):
            if mixed:
                st = dft.gemm_mixed_f32(input_type, M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N,
                                        handle, v)
            else:
                st = dft.gemm_f32_ex(M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N, handle, v)
            if st != dft.GEMM_OK:
                raise dft.GemmError(st, f"{shape} variant {v}")

        settle(lambda: step(variants[0]), torch, args.settle_ms)
        per_variant = {v: [] for v in variants}
        for rep in range(args.sweep_reps):
            # rotate the order each round: a variant timed right after a slower
            # one was seen to run a few percent faster (clock headroom)
            for v in variants[rep % len(variants):] + variants[:rep % len(variants)]:
                for _ in range(args.warmup):
                    step(v)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(args.steps):
                    step(v)
                e1.record(stream)
                torch.cuda.synchronize()
                avg = e0.elapsed_time(e1) / args.steps / 1e3
                per_variant[v].append(2.0 * M * N * K / avg / 1e12)
        for v in variants:
            rates = sorted(per_variant[v])
            vname = (dft.MIXED_NAMES if mixed else dft.VARIANT_NAMES)[v]
            resolved = (dft.MIXED_NAMES if mixed else dft.VARIANT_NAMES)[auto] if v == 0 else vname
            out.write(json.dumps({"shape": shape, "input": args.input, "variant": vname, "runs": resolved,
                                  "tflops_median": rates[len(rates) // 2], "tflops_all": rates,
                                  "device": meta["device"]}) + "\n")
            out.flush()
    if out is not sys.stdout:
        out.close()
    return 0


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
    if args.sweep:
        return sweep(args, names, mixed)
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
        """(wall seconds per step, kernel seconds per launch, median and min
        of single launches).  The timed region is bracketed by device
        synchronisation for the wall clock and by two HIP events on the launch
        stream for the kernel time: the launches run back to back, so the
        events' span over `steps` is the kernels' own time (a pair of events
        around each launch adds a few microseconds to a short kernel; those
        single-launch figures are taken afterwards, for the median and min)."""
        for _ in range(warmup):
            step(v)
        torch.cuda.synchronize()
        span0, span1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        span0.record(stream)
        for _ in range(steps):
            step(v)
        span1.record(stream)
        torch.cuda.synchronize()
        wall_s = (time.perf_counter() - t0) / steps
        kernel_s = span0.elapsed_time(span1) / 1e3 / steps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in ev:
            e0.record(stream)
            step(v)
            e1.record(stream)
        torch.cuda.synchronize()
        durs = sorted(e0.elapsed_time(e1) / 1e3 for e0, e1 in ev)
        return wall_s, kernel_s, durs[len(durs) // 2], durs[0]

    settled = settle(step, torch, args.settle_ms)
    props = torch.cuda.get_device_properties(dev)
    meta = run_metadata(torch, dev)
    meta["sclk_mhz_before"] = sclk_mhz(props)
    wall_s, kern_avg_s, kern_med_s, kern_min_s = time_variant(variant, args.steps, args.warmup)
    meta["sclk_mhz_after"] = sclk_mhz(props)

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
            # the library's own choice for these operands: packed rows (lda = K, ldb = N) on aligned bases
            resolved = dft.gemm_f32_auto_variant_ex(M, N, K, cus, K % 4 == 0, N % 4 == 0)
        else:
            resolved = variant
        tile = dft.gemm_f32_tile_config(resolved)
        run_name = dft.VARIANT_NAMES[resolved] + (f"+splitk{splits_used}" if args.splits >= 0 else "")
    peak = PEAK_16BIT_TFLOPS if mixed else PEAK_FP32_TFLOPS if tile["mfma_block"] else PEAK_VALU_FMA_TFLOPS

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
        "settle": settled,
        "run": meta,
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
