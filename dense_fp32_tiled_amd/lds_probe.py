"""Measure the gfx950 LDS bank geometry with liblds_probe.so.

    python -m dense_fp32_tiled_amd.lds_probe [--out FILE]

Times a fixed set of one-instruction LDS access patterns (strided 4/8/16-byte
reads and stores, two-address reads, patterns that isolate which lanes share
a pass, and with --kernels every fragment read and store of the MFMA
kernels with their built layouts) and prints the LDS cycles per instruction
next to what the bank model the layout search uses predicts for it
(gemm_lds_access_cycles, or the issue floor of a conflict-free
instruction).
"""

from __future__ import annotations

import argparse
import ctypes
import json
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
PROBE_LIB = PKG / "liblds_probe.so"
LDS_PROBE_WORDS = 16384  # the probe kernel's LDS buffer (include/lds_probe.h)



def load():
    if not PROBE_LIB.exists():
        raise ImportError(f"{PROBE_LIB} is not built; run `python -m dense_fp32_tiled_amd.build`")
    import dense_fp32_tiled_amd as dft

    dft._share_torch_hip_runtime()
    lib = ctypes.CDLL(str(PROBE_LIB))
    # Every entry point gets its full signature: an undeclared argument is
    # passed as a C int, which would truncate a 64-bit device pointer.
    lib.lds_probe_run.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.lds_probe_run.restype = ctypes.c_int
    lib.probe_xcc_ids.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.probe_xcc_ids.restype = ctypes.c_int
    lib.probe_copy_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.probe_copy_f32.restype = ctypes.c_int
    lib.probe_dma_throughput.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_dma_throughput.restype = ctypes.c_int
    lib.probe_valu_fma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_valu_fma.restype = ctypes.c_int
    lib.probe_mfma_f32.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.probe_mfma_f32.restype = ctypes.c_int
    return lib


def valu_fma_throughput(reps: int = 20000, blocks: int = 256, waves_list=(4, 8, 16)):
    """v_fmac_f32 instructions per cycle per SIMD (one workgroup per CU, its
    waves spread over the CU's 4 SIMDs) and the fp32 rate that implies at
    2.4 GHz on 256 CUs."""
    import torch

    lib = load()
    out = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")
    rows = []
    for waves in waves_list:
        st = lib.probe_valu_fma(blocks, waves, reps, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"probe_valu_fma failed ({st}), {waves} waves")
        torch.cuda.synchronize()
        worst = max(out[:blocks * waves].cpu().tolist())
        ipc = (waves / 4) * reps * 64 / worst  # per SIMD
        rows.append({"waves_per_cu": waves, "cycles": worst, "fma_instr_per_cycle_per_simd": ipc,
                     "cycles_per_fma_instr": 1.0 / ipc, "tflops_at_2400mhz_256cu": ipc * 64 * 2 * 1024 * 2.4e9 / 1e12})
    return rows


def mfma_throughput(reps: int = 4000, blocks: int = 256, waves_list=(4, 8, 16)):
    """v_mfma_f32_32x32x2_f32 instructions per cycle per SIMD (one workgroup
    per CU, its waves spread over the CU's 4 SIMDs), accumulators in VGPRs
    and in AGPRs, and the fp32 rate that implies at 2.4 GHz on 256 CUs."""
    import torch

    lib = load()
    out = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")
    rows = []
    for agpr in (0, 1):
        for waves in waves_list:
            st = lib.probe_mfma_f32(blocks, waves, reps, agpr, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise RuntimeError(f"probe_mfma_f32 failed ({st}), {waves} waves")
            torch.cuda.synchronize()
            worst = max(out[:blocks * waves].cpu().tolist())
            ipc = (waves / 4) * reps * 16 / worst  # per SIMD
            rows.append({"accumulators": "AGPR" if agpr else "VGPR", "waves_per_cu": waves, "cycles": worst,
                         "mfma_instr_per_cycle_per_simd": ipc, "cycles_per_mfma_instr": 1.0 / ipc,
                         "tflops_at_2400mhz_256cu": ipc * 4096 * 1024 * 2.4e9 / 1e12})
    return rows


def platform_gemm(shapes=((4096, 4096, 4096), (8192, 8192, 8192)), reps: int = 20):
    """Context only, not part of the library: the platform's own GEMM
    (torch.matmul on the GPU, fp32 with TF32 off, then bf16 inputs) timed
    with HIP events over `reps` launches after 5 untimed ones."""
    import torch

    torch.backends.cuda.matmul.allow_tf32 = False
    rows = []
    for dtype in (torch.float32, torch.bfloat16):
        for M, N, K in shapes:
            g = torch.Generator(device="cuda").manual_seed(M + N + K)
            a = torch.rand(M, K, device="cuda", dtype=torch.float32, generator=g).to(dtype)
            b = torch.rand(K, N, device="cuda", dtype=torch.float32, generator=g).to(dtype)
            for _ in range(5):
                torch.matmul(a, b)
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            for _ in range(reps):
                torch.matmul(a, b)
            stop.record()
            torch.cuda.synchronize()
            ms = start.elapsed_time(stop) / reps
            rows.append({"dtype": str(dtype).replace("torch.", ""), "shape": f"{M}x{N}x{K}", "ms": ms,
                         "tflops": 2.0 * M * N * K / (ms * 1e-3) / 1e12})
            del a, b
    return rows


# Direct-copy pieces as the 64x64x32 fp32 kernel issues them: (label, bytes per
# lane, lanes per row, row pitch in bytes, byte offset of the first row).
DMA_CASES = [
    ("16-byte, A tile rows (8 lanes per 128-byte row, pitch 2048 B)", 16, 8, 2048, 0),
    ("4-byte, A tile rows (32 lanes per row, pitch 2048 B)", 4, 32, 2048, 0),
    ("4-byte, A tile rows (32 lanes per row, pitch 2052 B, odd lda)", 4, 32, 2052, 4),
    ("4-byte, B tile rows (64 lanes per row, pitch 3996 B, odd ldb)", 4, 64, 3996, 4),
    ("16-byte, B tile rows (16 lanes per row, pitch 4096 B)", 16, 16, 4096, 0),
]


def dma_throughput(reps: int = 200, blocks: int = 256, waves_list=(1, 2, 4, 8, 16)):
    """Copies per CU per 1000 cycles for each DMA_CASES piece and wave count
    (one workgroup per CU: `blocks` no larger than the CU count)."""
    import torch

    lib = load()
    src_bytes = 128 << 20
    src = torch.zeros(src_bytes // 4, dtype=torch.float32, device="cuda")
    out = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")
    rows = []
    for label, width, row_lanes, ld, off0 in DMA_CASES:
        for waves in waves_list:
            # each wave reads its own 64 rows' worth of a window that stays in L2 and MALL
            wave_stride = ((64 // row_lanes) * ld + 15) // 16 * 16
            st = lib.probe_dma_throughput(src.data_ptr(), src_bytes, width, blocks, waves, reps, off0, wave_stride,
                                          ld, row_lanes, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise RuntimeError(f"probe_dma_throughput failed ({st}) for {label}, {waves} waves")
            torch.cuda.synchronize()
            cyc = out[:blocks * waves].cpu().tolist()
            worst = max(cyc)
            rows.append({"case": label, "bytes_per_lane": width, "waves": waves,
                         "cycles_per_copy_per_wave": worst / (reps * 16),
                         "copies_per_kcycle_per_cu": 1000.0 * waves * reps * 16 / worst,
                         "bytes_per_cycle_per_cu": waves * reps * 16 * 64 * width / worst})
    return rows


def patterns():
    """(name, width_words, lane -> dword address list)."""
    pats = []
    for s in (0, 1, 2, 3, 4, 8, 16, 32, 33, 64, 65, 128):
        pats.append((f"b32 stride {s}", 1, [l * s for l in range(64)]))
    for s in (2, 4, 8, 16, 32, 64, 128):
        pats.append((f"b64 stride {s}", 2, [l * s for l in range(64)]))
    for s in (4, 8, 12, 16, 20, 24, 28, 32, 36, 64, 128):
        pats.append((f"b128 stride {s}", 4, [l * s for l in range(64)]))
    # which lanes share a pass: lanes >= G repeat lanes < G's banks at another address
    for g in (8, 16, 32):
        pats.append((f"b32 halves at lane {g}", 1, [(l % g) + (l // g) * 1024 for l in range(64)]))
        pats.append((f"b128 groups of {g}", 4, [4 * (l % g) + (l // g) * 1024 for l in range(64)]))
    # the GEMM kernels' own fragment reads
    for pad in (0, 4, 8, 12):
        stride = 16 + pad
        pats.append((f"mfma A read, row stride {stride}", 4, [(l % 32) * stride + (l // 32) * 8 for l in range(64)]))
    for pad in (0, 4, 8, 16, 32):
        stride = 128 + pad
        pats.append((f"mfma B read, row stride {stride}", 1, [(l // 32) * 8 * stride + (l % 32) for l in range(64)]))
    # two-address reads (ds_read2_b32): MFMA B fragments of block columns 2p, 2p+1
    for stride in (128, 132, 136, 144):
        pats.append((f"read2 +16, mfma16 B, row stride {stride}", -16,
                     [(l // 16) * 4 * stride + (l % 16) for l in range(64)]))
        pats.append((f"read2 +32, mfma32 B, row stride {stride}", -32,
                     [(l // 32) * 8 * stride + (l % 32) for l in range(64)]))
    pats.append(("read2 +16, consecutive lanes", -16, list(range(64))))
    pats.append(("read2 +32, consecutive lanes", -32, list(range(64))))
    pats.append(("read2 +16, lanes 32 apart", -16, [(l % 32) + (l // 32) * 1024 for l in range(64)]))
    # writes, to check that stores follow the read geometry of the same width
    for s_ in (1, 2, 32, 33, 64):
        pats.append((f"write b32 stride {s_}", 101, [l * s_ for l in range(64)]))
    for s_ in (4, 8, 16, 20, 32, 64):
        pats.append((f"write b128 stride {s_}", 104, [l * s_ for l in range(64)]))
    for g in (8, 16, 32):
        pats.append((f"write b128 groups of {g}", 104, [4 * (l % g) + (l // g) * 1024 for l in range(64)]))
    # 8-byte stores: strides, and which lanes share a pass
    for s_ in (2, 4, 8, 16, 32, 64):
        pats.append((f"write b64 stride {s_}", 102, [l * s_ for l in range(64)]))
    for g in (8, 16, 32):
        pats.append((f"write b64 groups of {g}", 102, [2 * (l % g) + (l // g) * 1024 for l in range(64)]))
    # which lanes of a 16-byte read share a pass: rows 0..15 of a 16-word-stride
    # tile, 4-word group g ^ ((row >> 2) & 3); the lanes named carry the pattern,
    # every other lane reads lane 0's address (a broadcast)
    def quad(row, g):
        return row * 16 + 4 * (g ^ ((row >> 2) & 3))
    sel = {"0-15": range(0, 16), "16-31": range(16, 32), "0-31": range(0, 32), "0-15,32-47": [*range(16), *range(32, 48)],
           "0-7,16-23": [*range(8), *range(16, 24)], "0-15,48-63": [*range(16), *range(48, 64)]}
    for label, lanes in sel.items():
        lanes = set(lanes)
        pats.append((f"b128 rows x groups, lanes {label} (g = l / 16)", 4,
                     [quad(l % 16, l // 16) if l in lanes else 0 for l in range(64)]))
    pats.append(("b128 rows x groups, all lanes (g = l / 32, rows 0..31)", 4, [quad(l % 32, l // 32) for l in range(64)]))
    # One pass alone (lanes 0-15; the others read lane 0's address): 16
    # distinct 16-byte bank quads, spread over 256-byte rows in different ways.
    def one_pass(words16):
        return [words16[l] if l < 16 else words16[0] for l in range(64)]
    mfma16_quad = [4 * (l % 4) + l // 4 for l in range(16)]
    for label, words16 in (
            ("quads in order, one row", [4 * l for l in range(16)]),
            ("quads in order, row per lane", [4 * l + 64 * l for l in range(16)]),
            ("quads 4(l%4)+l/4, one row", [4 * q for q in mfma16_quad]),
            ("quads 4(l%4)+l/4, row per lane", [4 * q + 64 * l for l, q in enumerate(mfma16_quad)]),
            ("quads in order, row l/4", [4 * l + 64 * (l // 4) for l in range(16)]),
            ("quads in order, row l%4", [4 * l + 64 * (l % 4) for l in range(16)]),
            ("quads in order, row l/8", [4 * l + 64 * (l // 8) for l in range(16)]),
            ("quads in order, row l%2", [4 * l + 64 * (l % 2) for l in range(16)]),
            ("mfma16 A rows (16-word rows, swizzle 4,2,3)",
             [16 * r + 4 * (0 ^ ((r >> 2) & 3)) for r in range(16)])):
        pats.append((f"b128 one pass, {label}", 4, one_pass(words16)))
    # Two passes whose quads coincide: lanes 0-15 and lanes 16k..16k+15 at
    # another row, one pair of passes at a time.
    for other in (1, 2, 3):
        pats.append((f"b128 passes 0 and {other} on the same quads", 4,
                     [4 * (l % 16) + (1024 if l // 16 == other else 0) if l // 16 in (0, other) else 0
                      for l in range(64)]))
    pats.append(("valu A read (broadcast groups of 16)", 4, [(l // 16) * 4 for l in range(64)]))
    pats.append(("valu B read", 4, [(l % 16) * 4 for l in range(64)]))
    return pats


def kernel_patterns(variant: int):
    """Every distinct LDS access pattern one K tile of an MFMA variant issues
    (fragment reads, ds_read2 pairs, and the cooperative stores of the
    register-path kernels), A tile at dword 0 and B tile at dword 8192 as in
    the kernel's stage-0 layout."""
    import dense_fp32_tiled_amd as dft

    c = dft.gemm_f32_tile_config(variant)
    mb = c["mfma_block"]
    kg = c["bk"] // (64 // mb)
    waves_n = c["bn"] // c["tn"]
    vec = c["vec_width"]
    base = {"a": 0, "b": 8192}

    def word(tile, row, col):
        unit, shift, mask = c[f"{tile}_swz_unit"], c[f"{tile}_swz_shift"], c[f"{tile}_swz_mask"]
        phys = col ^ (unit * ((row >> shift) & mask)) if unit else col
        return base[tile] + row * c[f"{tile}_row_stride"] + phys

    name = dft.VARIANT_NAMES[variant]
    seen, out = set(), []

    def add(label, mode, words):
        key = (mode, tuple(words))
        if key not in seen:
            seen.add(key)
            out.append((f"{name} {label}", mode, list(words)))

    for w in range(c["threads"] // 64):
        wm0, wn0 = (w // waves_n) * c["tm"], (w % waves_n) * c["tn"]
        for mi in range(c["tm"] // mb):
            for q in range(kg // 4):
                add(f"A read w{w} m{mi} q{q}", 4, [word("a", wm0 + mi * mb + l % mb, (l // mb) * kg + 4 * q)
                                                  for l in range(64)])
        for j in range(kg):
            for ni in range(0, c["tn"] // mb, 2):
                add(f"B read2 w{w} j{j} n{ni}", -mb,
                    [word("b", (l // mb) * kg + j, wn0 + ni * mb + l % mb) for l in range(64)])
        for tile, rows, cols in (("a", c["bm"], c["bk"]), ("b", c["bk"], c["bn"])):
            if c["direct_to_lds"]:
                break  # direct copies: no LDS store instructions
            vcols = cols // vec
            for i in range(rows * vcols // c["threads"]):
                idx = [w * 64 + l + i * c["threads"] for l in range(64)]
                add(f"{tile.upper()} store w{w} s{i}", 100 + vec, [word(tile, x // vcols, (x % vcols) * vec) for x in idx])
    return out


# Issue time of a conflict-free instruction (LDS cycles, measured with 4
# waves): the bank model's cycles (gemm_lds_access_cycles) exclude it, so a
# timing is predicted as the larger of the two.
ISSUE_FLOOR = {1: 3.4, 2: 3.4, 4: 4.0, -16: 4.0, -32: 4.0, 101: 4.0, 102: 7.2, 104: 13.1}


def model_cycles(words, mode) -> float:
    """Cycles per instruction the gfx950 bank model predicts (bank cycles or
    the issue floor, whichever is larger)."""
    import dense_fp32_tiled_amd as dft

    return max(ISSUE_FLOOR[mode], dft.gemm_lds_access_cycles(words, mode))


def xcc_map(blocks: int = 512, threads: int = 512):
    """XCD of each workgroup of a 1-D launch (probe_xcc_ids)."""
    import torch

    lib = load()
    out = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
    if lib.probe_xcc_ids(out.data_ptr(), blocks, threads, torch.cuda.current_stream().cuda_stream) != 0:
        raise RuntimeError("probe_xcc_ids failed")
    torch.cuda.synchronize()
    return out.cpu().tolist()


def run(reps: int = 2000, waves: int = 4, variants=(), trials: int = 3):
    """Time every pattern `trials` times and keep the fastest: a timing can
    only grow from interference (other work on the device, a clock change),
    never shrink."""
    import torch

    lib = load()
    out = torch.zeros(16, dtype=torch.int64, device="cuda")
    rows = []
    pats = list(patterns())
    for v in variants:
        pats += kernel_patterns(v)
    for name, width, words in pats:
        arr = (ctypes.c_int32 * 64)(*words)
        if max(words) + 4 + (-width if width < 0 else 0) > LDS_PROBE_WORDS:
            continue  # beyond the probe's LDS buffer (tiles of the largest kernels)
        per_instr = None
        for _ in range(trials):
            st = lib.lds_probe_run(arr, width, waves, reps, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise RuntimeError(f"lds_probe_run failed ({st}) for {name}")
            torch.cuda.synchronize()
            t = max(out[:waves].cpu().tolist()) / (reps * 16)
            per_instr = t if per_instr is None else min(per_instr, t)
        rows.append({"pattern": name, "width_bytes": 4 * (width % 100) if width > 0 else 8, "mode": width,
                     "words": list(words), "cycles_per_instr_per_wave": per_instr,
                     "cycles_per_instr": per_instr / waves,  # the waves share the LDS
                     "model_cycles": model_cycles(words, width)})
    return rows


def unique_patterns(rows):
    """Rows whose (mode, words) differ only by a whole number of 64-dword
    lines share bank behaviour: keep the first of each (its name, the median
    timing, how many there were)."""
    import statistics

    groups = {}
    for r in rows:
        base = (min(r["words"]) // 64) * 64
        groups.setdefault((r["mode"], tuple(w - base for w in r["words"])), []).append(r)
    out = []
    for (mode, words), rs in groups.items():
        out.append({"pattern": rs[0]["pattern"], "count": len(rs), "mode": mode, "words": list(words),
                    "cycles_per_instr": round(statistics.median(x["cycles_per_instr"] for x in rs), 3),
                    "model_cycles": rs[0]["model_cycles"]})
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default="")
    ap.add_argument("--reps", type=int, default=2000)
    ap.add_argument("--waves", type=int, default=4)
    ap.add_argument("--kernels", action="store_true",
                    help="also replay every LDS access pattern of the MFMA variants")
    ap.add_argument("--xcc", action="store_true", help="also report the XCD of each workgroup of a 512-block launch")
    ap.add_argument("--dma", action="store_true",
                    help="time the direct global->LDS copies instead (probe_dma_throughput, one workgroup per CU)")
    ap.add_argument("--valu", action="store_true",
                    help="time the vector ALU's v_fmac_f32 instead (probe_valu_fma, one workgroup per CU)")
    ap.add_argument("--mfma", action="store_true",
                    help="time the matrix pipe's v_mfma_f32_32x32x2_f32 instead (probe_mfma_f32, one workgroup per CU)")
    ap.add_argument("--platform-gemm", action="store_true",
                    help="time torch.matmul (fp32 with TF32 off, and bf16) at 4096^3 and 8192^3, for context")
    args = ap.parse_args(argv)
    if args.mfma:
        rows = mfma_throughput()
        lines = ["# command: python -m dense_fp32_tiled_amd.lds_probe --mfma --out <file>",
                 "# v_mfma_f32_32x32x2_f32 throughput: 256 workgroups (one per CU), each wave 4000 x 16 MFMAs on "
                 "4 independent accumulators, register operands; worst wave",
                 "accumulators | waves per CU | cycles | MFMA instructions per cycle per SIMD | "
                 "cycles per instruction | fp32 TFLOP/s at 2.4 GHz, 256 CUs"]
        for r in rows:
            lines.append(f"{r['accumulators']} | {r['waves_per_cu']} | {r['cycles']} | "
                         f"{r['mfma_instr_per_cycle_per_simd']:.4f} | {r['cycles_per_mfma_instr']:.2f} | "
                         f"{r['tflops_at_2400mhz_256cu']:.1f}")
        text = "\n".join(lines)
        print(text)
        if args.out:
            Path(args.out).write_text(text + "\n\n" + json.dumps(rows) + "\n")
        return 0
    if args.platform_gemm:
        rows = platform_gemm()
        lines = ["# command: python -m dense_fp32_tiled_amd.lds_probe --platform-gemm --out <file>",
                 "# torch.matmul on the GPU (context only; not part of the library), TF32 off; 20 timed launches "
                 "after 5 untimed, HIP events",
                 "dtype | M x N x K | ms per launch | TFLOP/s"]
        for r in rows:
            lines.append(f"{r['dtype']} | {r['shape']} | {r['ms']:.4f} | {r['tflops']:.1f}")
        text = "\n".join(lines)
        print(text)
        if args.out:
            Path(args.out).write_text(text + "\n\n" + json.dumps(rows) + "\n")
        return 0
    if args.valu:
        rows = valu_fma_throughput()
        lines = ["# v_fmac_f32 throughput: 256 workgroups (one per CU), each lane 20000 x 64 FMAs on 8 independent "
                 "accumulators; worst wave",
                 "waves per CU | cycles | FMA instructions per cycle per SIMD | cycles per instruction | "
                 "fp32 TFLOP/s at 2.4 GHz, 256 CUs"]
        for r in rows:
            lines.append(f"{r['waves_per_cu']} | {r['cycles']} | {r['fma_instr_per_cycle_per_simd']:.3f} | "
                         f"{r['cycles_per_fma_instr']:.2f} | {r['tflops_at_2400mhz_256cu']:.1f}")
        text = "\n".join(lines)
        print(text)
        if args.out:
            Path(args.out).write_text(text + "\n\n" + json.dumps(rows) + "\n")
        return 0
    if args.dma:
        rows = dma_throughput()
        lines = ["# direct global->LDS copy throughput: 256 workgroups (one per CU), each wave 200 x 16 copies, "
                 "waiting after each 16; worst wave",
                 "case | waves | cycles/copy/wave | copies per 1000 cycles per CU | bytes/cycle/CU"]
        for r in rows:
            lines.append(f"{r['case']} | {r['waves']} | {r['cycles_per_copy_per_wave']:.1f} | "
                         f"{r['copies_per_kcycle_per_cu']:.1f} | {r['bytes_per_cycle_per_cu']:.1f}")
        text = "\n".join(lines)
        print(text)
        if args.out:
            Path(args.out).write_text(text + "\n\n" + json.dumps(rows) + "\n")
        return 0
    import dense_fp32_tiled_amd as dft

    variants = [v for v in range(1, dft.VARIANT_COUNT)
                if dft.gemm_f32_tile_config(v)["mfma_block"] > 0] if args.kernels else ()
    rows = unique_patterns(run(args.reps, args.waves, variants))
    lines = ["# command: python -m dense_fp32_tiled_amd.lds_probe" + (" --kernels" if args.kernels else "") +
             " --out <file>",
             f"# LDS probe: {args.waves} waves x {args.reps} x 16 accesses per pattern, fastest of 3 timings; patterns that differ only "
             "by a whole number of 64-dword lines are timed once (count = how many the run had)",
             "# cycles per instruction of the LDS (per wave / waves); model = gemm_lds_access_cycles or the "
             "issue floor, whichever is larger",
             "pattern | count | mode | LDS cycles/instr | model"]
    for r in rows:
        lines.append(f"{r['pattern']} | {r['count']} | {r['mode']} | {r['cycles_per_instr']:.2f} | "
                     f"{r['model_cycles']:.1f}")
    if args.xcc:
        ids = xcc_map()
        rr = sum(1 for b, x in enumerate(ids) if x == b % 8)
        lines.append("")
        lines.append(f"XCD of workgroups 0..{len(ids) - 1} (512 threads each): {ids[:32]} ...")
        lines.append(f"workgroups with XCD == index % 8: {rr} of {len(ids)}")
    close = [r for r in rows if abs(r["model_cycles"] - r["cycles_per_instr"]) <= 0.15 * r["cycles_per_instr"]]
    lines.append("")
    lines.append(f"patterns the bank model times within 15 %: {len(close)} of {len(rows)} "
                 f"({sum(r['count'] for r in close)} of {sum(r['count'] for r in rows)} counting repeats)")
    lines.append("not within 15 %: " + "; ".join(r["pattern"] for r in rows if r not in close))
    text = "\n".join(lines)
    print(text)
    if args.out:
        Path(args.out).write_text(text + "\n\n" + json.dumps(rows, separators=(",", ":")) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
