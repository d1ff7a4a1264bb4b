"""Measure the gfx950 LDS bank geometry with liblds_probe.so.

    python -m dense_fp32_tiled_amd.lds_probe [--out FILE]

Times a fixed set of one-instruction LDS read patterns (strided 4/8/16-byte
reads, and the exact fragment-read patterns of the GEMM kernels at their
candidate paddings) and prints cycles per instruction next to the conflict
degree the bank model predicts for each candidate geometry.  The geometry
whose predictions track the measurements is the one the kernels' padding is
derived for.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
PROBE_LIB = PKG / "liblds_probe.so"

# candidate geometries: access width in dwords -> (banks, lanes serviced per pass)
GEOMETRIES = {
    "32 banks x 128 B/pass": {1: (32, 32), 2: (32, 16), 4: (32, 8)},
    "64 banks x 256 B/pass": {1: (64, 64), 2: (64, 32), 4: (64, 16)},
    "b32 32x32, b64 64x32, b128 64x16": {1: (32, 32), 2: (64, 32), 4: (64, 16)},
}


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
    pats.append(("valu A read (broadcast groups of 16)", 4, [(l // 16) * 4 for l in range(64)]))
    pats.append(("valu B read", 4, [(l % 16) * 4 for l in range(64)]))
    return pats


def kernel_patterns(variant: int):
    """Every distinct LDS access pattern one K tile of an MFMA variant issues
    (fragment reads, ds_read2 pairs, cooperative stores), A tile at dword 0
    and B tile at dword 8192 as in the kernel's stage-0 layout."""
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
            vcols = cols // vec
            for i in range(rows * vcols // c["threads"]):
                idx = [w * 64 + l + i * c["threads"] for l in range(64)]
                add(f"{tile.upper()} store w{w} s{i}", 100 + vec, [word(tile, x // vcols, (x % vcols) * vec) for x in idx])
    return out


def predicted(words, width, geom):
    import dense_fp32_tiled_amd as dft

    if width > 100:  # a store: modelled with the read geometry of its width
        width -= 100
    if width < 0:  # ds_read2_b32: two 4-byte accesses, one per address; report the worse
        banks, group = geom[1]
        return max(dft.gemm_lds_conflict_degree(words, 1, banks, group),
                   dft.gemm_lds_conflict_degree([w - width for w in words], 1, banks, group))
    banks, group = geom[width]
    return dft.gemm_lds_conflict_degree(words, width, banks, group)


def measured_degree(cycles_per_instr: float, width: int, waves: int, geom, issue_floor: float) -> int:
    """Conflict degree implied by a timing.  An instruction occupies the LDS
    for (64 / lanes per pass) passes of one cycle per unit of degree, and
    `waves` wavefronts share it, so cycles = waves * passes * degree unless
    that is below the issue floor (the time of a broadcast read), where every
    degree-1 access lands."""
    if cycles_per_instr < 1.1 * issue_floor:
        return 1
    width = width - 100 if width > 100 else width
    passes = 64 // geom[width][1] if width > 0 else 2 * (64 // geom[1][1])
    return max(1, round(cycles_per_instr / (waves * passes)))


def fit(rows, waves):
    """Patterns whose measured degree equals each geometry's prediction."""
    floor = next(r["cycles_per_instr_per_wave"] for r in rows if r["pattern"] == "b32 stride 0")
    score = {}
    for g, geom in GEOMETRIES.items():
        score[g] = sum(1 for r in rows
                       if measured_degree(r["cycles_per_instr_per_wave"], r.get("mode", r["width_bytes"] // 4), waves,
                                          geom, floor)
                       == r["predicted_degree"][g])
    return score


def xcc_map(blocks: int = 512, threads: int = 512):
    """XCD of each workgroup of a 1-D launch (probe_xcc_ids)."""
    import torch

    lib = load()
    out = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
    if lib.probe_xcc_ids(out.data_ptr(), blocks, threads, torch.cuda.current_stream().cuda_stream) != 0:
        raise RuntimeError("probe_xcc_ids failed")
    torch.cuda.synchronize()
    return out.cpu().tolist()


def run(reps: int = 2000, waves: int = 4, variants=()):
    import torch

    lib = load()
    out = torch.zeros(16, dtype=torch.int64, device="cuda")
    rows = []
    pats = list(patterns())
    for v in variants:
        pats += kernel_patterns(v)
    for name, width, words in pats:
        arr = (ctypes.c_int32 * 64)(*words)
        st = lib.lds_probe_run(arr, width, waves, reps, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"lds_probe_run failed ({st}) for {name}")
        torch.cuda.synchronize()
        cyc = out[:waves].cpu().tolist()
        per_instr = max(cyc) / (reps * 16)
        rows.append({"pattern": name, "width_bytes": 4 * (width % 100) if width > 0 else 8, "mode": width,
                     "cycles_per_instr_per_wave": per_instr,
                     "predicted_degree": {g: predicted(words, width, v) for g, v in GEOMETRIES.items()}})
    return rows


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
    args = ap.parse_args(argv)
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

    variants = (dft.VARIANT_MFMA, dft.VARIANT_MFMA16, dft.VARIANT_MFMA_128_BK32) if args.kernels else ()
    rows = run(args.reps, args.waves, variants)
    lines = [f"# LDS probe: {args.waves} waves x {args.reps} x 16 reads per pattern; cycles per instruction per wave",
             "pattern | bytes/lane | cycles/instr | " + " | ".join(f"degree[{g}]" for g in GEOMETRIES)]
    for r in rows:
        lines.append(f"{r['pattern']} | {r['width_bytes']} | {r['cycles_per_instr_per_wave']:.2f} | " +
                     " | ".join(str(r["predicted_degree"][g]) for g in GEOMETRIES))
    if args.xcc:
        ids = xcc_map()
        rr = sum(1 for b, x in enumerate(ids) if x == b % 8)
        lines.append("")
        lines.append(f"XCD of workgroups 0..{len(ids) - 1} (512 threads each): {ids[:32]} ...")
        lines.append(f"workgroups with XCD == index % 8: {rr} of {len(ids)}")
    score = fit(rows, args.waves)
    lines.append("")
    lines.append("patterns whose timing matches the predicted degree (of %d):" % len(rows))
    for g, ok in score.items():
        lines.append(f"  {g}: {ok}")
    text = "\n".join(lines)
    print(text)
    if args.out:
        Path(args.out).write_text(text + "\n\n" + json.dumps(rows) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
