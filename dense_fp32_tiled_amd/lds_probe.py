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
    lib.lds_probe_run.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.lds_probe_run.restype = ctypes.c_int
    return lib


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
    pats.append(("valu A read (broadcast groups of 16)", 4, [(l // 16) * 4 for l in range(64)]))
    pats.append(("valu B read", 4, [(l % 16) * 4 for l in range(64)]))
    return pats


def predicted(words, width, geom):
    import dense_fp32_tiled_amd as dft

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


def run(reps: int = 2000, waves: int = 4):
    import torch

    lib = load()
    out = torch.zeros(16, dtype=torch.int64, device="cuda")
    rows = []
    for name, width, words in patterns():
        arr = (ctypes.c_int32 * 64)(*words)
        st = lib.lds_probe_run(arr, width, waves, reps, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"lds_probe_run failed ({st}) for {name}")
        torch.cuda.synchronize()
        cyc = out[:waves].cpu().tolist()
        per_instr = max(cyc) / (reps * 16)
        rows.append({"pattern": name, "width_bytes": 4 * width if width > 0 else 8, "mode": width,
                     "cycles_per_instr_per_wave": per_instr,
                     "predicted_degree": {g: predicted(words, width, v) for g, v in GEOMETRIES.items()}})
    return rows


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default="")
    ap.add_argument("--reps", type=int, default=2000)
    ap.add_argument("--waves", type=int, default=4)
    args = ap.parse_args(argv)
    rows = run(args.reps, args.waves)
    lines = [f"# LDS probe: {args.waves} waves x {args.reps} x 16 reads per pattern; cycles per instruction per wave",
             "pattern | bytes/lane | cycles/instr | " + " | ".join(f"degree[{g}]" for g in GEOMETRIES)]
    for r in rows:
        lines.append(f"{r['pattern']} | {r['width_bytes']} | {r['cycles_per_instr_per_wave']:.2f} | " +
                     " | ".join(str(r["predicted_degree"][g]) for g in GEOMETRIES))
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
