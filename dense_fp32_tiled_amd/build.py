"""Build the gfx950 HIP library in-tree with hipcc.

    python -m dense_fp32_tiled_amd.build

first runs the host LDS layout search (csrc/layout_gen.cpp -> 
csrc/generated/mfma_layouts.hpp), then produces
dense_fp32_tiled_amd/libdense_fp32_tiled.so from csrc/gemm_api.hip and the
LDS bank-geometry probe liblds_probe.so from csrc/lds_probe.hip.
Packed fp32 VALU instructions are disabled for all device code
(-packed-fp32-ops); hipcc's host pass warns that it does not know that
feature, which is harmless.
"""

from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libdense_fp32_tiled.so"
SOURCES = [CSRC / "gemm_api.hip"]
PROBE_LIB = PKG / "liblds_probe.so"
PROBE_SOURCES = [CSRC / "lds_probe.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return str(Path(rocm) / "bin" / "hipcc")


GENERATED = CSRC / "generated"
LAYOUT_GEN_SRC = CSRC / "layout_gen.cpp"
LAYOUT_HEADER = GENERATED / "mfma_layouts.hpp"


def generate_layouts() -> Path:
    """Compile and run the host layout search (layout_gen.cpp, plain C++17
    with g++), writing csrc/generated/mfma_layouts.hpp for the kernels."""
    GENERATED.mkdir(exist_ok=True)
    exe = GENERATED / "layout_gen"
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", f"-I{CSRC}", str(LAYOUT_GEN_SRC), "-o", str(exe)],
                   check=True)
    text = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    tmp = LAYOUT_HEADER.with_suffix(".tmp")
    tmp.write_text(text)
    os.replace(tmp, LAYOUT_HEADER)
    return LAYOUT_HEADER


def build(out: Path = LIB, extra: list[str] | None = None, sources: list[Path] | None = None) -> Path:
    """Compile the library (always recompiles)."""
    tmp = out.with_name(out.name + ".tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), f"-I{ROOT / 'include'}", f"-I{CSRC}",
           *[str(s) for s in (sources or SOURCES)], "-o", str(tmp)]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stderr)
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}")
    os.replace(tmp, out)
    return out


def build_all() -> list[Path]:
    generate_layouts()
    return [build(LIB, sources=SOURCES), build(PROBE_LIB, sources=PROBE_SOURCES)]


if __name__ == "__main__":
    for p in build_all():
        print(p)
