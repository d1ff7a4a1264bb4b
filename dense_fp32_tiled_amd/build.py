"""Build the gfx950 HIP library in-tree with hipcc.

    python -m dense_fp32_tiled_amd.build

first runs the host LDS layout search (csrc/layout_gen.cpp ->
csrc/generated/mfma_layouts.hpp), then produces
dense_fp32_tiled_amd/libdense_fp32_tiled.so from csrc/gemm_api.hip and
csrc/gemm_default.hip, the same library built with DFT_LDS_POISON=1
(libdense_fp32_tiled_poison.so, for the LDS-poison parity tests), and the
measurement probes liblds_probe.so from csrc/lds_probe.hip.
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
POISON_LIB = PKG / "libdense_fp32_tiled_poison.so"
SOURCES = [CSRC / "gemm_api.hip", CSRC / "gemm_default.hip"]
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
    with g++), writing csrc/generated/mfma_layouts.hpp for the kernels.
    Safe to run from several processes at once: the search is built in a
    private directory and the header replaced atomically."""
    import tempfile

    GENERATED.mkdir(exist_ok=True)
    with tempfile.TemporaryDirectory() as work:
        exe = Path(work) / "layout_gen"
        subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", f"-I{CSRC}", str(LAYOUT_GEN_SRC), "-o", str(exe)],
                       check=True)
        text = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    fd, tmp = tempfile.mkstemp(dir=GENERATED, prefix=".mfma_layouts.", suffix=".tmp")
    with os.fdopen(fd, "w") as f:
        f.write(text)
    os.replace(tmp, LAYOUT_HEADER)
    return LAYOUT_HEADER


def _start(out: Path, extra: list[str] | None, sources: list[Path] | None):
    tmp = out.with_name(f"{out.name}.{os.getpid()}.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), f"-I{ROOT / 'include'}", f"-I{CSRC}",
           *[str(s) for s in (sources or SOURCES)], "-o", str(tmp)]
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    return proc, tmp, out, cmd


def _finish(job) -> Path:
    proc, tmp, out, cmd = job
    _, err = proc.communicate()
    if proc.returncode != 0:
        sys.stderr.write(err)
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}")
    os.replace(tmp, out)
    return out


def build(out: Path = LIB, extra: list[str] | None = None, sources: list[Path] | None = None) -> Path:
    """Compile the library (always recompiles)."""
    return _finish(_start(out, extra, sources))


def build_all() -> list[Path]:
    """The library, its LDS-poison debug build (every kernel fills its LDS
    with NaN before the first copy: DFT_LDS_POISON=1) and the probe library,
    compiled concurrently."""
    generate_layouts()
    jobs = [_start(LIB, None, SOURCES), _start(POISON_LIB, ["-DDFT_LDS_POISON=1"], SOURCES),
            _start(PROBE_LIB, None, PROBE_SOURCES)]
    return [_finish(j) for j in jobs]


def device_assembly(source: Path | None = None) -> str:
    """The gfx950 assembly hipcc emits for the library's device code (the
    same flags as the build), as text: of `source`, or of every library
    source concatenated."""
    import tempfile

    if source is None:
        return "\n".join(device_assembly(src) for src in SOURCES)
    generate_layouts()
    with tempfile.TemporaryDirectory() as tmp:
        out = Path(tmp) / "device.s"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "--cuda-device-only", "-S", f"-I{ROOT / 'include'}", f"-I{CSRC}",
               str(source), "-o", str(out)]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            sys.stderr.write(proc.stderr)
            raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}")
        return out.read_text()


def resource_report(source: Path | None = None) -> dict[str, dict[str, int]]:
    """The compiler's per-kernel resource usage for the library's device code
    (hipcc -Rpass-analysis=kernel-resource-usage): {mangled kernel name:
    {"vgpr", "agpr", "scratch" (bytes per lane), "occupancy" (waves per SIMD),
    "lds" (bytes per workgroup)}}, of `source` or of every library source.
    Compiles device code only, to a temporary object."""
    import re
    import tempfile

    if source is None:
        merged: dict[str, dict[str, int]] = {}
        for src in SOURCES:
            merged.update(resource_report(src))
        return merged
    generate_layouts()
    fields = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
              "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "--cuda-device-only", "-c", f"-I{ROOT / 'include'}", f"-I{CSRC}",
               str(source), "-o", str(Path(tmp) / "device.o"), "-Rpass-analysis=kernel-resource-usage"]
        proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stderr)
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}")
    report: dict[str, dict[str, int]] = {}
    current = None
    for line in proc.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            current = report.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(.+?): (\d+) \[-Rpass", line)
        if m and current is not None and m.group(1) in fields:
            current[fields[m.group(1)]] = int(m.group(2))
    return report


if __name__ == "__main__":
    for p in build_all():
        print(p)
