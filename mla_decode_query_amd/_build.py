"""Builds libmlaq.so in-tree with hipcc for gfx950.

    python -m mla_decode_query_amd._build

Every HIP source is compiled with packed-FP32 code generation switched off
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know the feature, which is harmless. ``-ffp-contract=off`` keeps every
multiply and add as written (the epilogue's division correction relies on
explicit FMAs only).
"""

from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libmlaq.so"
SOURCES = [CSRC / "mlaq_kernels.hip", CSRC / "mlaq_uv.hip", CSRC / "mlaq_attn.hip", CSRC / "mlaq_scratch.hip",
           CSRC / "mlaq_api.cpp"]
# Measurement floors used by bench.py (not part of the fused path).
DIAG_LIB = PKG / "libmlaq_diag.so"
DIAG_SOURCES = [CSRC / "mlaq_diag.hip"]
HEADERS = [ROOT / "include" / "mlaq.h", CSRC / "mlaq_internal.h", CSRC / "mlaq_device.h"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
    # MFMA accumulators in ordinary VGPRs (gfx90a+ form): saves the AGPR read-back
    # of every partial tile before the LDS reduction.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # Kernel-argument preloading (gfx950): the first 14 dwords of a kernel's
    # scalar arguments arrive in SGPRs with the wave, so no wave waits for a
    # kernel-argument load before its first memory request (the code object
    # keeps a load-based entry for firmware without it). Kernels whose early
    # arguments fit take scalar arguments, not a struct, for this.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


def build(out: Path | None = None, extra_flags: list[str] | None = None, quiet: bool = True,
          sources: list[Path] | None = None) -> Path:
    """Compile the sources (default: the fused-path library) into one shared
    library; returns its path."""
    out = Path(out) if out is not None else LIB
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{ROOT / 'include'}", f"-I{CSRC}",
           "-o", str(tmp), *map(str, sources or SOURCES)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if not quiet:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


def build_all(quiet: bool = True) -> list[Path]:
    """The fused-path library and the benchmark's floor library."""
    return [build(quiet=quiet), build(DIAG_LIB, quiet=quiet, sources=DIAG_SOURCES)]


def is_stale(lib: Path = LIB) -> bool:
    if not lib.exists():
        return True
    t = lib.stat().st_mtime
    return any(p.stat().st_mtime > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    for p in build_all(quiet=False):
        print(p)
