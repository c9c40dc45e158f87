"""Build step for the HIP library: compiles csrc/ into an in-tree shared
library for gfx950 with hipcc (run ``python -m dense_tiled_gemm_tile_amd.build``)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "_lib" / "libtile_gemm.so"
SOURCES = [CSRC / "api.cpp", CSRC / "gemm_kernels.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # keep packed-fp32 VALU forms out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False) -> Path:
    """Compile every source for gfx950 and link the shared library (always rebuilds)."""
    LIB.parent.mkdir(parents=True, exist_ok=True)
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [hipcc(), *compile_flags(), "-shared", "-o", str(tmp), *map(str, SOURCES)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def asm(out_dir: Path) -> list[Path]:
    """Write the gfx950 assembly of the kernels (our own build) for inspection."""
    out_dir.mkdir(parents=True, exist_ok=True)
    out = out_dir / "gemm_kernels-gfx950.s"
    cmd = [hipcc(), *compile_flags(), "--cuda-device-only", "-S", "-o", str(out), str(CSRC / "gemm_kernels.hip")]
    subprocess.run(cmd, check=True)
    return [out]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
