"""Build step for the HIP library: compiles csrc/ into an in-tree shared
library for gfx950 with hipcc (run ``python -m dense_tiled_gemm_tile_amd.build``).

Every translation unit is compiled to its own object in parallel (the kernel
instances are spread over several units for that reason), then the objects
are linked into ``_lib/libtile_gemm.so``."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "_lib" / "libtile_gemm.so"
# host-side units first, then the kernel units (largest first, so the
# parallel build ends sooner)
SOURCES = [CSRC / "gemm_wide16.hip", CSRC / "gemm_rs.hip", CSRC / "gemm_wide8.hip", CSRC / "gemm_wide32.hip",
           CSRC / "gemm_wide4.hip", CSRC / "gemm_wide6.hip", CSRC / "gemm_wide_m16.hip", CSRC / "gemm_stream.hip", CSRC / "gemm_kslice.hip",
           CSRC / "gemm_aux.hip",
           CSRC / "api.cpp", CSRC / "kernel_table.cpp"]
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


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n, len(SOURCES)))


def build(verbose: bool = False) -> Path:
    """Compile every source for gfx950 and link the shared library (always rebuilds)."""
    LIB.parent.mkdir(parents=True, exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="tg_build_") as tmpdir:
        objs = [Path(tmpdir) / (src.name + ".o") for src in SOURCES]

        def compile_one(pair):
            src, obj = pair
            cmd = [hipcc(), *compile_flags(), "-c", "-o", str(obj), str(src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)

        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            list(pool.map(compile_one, zip(SOURCES, objs)))
        tmp = LIB.with_name(LIB.name + ".tmp")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", str(tmp), *map(str, objs)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def asm(out_dir: Path, source: str = "gemm_wide16.hip") -> list[Path]:
    """Write the gfx950 assembly of one kernel unit (our own build) for inspection."""
    out_dir.mkdir(parents=True, exist_ok=True)
    out = out_dir / (Path(source).stem + "-gfx950.s")
    cmd = [hipcc(), *compile_flags(), "--cuda-device-only", "-S", "-o", str(out), str(CSRC / source)]
    subprocess.run(cmd, check=True)
    return [out]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
