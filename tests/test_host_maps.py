"""Index maps of the kernels (csrc/tile_math.h), checked on the host: tile
order bijection, unique and conflict-free LDS staging, conflict-free fragment
reads with matching k sets, and accumulator ownership (see
tests/tile_math_check.cpp for the list)."""
import subprocess
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent


def test_index_map_properties(tmp_path):
    exe = tmp_path / "tile_math_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror",
                    f"-I{ROOT / 'dense_tiled_gemm_tile_amd' / 'csrc'}",
                    str(ROOT / "tests" / "tile_math_check.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
