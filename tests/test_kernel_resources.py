"""Register and scratch budget of the wide-kernel instances, checked on the
host from the gfx950 assembly of our own build (no GPU needed).

The wide kernels use the whole register file (256 accumulators in AGPRs and
up to 256 VGPRs); a few bytes of spill per lane are tolerated only outside
the main loop.  A spill reload inside the loop comes with a wait for every
memory operation in flight (measured: it drained the LDS-DMA copies and cost
the block-scaled 8-bit instances a sixth of their throughput), so any scratch
access between a loop header and its back-edge fails this test.
"""
from __future__ import annotations

import re
import shutil
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

from dense_tiled_gemm_tile_amd import build as tgbuild

UNITS = ["gemm_wide16.hip", "gemm_wide8.hip", "gemm_wide32.hip", "gemm_wide4.hip", "gemm_wide6.hip",
         "gemm_wide_m16.hip"]


@pytest.fixture(scope="module")
def wide_asm():
    try:
        tgbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory(prefix="tg_asm_") as tmp:
        with ThreadPoolExecutor(len(UNITS)) as pool:
            outs = list(pool.map(lambda u: tgbuild.asm(Path(tmp), u)[0], UNITS))
        yield "\n".join(p.read_text() for p in outs)


def _kernels(text: str):
    """(name, body lines, metadata dict) of every wide kernel in the assembly."""
    meta = {}
    for block in re.findall(r"^  - \.agpr_count:.*?(?=^  - \.agpr_count:|^amdhsa\.target|\Z)", text, re.S | re.M):
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        meta[name] = {k: int(v) for k, v in re.findall(r"\.(agpr_count|vgpr_count|private_segment_fixed_size):\s+(\d+)",
                                                         block)}
    for name, body in re.findall(r"^(_ZN2tg(?:16gemm_wide_kernel|20gemm_wide_m16_kernel)\w+):[^\n]*\n(.*?)^\.Lfunc_end",
                                 text, re.S | re.M):
        yield name, body.split("\n"), meta[name]


def _loops(lines):
    """(header, back-edge) line index pairs of the loops in a function body
    (the compiler marks loop headers with a comment; the label is on that
    line or the one before)."""
    out = []
    for h, line in enumerate(lines):
        if "Loop Header" not in line:
            continue
        lab = next(lines[i] for i in range(h, -1, -1) if lines[i].startswith(".LBB"))
        label = lab.split(":")[0]
        back = [i for i, l in enumerate(lines) if i > h and re.search(r"s_c?branch\w* " + re.escape(label) + r"\b", l)]
        if back:
            out.append((h, max(back)))
    return out


def test_wide_kernels_keep_their_loops_free_of_spills(wide_asm):
    seen = 0
    for name, lines, meta in _kernels(wide_asm):
        seen += 1
        # template arguments: <DT, GM, NS, RS, ADDR, SCHED, EPI, LC>, or
        # <DT, GM, EPI> for the 16x16x32 kernel (no softmax epilogue)
        args = [int(a) for a in re.findall(r"Li(\d+)E", name)]
        epi = args[6] if "gemm_wide_kernel" in name else 0
        loops = _loops(lines)
        assert loops, name
        # the K loop: the innermost loop with MFMAs (an outer loop walks the tiles)
        mfma_loop = [(a, b) for a, b in loops if any("v_mfma" in lines[i] for i in range(a, b + 1))
                     and not any(a < h <= b for h, _ in loops)]
        assert len(mfma_loop) == 1, (name, loops)
        a, b = mfma_loop[0]
        spills = [lines[i].strip() for i in range(a, b + 1) if re.search(r"\bscratch_(load|store)", lines[i])]
        assert not spills, (name, spills[:4])
        assert meta["agpr_count"] == 256, (name, meta)      # the 128 x 128 accumulator tile of a wave
        assert meta["vgpr_count"] <= 512, (name, meta)
        # a few bytes of spill outside the loop (12-20 measured); the softmax
        # epilogue (EPI bit 3) takes more
        limit = 128 if epi & 8 else 24
        assert meta["private_segment_fixed_size"] <= limit, (name, meta)
    assert seen >= 32  # every wide instance of the six units


def test_m16_copies_follow_their_own_m0_writes(wide_asm):
    """The 16x16x32 kernel loads M0 once per group of four LDS-DMA copies with
    its own `s_mov_b32 m0` + `s_nop 0`, and the copies read M0 without naming
    it: so no other instruction may write or read M0 in those kernels, every
    M0 write must carry its wait state, and no copy may come before the first
    write."""
    seen = 0
    for name, body in re.findall(r"^(_ZN2tg20gemm_wide_m16_kernel\w+):[^\n]*\n(.*?)^\.Lfunc_end", wide_asm, re.S | re.M):
        seen += 1
        lines = [l.split(";")[0].strip() for l in body.split("\n")]
        lines = [l for l in lines if l and not (l.startswith(".") and not l.startswith(".LBB"))]
        writes = [i for i, l in enumerate(lines) if re.match(r"s_\w+\s+m0\s*,", l)]
        assert writes, name
        for i in writes:
            assert lines[i].startswith("s_mov_b32 m0,") and lines[i + 1] == "s_nop 0", (name, lines[i:i + 2])
        loads = [i for i, l in enumerate(lines) if l.startswith("buffer_load") and l.endswith(" lds")]
        assert loads and loads[0] > writes[0], name
        others = [l for l in lines if re.search(r"\bm0\b", l) and not l.startswith("s_mov_b32 m0,")]
        assert not others, (name, others[:3])
    assert seen == 4
