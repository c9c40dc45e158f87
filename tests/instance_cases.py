"""Shared helpers of the every-instance GPU tests: operand type names and
leading strides that give operand rows exactly an instance's alignment class."""
from __future__ import annotations

import dense_tiled_gemm_tile_amd as tg

DT_NAMES = {tg.BF16: "bf16", tg.F16: "f16", tg.F32: "f32", tg.E4M3: "e4m3", tg.E5M2: "e5m2"}
ELEM_SIZE = {"bf16": 2, "f16": 2, "f32": 4, "e4m3": 1, "e5m2": 1}


def dtype_name(info) -> str:
    return DT_NAMES[info.dtype]


def unpacked_instances() -> list:
    """Ids of the instances whose operands are whole bytes or more; the
    packed 4-bit instances have tests of their own (test_gpu_fp4.py)."""
    return [k for k in range(tg.kernel_count()) if tg.kernel_info(k).dtype in DT_NAMES]


def strides_for_class(cls: int, K: int, es: int):
    """(lda, ldb) >= K, in elements, whose row byte offsets (from a 256-byte
    aligned base) are aligned to exactly `cls` bytes for odd rows."""
    def smallest(residue):  # smallest ld >= K with ld*es = residue (mod 16)
        ld = K
        while (ld * es) % 16 != residue:
            ld += 1
        return ld
    if cls == 16:
        lda = smallest(0)
        return lda, lda + 16 // es
    if cls == 4:
        lda = smallest(4)
        return lda, smallest(4) + 16 // es
    if cls == 2:
        lda = smallest(2 if es == 2 else 6)  # 16-bit: 2 (mod 16); 8-bit: 6 (mod 16)
        return lda, lda + 8 // es
    lda = smallest(1 if es == 1 else 0)
    return lda, lda + 2
