"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/tile_gemm.h declares, validates arguments with the documented
status codes before touching HIP, and plans every benchmark workload the way
the kernels require."""
import ctypes
import json
from pathlib import Path

import pytest

import dense_tiled_gemm_tile_amd as tg
import seeded_inputs as si

GOLDEN = Path(__file__).resolve().parent / "golden"


def test_library_exports_every_declared_function():
    lib = tg.load_library()
    declared = tg.header_functions()
    assert {"tile_gemm", "tile_gemm_out", "tile_gemm_batched", "tile_gemm_query_plan",
            "tile_gemm_strerror"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name
    assert tg.abi_version() == 9


def test_library_neither_allocates_nor_synchronises():
    """The library borrows every buffer from the caller and only enqueues work
    (Tylo.jl manual, "Walk through GEMM", sections 2 and 4: views borrow
    storage, no hidden allocation or barrier): its dynamic symbol table
    imports no HIP allocation, free or synchronisation routine."""
    import shutil
    import subprocess

    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is not available")
    out = subprocess.run([nm, "-D", "--undefined-only", str(tg.LIB_PATH)], check=True, capture_output=True,
                         text=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    assert "hipLaunchKernel" in imported  # the table really is the dynamic imports
    forbidden = {name for name in imported
                 if name.startswith(("hipMalloc", "hipFree", "hipExtMalloc", "hipHostMalloc", "hipMallocAsync",
                                     "hipStreamSynchronize", "hipDeviceSynchronize", "hipEventSynchronize",
                                     "hipStreamWaitEvent", "hipMemcpy", "hipMemset"))}
    assert not forbidden, forbidden


def test_strerror_covers_every_status():
    for code, name in tg.STATUS.items():
        msg = tg.strerror(code)
        assert msg and msg != "unknown status", name
    assert tg.strerror(-1234) == "unknown status"


# fake but well-aligned device addresses: validation only inspects them
A, B, D = 0x7F0000000000, 0x7F0010000000, 0x7F0020000000


@pytest.mark.parametrize("args,code", [
    (dict(M=-1), -1), (dict(N=-5), -1), (dict(K=-1), -1), (dict(M=(1 << 30) + 1), -1),
    (dict(lda=63), -2), (dict(ldb=10), -2), (dict(ldd=63), -2),
    (dict(A=0), -3), (dict(B=0), -3), (dict(D=0), -3),
    (dict(A=A + 1), -4), (dict(D=D + 2), -4), (dict(dtype=3, B=B + 2), -4),
    (dict(dtype=0), -5), (dict(dtype=9), -5),
    (dict(D=A + 64), -6), (dict(D=B - 16), -6),
])
def test_validation_codes(args, code):
    p = dict(M=64, N=48, K=64, alpha=1.0, relu=0, A=A, lda=64, B=B, ldb=64, D=D, ldd=64, dtype=1)
    p.update(args)
    rc = tg.tile_gemm(p["M"], p["N"], p["K"], p["alpha"], p["relu"], p["A"], p["lda"], p["B"],
                      p["ldb"], p["D"], p["ldd"], p["dtype"], None)
    assert rc == code, tg.STATUS.get(rc, rc)
    info = tg.PlanInfo()
    rc2 = tg.load_library().tile_gemm_query_plan(p["M"], p["N"], p["K"], p["dtype"], p["A"], p["lda"],
                                                 p["B"], p["ldb"], p["D"], p["ldd"], ctypes.byref(info))
    assert rc2 == code


@pytest.mark.parametrize("args,code", [
    (dict(out=0), -5), (dict(out=9), -5),
    (dict(out=1, D=D + 1), -4), (dict(out=2, D=D + 3), -4), (dict(out=3, D=D + 2), -4),
    (dict(out=1, D=D + 2), None), (dict(out=2, D=D + 6), None),
    # the output range scales with the output element size
    (dict(out=3, D=A - 64 * 48 * 4 + 8), -6), (dict(out=1, D=A - 64 * 48 * 4 + 8), None),
])
def test_low_precision_output_validation(args, code):
    """tile_gemm_out validates the output type, D's alignment to it and the
    overlap of D's byte range, before any HIP call (no GPU here: a valid call
    reports the missing device)."""
    import torch

    p = dict(M=64, N=48, K=64, A=A, B=B, D=D, out=1)
    p.update(args)
    rc = tg.tile_gemm_out(p["M"], p["N"], p["K"], 1.0, 0, p["A"], 64, p["B"], 64, p["D"], 64, 1, p["out"],
                          None, -1)
    info = tg.PlanInfo()
    rq = tg.load_library().tile_gemm_query_plan_out(p["M"], p["N"], p["K"], 1, p["A"], 64, p["B"], 64,
                                                    p["D"], 64, p["out"], -1, ctypes.byref(info))
    assert rq == (0 if code is None else code)
    if code is None:
        code = 0 if torch.cuda.is_available() else -8
        if code == 0:
            pytest.skip("fake pointers cannot be launched on a GPU")
    assert rc == code, tg.STATUS.get(rc, rc)


def test_degenerate_shapes_need_no_operands():
    # M = 0 or N = 0: no-op, nothing is read or written, no device needed
    assert tg.tile_gemm(0, 5, 7, 1.0, 0, 0, 7, 0, 7, 0, 1, 1, None) == 0
    assert tg.tile_gemm(5, 0, 7, 1.0, 0, 0, 7, 0, 7, 0, 5, 1, None) == 0
    # K = 0: A and B are not read, so they may be NULL; D still required
    assert tg.query_plan(5, 4, 0, 1, 0, 1, 0, 1, D, 5).grid == 1
    with pytest.raises(tg.TileGemmError):
        tg.query_plan(5, 4, 0, 1, 0, 1, 0, 1, 0, 5)


def test_valid_call_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert tg.tile_gemm(64, 48, 64, 1.0, 0, A, 64, B, 64, D, 64, 1, None) == -8


def _plan(w: si.Workload, a=A, b=B, d=D, kernel_id=-1):
    return tg.query_plan(w.M, w.N, w.K, tg.DTYPE_CODES[w.dtype], a, w.lda, b, w.ldb, d, w.ldd, kernel_id)


def test_plans_for_the_workloads():
    W = si.WORKLOADS
    big = _plan(W["square_8192_bf16_relu"])
    assert (big.block_m, big.block_n, big.load_class, big.grid) == (256, 256, 16, 1024)
    assert big.lds_bytes <= 160 * 1024
    assert tg.kernel_info(big.kernel_id).load_class == 16  # a streaming instance
    assert _plan(W["square_8192_f16_relu"]).dtype == tg.F16
    # 2-byte aligned rows run directly (tile_gemm never copies the operands)
    ragged = _plan(W["ragged_strided_12289x5003x4099_bf16"])
    assert ragged.staged == 0 and ragged.load_class == 2 and (ragged.tiles_m, ragged.tiles_n) == (49, 20)
    assert tg.kernel_info(ragged.kernel_id).block_m == 256 and big.staged == 0
    assert big.kernel_id == 67  # the 16x16x32 wide kernel: a full round of tiles and 128 K stages
    assert _plan(W["square_8192_f16_relu"]).kernel_id == 68
    # small problems take small tiles so that more CUs get work (and are not staged)
    tiny = _plan(W["tiny_bounded_65x97x73_bf16"])
    assert tiny.staged == 0 and tiny.load_class == 2 and (tiny.block_m, tiny.grid) == (64, 4)
    mid = _plan(W["full_tile_1024_bf16"])
    assert (mid.block_m, mid.block_n, mid.grid) == (64, 64, 256)
    f32 = _plan(W["fp32_2048"])
    assert f32.dtype == tg.F32 and f32.grid == 256 and (f32.block_m, f32.block_k) == (128, 16)


def test_plan_alignment_classes_and_forced_instances():
    W = si.WORKLOADS["square_8192_bf16_relu"]
    for off_a, off_b, cls in ((4, 0, 4), (0, 2, 2)):
        p = _plan(W, a=A + off_a, b=B + off_b)
        assert p.staged == 0 and p.load_class == cls and p.grid == 1024
    w = si.Workload("mid", 300, 200, 130, "bf16", "uniform_pm1", 1.0, False, 130, 130, 300, 1, 2)
    assert (_plan(w, a=A + 4).load_class, _plan(w, a=A + 4).staged) == (4, 0)
    assert (_plan(w, b=B + 2).load_class, _plan(w, b=B + 2).staged) == (2, 0)
    # a 2-byte aligned operand cannot run an instance that needs 4-byte rows
    narrow = [k for k in range(tg.kernel_count()) if tg.kernel_info(k).load_class == 4
              and tg.kernel_info(k).dtype == tg.BF16]
    with pytest.raises(tg.TileGemmError) as e:
        _plan(W, b=B + 2, kernel_id=narrow[0])
    assert e.value.code == -9
    with pytest.raises(tg.TileGemmError):
        _plan(W, kernel_id=tg.kernel_count())


def test_every_instance_has_consistent_ownership_arithmetic():
    """acc/lane * threads == tile size, as in the worked plan of the Tylo manual
    (golden/tylo_plan_example.json): 32 accumulators x 128 threads own 64x64."""
    ex = json.loads((GOLDEN / "tylo_plan_example.json").read_text())
    tm, tn, _ = ex["tile_mnk"]
    assert ex["acc_per_thread"] * ex["threads"] == tm * tn
    assert ex["threads"] == 32 * ex["warps"][0] * ex["warps"][1]
    atom_m, atom_n, _ = ex["atom_mnk"]
    assert ex["warps"][0] * ex["reps"][0] * atom_m == tm and ex["warps"][1] * ex["reps"][1] * atom_n == tn
    for k in range(tg.kernel_count()):
        info = tg.kernel_info(k)
        assert info.kernel_id == k
        # K-sliced instances hold k_slices copies of the tile (summed at the end)
        assert info.acc_per_lane * info.threads == info.block_m * info.block_n * info.k_slices
        assert info.threads == 64 * info.waves_m * info.waves_n * info.k_slices
        assert info.wave_tile_m * info.waves_m == info.block_m
        assert info.wave_tile_n * info.waves_n == info.block_n
        bits = {tg.F32: 32, tg.E4M3: 8, tg.E5M2: 8, tg.E2M1: 4, tg.E2M3: 6, tg.E3M2: 6}.get(info.dtype, 16)
        row_bytes = info.block_k * bits // 8
        # a stage covers 64 or 128 bytes of each row (6-bit: 96 of a 128-byte LDS row)
        assert row_bytes in (64, 128) or (bits == 6 and row_bytes == 96)
        row_bytes = 128 if bits == 6 else row_bytes
        # every instance keeps at least its A stages in LDS, within the 160 KiB of a CU
        assert info.stages * info.block_m * row_bytes <= info.lds_bytes <= 160 * 1024


def test_row_stride_limited_instances_are_refused_for_huge_strides():
    """Instances that address a tile through 32-bit byte offsets (256 rows x
    stride < 2^31) refuse larger strides; the planner then takes another."""
    W = si.WORKLOADS["square_8192_bf16_relu"]
    huge = (1 << 22) + 64  # elements: 8 MiB + 128 bytes per bf16 row
    a, b, d = 0x100000000000, 0x200000000000, 0x300000000000  # far apart: no overlap
    small_plan = _plan(W)
    refused = []
    for k in range(tg.kernel_count()):
        info = tg.kernel_info(k)
        if info.dtype != tg.BF16:
            continue
        try:
            tg.query_plan(512, 512, W.K, tg.BF16, a, huge, b, huge, d, 512, k)
        except tg.TileGemmError as e:
            assert e.code == -9
            refused.append(k)
    assert refused, "no stride-limited instance"
    assert small_plan.kernel_id in refused  # the default for ordinary strides is one of them
    p = tg.query_plan(512, 512, W.K, tg.BF16, a, huge, b, huge, d, 512, -1)
    assert p.kernel_id not in refused and p.load_class == 16


@pytest.mark.parametrize("args,code", [
    (dict(batch=-1), -1), (dict(batch=65536), -1),
    (dict(sa=-1), -2), (dict(sb=-64), -2), (dict(sd=-1), -2), (dict(sa=(1 << 40) + 1), -2),
    (dict(sd=64 * 47 + 63), -2),                # outputs of consecutive products would overlap
    (dict(sd=64 * 48), None), (dict(sa=0, sb=0), None), (dict(batch=1, sd=0), None),
    (dict(batch=0, A=0, B=0, D=0), 0),          # nothing to do
    (dict(sa=4 * 64 * 64, D=A + 4 * 64 * 64 * 2 + 4096), -6),  # A's span reaches into D's
    (dict(sa=64 * 64 + 3), None),               # a batch stride that breaks 16-byte rows is legal
])
def test_batched_validation(args, code):
    """tile_gemm_batched's extra checks (batch range, strides, non-overlapping
    outputs, whole-span aliasing), before any HIP call."""
    import torch

    p = dict(M=64, N=48, K=64, A=A, B=B, D=D, sa=64 * 64, sb=48 * 64, sd=64 * 48 + 16, batch=4)
    p.update(args)
    rc = tg.tile_gemm_batched(p["M"], p["N"], p["K"], 1.0, 0, p["A"], 64, p["sa"], p["B"], 64, p["sb"],
                              p["D"], 64, p["sd"], p["batch"], 1, 3, None, -1)
    if code is None:
        if torch.cuda.is_available():
            pytest.skip("fake pointers cannot be launched on a GPU")
        code = -8
    assert rc == code, tg.STATUS.get(rc, rc)


def test_batched_plan_counts_every_product():
    """The plan of a batch weighs all its workgroups: 16 products of 1024^3
    bf16 fill the chip with 256x256 tiles (16 tiles each)."""
    w = si.WORKLOADS["batched_16x1024_bf16"]
    info = tg.PlanInfo()
    D2 = 0x7F4000000000
    rc = tg.load_library().tile_gemm_query_plan_batched(
        w.M, w.N, w.K, tg.BF16, A, w.lda, w.M * w.lda, B, w.ldb, w.N * w.ldb, D2, w.ldd, w.N * w.ldd,
        w.batch, tg.F32, -1, ctypes.byref(info))
    assert rc == 0
    assert (info.block_m, info.block_n, info.grid) == (256, 256, 256)
    single = _plan(si.WORKLOADS["full_tile_1024_bf16"])
    assert (single.block_m, single.block_n) == (64, 64)


def test_splitk_workspace_size_and_validation():
    """Split-K: workspace size, the splits range and the workspace checks, all
    before any HIP call."""
    import torch

    assert tg.splitk_workspace_bytes(1024, 512, 4) == 4 * 1024 * 512 * 4
    assert tg.splitk_workspace_bytes(1024, 512, 1) == 0
    assert tg.splitk_workspace_bytes(0, 512, 4) == 0
    assert tg.splitk_workspace_bytes(-1, 5, 2) == -1 and tg.splitk_workspace_bytes(5, 5, 257) == -1
    W = 0x7F8000000000
    M, N, K = 256, 128, 1024
    need = tg.splitk_workspace_bytes(M, N, 4)

    def call(splits=4, ws=W, ws_bytes=need, **kw):
        p = dict(A=A, B=B, D=D, lda=K)
        p.update(kw)
        return tg.tile_gemm_splitk(M, N, K, 1.0, 1, p["A"], p["lda"], p["B"], K, p["D"], M, tg.BF16, tg.F32,
                                   splits, ws, ws_bytes, None, -1)
    no_gpu = 0 if torch.cuda.is_available() else -8
    assert call(splits=-1) == -1 and call(splits=257) == -1
    assert tg.splitk_workspace_bytes(1024, 512, 0) == 64 * 1024 * 512 * 4
    assert call(ws=0) == -10 and call(ws_bytes=need - 1) == -10 and call(ws=W + 8) == -10
    assert call(ws=D) == -6                   # workspace on top of D
    assert call(lda=K - 1) == -2              # ordinary validation still applies
    if no_gpu:
        assert call() == -8
        # K with fewer stages than splits: the unused splits need no workspace
        assert tg.tile_gemm_splitk(M, N, 100, 1.0, 0, A, 100, B, 100, D, M, tg.BF16, tg.F32, 8, W,
                                   tg.splitk_workspace_bytes(M, N, 2), None, -1) == -8


def test_softmax_validation_without_gpu():
    """tile_gemm_softmax validates like tile_gemm_out; the fused path needs an
    instance whose tile spans N, the two-pass path an fp32 D."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    call = lambda N, out, kid=-1, lda=64: tg.tile_gemm_softmax(256, N, 64, 1.0, A, lda, B, 64, D, 256, tg.BF16,
                                                               out, None, kid)
    assert call(256, tg.BF16) == -8       # fused, valid: no device here
    assert call(1000, tg.F32) == -8       # two passes, valid
    assert call(1000, tg.BF16) == -1      # two passes need an fp32 D
    assert call(256, tg.BF16, lda=63) == -2
    assert call(256, 9) == -5
    big = [k for k in range(tg.kernel_count()) if tg.kernel_info(k).block_n == 256
           and tg.kernel_info(k).dtype == tg.BF16 and tg.kernel_info(k).load_class != 16]
    wide = [k for k in range(tg.kernel_count()) if tg.kernel_info(k).load_class == 16
            and tg.kernel_info(k).dtype == tg.BF16]
    codes = {call(256, tg.F32, k) for k in big}
    assert codes == {-8, -9}                # some 256-wide instances carry the softmax epilogue, some not
    assert call(256, tg.F32, wide[0]) == -9   # streaming instances have no softmax epilogue


def test_staged_workspace_size_and_validation():
    """tile_gemm_staged: workspace size formula, and the argument checks that
    happen before any HIP call."""
    M, N, K = 12289, 5003, 4099
    rb = -(-K * 2 // 128) * 128
    assert rb == 8320
    assert tg.staged_workspace_bytes(M, N, K, tg.BF16) == -(-M * rb // 256) * 256 + N * rb
    assert tg.staged_workspace_bytes(M, N, 33, tg.F32) == -(-M * 256 // 256) * 256 + N * 256
    assert tg.staged_workspace_bytes(M, N, 0, tg.BF16) == 0
    assert tg.staged_workspace_bytes(0, N, K, tg.BF16) == 0
    assert tg.staged_workspace_bytes(M, N, K, 9) == -1
    assert tg.staged_workspace_bytes(-1, N, K, tg.BF16) == -1
    m, n, k = 300, 200, 130
    need = tg.staged_workspace_bytes(m, n, k, tg.BF16)
    W = 0x7F4000000000  # far from A, B and D
    call = lambda ws, nbytes, mode, d=D: tg.tile_gemm_staged(m, n, k, 1.0, 0, A + 2, k, B, k, d, m, tg.BF16, tg.F32,
                                                             ws, nbytes, None, mode)
    assert call(0, 0, 1) == -10            # mode 1 needs a workspace
    assert call(W, need - 1, 1) == -10     # too short
    assert call(W + 16, need, 1) == -10    # not 256-byte aligned
    assert call(W, need, 2) == -9          # unknown mode
    assert call(A - 256, need, 1) == -6    # overlaps A
    assert call(W, need, 1, d=W + 512) == -6   # overlaps D
    import torch
    if not torch.cuda.is_available():
        assert call(W, need, 1) == -8      # valid: only the device is missing
        assert call(0, 0, -1) == -8        # automatic without a workspace: direct plan
        assert call(0, 0, 0) == -8


def test_staging_decision_scales_with_the_problem():
    """tile_gemm_staged (mode -1) copies misaligned rows only when the copy
    pays and the caller's workspace holds the copies: 16384^3 and the ragged
    workload yes (the direct 2-byte-row path of the wide kernel runs about
    0.8 of the aligned rate), 4096^3 and 1024^3 no (the copy costs more than
    it saves); aligned rows never; mode 1 always (with a workspace), mode 0
    never."""
    A2, B2, D2, W2 = 0x100000000000, 0x200000000000, 0x300000000000, 0x400000000000
    for n, staged in ((16384, 1), (4096, 0), (1024, 0)):
        need = tg.staged_workspace_bytes(n, n, n, tg.BF16)
        q = lambda b, mode=-1, ws=W2, nbytes=need: tg.query_plan_staged(n, n, n, tg.BF16, A2, n, b, n, D2, n, tg.F32,
                                                                        ws, nbytes, mode)
        p = q(B2 + 2)
        assert p.staged == staged, n
        if staged:
            assert p.load_class == 16 and tg.kernel_info(p.kernel_id).load_class == 16
        assert q(B2 + 2, ws=0, nbytes=0).staged == 0          # no workspace: the direct plan
        assert q(B2 + 2, nbytes=need - 1).staged == 0         # too short: the direct plan
        assert q(B2).staged == 0                              # aligned rows never need it
        assert q(B2, mode=1).staged == 1 and q(B2 + 2, mode=0).staged == 0
        with pytest.raises(tg.TileGemmError) as e:
            q(B2, mode=1, ws=0, nbytes=0)
        assert e.value.code == -10
    # the ragged workload: rows of K + 8 elements (2-byte aligned), D columns of M + 16
    M, N, K = 12289, 5003, 4099
    need = tg.staged_workspace_bytes(M, N, K, tg.BF16)
    p = tg.query_plan_staged(M, N, K, tg.BF16, A2, K + 8, B2, K + 8, D2, M + 16, tg.F32, W2, need, -1)
    assert p.staged == 1 and tg.kernel_info(p.kernel_id).load_class == 16


def test_plan_choices_follow_the_kernel_trace_table():
    """The automatic choice for aligned bf16 operands is the instance that was
    fastest in the kernel trace for each of these shapes (the K-sliced 64^2
    when at most half the CUs get a tile, small streaming 64^2 for 1024^2
    outputs, 128^2 at 2048^2, the wide kernel beyond: on 16x16x32 MFMAs when
    K has at least 16 stages, else on 32x32x16)."""
    A2, B2, D2 = 0x7F0000000000, 0x7F4000000000, 0x7F8000000000
    expect = {(1024, 1024, 1024): 14, (2048, 2048, 2048): 16, (512, 512, 16384): 48, (1024, 1024, 4096): 14,
              (2048, 2048, 8192): 16, (4096, 4096, 1024): 67, (3072, 3072, 3072): 67, (4096, 4096, 4096): 67,
              (8192, 8192, 1024): 67, (8192, 8192, 2048): 67, (4096, 4096, 512): 0, (8192, 8192, 768): 0}
    for (M, N, K), kid in expect.items():
        assert tg.query_plan(M, N, K, tg.BF16, A2, K, B2, K, D2, M).kernel_id == kid, (M, N, K)


def test_fp32_plan_choices():
    """fp32 operands: the wide kernel at 4096^3 (ids 8, or 9 with plain
    stores when D columns are not line-aligned), the 128^2 streaming instance
    at 2048^3, the register-staged 64^2 for 1024x1024x4096."""
    A2, B2, D2 = 0x7F0000000000, 0x7F4000000000, 0x7F8000000000
    q = lambda M, N, K, ldd=None: tg.query_plan(M, N, K, tg.F32, A2, K, B2, K, D2, ldd or M).kernel_id
    assert q(4096, 4096, 4096) == 8
    assert q(4096, 4096, 4096, ldd=4097) == 9
    assert q(2048, 2048, 2048) == 18
    assert q(1024, 1024, 4096) == 26


def test_scaled_entry_point_validation():
    """tile_gemm_scaled: scales only with 8-bit operands, whole dwords of
    scales per 128-k stage, 4-byte aligned, not overlapping D."""
    M, N, K = 300, 200, 300
    S = 0x7F4000000000  # far from A, B and D
    need = 4 * -(-K // 128)
    call = lambda dt, sa, la, sb, lb, d=D: tg.tile_gemm_scaled(M, N, K, 1.0, 0, A, K, sa, la, B, K, sb, lb, d, M, dt,
                                                               tg.F32, None, -1)
    assert call(tg.BF16, S, need, 0, 0) == -5
    assert call(tg.E4M3, S, need - 4, 0, 0) == -2
    assert call(tg.E4M3, 0, 0, S, need + 2, ) == -2
    assert call(tg.E4M3, S + 2, need, 0, 0) == -4
    assert call(tg.E4M3, S, need, 0, 0, d=S + 64) == -6
    import torch
    if not torch.cuda.is_available():
        assert call(tg.E4M3, S, need, S + (1 << 20), need) == -8
        assert call(tg.E5M2, 0, 0, 0, 0) == -8
    # 8-bit plans: rows aligned to a single byte take the 1-byte class
    p = tg.query_plan(M, N, K, tg.E4M3, A + 1, K, B, K, D, M)
    assert p.load_class == 1 and tg.kernel_info(p.kernel_id).dtype == tg.E4M3
    assert tg.query_plan(8192, 8192, 8192, tg.E4M3, A, 8192, B, 8192, D, 8192).block_k == 128


def test_4bit_validation_and_plans():
    """Packed 4-bit operands: rows must start on a byte (even strides), block
    scales come in 16-byte pieces per two 256-k stages (16-byte aligned),
    staging is refused, and the plans take the 4-bit instances: the
    streaming one for aligned rows (256 k per stage), the register-staged one
    for rows on odd bytes (the register-staged ones for small or scaled
    products)."""
    import torch

    A2, B2, D2, S2, W2 = 0x7F0000000000, 0x7F4000000000, 0x7F8000000000, 0x7FC000000000, 0x7E0000000000
    M, N, K = 300, 200, 701
    gpu = torch.cuda.is_available()
    ok = 0 if gpu else -8
    ex = lambda lda, ldb, a=A2, b=B2: tg.tile_gemm_ex(M, N, K, 1.0, 0, a, lda, b, ldb, D2, M, tg.E2M1, None, -1)
    if not gpu:
        assert ex(702, 704) == -8                 # valid: reaches the device check
        assert ex(702, 704, a=A2 + 1) == -8       # byte alignment is enough
    assert ex(703, 704) == -2 and ex(702, 705) == -2   # a row would start mid-byte
    assert ex(700, 704) == -2                          # lda < K
    # batch strides must keep whole bytes too
    assert tg.tile_gemm_batched(M, N, K, 1.0, 0, A2, 702, 702 * M + 1, B2, 702, 702 * N, D2, M, M * N, 2, tg.E2M1,
                                tg.F32, None, -1) == -2
    # staging: packed operands are never staged
    assert tg.staged_workspace_bytes(M, N, K, tg.E2M1) == -1
    assert tg.tile_gemm_staged(M, N, K, 1.0, 0, A2, 702, B2, 702, D2, M, tg.E2M1, tg.F32, W2, 1 << 30, None,
                               1) == -5
    # scales: 16*ceil(K/512) bytes per row, multiples of 16, 16-byte aligned
    need = 16 * -(-K // 512)
    sc = lambda sa, la, sb=0, lb=0, lda=704: tg.tile_gemm_scaled(M, N, K, 1.0, 0, A2, lda, sa, la, B2, lda, sb, lb, D2,
                                                               M, tg.E2M1, tg.F32, None, -1)
    assert sc(S2, need - 16) == -2 and sc(S2, need + 4) == -2
    assert sc(S2 + 4, need) == -4
    p = tg.query_plan_scaled(M, N, K, tg.E2M1, A2, 706, S2, need, B2, 706, 0, 0, D2, M)
    assert p.load_class == 1 and p.block_scales == 1   # rows on odd bytes: the register-staged instance
    if not gpu:
        assert sc(S2, need, S2 + (1 << 20), need) == -8
    # plans
    p = tg.query_plan(8192, 8192, 8192, tg.E2M1, A2, 8192, B2, 8192, D2, 8192)
    assert p.kernel_id == 51 and p.block_k == 256 and p.load_class == 16
    assert tg.query_plan(8192, 8192, 8192, tg.E2M1, A2, 8192, B2, 8192, D2, 8193).kernel_id == 52
    p = tg.query_plan(4096, 4096, K, tg.E2M1, A2, 706, B2, 706, D2, 4096)
    assert p.kernel_id == 53 and p.load_class == 1
    p = tg.query_plan(M, N, K, tg.E2M1, A2, 706, B2, 706, D2, M)   # small: the 64 x 64 register-staged one
    assert p.kernel_id == 62 and p.load_class == 1
    p = tg.query_plan_scaled(8192, 8192, 8192, tg.E2M1, A2, 8192, S2, 256, B2, 8192, S2 + (1 << 24), 256, D2, 8192)
    assert p.kernel_id == 54 and p.block_scales == 1
    assert tg.kernel_info(51).block_scales == 0 and tg.kernel_info(55).block_scales == 1
    assert ok in (0, -8)


def test_6bit_validation_and_plans():
    """Packed 6-bit operands: rows must start on a byte (strides multiples of
    4 elements), the streaming instances take 16-byte aligned rows (strides
    multiples of 64 elements) and the register-staged ones any other, block
    scales follow the 8-bit rule (a dword per 128-k stage), a stage is 128
    elements (96 bytes), and staging is refused."""
    import torch

    A2, B2, D2, S2, W2 = 0x7F0000000000, 0x7F4000000000, 0x7F8000000000, 0x7FC000000000, 0x7E0000000000
    M, N, K = 300, 200, 701
    for dt in (tg.E2M3, tg.E3M2):
        ex = lambda lda, ldb: tg.tile_gemm_ex(M, N, K, 1.0, 0, A2, lda, B2, ldb, D2, M, dt, None, -1)
        assert ex(702, 704) == -2 and ex(704, 706) == -2         # a row would start mid-byte
        p = tg.query_plan(M, N, K, dt, A2, 704, B2, 708, D2, M)    # rows on 3-byte boundaries
        assert p.load_class == 1 and p.block_m in (64, 256) and p.block_k == 128
        if not torch.cuda.is_available():
            assert ex(704, 768) == -8 and ex(704, 708) == -8
        assert tg.staged_workspace_bytes(M, N, K, dt) == -1
        p = tg.query_plan(8192, 8192, 8192, dt, A2, 8192, B2, 8192, D2, 8192)
        assert p.block_k == 128 and p.load_class == 16 and p.block_scales == 0
        q = tg.query_plan_scaled(8192, 8192, 8192, dt, A2, 8192, S2, 256, B2, 8192, 0, 0, D2, 8192)
        assert q.block_scales == 1 and q.kernel_id != p.kernel_id
        sc = lambda la: tg.tile_gemm_scaled(M, N, K, 1.0, 0, A2, 704, S2, la, B2, 768, 0, 0, D2, M, dt, tg.F32, None,
                                            -1)
        assert sc(4 * 5) == -2 and sc(4 * 6 + 2) == -2
        if not torch.cuda.is_available():
            assert sc(4 * 6) == -8


def test_8bit_staging_and_streaming_plans():
    """8-bit operands: aligned rows run the streaming 8-bit instance; a large
    product with 1-byte aligned rows runs the 1-byte loader directly, or is
    staged onto the streaming instance through tile_gemm_staged; a small one
    is not staged."""
    A2, B2, D2, W2 = 0x7F0000000000, 0x7F4000000000, 0x7F8000000000, 0x7FC000000000
    p = tg.query_plan(4096, 4096, 4096, tg.E4M3, A2, 4096, B2, 4096, D2, 4096)
    assert p.staged == 0 and p.kernel_id == 10 and p.block_k == 128
    p = tg.query_plan(4096, 4096, 4096, tg.E5M2, A2 + 1, 4097, B2, 4097, D2, 4096)
    assert p.staged == 0 and p.load_class == 1
    need = tg.staged_workspace_bytes(4096, 4096, 4096, tg.E5M2)
    p = tg.query_plan_staged(4096, 4096, 4096, tg.E5M2, A2 + 1, 4097, B2, 4097, D2, 4096, tg.F32, W2, need)
    assert p.staged == 1 and p.kernel_id == 11
    p = tg.query_plan(300, 200, 130, tg.E4M3, A2 + 1, 131, B2, 131, D2, 300)
    assert p.staged == 0 and p.load_class == 1


def test_scaled_call_refuses_instances_without_scales():
    """A forced instance that does not apply block scales (the plain 8-bit
    streaming one) is refused before any device call, as is a scaled
    streaming instance whose scale rows are too long for its 32-bit offsets."""
    A2, B2, D2, S2 = 0x7F0000000000, 0x7F4000000000, 0x7F8000000000, 0x7FC000000000
    M = N = K = 4096
    need = 4 * (K // 128)
    rc = tg.tile_gemm_scaled(M, N, K, 1.0, 0, A2, K, S2, need, B2, K, 0, 0, D2, M, tg.E4M3, tg.F32, None, 10)
    assert rc == -9
    big = 1 << 24  # bytes per scale row, beyond 8 MiB
    rc = tg.tile_gemm_scaled(M, N, K, 1.0, 0, A2, K, S2, big, B2, K, 0, 0, D2, M, tg.E4M3, tg.F32, None, 12)
    assert rc == -9
    # the automatic choice with scales is the scaled streaming instance
    p = tg.query_plan_scaled(M, N, K, tg.E4M3, A2, K, S2, need, B2, K, 0, 0, D2, M)
    assert p.kernel_id == 12 and tg.kernel_info(12).load_class == 16


def _chosen_instances():
    """Every instance some automatic plan picks, over a grid of shapes, dtypes,
    row alignments, D line alignments and entry points."""
    A2, B2, D2, S2, W2 = 0x100000000000, 0x200000000000, 0x300000000000, 0x400000000000, 0x500000000000
    bits_of = {tg.BF16: 16, tg.F16: 16, tg.F32: 32, tg.E4M3: 8, tg.E5M2: 8, tg.E2M1: 4, tg.E2M3: 6, tg.E3M2: 6}
    dims = [17, 65, 200, 512, 1024, 2048, 4096, 8192, 12289]
    Ks = [9, 73, 1024, 4099, 8192, 16384]
    chosen = set()

    def stride(K, bits, cls):
        for ld in range(K, K + 256):
            if (ld * bits) % 8:
                continue
            b = ld * bits // 8
            c = 16 if b % 16 == 0 else 4 if b % 4 == 0 else 2 if b % 2 == 0 else 1
            if c == cls:
                return ld
        return None

    for dt, bits in bits_of.items():
        classes = [c for c in (16, 4, 2, 1) if 8 * c >= bits]
        for M in dims:
            for N in dims[::2]:
                for K in Ks:
                    for cls in classes:
                        ld = stride(K, bits, cls)
                        for ldd in (-(-M // 32) * 32, M + 1):
                            chosen.add(tg.query_plan(M, N, K, dt, A2, ld, B2, ld, D2, ldd, -1, tg.F32).kernel_id)
                            if bits <= 8:
                                sc = 16 * -(-K // 512) if bits == 4 else 4 * -(-K // 128)
                                chosen.add(tg.query_plan_scaled(M, N, K, dt, A2, ld, S2, sc, B2, ld, 0, 0, D2,
                                                                ldd).kernel_id)
                            elif N <= 256:
                                p = tg.query_plan_softmax(M, N, K, dt, A2, ld, B2, ld, D2, ldd)
                                chosen.add(p.kernel_id)
        # operand rows longer than 8 MiB (6-bit instances address rows through
        # 32-bit offsets only)
        K = -(-((1 << 23) * 8 // bits + 64) // 64) * 64
        if bits != 6:
            chosen.add(tg.query_plan(8192, 8192, K, dt, A2, K, B2, K, D2, 8192, -1, tg.F32).kernel_id)
    chosen.discard(-1)
    return chosen


def test_every_instance_is_chosen_by_some_plan():
    """The instance table holds only instances that an automatic plan picks
    for some call (no experiment variants ship)."""
    chosen = _chosen_instances()
    assert chosen == set(range(tg.kernel_count())), sorted(set(range(tg.kernel_count())) - chosen)


def test_noalloc_splitk_refuses_partials_beyond_the_static_scratch():
    """tile_gemm_splitk_noalloc checks the partials against its static scratch
    before any HIP call (no GPU here: a call that fits reports the device)."""
    import torch

    M = N = 2048
    K = 8192
    call = lambda splits: tg.tile_gemm_splitk_noalloc(M, N, K, 1.0, 0, A, K, B, K, D, M, tg.BF16, tg.F32, splits,
                                                      None, -1)
    assert call(3) == -10                      # 3 x 16 MiB > 32 MiB
    assert call(-1) == -1 and call(257) == -1
    if not torch.cuda.is_available():
        assert call(2) == -8                   # exactly 32 MiB fits
        assert call(0) == -8
