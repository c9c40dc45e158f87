"""Staged operand copies (tile_gemm_staged, with the caller's workspace)
against the oracle, on the GPU.

The staging launch copies A and B into 16-byte aligned rows padded with zeros
to whole K stages; the product of the copies must equal the oracle's result
exactly on integer data (the padding adds exact zeros) and leave D's padding
alone.  Operand storage carries NaN past K in every row, so a copy that read
beyond K would show.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_tiled_gemm_tile_amd as tg
import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

DT = {"bf16": tg.BF16, "f16": tg.F16, "f32": tg.F32, "e4m3": tg.E4M3, "e5m2": tg.E5M2}


def _log(msg):
    print(msg, flush=True)


def _device_operand(st: torch.Tensor, off: int):
    """Device copy of a row-major storage starting `off` elements into a flat
    buffer (so that off = 1 makes every row start misaligned)."""
    dev = torch.device("cuda:0")
    n = st.numel() + off + 8
    if st.element_size() == 1:  # 8-bit formats: zero bytes, viewed as the format
        flat = torch.zeros(n, dtype=torch.uint8, device=dev).view(st.dtype)
    else:
        flat = torch.zeros(n, dtype=st.dtype, device=dev)
    flat[off:off + st.numel()] = st.reshape(-1).to(dev)
    return flat, flat.data_ptr() + off * flat.element_size()


def run(A_st, B_st, M, N, K, alpha, relu, dt, mode, a_off=0, b_off=0, ldd=None, workspace="fit"):
    dev = torch.device("cuda:0")
    ldd = M if ldd is None else ldd
    A_keep, pa = _device_operand(A_st, a_off)
    B_keep, pb = _device_operand(B_st, b_off)
    D = si.out_storage(M, N, ldd).to(dev)
    need = tg.staged_workspace_bytes(M, N, K, DT[dt])
    ws = None
    if workspace == "fit":
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        ws.fill_(0xFF)  # NaN-like garbage: prior contents are irrelevant
        wp, wn = ws.data_ptr(), ws.numel()
    elif workspace == "short":
        ws = torch.empty(max(need // 2, 256), dtype=torch.uint8, device=dev)
        wp, wn = ws.data_ptr(), ws.numel()
    else:
        wp, wn = 0, 0
    rc = tg.tile_gemm_staged(M, N, K, alpha, relu, pa, A_st.shape[1], pb, B_st.shape[1], D.data_ptr(), ldd, DT[dt],
                             tg.F32, wp, wn, torch.cuda.current_stream().cuda_stream, mode)
    assert rc == 0, tg.strerror(rc)
    torch.cuda.synchronize()
    del A_keep, B_keep, ws
    return D.cpu()


def check_exact(D_st, A_st, B_st, M, N, K, alpha, relu, dt):
    ref, _ = oracle.gemm(M, N, K, alpha, relu, si.bits(A_st), A_st.shape[1], si.bits(B_st), B_st.shape[1], dt)
    d = D_st[:, :M].double().numpy()
    bad = np.argwhere(d != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first {tuple(bad[0])}: {d[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
    assert bool((D_st[:, M:] == si.D_SENTINEL).all()), "D padding was written"


# (M, N, K, lda - K, ldb - K, A offset, B offset) in elements
SHAPES = [
    (70, 50, 1, 0, 3, 0, 1),
    (130, 257, 7, 1, 0, 1, 0),
    (257, 129, 63, 2, 5, 1, 1),
    (300, 260, 64, 0, 0, 1, 0),
    (513, 300, 65, 3, 1, 0, 1),
    (260, 513, 200, 1, 1, 1, 1),
    (64, 64, 130, 6, 2, 0, 0),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}" for s in SHAPES])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32", "e4m3", "e5m2"])
def test_staged_exact_on_integer_data(dt, shape):
    """mode 1 (always stage): misaligned rows, odd strides, K below, at and
    past one stage; exact against the oracle with alpha < 0 and ReLU."""
    M, N, K, pa, pb, oa, ob = shape
    A_st, B_st = si.int_operands(M, N, K, dt, seed=M + N + K, lda=K + pa, ldb=K + pb)
    _log(f"[staged] {dt} {M}x{N}x{K} lda={K + pa} ldb={K + pb} offsets {oa},{ob}")
    D_st = run(A_st, B_st, M, N, K, -1.5, True, dt, 1, a_off=oa, b_off=ob, ldd=M + 3)
    check_exact(D_st, A_st, B_st, M, N, K, -1.5, True, dt)


def test_automatic_mode_and_short_workspace():
    """mode -1 on a small problem and mode -1 with a short workspace run the
    direct plan: same bits as mode 0; with room, mode -1 gives the bits of
    the plan the staging decision names (mode 1 if it stages, else mode 0)."""
    M, N, K = 300, 200, 130
    A_st, B_st = si.operands(M, N, K, "bf16", "uniform_pm1", 1, 2, lda=K + 1)
    direct = run(A_st, B_st, M, N, K, 0.5, False, "bf16", 0, a_off=1, workspace=None)
    assert torch.equal(run(A_st, B_st, M, N, K, 0.5, False, "bf16", -1, a_off=1), direct)
    big = 4096
    A_st, B_st = si.operands(big, big, big, "bf16", "normal_invsqrtk", 3, 4, lda=big + 1, ldb=big + 3)
    staged = run(A_st, B_st, big, big, big, 0.5, True, "bf16", 1)
    auto = run(A_st, B_st, big, big, big, 0.5, True, "bf16", -1)
    short = run(A_st, B_st, big, big, big, 0.5, True, "bf16", -1, workspace="short")
    plain = run(A_st, B_st, big, big, big, 0.5, True, "bf16", 0, workspace=None)
    assert torch.equal(short, plain), "mode -1 without room runs the direct plan"
    need = tg.staged_workspace_bytes(big, big, big, tg.BF16)
    decided = tg.query_plan_staged(big, big, big, tg.BF16, 0x100000000000, big + 1, 0x200000000000, big + 3,
                                   0x300000000000, big, tg.F32, 0x400000000000, need, -1).staged
    assert torch.equal(auto, staged if decided else plain), f"mode -1 with room (staged={decided})"
    # both within the fp32 bound on sampled rows
    rows = torch.arange(0, big, 61)
    a_rows = A_st[rows].contiguous()
    ref, mag = oracle.gemm(len(rows), big, big, 0.5, True, si.bits(a_rows), a_rows.shape[1], si.bits(B_st),
                           B_st.shape[1], "bf16")
    for D_st in (staged, plain):
        ok, r = oracle.check(D_st[:, rows].double().numpy(), ref, mag, big)
        assert ok, f"worst ratio {r}"


def test_graph_capture_of_misaligned_rows():
    """tile_gemm on misaligned rows, captured into a graph: the library only
    enqueues kernels, so every replay equals the eager result."""
    dev = torch.device("cuda:0")
    M = N = K = 4096
    A_st, B_st = si.operands(M, N, K, "bf16", "normal_invsqrtk", 31, 32, lda=K + 1, ldb=K + 1)
    A, B = A_st.to(dev), B_st.to(dev)
    eager = run(A_st, B_st, M, N, K, 0.5, True, "bf16", 0, workspace=None)
    D = si.out_storage(M, N).to(dev)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tg.gemm(A[:, :K], B[:, :K].t(), D.t(), 0.5, True)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        D.fill_(si.D_SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(D.cpu(), eager), f"replay {rep}"
    del g
