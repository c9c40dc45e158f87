"""tile_gemm_splitk_noalloc (the split-K product with its partials in the
library's static scratch array, for callers that cannot allocate) against
tile_gemm_splitk with a caller workspace, through the C ABI, on the GPU.

Both run the same kernels with the same split, so their results must be the
same bits; two calls in a row (the second on a smaller problem, so that the
scratch still holds the first call's partials past the second's) must each
match, and integer-valued inputs must match the oracle exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_tiled_gemm_tile_amd as tg
import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _call(entry, A, B, D, M, N, K, lda, ldb, ldd, alpha, relu, splits, dtype, out, ws=None):
    stream = torch.cuda.current_stream().cuda_stream
    if entry == "noalloc":
        rc = tg.tile_gemm_splitk_noalloc(M, N, K, alpha, relu, A.data_ptr(), lda, B.data_ptr(), ldb, D.data_ptr(),
                                         ldd, dtype, out, splits, stream, -1)
    else:
        rc = tg.tile_gemm_splitk(M, N, K, alpha, relu, A.data_ptr(), lda, B.data_ptr(), ldb, D.data_ptr(), ldd,
                                 dtype, out, splits, ws.data_ptr(), ws.numel(), stream, -1)
    assert rc == 0, tg.STATUS.get(rc, rc)


CASES = [
    # (M, N, K, splits, dtype, integer data)
    (512, 512, 16384, 0, "bf16", False),   # automatic split (8 splits of 2048)
    (300, 200, 4100, 8, "bf16", True),     # smaller than the first: the scratch keeps stale partials past it
    (130, 70, 1100, 3, "f16", False),
    (96, 64, 777, 2, "f32", True),
]


def test_noalloc_matches_workspace_splitk_on_consecutive_calls():
    dev = torch.device("cuda:0")
    for i, (M, N, K, splits, dt, integer) in enumerate(CASES):
        lda, ldb, ldd = K + 3, K + 5, M + 7
        if integer:
            A_st, B_st = si.int_operands(M, N, K, dt, seed=50 + i, lda=lda, ldb=ldb)
        else:
            A_st, B_st = si.operands(M, N, K, dt, "normal_invsqrtk", 60 + i, 70 + i, lda=lda, ldb=ldb)
        A, B = A_st.to(dev), B_st.to(dev)
        code = tg.DTYPE_CODES[dt]
        d_na = si.out_storage(M, N, ldd).to(dev)
        d_ws = si.out_storage(M, N, ldd).to(dev)
        _log(f"[no-alloc split-K] call {i}: {dt} {M}x{N}x{K} splits={splits}")
        _call("noalloc", A, B, d_na, M, N, K, lda, ldb, ldd, -0.75, True, splits, code, tg.F32)
        ws = torch.full((max(tg.splitk_workspace_bytes(M, N, splits), 16),), 0xFF, dtype=torch.uint8, device=dev)
        _call("workspace", A, B, d_ws, M, N, K, lda, ldb, ldd, -0.75, True, splits, code, tg.F32, ws)
        torch.cuda.synchronize()
        got, want = d_na.cpu(), d_ws.cpu()
        assert torch.equal(got, want), f"call {i}: differs from tile_gemm_splitk"
        assert bool((got[:, M:] == si.D_SENTINEL).all()), "D padding was written"
        if integer:
            ref, _ = oracle.gemm(M, N, K, -0.75, True, si.bits(A_st), lda, si.bits(B_st), ldb, dt)
            assert np.array_equal(got[:, :M].double().numpy(), ref)
        else:
            ref, mag = oracle.gemm(M, N, K, -0.75, True, si.bits(A_st), lda, si.bits(B_st), ldb, dt)
            ok, r = oracle.check(got[:, :M].double().numpy(), ref, mag, K)
            assert ok, f"call {i}: worst ratio {r}"


def test_noalloc_rejects_partials_beyond_the_scratch():
    """Partials that do not fit the static scratch are refused before any
    launch; the automatic split stays within it."""
    dev = torch.device("cuda:0")
    M = N = 2048
    K = 8192
    A = torch.zeros(M, K, dtype=torch.bfloat16, device=dev)
    B = torch.zeros(N, K, dtype=torch.bfloat16, device=dev)
    D = torch.zeros(N, M, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    # 3 splits x 2048 x 2048 x 4 bytes = 48 MiB > 32 MiB
    rc = tg.tile_gemm_splitk_noalloc(M, N, K, 1.0, False, A.data_ptr(), K, B.data_ptr(), K, D.data_ptr(), M,
                                     tg.BF16, tg.F32, 3, stream, -1)
    assert rc == -10
    rc = tg.tile_gemm_splitk_noalloc(M, N, K, 1.0, False, A.data_ptr(), K, B.data_ptr(), K, D.data_ptr(), M,
                                     tg.BF16, tg.F32, 2, stream, -1)
    assert rc == 0
    torch.cuda.synchronize()
    assert bool((D == 0).all())


def test_noalloc_replays_from_a_graph():
    """The no-allocation split-K captured into a graph (the callers it is for):
    every replay equals the eager call bit for bit, also when other eager
    calls have rewritten the static scratch between replays."""
    dev = torch.device("cuda:0")
    M, N, K, splits = 512, 384, 8192 + 40, 4
    lda, ldb, ldd = K + 8, K + 8, M + 4
    A_st, B_st = si.operands(M, N, K, "bf16", "normal_invsqrtk", 81, 82, lda=lda, ldb=ldb)
    A, B = A_st.to(dev), B_st.to(dev)
    eager = si.out_storage(M, N, ldd).to(dev)
    _log(f"[no-alloc graph] eager {M}x{N}x{K} splits={splits}")
    _call("noalloc", A, B, eager, M, N, K, lda, ldb, ldd, 0.5, True, splits, tg.BF16, tg.F32)
    torch.cuda.synchronize()
    want = eager.cpu()
    ref, mag = oracle.gemm(M, N, K, 0.5, True, si.bits(A_st), lda, si.bits(B_st), ldb, "bf16")
    ok, r = oracle.check(want[:, :M].double().numpy(), ref, mag, K)
    assert ok, f"eager: worst ratio {r}"
    # another problem whose partials overwrite the scratch between replays
    M2, N2, K2 = 256, 256, 4096
    A2 = torch.ones(M2, K2, dtype=torch.bfloat16, device=dev)
    B2 = torch.ones(N2, K2, dtype=torch.bfloat16, device=dev)
    D2 = torch.zeros(N2, M2, device=dev)

    D = si.out_storage(M, N, ldd).to(dev)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    _log("[no-alloc graph] capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _call("noalloc", A, B, D, M, N, K, lda, ldb, ldd, 0.5, True, splits, tg.BF16, tg.F32)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        D.fill_(si.D_SENTINEL)
        _call("noalloc", A2, B2, D2, M2, N2, K2, K2, K2, M2, 1.0, False, 2, tg.BF16, tg.F32)
        torch.cuda.synchronize()
        assert bool((D2 == float(K2)).all()), f"replay {rep}: the eager call in between"
        _log(f"[no-alloc graph] replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(D.cpu(), want), f"replay {rep} differs from the eager call"
    del g
