"""Split-K (tile_gemm_splitk) against the oracle, on the GPU.

The fp32 partial products of the K ranges are summed in split order before
the epilogue, so: integer-valued inputs must match the oracle exactly (every
partial and every sum is exact), random inputs must meet the fp32 bound
|d - ref| <= 4*K*2^-24*sum|alpha*a*b| + 1e-6, repeated calls must give the same
bits, and nothing outside [0,M) x [0,N) of D may be written.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_tiled_gemm_tile_amd as tg
import oracle
import seeded_inputs as si
from instance_cases import ELEM_SIZE, dtype_name, strides_for_class, unpacked_instances

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def run_splitk(A_st, B_st, M, N, K, alpha, relu, splits, ldd=None, kernel_id=-1, out="f32", garbage=True):
    ldd = M if ldd is None else ldd
    dev = torch.device("cuda:0")
    A, B = A_st.to(dev), B_st.to(dev)
    odt = {"f32": torch.float32, "bf16": torch.bfloat16}[out]
    D = si.out_storage(M, N, ldd).to(odt).to(dev)
    need = max(tg.splitk_workspace_bytes(M, N, splits), 16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if garbage:
        ws.view(torch.float32)[: need // 4].fill_(float("nan"))  # prior contents are irrelevant
    tg.gemm_splitk(A[:, :K], B[:, :K].t(), D[:, :M].t(), alpha, relu, splits=splits, workspace=ws,
                   kernel_id=kernel_id)
    torch.cuda.synchronize()
    return D.cpu()


def check(D_st, A_st, B_st, M, N, K, alpha, relu, dt, exact, out="f32"):
    ref, mag = oracle.gemm(M, N, K, alpha, relu, si.bits(A_st), A_st.shape[1], si.bits(B_st),
                           B_st.shape[1], dt)
    if out == "f32":
        d = D_st[:, :M].double().numpy()
        if exact:
            bad = np.argwhere(d != ref)
            assert bad.size == 0, f"{len(bad)} mismatches, first {tuple(bad[0])}: {d[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
            ratio = 0.0
        else:
            ok, ratio = oracle.check(d, ref, mag, K)
            assert ok, f"worst ratio {ratio}"
    else:
        raw = D_st[:, :M].contiguous().view(torch.int16).numpy().view(np.uint16)
        ok, ratio = oracle.check_out(oracle.decode(raw, out), ref, mag, K, out)
        assert ok, f"worst ratio {ratio}"
    sentinel = torch.tensor(si.D_SENTINEL).to(D_st.dtype)
    assert bool((D_st[:, M:] == sentinel).all()), "D padding was written"
    return ratio


@pytest.mark.parametrize("kid", unpacked_instances())
def test_every_instance_splitk(kid):
    """Every instance as the partial-product kernel, 3 splits of a ragged K, exact."""
    info = tg.kernel_info(kid)
    dt = dtype_name(info)
    es = ELEM_SIZE[dt]
    M, N, K = info.block_m + 19, info.block_n + 3, 5 * info.block_k + 7
    lda, ldb = strides_for_class(info.load_class, K, es)
    _log(f"[split-K] instance {kid} ({dt}): {M}x{N}x{K}, 3 splits")
    A_st, B_st = si.int_operands(M, N, K, dt, seed=900 + kid, lda=lda, ldb=ldb)
    D_st = run_splitk(A_st, B_st, M, N, K, -1.5, True, 3, ldd=M + 2, kernel_id=kid)
    check(D_st, A_st, B_st, M, N, K, -1.5, True, dt, exact=True)


@pytest.mark.parametrize("kid", unpacked_instances())
def test_every_instance_splitk_whole_splits_per_xcd(kid):
    """Every instance on the split-K grid of splits by tiles (eight splits
    used, each run whole on one XCD), the last split ragged, exact."""
    info = tg.kernel_info(kid)
    dt = dtype_name(info)
    es = ELEM_SIZE[dt]
    # 15 stages and a ragged tail: 8 splits of 2 stages, all used, the last short
    M, N, K = info.block_m + 19, info.block_n + 3, 15 * info.block_k + 7
    lda, ldb = strides_for_class(info.load_class, K, es)
    _log(f"[split-K on XCDs] instance {kid} ({dt}): {M}x{N}x{K}, 8 splits")
    A_st, B_st = si.int_operands(M, N, K, dt, seed=950 + kid, lda=lda, ldb=ldb)
    D_st = run_splitk(A_st, B_st, M, N, K, 0.5, False, 8, ldd=M + 4, kernel_id=kid)
    check(D_st, A_st, B_st, M, N, K, 0.5, False, dt, exact=True)


@pytest.mark.parametrize("splits", [2, 4, 6, 7, 16, 64])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_splitk_random_within_bound(dt, splits):
    M, N, K = 300, 200, 2011
    A_st, B_st = si.operands(M, N, K, dt, "normal_invsqrtk", 31 + splits, 41 + splits)
    D_st = run_splitk(A_st, B_st, M, N, K, 0.5, True, splits, ldd=M + 5)
    ratio = check(D_st, A_st, B_st, M, N, K, 0.5, True, dt, exact=False)
    _log(f"[split-K] {dt} splits {splits}: worst ratio {ratio:.3g}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_full_tile_workload_splitk(out):
    """The 1024^3 bf16 workload (few output tiles, long K) with 4 splits, in full."""
    w = si.WORKLOADS["full_tile_1024_bf16"]
    A_st, B_st = si.workload_operands(w)
    D_st = run_splitk(A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, 4, ldd=w.ldd, out=out)
    ratio = check(D_st, A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.dtype, exact=False, out=out)
    _log(f"[split-K] {w.name} out {out}: worst ratio {ratio:.3g}")


def test_splitk_repeatable_and_edge_cases():
    """Three calls give the same bits; more splits than stages use fewer; K = 0
    writes zeros; splits = 1 is the plain product."""
    M, N, K = 513, 257, 1500
    A_st, B_st = si.operands(M, N, K, "bf16", "uniform_pm1", 5, 6)
    outs = [run_splitk(A_st, B_st, M, N, K, 1.25, False, 6) for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    check(outs[0], A_st, B_st, M, N, K, 1.25, False, "bf16", exact=False)
    # 70 elements of K = 2 stages of 64: 8 requested splits become 2
    A_st, B_st = si.int_operands(M, N, 70, "f16", seed=8)
    D_st = run_splitk(A_st, B_st, M, N, 70, 1.0, True, 8)
    check(D_st, A_st, B_st, M, N, 70, 1.0, True, "f16", exact=True)
    # K = 0
    D_st = run_splitk(torch.zeros(M, 1, dtype=torch.bfloat16), torch.zeros(N, 1, dtype=torch.bfloat16),
                      M, N, 0, 3.0, False, 4, ldd=M + 1)
    assert bool((D_st[:, :M] == 0).all())
    # splits = 1
    A_st, B_st = si.operands(M, N, K, "bf16", "uniform_pm1", 9, 10)
    one = run_splitk(A_st, B_st, M, N, K, 0.5, True, 1)
    dev = torch.device("cuda:0")
    D = si.out_storage(M, N).to(dev)
    tg.gemm(A_st.to(dev), B_st.to(dev).t(), D.t(), 0.5, True)
    torch.cuda.synchronize()
    assert torch.equal(one, D.cpu())


def test_short_workspace_is_refused():
    M, N, K = 128, 128, 512
    dev = torch.device("cuda:0")
    A = torch.ones(M, K, dtype=torch.bfloat16, device=dev)
    D = torch.zeros(N, M, device=dev)
    need = tg.splitk_workspace_bytes(M, N, 4)
    ws = torch.empty(need - 4, dtype=torch.uint8, device=dev)
    rc = tg.tile_gemm_splitk(M, N, K, 1.0, 0, A.data_ptr(), K, A.data_ptr(), K, D.data_ptr(), M, tg.BF16, tg.F32,
                             4, ws.data_ptr(), need - 4, None, -1)
    assert rc == -10


@pytest.mark.parametrize("M,N,K,integer", [(384, 384, 32768, True), (1024, 512, 16384, False)])
def test_automatic_splits_on_long_k(M, N, K, integer):
    """splits = 0 on long-K shapes whose automatic count is a multiple of eight
    (16 and 8 splits of about 32 stages, each split whole on one XCD): exact
    on small-integer data, within the bound on random data."""
    lda = ldb = K + 8
    if integer:
        A_st, B_st = si.int_operands(M, N, K, "bf16", seed=M + K, lda=lda, ldb=ldb)
    else:
        A_st, B_st = si.operands(M, N, K, "bf16", "normal_invsqrtk", M + 1, K + 1, lda=lda, ldb=ldb)
    _log(f"[split-K auto long K] {M}x{N}x{K} integer={integer}")
    D_st = run_splitk(A_st, B_st, M, N, K, 0.75, True, 0, ldd=M + 3)
    ratio = check(D_st, A_st, B_st, M, N, K, 0.75, True, "bf16", exact=integer)
    _log(f"[split-K auto long K] worst ratio {ratio:.3g}")


def test_automatic_splits():
    """splits = 0: the tall-K workload is split (and stays within the bound), the
    1024^3 workload (already one tile per CU) is not (same bits as the plain
    call)."""
    w = si.WORKLOADS["tall_k_512x512x16384_bf16"]
    A_st, B_st = si.workload_operands(w)
    D_st = run_splitk(A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, 0)
    ratio = check(D_st, A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.dtype, exact=False)
    _log(f"[split-K auto] {w.name}: worst ratio {ratio:.3g}")
    w = si.WORKLOADS["full_tile_1024_bf16"]
    A_st, B_st = si.workload_operands(w)
    auto = run_splitk(A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, 0)
    dev = torch.device("cuda:0")
    D = si.out_storage(w.M, w.N).to(dev)
    tg.gemm(A_st.to(dev), B_st.to(dev).t(), D.t(), w.alpha, w.relu)
    torch.cuda.synchronize()
    assert torch.equal(auto, D.cpu())
