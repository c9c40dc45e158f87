"""Low-precision output D (tile_gemm_out): the fp32 epilogue value rounded to
nearest-even bf16 or fp16 on the way out (cuTile.jl tutorial "Matrix
Multiplication", Step 4), checked against the oracle on the GPU.

Bars: integer-valued inputs make every fp32 value exact, so the stored bits
must equal the oracle's own rounding of the exact result; random inputs must
lie within the fp32 bound plus half a unit of the output format; storage
outside [0,M) x [0,N) keeps its sentinel bits.
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

OUT = {"bf16": (tg.BF16, torch.bfloat16), "f16": (tg.F16, torch.float16)}
SENTINEL = {"bf16": 0x7FAB, "f16": 0x7E55}  # NaN payloads the product never writes


def _log(msg):
    print(msg, flush=True)


def out_storage(M, N, ldd, out):
    """(N, ldd) storage of the output type filled with the sentinel bit pattern."""
    return torch.full((N, ldd), SENTINEL[out], dtype=torch.int16).view(OUT[out][1])


def run_out(A_st, B_st, M, N, K, alpha, relu, out, ldd=None, kernel_id=-1):
    ldd = M if ldd is None else ldd
    dev = torch.device("cuda:0")
    A, B = A_st.to(dev), B_st.to(dev)
    D = out_storage(M, N, ldd, out).to(dev)
    tg.gemm(A[:, :K], B[:, :K].t(), D[:, :M].t(), alpha, relu, kernel_id=kernel_id)
    torch.cuda.synchronize()
    return D.cpu()


def _bits16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _plus_zero(bits):
    return np.where(bits == 0x8000, np.uint16(0), bits)


def check_padding(D_st, M, out):
    if D_st.shape[1] > M:
        assert bool((_bits16(D_st[:, M:]) == SENTINEL[out]).all()), "D padding was written"


def check_exact(D_st, A_st, B_st, M, N, K, alpha, relu, dt, out):
    ref, _ = oracle.gemm(M, N, K, alpha, relu, si.bits(A_st), A_st.shape[1], si.bits(B_st),
                         B_st.shape[1], dt)
    # signed zeros compare equal (the pages leave the sign of a zero result open)
    want = _plus_zero(oracle.encode(ref, out))
    got = _plus_zero(_bits16(D_st[:, :M]))
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{len(bad)} mismatches, first (n,m)={tuple(bad[0])}: "
                           f"{hex(got[tuple(bad[0])])} vs {hex(want[tuple(bad[0])])}")
    check_padding(D_st, M, out)


def check_tol(D_st, A_st, B_st, M, N, K, alpha, relu, dt, out):
    ref, mag = oracle.gemm(M, N, K, alpha, relu, si.bits(A_st), A_st.shape[1], si.bits(B_st),
                           B_st.shape[1], dt)
    d = oracle.decode(_bits16(D_st[:, :M]), out)
    ok, ratio = oracle.check_out(d, ref, mag, K, out)
    assert ok, f"tolerance exceeded: worst |d-ref|/bound = {ratio}"
    check_padding(D_st, M, out)
    return ratio


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("kid", unpacked_instances())
def test_every_instance_low_precision_output(kid, out):
    """Every instance, forced, writes bf16/fp16 D: exact on integer data (large
    enough sums that the output format has to round), within the bound on
    random data."""
    info = tg.kernel_info(kid)
    dt = dtype_name(info)
    es = ELEM_SIZE[dt]
    M, N = info.block_m + 37, 2 * info.block_n + 11
    K = 3 * info.block_k + 9
    lda, ldb = strides_for_class(info.load_class, K, es)
    _log(f"[out {out}] instance {kid} ({dt}, {info.block_m}x{info.block_n}): {M}x{N}x{K}")
    A_st, B_st = si.int_operands(M, N, K, dt, seed=300 + kid, lda=lda, ldb=ldb)
    D_st = run_out(A_st, B_st, M, N, K, -1.5, True, out, M + 3, kernel_id=kid)
    check_exact(D_st, A_st, B_st, M, N, K, -1.5, True, dt, out)
    A_st, B_st = si.operands(M, N, K, dt, "uniform_pm1", 400 + kid, 500 + kid, lda=lda, ldb=ldb)
    D_st = run_out(A_st, B_st, M, N, K, 0.75, False, out, M + 1, kernel_id=kid)
    check_tol(D_st, A_st, B_st, M, N, K, 0.75, False, dt, out)


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("name", ["tiny_bounded_65x97x73_bf16", "full_tile_1024_bf16", "fp32_2048"])
def test_small_workloads_low_precision_output(name, out):
    w = si.WORKLOADS[name]
    _log(f"[out {out}] {name}")
    A_st, B_st = si.workload_operands(w)
    D_st = run_out(A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, out, w.ldd)
    ratio = check_tol(D_st, A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.dtype, out)
    _log(f"  worst |d-ref|/bound = {ratio:.3g}")


@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_large_square_low_precision_output_sampled(out):
    """The 8192^3 bf16 workload in its measured launch configuration, with a
    16-bit D, on 20000 sampled entries plus the edge bands."""
    w = si.WORKLOADS["square_8192_bf16_relu"]
    _log(f"[out {out}] {w.name} sampled")
    A_st, B_st = si.workload_operands(w)
    D_st = run_out(A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, out, w.ldd)
    ms, ns = si.sample_coords(w.M, w.N, 20000, seed=21)
    ref, mag = oracle.gemm_entries(w.M, w.N, w.K, w.alpha, w.relu, si.bits(A_st), w.lda,
                                   si.bits(B_st), w.ldb, w.dtype, ms, ns)
    d = oracle.decode(_bits16(D_st[torch.from_numpy(ns), torch.from_numpy(ms)]), out)
    ok, ratio = oracle.check_out(d, ref, mag, w.K, out)
    assert ok, ratio
    _log(f"  worst |d-ref|/bound = {ratio:.3g}")


def test_fp16_output_range():
    """fp16 D: sums beyond 65504 become +inf (-inf without ReLU for negative
    sums), ReLU with a negative scale gives zeros, results below 2^-14 are
    stored as subnormals."""
    M, N, K = 64, 64, 2
    A_st = torch.full((M, K), 256.0, dtype=torch.bfloat16)
    B_st = torch.full((N, K), 256.0, dtype=torch.bfloat16)        # S = 131072
    D_st = run_out(A_st, B_st, M, N, K, 1.0, False, "f16")
    assert bool(torch.isinf(D_st[:, :M]).all() and (D_st[:, :M] > 0).all())
    D_st = run_out(A_st, B_st, M, N, K, -1.0, False, "f16")
    assert bool(torch.isinf(D_st[:, :M]).all() and (D_st[:, :M] < 0).all())
    D_st = run_out(A_st, B_st, M, N, K, -1.0, True, "f16")
    assert bool((D_st[:, :M] == 0).all())
    D_st = run_out(A_st, B_st, M, N, K, 2.0 ** -40, False, "f16")  # 2^17 * 2^-40 = 2^-23
    assert bool((_bits16(D_st[:, :M]) == 0x0002).all())


def test_odd_output_stride_and_offset():
    """A 16-bit D needs only 2-byte alignment: odd ldd and an odd element offset."""
    M, N, K = 131, 77, 200
    A_st, B_st = si.int_operands(M, N, K, "bf16", seed=91)
    dev = torch.device("cuda:0")
    D = out_storage(M + 4, N, M + 5, "bf16").to(dev)
    Dv = D[:, 1:M + 1].t()  # starts one element in: 2-byte aligned only
    tg.gemm(A_st.to(dev), B_st.to(dev).t(), Dv, 1.0, False)
    torch.cuda.synchronize()
    Dh = D.cpu()
    ref, _ = oracle.gemm(M, N, K, 1.0, False, si.bits(A_st), K, si.bits(B_st), K, "bf16")
    assert np.array_equal(_plus_zero(_bits16(Dh[:, 1:M + 1])), _plus_zero(oracle.encode(ref, "bf16")))
    assert bool((_bits16(Dh[:, :1]) == SENTINEL["bf16"]).all())
    assert bool((_bits16(Dh[:, M + 1:]) == SENTINEL["bf16"]).all())
