"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Bars: integer-valued inputs must match the oracle exactly; random inputs must
satisfy |d - ref| <= 4*K*2^-24*sum|alpha*a*b| + 1e-6 elementwise (and, for the
fp32 workload, the norm-wise relative error 1e-4 of the cuTile.jl tutorial's
checks); D storage outside [0,M) x [0,N) must keep its sentinel.
Workloads too large for a full oracle pass are checked on a seeded sample of
entries that always includes every entry of the last row and column bands.
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


def run(A_st, B_st, M, N, K, alpha, relu, ldd=None, kernel_id=-1, D_st=None, stream=None):
    """Copy storages to the GPU, run tile_gemm, return the D storage on the host."""
    ldd = M if ldd is None else ldd
    dev = torch.device("cuda:0")
    A = A_st.to(dev)
    B = B_st.to(dev)
    D = (si.out_storage(M, N, ldd) if D_st is None else D_st).to(dev)
    tg.gemm(A[:, :K], B[:, :K].t(), D[:, :M].t(), alpha, relu, kernel_id=kernel_id, stream=stream)
    torch.cuda.synchronize()
    return D.cpu()


def check_full(D_st, A_st, B_st, M, N, K, alpha, relu, dtype, exact=False):
    ref, mag = oracle.gemm(M, N, K, alpha, relu, si.bits(A_st), A_st.shape[1], si.bits(B_st),
                           B_st.shape[1], dtype)
    d = D_st[:, :M].double().numpy()
    if exact:
        bad = np.argwhere(d != ref)
        assert bad.size == 0, f"{len(bad)} mismatches, first (n,m)={tuple(bad[0])}: {d[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
        ratio = 0.0
    else:
        ok, ratio = oracle.check(d, ref, mag, K)
        assert ok, f"tolerance exceeded: worst |d-ref|/tol = {ratio}"
    pad = D_st[:, M:]
    assert bool((pad == si.D_SENTINEL).all()), "D padding was written"
    return ratio, d, ref


def check_sampled(D_st, A_st, B_st, M, N, K, alpha, relu, dtype, count, seed, exact=False):
    ms, ns = si.sample_coords(M, N, count, seed)
    ref, mag = oracle.gemm_entries(M, N, K, alpha, relu, si.bits(A_st), A_st.shape[1],
                                   si.bits(B_st), B_st.shape[1], dtype, ms, ns)
    d = D_st[torch.from_numpy(ns), torch.from_numpy(ms)].double().numpy()
    if exact:
        bad = np.nonzero(d != ref)[0]
        assert bad.size == 0, f"{bad.size} mismatches, first (m,n)=({ms[bad[0]]},{ns[bad[0]]}): {d[bad[0]]} vs {ref[bad[0]]}"
        ratio = 0.0
    else:
        ok, ratio = oracle.check(d, ref, mag, K)
        assert ok, f"tolerance exceeded: worst |d-ref|/tol = {ratio}"
    if D_st.shape[1] > M:
        assert bool((D_st[:, M:] == si.D_SENTINEL).all()), "D padding was written"
    assert not torch.isnan(D_st[:, :M]).any()
    return ratio


SMALL = ["tiny_bounded_65x97x73_bf16", "full_tile_1024_bf16", "fp32_2048"]
LARGE = ["square_8192_bf16_relu", "square_8192_f16_relu", "ragged_strided_12289x5003x4099_bf16"]


@pytest.mark.parametrize("name", SMALL)
def test_workload_parity_full(name):
    w = si.WORKLOADS[name]
    _log(f"[parity full] {name}")
    A_st, B_st = si.workload_operands(w)
    D_st = run(A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.ldd)
    ratio, d, ref = check_full(D_st, A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.dtype)
    _log(f"  worst |d-ref|/tol = {ratio:.3g}")
    if w.dtype == "f32":
        rel = np.linalg.norm(d - ref) / max(np.linalg.norm(d), np.linalg.norm(ref))
        assert rel <= 1e-4, rel


@pytest.mark.parametrize("name", LARGE)
def test_workload_parity_sampled(name):
    w = si.WORKLOADS[name]
    _log(f"[parity sampled] {name}")
    A_st, B_st = si.workload_operands(w)
    D_st = run(A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.ldd)
    ratio = check_sampled(D_st, A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.dtype, 20000, seed=7)
    _log(f"  worst |d-ref|/tol = {ratio:.3g}")


@pytest.mark.parametrize("name", SMALL + LARGE)
def test_workload_integer_exact(name):
    """Small-integer operands at every workload's shape and strides: every fp32
    summation order is exact, so the result must equal the oracle bit for bit."""
    w = si.WORKLOADS[name]
    _log(f"[integer exact] {name}")
    A_st, B_st = si.int_operands(w.M, w.N, w.K, w.dtype, seed=w.seed_a, lda=w.lda, ldb=w.ldb)
    D_st = run(A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.ldd)
    if name in SMALL:
        check_full(D_st, A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.dtype, exact=True)
    else:
        check_sampled(D_st, A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, w.dtype, 100000, seed=11,
                      exact=True)


def _instances():
    return unpacked_instances()


@pytest.mark.parametrize("kid", _instances())
def test_every_kernel_instance(kid):
    """Each compiled instance, forced, on a problem spanning several tiles with
    ragged M, N and K, at the narrowest row alignment it accepts."""
    info = tg.kernel_info(kid)
    dt = dtype_name(info)
    M, N = 2 * info.block_m + 37, 2 * info.block_n + 11
    K = 3 * info.block_k + 9
    es = ELEM_SIZE[dt]
    # narrowest accepted row alignment: lda*es odd for class 1, 2 (mod 4)
    # for class 2, 4 (mod 16) for class 4
    lda, ldb = strides_for_class(info.load_class, K, es)
    want = {1: tuple(range(1, 16, 2)), 2: (2, 6, 10, 14), 4: (4, 12), 16: (0,)}[info.load_class]
    assert (lda * es) % 16 in want
    _log(f"[instance {kid}] {dt} {info.block_m}x{info.block_n} class {info.load_class}: {M}x{N}x{K} lda={lda} ldb={ldb}")
    A_st, B_st = si.int_operands(M, N, K, dt, seed=kid, lda=lda, ldb=ldb)
    D_st = run(A_st, B_st, M, N, K, -1.5, True, M + 3, kernel_id=kid)
    check_full(D_st, A_st, B_st, M, N, K, -1.5, True, dt, exact=True)
    A_st, B_st = si.operands(M, N, K, dt, "uniform_pm1", 100 + kid, 200 + kid, lda=lda, ldb=ldb)
    D_st = run(A_st, B_st, M, N, K, 0.75, False, M, kernel_id=kid)
    check_full(D_st, A_st, B_st, M, N, K, 0.75, False, dt)


@pytest.mark.parametrize("kid", [67, 68, 69, 70])
def test_wide_m16_ragged_long_k(kid):
    """The 16x16x32 wide instances on a product with ragged M, N and K and 64
    full stages: every unrolled stage of the K loop and each of its exits,
    edge rows past M and N (copied as zeros), the register-staged K tail;
    integer data exactly, random data within the bound (sampled)."""
    info = tg.kernel_info(kid)
    dt = dtype_name(info)
    M, N, K = 4100, 2900, 4159
    lda, ldb = K + 1, K + 9  # 16-byte aligned rows (4160 and 4168 elements)
    _log(f"[m16 long K] instance {kid} ({dt}): {M}x{N}x{K}")
    A_st, B_st = si.int_operands(M, N, K, dt, seed=1300 + kid, lda=lda, ldb=ldb)
    D_st = run(A_st, B_st, M, N, K, -0.5, True, M + 4, kernel_id=kid)
    check_sampled(D_st, A_st, B_st, M, N, K, -0.5, True, dt, 20000, seed=kid, exact=True)
    A_st, B_st = si.operands(M, N, K, dt, "normal_invsqrtk", 1400 + kid, 1500 + kid, lda=lda, ldb=ldb)
    D_st = run(A_st, B_st, M, N, K, 1.25, False, M, kernel_id=kid)
    check_sampled(D_st, A_st, B_st, M, N, K, 1.25, False, dt, 20000, seed=100 + kid)


EDGE_DIMS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _stream_instances():
    return [k for k in unpacked_instances() if tg.kernel_info(k).load_class == 16]


@pytest.mark.parametrize("kid", _stream_instances())
def test_stream_instance_k_sweep(kid):
    """The streaming instances across K: fewer full stages than pipeline
    depth, exact multiples of the stage, and ragged tails."""
    info = tg.kernel_info(kid)
    dt = dtype_name(info)
    bk = info.block_k
    M, N = info.block_m + 45, 2 * info.block_n - 3
    Ks = sorted({1, bk // 2, bk - 1, bk, bk + 1, 2 * bk, 2 * bk + 7, 3 * bk, 3 * bk + 1,
                 4 * bk, 5 * bk - 1, 9 * bk, 9 * bk + 3})
    _log(f"[stream K sweep] instance {kid}: K in {Ks}")
    for K in Ks:
        lda = K + (-K) % (16 // ELEM_SIZE[dt])  # 16-byte aligned rows
        A_st, B_st = si.int_operands(M, N, K, dt, seed=K, lda=lda, ldb=lda)
        D_st = run(A_st, B_st, M, N, K, 1.0, False, M + 5, kernel_id=kid)
        check_full(D_st, A_st, B_st, M, N, K, 1.0, False, dt, exact=True)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_boundary_sweep(dt):
    """Partial tiles along every dimension (the auto plan), integer data, exact."""
    cases = [(v, 33, 65) for v in EDGE_DIMS] + [(33, v, 65) for v in EDGE_DIMS] + \
            [(40, 70, v) for v in EDGE_DIMS] + [(v, v, v) for v in EDGE_DIMS] + [(65, 97, 73), (200, 100, 300)]
    _log(f"[boundary sweep] {dt}: {len(cases)} shapes")
    for i, (M, N, K) in enumerate(cases):
        A_st, B_st = si.int_operands(M, N, K, dt, seed=1000 + i)
        D_st = run(A_st, B_st, M, N, K, 1.0, False, M + 1)
        check_full(D_st, A_st, B_st, M, N, K, 1.0, False, dt, exact=True)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_identity_and_permutation(dt):
    """B a permutation: D[:, n] = relu(alpha*A[:, pi(n)]) exactly.  Pins the MFMA
    operand and accumulator lane layouts on the hardware."""
    M, K = 300, 260
    N = K
    g = torch.Generator().manual_seed(5)
    A_st, _ = si.operands(M, 1, K, dt, "uniform_pm1", 31, 32)
    for perm in (torch.arange(K), torch.randperm(K, generator=g)):
        B_st = torch.zeros(N, K, dtype=si.TORCH_DTYPES[dt])
        B_st[torch.arange(N), perm] = 1
        D_st = run(A_st, B_st, M, N, K, 2.0, True)
        want = torch.clamp(2.0 * A_st[:, perm].double(), min=0).t()
        assert torch.equal(D_st[:, :M].double(), want)


def test_rank1_closed_form():
    M, N, K = 257, 130, 515
    g = torch.Generator().manual_seed(9)
    u = torch.randint(-2, 3, (M,), generator=g).double()
    v = torch.randint(-2, 3, (N,), generator=g).double()
    w = torch.randint(-3, 4, (K,), generator=g).double()
    A_st = (u[:, None] * w[None, :]).to(torch.bfloat16)
    B_st = (v[:, None] * w[None, :]).to(torch.bfloat16)
    D_st = run(A_st, B_st, M, N, K, 0.5, False)
    want = 0.5 * torch.outer(v, u) * float((w * w).sum())
    assert torch.equal(D_st[:, :M].double(), want)


def test_nan_padding_never_reaches_d():
    """NaN in the lda/ldb padding (ReLU off, so nothing can hide it) and D
    sentinels outside the output window."""
    M, N, K = 259, 300, 131
    for dt, padk in [("bf16", 8), ("bf16", 5), ("f16", 3), ("f32", 7)]:
        A_st, B_st = si.operands(M, N, K, dt, "uniform_pm1", 3, 4, lda=K + padk, ldb=K + padk + 1)
        D_st = run(A_st, B_st, M, N, K, 1.0, False, M + 16)
        assert not torch.isnan(D_st).any()
        check_full(D_st, A_st, B_st, M, N, K, 1.0, False, dt)


def test_repeated_launches_bitwise_identical():
    """Three launches into the same D (pre-filled with garbage) give identical bits."""
    M, N, K = 1000, 777, 1031
    A_st, B_st = si.operands(M, N, K, "bf16", "normal_invsqrtk", 13, 14)
    dev = torch.device("cuda:0")
    A, B = A_st.to(dev), B_st.to(dev)
    D = torch.randn(N, M + 4, device=dev) * 1e30
    pad = D[:, M:].clone()
    outs = []
    for _ in range(3):
        tg.gemm(A, B.t(), D[:, :M].t(), 0.5, True)
        torch.cuda.synchronize()
        outs.append(D.clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    assert torch.equal(outs[0][:, M:], pad)
    ok, _ = oracle.check(outs[0][:, :M].double().cpu().numpy(),
                         *oracle.gemm(M, N, K, 0.5, True, si.bits(A_st), K, si.bits(B_st), K, "bf16"), K)
    assert ok


def test_degenerate_shapes():
    dev = torch.device("cuda:0")
    # K = 0: D = 0 (and relu(alpha*0) = 0); padding untouched
    D = si.out_storage(37, 21, 40).to(dev)
    A = torch.empty(37, 0, dtype=torch.bfloat16, device=dev)
    B = torch.empty(0, 21, dtype=torch.bfloat16, device=dev)
    tg.gemm(A, B, D[:, :37].t(), 3.0, False)
    torch.cuda.synchronize()
    assert bool((D[:, :37] == 0).all()) and bool((D[:, 37:] == si.D_SENTINEL).all())
    # M = 0 / N = 0: nothing written
    D = si.out_storage(8, 8).to(dev)
    A = torch.ones(8, 8, dtype=torch.float16, device=dev)
    B = torch.ones(8, 8, dtype=torch.float16, device=dev).t()  # (K, N), K-contiguous
    tg.gemm(A[:0], B, D[:, :0].t(), 1.0, False)
    tg.gemm(A, B[:, :0], D[:0, :].t(), 1.0, False)
    torch.cuda.synchronize()
    assert bool((D == si.D_SENTINEL).all())


def test_non_default_stream():
    M, N, K = 513, 129, 257
    A_st, B_st = si.int_operands(M, N, K, "f16", seed=77)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        D_st = run(A_st, B_st, M, N, K, 1.0, True, stream=s)
    check_full(D_st, A_st, B_st, M, N, K, 1.0, True, "f16", exact=True)


def test_fp16_subnormal_operands():
    """a = 2^-20 (an fp16 subnormal) times b = 2^10 gives 2^-10 exactly."""
    M, N, K = 64, 64, 64
    A_st = torch.full((M, K), 2.0 ** -20, dtype=torch.float16)
    B_st = torch.zeros(N, K, dtype=torch.float16)
    B_st[:, 0] = 2.0 ** 10
    D_st = run(A_st, B_st, M, N, K, 1.0, False)
    assert bool((D_st[:, :M] == 2.0 ** -10).all()), D_st[0, :4]


def test_invalid_arguments_return_codes_on_gpu():
    dev = torch.device("cuda:0")
    A = torch.ones(64, 64, dtype=torch.bfloat16, device=dev)
    D = torch.zeros(64, 64, device=dev)
    rc = tg.tile_gemm(64, 64, 64, 1.0, 0, A.data_ptr(), 64, A.data_ptr(), 63, D.data_ptr(), 64, 1, None)
    assert rc == -2
    rc = tg.tile_gemm(64, 64, 64, 1.0, 0, A.data_ptr(), 64, A.data_ptr(), 64, A.data_ptr(), 64, 1, None)
    assert rc == -6
    with pytest.raises(ValueError):
        tg.gemm(A, A, D, 1.0)  # D is not M-contiguous


def test_bound_gemm_repeats_the_same_call():
    """The pre-marshalled callable enqueues exactly what gemm does (fp32 and
    bf16 D), every time it is called."""
    dev = torch.device("cuda:0")
    M, N, K = 300, 200, 130
    A_st, B_st = si.operands(M, N, K, "bf16", "normal_invsqrtk", 5, 6)
    A, B = A_st.to(dev), B_st.to(dev)
    for odt in (torch.float32, torch.bfloat16):
        D1 = si.out_storage(M, N).to(odt).to(dev)
        D2 = si.out_storage(M, N).to(odt).to(dev)
        tg.gemm(A, B.t(), D1.t(), 0.5, True)
        call = tg.bound_gemm(A, B.t(), D2.t(), 0.5, True)
        call()
        torch.cuda.synchronize()
        assert torch.equal(D1.cpu(), D2.cpu())
        D2.fill_(si.D_SENTINEL)
        call()
        torch.cuda.synchronize()
        assert torch.equal(D1.cpu(), D2.cpu())
    bad = tg.bound_gemm(A, B.t(), D1.t(), 0.5, True, kernel_id=tg.kernel_count())
    with pytest.raises(tg.TileGemmError) as e:
        bad()
    assert e.value.code == -9
