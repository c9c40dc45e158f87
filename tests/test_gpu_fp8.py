"""8-bit operands (e4m3, e5m2) with and without block scales, on the GPU,
against the oracle.

Integer-valued operands and scales within 2^-3..2^3 keep every product and
every partial sum exact in fp32, so the result must equal the oracle's bit
for bit; scale bytes of blocks past the last one of K are set to 255 (NaN) and
must be ignored.  Random data must meet |d - ref| <= 4*K*2^-24*sum|alpha*a*b| + 1e-6.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_tiled_gemm_tile_amd as tg
import oracle
import seeded_inputs as si
from instance_cases import strides_for_class

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def scales(rows, K, seed, pad=4):
    """(rows, lds) exponents in 124..130 for the ceil(K/32) live blocks, 255
    (NaN) in every byte past them."""
    nblk = -(-K // 32)
    lds = 4 * -(-K // 128) + pad
    g = np.random.default_rng(seed)
    s = np.full((rows, lds), 255, dtype=np.uint8)
    s[:, :nblk] = g.integers(124, 131, size=(rows, nblk), dtype=np.uint8)
    return s, lds


def run(A_st, B_st, M, N, K, alpha, relu, sa=None, sb=None, ldd=None, kernel_id=-1, out=torch.float32):
    dev = torch.device("cuda:0")
    ldd = M if ldd is None else ldd
    A, B = A_st.to(dev), B_st.to(dev)
    D = si.out_storage(M, N, ldd).to(out).to(dev)
    ta = torch.from_numpy(sa).to(dev) if sa is not None else None
    tb = torch.from_numpy(sb).to(dev) if sb is not None else None
    tg.gemm_scaled(A[:, :K], B[:, :K].t(), D[:, :M].t(), ta, tb, alpha, relu, kernel_id=kernel_id)
    torch.cuda.synchronize()
    return D.cpu()


def _fp8_instances(dt):
    code = tg.DTYPE_CODES[dt]
    return [k for k in range(tg.kernel_count()) if tg.kernel_info(k).dtype == code]


SHAPES = [(70, 50, 1), (130, 257, 33), (257, 129, 128), (300, 260, 200), (513, 300, 1000)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}" for s in SHAPES])
@pytest.mark.parametrize("dt", ["e4m3", "e5m2"])
def test_block_scaled_exact(dt, shape):
    M, N, K = shape
    sa, lda_s = scales(M, K, 1 + K)
    sb, ldb_s = scales(N, K, 2 + K)
    refused = []
    for kid in [-1] + _fp8_instances(dt):
        # operand rows at exactly the instance's alignment class
        cls = tg.kernel_info(kid).load_class if kid >= 0 else 1
        lda, ldb = strides_for_class(cls, K, 1)
        A_st, B_st = si.int_operands(M, N, K, dt, seed=M + K + kid, lda=lda, ldb=ldb)
        ref, _ = oracle.gemm(M, N, K, -0.75, True, si.bits(A_st), lda, si.bits(B_st), ldb, dt,
                             scale_a=sa, lds_a=lda_s, scale_b=sb, lds_b=ldb_s)
        try:
            D_st = run(A_st, B_st, M, N, K, -0.75, True, sa, sb, ldd=M + 2, kernel_id=kid)
        except tg.TileGemmError as e:
            # an instance without block scales refuses the scaled call (and
            # still runs the same operands without scales)
            assert e.code == -9 and kid >= 0, (kid, e.code)
            run(A_st, B_st, M, N, K, -0.75, True, ldd=M + 2, kernel_id=kid)
            refused.append(kid)
            continue
        d = D_st[:, :M].double().numpy()
        bad = np.argwhere(d != ref)
        assert bad.size == 0, f"instance {kid}: {len(bad)} mismatches, first {tuple(bad[0])}: " \
                              f"{d[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
        assert bool((D_st[:, M:] == si.D_SENTINEL).all()), "D padding was written"
    assert len(refused) == 1, refused  # only the plain streaming 8-bit instance lacks scales
    _log(f"[fp8 scaled] {dt} {M}x{N}x{K}: exact on every instance that applies block scales")


@pytest.mark.parametrize("side", ["a", "b", "none"])
def test_one_sided_and_unscaled(side):
    M, N, K = 300, 200, 300
    A_st, B_st = si.int_operands(M, N, K, "e4m3", seed=7, lda=K + 1, ldb=K + 2)
    sa, la = scales(M, K, 3)
    sb, lb = scales(N, K, 4)
    sa = sa if side == "a" else None
    sb = sb if side == "b" else None
    ref, _ = oracle.gemm(M, N, K, 1.0, False, si.bits(A_st), A_st.shape[1], si.bits(B_st), B_st.shape[1], "e4m3",
                         scale_a=sa, lds_a=la, scale_b=sb, lds_b=lb)
    D_st = run(A_st, B_st, M, N, K, 1.0, False, sa, sb)
    assert np.array_equal(D_st[:, :M].double().numpy(), ref)
    if side == "none":  # the plain entry point gives the same bits
        dev = torch.device("cuda:0")
        D = si.out_storage(M, N).to(dev)
        tg.gemm(A_st.to(dev)[:, :K], B_st.to(dev)[:, :K].t(), D.t(), 1.0, False)
        torch.cuda.synchronize()
        assert torch.equal(D.cpu(), D_st)


@pytest.mark.parametrize("dt", ["e4m3", "e5m2"])
def test_random_within_bound_and_low_precision_out(dt):
    M, N, K = 777, 555, 1500
    A_st, B_st = si.operands(M, N, K, dt, "uniform_pm1", 21, 22)
    sa, la = scales(M, K, 5)
    sb, lb = scales(N, K, 6)
    ref, mag = oracle.gemm(M, N, K, 0.5, True, si.bits(A_st), A_st.shape[1], si.bits(B_st), B_st.shape[1], dt,
                           scale_a=sa, lds_a=la, scale_b=sb, lds_b=lb)
    D_st = run(A_st, B_st, M, N, K, 0.5, True, sa, sb)
    ok, r = oracle.check(D_st[:, :M].double().numpy(), ref, mag, K)
    assert ok, f"worst ratio {r}"
    D_st = run(A_st, B_st, M, N, K, 0.5, True, sa, sb, out=torch.bfloat16)
    raw = D_st[:, :M].contiguous().view(torch.int16).numpy().view(np.uint16)
    ok, r2 = oracle.check_out(oracle.decode(raw, "bf16"), ref, mag, K, "bf16")
    assert ok, f"bf16 out: worst ratio {r2}"
    _log(f"[fp8 random] {dt}: worst ratio {r:.3g} (fp32 D), {r2:.3g} (bf16 D)")


def test_fp8_workload_sampled():
    """The measured 8-bit workload at full size, sampled entries (edges included)."""
    w = si.WORKLOADS["square_8192_e4m3_relu"]
    A_st, B_st = si.workload_operands(w)
    dev = torch.device("cuda:0")
    D = si.out_storage(w.M, w.N, w.ldd).to(dev)
    tg.gemm(A_st.to(dev)[:, :w.K], B_st.to(dev)[:, :w.K].t(), D[:, :w.M].t(), w.alpha, w.relu)
    torch.cuda.synchronize()
    ms, ns = si.sample_coords(w.M, w.N, 3000, 17)
    ref, mag = oracle.gemm_entries(w.M, w.N, w.K, w.alpha, w.relu, si.bits(A_st), w.lda, si.bits(B_st), w.ldb,
                                   w.dtype, ms, ns)
    d = D.cpu()[torch.from_numpy(ns), torch.from_numpy(ms)].double().numpy()
    ok, r = oracle.check(d, ref, mag, w.K)
    assert ok, f"worst ratio {r}"
    _log(f"[fp8 workload] {w.name}: {ms.size} sampled entries, worst ratio {r:.3g}")


def test_softmax_over_8bit_logits():
    """Row softmax of an 8-bit product: no 8-bit instance carries the fused
    softmax, so the fp32 logits are written and normalised in a second pass."""
    M, N, K = 300, 300, 256
    A_st, B_st = si.operands(M, N, K, "e4m3", "uniform_pm1", 31, 32)
    dev = torch.device("cuda:0")
    D = si.out_storage(M, N, M + 1).to(dev)
    tg.gemm_softmax(A_st.to(dev), B_st.to(dev).t(), D[:, :M].t(), 0.25)
    torch.cuda.synchronize()
    ref, mag = oracle.gemm(M, N, K, 0.25, False, si.bits(A_st), K, si.bits(B_st), K, "e4m3")
    ok, r = oracle.check_softmax(D.cpu()[:, :M].double().numpy(), ref, mag, K)
    assert ok, f"worst ratio {r}"


def test_block_scaled_workload_sampled():
    """The measured 8-bit workload with seeded block scales (as bench.py
    --block-scales draws them), full size, sampled entries (edges included)."""
    w = si.WORKLOADS["square_8192_e4m3_relu"]
    A_st, B_st = si.workload_operands(w)
    sa = si.block_scales(w.M, w.K, w.seed_a + 50)
    sb = si.block_scales(w.N, w.K, w.seed_b + 50)
    D_st = run(A_st, B_st, w.M, w.N, w.K, w.alpha, w.relu, sa, sb, ldd=w.ldd)
    ms, ns = si.sample_coords(w.M, w.N, 2000, 19)
    ref, mag = oracle.gemm_entries(w.M, w.N, w.K, w.alpha, w.relu, si.bits(A_st), w.lda, si.bits(B_st), w.ldb,
                                   w.dtype, ms, ns, scale_a=sa, lds_a=sa.shape[1], scale_b=sb, lds_b=sb.shape[1])
    d = D_st[torch.from_numpy(ns), torch.from_numpy(ms)].double().numpy()
    ok, r = oracle.check(d, ref, mag, w.K)
    assert ok, f"worst ratio {r}"
    _log(f"[fp8 scaled workload] {w.name}: {ms.size} sampled entries, worst ratio {r:.3g}")


@pytest.mark.parametrize("K", [4096, 4099])
def test_block_scaled_misaligned_rows(K):
    """A large block-scaled product with 1-byte aligned rows (and a K that is
    not a whole number of 128-k stages): the automatic plan runs a 1-byte
    aligned instance that applies the scales, and it and every such instance
    match the oracle on sampled entries."""
    M = N = 4096
    lda = K + 1 if (K + 1) % 2 else K + 2  # odd strides: rows 1-byte aligned
    ldb = lda + 2
    A_st, B_st = si.operands(M, N, K, "e4m3", "uniform_pm1", 41, 42, lda=lda, ldb=ldb)
    sa = si.block_scales(M, K, 43, pad=4)
    sb = si.block_scales(N, K, 44, pad=8)
    ms, ns = si.sample_coords(M, N, 1500, 23)
    ref, mag = oracle.gemm_entries(M, N, K, 0.01, True, si.bits(A_st), lda, si.bits(B_st), ldb, "e4m3", ms, ns,
                                   scale_a=sa, lds_a=sa.shape[1], scale_b=sb, lds_b=sb.shape[1])
    dev = torch.device("cuda:0")
    A, B = A_st.to(dev), B_st.to(dev)
    D = torch.empty(N, M, device=dev)
    ta, tb = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
    plan = tg.query_plan_scaled(M, N, K, tg.E4M3, A.data_ptr(), lda, ta.data_ptr(), sa.shape[1], B.data_ptr(),
                                ldb, tb.data_ptr(), sb.shape[1], D.data_ptr(), M)
    assert plan.load_class == 1 and plan.staged == 0
    direct = [k for k in _fp8_instances("e4m3") if tg.kernel_info(k).load_class == 1]
    assert plan.kernel_id in direct
    for kid in [-1] + direct:
        D_st = run(A_st, B_st, M, N, K, 0.01, True, sa, sb, kernel_id=kid)
        d = D_st[torch.from_numpy(ns), torch.from_numpy(ms)].double().numpy()
        ok, r = oracle.check(d, ref, mag, K)
        assert ok, f"instance {kid}: worst ratio {r}"
        _log(f"[fp8 scaled misaligned] K={K} instance {kid}: worst ratio {r:.3g}")
