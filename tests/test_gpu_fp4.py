"""4-bit (e2m1) operands, packed two per byte, with and without block
scales, on the GPU, against the oracle.

Every e2m1 value is a multiple of 1/2 of magnitude at most 6.  Without scales
every product is then a multiple of 1/4 below 36, so every partial sum of
fewer than 2^16 products is exact in fp32 and the result must equal the
oracle's bit for bit, whatever the summation order.  With block scales in
2^0..2^3 and K <= 2048 every partial sum is a multiple of 1/4 below 2^23, so
the same holds.  Scale bytes of blocks past the last one of K are 255 (NaN)
and must be ignored.  Random scales spanning 2^-4..2^4 meet
|d - ref| <= 4*K*2^-24*sum|alpha*a*b| + 1e-6.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_tiled_gemm_tile_amd as tg
import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

DT = "e2m1"
OUT = {torch.float32: tg.F32, torch.bfloat16: tg.BF16, torch.float16: tg.F16}


def _log(msg):
    print(msg, flush=True)


def _instances():
    return [k for k in range(tg.kernel_count()) if tg.kernel_info(k).dtype == tg.E2M1]


def strides(K, aligned):
    """Element strides whose rows are 16-byte aligned (aligned) or start on
    odd bytes (lda/2 odd), padding included."""
    if aligned:
        lda = -(-K // 32) * 32 + 32
        return lda, lda + 32
    b = -(-K // 2) + 1
    b += 1 - (b & 1)  # odd byte stride
    return 2 * b, 2 * (b + 2)


def scales(rows, K, seed, lo=127, hi=130, pad=16):
    """(rows, lds) exponents in lo..hi for the ceil(K/32) live blocks, 255
    (NaN) in every byte past them; lds a multiple of 16."""
    s = si.block_scales(rows, K, seed, lo, hi, pad=pad, dtype=DT, fill=255)
    return s, s.shape[1]


def run(A, B, M, N, K, lda, ldb, alpha, relu, sa=None, sb=None, ldd=None, kernel_id=-1, out=torch.float32,
        scaled_call=None):
    """One call through the C ABI on packed byte storages (numpy uint8)."""
    dev = torch.device("cuda:0")
    ldd = M if ldd is None else ldd
    tA = torch.from_numpy(np.ascontiguousarray(A)).to(dev)
    tB = torch.from_numpy(np.ascontiguousarray(B)).to(dev)
    D = si.out_storage(M, N, ldd).to(out).to(dev)
    stream = torch.cuda.current_stream().cuda_stream
    scaled_call = (sa is not None or sb is not None) if scaled_call is None else scaled_call
    if scaled_call:
        ta = torch.from_numpy(sa).to(dev) if sa is not None else None
        tb = torch.from_numpy(sb).to(dev) if sb is not None else None
        rc = tg.tile_gemm_scaled(M, N, K, alpha, relu, tA.data_ptr(), lda, ta.data_ptr() if ta is not None else None,
                                 sa.shape[1] if sa is not None else 0, tB.data_ptr(), ldb,
                                 tb.data_ptr() if tb is not None else None, sb.shape[1] if sb is not None else 0,
                                 D.data_ptr(), ldd, tg.E2M1, OUT[out], stream, kernel_id)
    else:
        rc = tg.tile_gemm_out(M, N, K, alpha, relu, tA.data_ptr(), lda, tB.data_ptr(), ldb, D.data_ptr(), ldd,
                              tg.E2M1, OUT[out], stream, kernel_id)
    if rc != tg.TG_OK:
        raise tg.TileGemmError(rc, tg.strerror(rc))
    torch.cuda.synchronize()
    return D.cpu()


def _exact(D_st, ref, M, what):
    d = D_st[:, :M].double().numpy()
    bad = np.argwhere(d != ref)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first {tuple(bad[0])}: {d[tuple(bad[0])]} vs " \
                          f"{ref[tuple(bad[0])]}"
    assert bool((D_st[:, M:] == si.D_SENTINEL).all()), f"{what}: D padding was written"


SHAPES = [(70, 50, 1), (130, 257, 33), (300, 260, 701), (513, 300, 1000), (257, 513, 2048)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}" for s in SHAPES])
def test_exact_every_instance(shape):
    """Every 4-bit instance (and the automatic plan) on operand rows of its
    alignment class, odd K included: bit-exact, padding untouched."""
    M, N, K = shape
    for kid in [-1] + _instances():
        info = tg.kernel_info(kid) if kid >= 0 else None
        for aligned in ([True, False] if kid < 0 else [info.load_class == 16]):
            lda, ldb = strides(K, aligned)
            A, B = si.packed_operands(M, N, K, DT, M + K + kid, N + K + kid, lda, ldb)
            ref, _ = oracle.gemm(M, N, K, -0.75, True, A, lda, B, ldb, DT)
            D_st = run(A, B, M, N, K, lda, ldb, -0.75, True, ldd=M + 3, kernel_id=kid)
            _exact(D_st, ref, M, f"instance {kid} aligned={aligned}")
    _log(f"[fp4] {M}x{N}x{K}: exact on every 4-bit instance")


@pytest.mark.parametrize("kid", _instances())
def test_instance_k_sweep(kid):
    """Each 4-bit instance across K: no full stage, exactly one or two, fewer
    full stages than the pipeline holds, ragged tails (odd K included), with
    and (scaled instances) without block scales."""
    info = tg.kernel_info(kid)
    M, N = info.block_m + 45, 2 * info.block_n - 3
    for K in (1, 255, 256, 257, 512, 513, 767, 768, 1031, 2304):
        lda, ldb = strides(K, info.load_class == 16)
        A, B = si.packed_operands(M, N, K, DT, 50 + K, 60 + K, lda, ldb)
        ref, _ = oracle.gemm(M, N, K, 1.25, False, A, lda, B, ldb, DT)
        _exact(run(A, B, M, N, K, lda, ldb, 1.25, False, kernel_id=kid), ref, M, f"instance {kid} K={K}")
        if info.block_scales:
            sa, _ = scales(M, K, 70 + K)
            sb, _ = scales(N, K, 80 + K)
            ref, _ = oracle.gemm(M, N, K, 1.25, False, A, lda, B, ldb, DT, scale_a=sa, lds_a=sa.shape[1],
                                 scale_b=sb, lds_b=sb.shape[1])
            _exact(run(A, B, M, N, K, lda, ldb, 1.25, False, sa, sb, kernel_id=kid), ref, M,
                   f"instance {kid} K={K} scaled")
    _log(f"[fp4 K sweep] instance {kid}: exact")


@pytest.mark.parametrize("shape", SHAPES[1:], ids=[f"{s[0]}x{s[1]}x{s[2]}" for s in SHAPES[1:]])
def test_block_scaled_exact(shape):
    """Block scales in 2^0..2^3 on both sides, NaN bytes past the live blocks:
    bit-exact on every instance that applies scales; the others refuse."""
    M, N, K = shape
    lda, ldb = strides(K, True)
    A, B = si.packed_operands(M, N, K, DT, 5 + K, 6 + K, lda, ldb)
    sa, _ = scales(M, K, 1 + K)
    sb, _ = scales(N, K, 2 + K)
    ref, _ = oracle.gemm(M, N, K, 0.5, False, A, lda, B, ldb, DT, scale_a=sa, lds_a=sa.shape[1], scale_b=sb,
                         lds_b=sb.shape[1])
    ran = 0
    for kid in [-1] + _instances():
        try:
            D_st = run(A, B, M, N, K, lda, ldb, 0.5, False, sa, sb, ldd=M + 1, kernel_id=kid)
        except tg.TileGemmError as e:
            assert e.code == -9 and kid >= 0 and not tg.kernel_info(kid).block_scales, (kid, e.code)
            continue
        _exact(D_st, ref, M, f"instance {kid}")
        ran += 1
    assert ran >= 3
    _log(f"[fp4 scaled] {M}x{N}x{K}: exact on {ran - 1} instances and the plan")


def test_block_scaled_rows_on_odd_bytes():
    """Rows starting on odd bytes with block scales: the register-staged
    instances (large and small products), bit-exact."""
    for M, N, K in ((600, 700, 1001), (70, 90, 260)):
        lda, ldb = strides(K, False)
        A, B = si.packed_operands(M, N, K, DT, 3 + K, 4 + K, lda, ldb)
        sa, _ = scales(M, K, 5 + K)
        sb, _ = scales(N, K, 6 + K)
        ref, _ = oracle.gemm(M, N, K, 2.0, True, A, lda, B, ldb, DT, scale_a=sa, lds_a=sa.shape[1], scale_b=sb,
                             lds_b=sb.shape[1])
        _exact(run(A, B, M, N, K, lda, ldb, 2.0, True, sa, sb), ref, M, f"{M}x{N}x{K} odd rows scaled")


@pytest.mark.parametrize("side", ["a", "b"])
def test_one_sided_scales(side):
    M, N, K = 300, 270, 1100
    lda, ldb = strides(K, True)
    A, B = si.packed_operands(M, N, K, DT, 11, 12, lda, ldb)
    sa, _ = scales(M, K, 3)
    sb, _ = scales(N, K, 4)
    sa = sa if side == "a" else None
    sb = sb if side == "b" else None
    ref, _ = oracle.gemm(M, N, K, 1.0, True, A, lda, B, ldb, DT, scale_a=sa, lds_a=sa.shape[1] if sa is not None else 0,
                         scale_b=sb, lds_b=sb.shape[1] if sb is not None else 0)
    _exact(run(A, B, M, N, K, lda, ldb, 1.0, True, sa, sb), ref, M, f"scales on {side} only")


def test_nan_scale_poisons_its_row():
    """A NaN scale of one A row's live block makes exactly that output row NaN."""
    M, N, K = 260, 300, 600
    lda, ldb = strides(K, True)
    A, B = si.packed_operands(M, N, K, DT, 13, 14, lda, ldb, pool=[2, 3, 4])  # positive codes only
    sa, _ = scales(M, K, 5)
    sb, _ = scales(N, K, 6)
    sa[17, 9] = 255
    D_st = run(A, B, M, N, K, lda, ldb, 1.0, False, sa, sb)
    d = D_st[:, :M].numpy()
    assert np.isnan(d[:, 17]).all()
    assert np.isfinite(np.delete(d, 17, axis=1)).all()


def test_random_scales_within_bound_and_low_precision_out():
    M, N, K = 777, 555, 4099
    lda, ldb = strides(K, True)
    A, B = si.packed_operands(M, N, K, DT, 21, 22, lda, ldb)
    sa, _ = scales(M, K, 7, lo=123, hi=131)
    sb, _ = scales(N, K, 8, lo=123, hi=131)
    ref, mag = oracle.gemm(M, N, K, 0.5, True, A, lda, B, ldb, DT, scale_a=sa, lds_a=sa.shape[1], scale_b=sb,
                           lds_b=sb.shape[1])
    D_st = run(A, B, M, N, K, lda, ldb, 0.5, True, sa, sb)
    ok, r = oracle.check(D_st[:, :M].double().numpy(), ref, mag, K)
    assert ok, f"worst ratio {r}"
    D_st = run(A, B, M, N, K, lda, ldb, 0.5, True, sa, sb, out=torch.bfloat16)
    raw = D_st[:, :M].contiguous().view(torch.int16).numpy().view(np.uint16)
    ok, r2 = oracle.check_out(oracle.decode(raw, "bf16"), ref, mag, K, "bf16")
    assert ok, f"bf16 out: worst ratio {r2}"
    _log(f"[fp4 random scales] worst ratio {r:.3g} (fp32 D), {r2:.3g} (bf16 D)")


def test_fp4_workload_sampled():
    """The measured 4-bit workload at full size through the torch-view entry
    point (float4_e2m1fn_x2 views), sampled entries (edges included): exact."""
    w = si.WORKLOADS["square_8192_e2m1_relu"]
    A_st, B_st = si.workload_operands(w)
    dev = torch.device("cuda:0")
    A = A_st.to(dev).view(torch.float4_e2m1fn_x2)
    B = B_st.to(dev).view(torch.float4_e2m1fn_x2)
    D = si.out_storage(w.M, w.N, w.ldd).to(dev)
    tg.gemm(A[:, :w.K // 2], B[:, :w.K // 2].t(), D[:, :w.M].t(), w.alpha, w.relu)
    torch.cuda.synchronize()
    ms, ns = si.sample_coords(w.M, w.N, 3000, 19)
    ref, _ = oracle.gemm_entries(w.M, w.N, w.K, w.alpha, w.relu, A_st.numpy(), w.lda, B_st.numpy(), w.ldb, w.dtype,
                                 ms, ns)
    d = D.cpu()[torch.from_numpy(ns), torch.from_numpy(ms)].double().numpy()
    assert np.array_equal(d, ref), f"{int((d != ref).sum())} of {d.size} sampled entries differ"
    _log(f"[fp4 workload] {w.name}: {ms.size} sampled entries exact")


def test_splitk_and_batched():
    """Split-K (K ranges of whole stages, byte offsets of packed rows) and a
    batch with element strides: exact."""
    dev = torch.device("cuda:0")
    M, N, K = 300, 200, 8192 + 64
    lda, ldb = strides(K, True)
    A, B = si.packed_operands(M, N, K, DT, 31, 32, lda, ldb)
    ref, _ = oracle.gemm(M, N, K, 1.0, False, A, lda, B, ldb, DT)
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    D = si.out_storage(M, N).to(dev)
    ws = torch.empty(tg.splitk_workspace_bytes(M, N, 8), dtype=torch.uint8, device=dev)
    rc = tg.tile_gemm_splitk(M, N, K, 1.0, False, tA.data_ptr(), lda, tB.data_ptr(), ldb, D.data_ptr(), M, tg.E2M1,
                             tg.F32, 8, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, tg.strerror(rc)
    torch.cuda.synchronize()
    _exact(D.cpu(), ref, M, "split-K")
    # three products stored back to back (element strides, whole bytes)
    Mb, Nb, Kb, batch = 130, 140, 300, 3
    lda, ldb = strides(Kb, False)
    A, B = si.packed_operands(batch * Mb, batch * Nb, Kb, DT, 33, 34, lda, ldb)
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    D = si.out_storage(Mb, batch * Nb).to(dev)
    rc = tg.tile_gemm_batched(Mb, Nb, Kb, 2.0, True, tA.data_ptr(), lda, Mb * lda, tB.data_ptr(), ldb, Nb * ldb,
                              D.data_ptr(), Mb, Nb * Mb, batch, tg.E2M1, tg.F32,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0, tg.strerror(rc)
    torch.cuda.synchronize()
    for b in range(batch):
        ref, _ = oracle.gemm(Mb, Nb, Kb, 2.0, True, A[b * Mb:(b + 1) * Mb], lda, B[b * Nb:(b + 1) * Nb], ldb, DT)
        _exact(D.cpu()[b * Nb:(b + 1) * Nb], ref, Mb, f"batch entry {b}")


def test_softmax_over_fp4_logits():
    """Row softmax of a 4-bit product: the two-pass path (fp32 logits, then
    the row pass)."""
    M, N, K = 300, 300, 512
    lda, ldb = strides(K, True)
    A, B = si.packed_operands(M, N, K, DT, 41, 42, lda, ldb)
    dev = torch.device("cuda:0")
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    D = si.out_storage(M, N, M + 1).to(dev)
    rc = tg.tile_gemm_softmax(M, N, K, 0.125, tA.data_ptr(), lda, tB.data_ptr(), ldb, D.data_ptr(), M + 1, tg.E2M1,
                              tg.F32, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, tg.strerror(rc)
    torch.cuda.synchronize()
    ref, mag = oracle.gemm(M, N, K, 0.125, False, A, lda, B, ldb, DT)
    ok, r = oracle.check_softmax(D.cpu()[:, :M].double().numpy(), ref, mag, K)
    assert ok, f"worst ratio {r}"
