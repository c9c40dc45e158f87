"""6-bit operands (e2m3, e3m2), packed four per three bytes, with and without
block scales, on the GPU, against the oracle.

e2m3 values are multiples of 1/8 of magnitude at most 7.5, so without scales
(or with scales in 2^0..2^1 and K <= 1024) every product is a multiple of
1/64 and every partial sum stays below 2^18: exact in fp32, so the result must
equal the oracle's bit for bit.  For e3m2 the exact cases draw codes with
exponent fields 2..5 (values 0.25..7): products are multiples of 2^-6 below
49 and K <= 2048 keeps the sums below 2^17.  Full-range codes and scales
spanning 2^-4..2^4 meet |d - ref| <= 4*K*2^-24*sum|alpha*a*b| + 1e-6.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_tiled_gemm_tile_amd as tg
import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

DTS = ["e2m3", "e3m2"]
OUT = {torch.float32: tg.F32, torch.bfloat16: tg.BF16}
# e3m2 codes with exponent fields 2..5, both signs (values 0.25..7)
E3M2_POOL = [c for c in range(64) if 2 <= ((c >> 2) & 7) <= 5]


def _log(msg):
    print(msg, flush=True)


def _instances(dt):
    return [k for k in range(tg.kernel_count()) if tg.kernel_info(k).dtype == tg.DTYPE_CODES[dt]]


def strides(K, aligned=True):
    """Element strides whose rows start 16-byte aligned (multiples of 64
    elements, 48 bytes), or (aligned False) only on whole bytes (multiples of
    4 elements, 3 bytes, that are not multiples of 64), padding included."""
    if aligned:
        lda = -(-K // 64) * 64 + 64
        return lda, lda + 128
    lda = -(-K // 64) * 64 + 4
    return lda, lda + 8


def pool(dt):
    return None if dt == "e2m3" else E3M2_POOL


def scales(rows, K, seed, lo=127, hi=128, pad=4):
    """(rows, lds) exponents in lo..hi for the ceil(K/32) live blocks, 255
    (NaN) in every byte past them."""
    s = si.block_scales(rows, K, seed, lo, hi, pad=pad, dtype="e2m3", fill=255)
    return s, s.shape[1]


def run(dt, A, B, M, N, K, lda, ldb, alpha, relu, sa=None, sb=None, ldd=None, kernel_id=-1, out=torch.float32):
    dev = torch.device("cuda:0")
    ldd = M if ldd is None else ldd
    tA = torch.from_numpy(np.ascontiguousarray(A)).to(dev)
    tB = torch.from_numpy(np.ascontiguousarray(B)).to(dev)
    D = si.out_storage(M, N, ldd).to(out).to(dev)
    stream = torch.cuda.current_stream().cuda_stream
    code = tg.DTYPE_CODES[dt]
    if sa is not None or sb is not None:
        ta = torch.from_numpy(sa).to(dev) if sa is not None else None
        tb = torch.from_numpy(sb).to(dev) if sb is not None else None
        rc = tg.tile_gemm_scaled(M, N, K, alpha, relu, tA.data_ptr(), lda, ta.data_ptr() if ta is not None else None,
                                 sa.shape[1] if sa is not None else 0, tB.data_ptr(), ldb,
                                 tb.data_ptr() if tb is not None else None, sb.shape[1] if sb is not None else 0,
                                 D.data_ptr(), ldd, code, OUT[out], stream, kernel_id)
    else:
        rc = tg.tile_gemm_out(M, N, K, alpha, relu, tA.data_ptr(), lda, tB.data_ptr(), ldb, D.data_ptr(), ldd, code,
                              OUT[out], stream, kernel_id)
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
@pytest.mark.parametrize("dt", DTS)
def test_exact_every_instance(dt, shape):
    """Every 6-bit instance of the type (and the automatic plan), ragged M, N
    and K: bit-exact, padding untouched."""
    M, N, K = shape
    for kid in [-1] + _instances(dt):
        for aligned in ([True, False] if kid < 0 else [tg.kernel_info(kid).load_class == 16]):
            lda, ldb = strides(K, aligned)
            A, B = si.packed_operands(M, N, K, dt, M + K + kid, N + K + kid, lda, ldb, pool=pool(dt))
            ref, _ = oracle.gemm(M, N, K, -0.75, True, A, lda, B, ldb, dt)
            _exact(run(dt, A, B, M, N, K, lda, ldb, -0.75, True, ldd=M + 3, kernel_id=kid), ref, M,
                   f"{dt} instance {kid} aligned={aligned}")
    _log(f"[fp6] {dt} {M}x{N}x{K}: exact on every instance")


@pytest.mark.parametrize("dt", DTS)
def test_instance_k_sweep(dt):
    """Each instance across K: no full stage, exactly one or two, fewer full
    stages than the pipeline holds, ragged tails (K not a multiple of 4
    included), with and (scaled instances) without block scales."""
    for kid in _instances(dt):
        info = tg.kernel_info(kid)
        M, N = info.block_m + 45, 2 * info.block_n - 3
        for K in (1, 3, 127, 128, 129, 256, 383, 384, 385, 640, 1031):
            lda, ldb = strides(K, info.load_class == 16)
            A, B = si.packed_operands(M, N, K, dt, 50 + K, 60 + K, lda, ldb, pool=pool(dt))
            ref, _ = oracle.gemm(M, N, K, 1.25, False, A, lda, B, ldb, dt)
            _exact(run(dt, A, B, M, N, K, lda, ldb, 1.25, False, kernel_id=kid), ref, M, f"instance {kid} K={K}")
            if info.block_scales:
                sa, _ = scales(M, K, 70 + K)
                sb, _ = scales(N, K, 80 + K)
                ref, _ = oracle.gemm(M, N, K, 1.25, False, A, lda, B, ldb, dt, scale_a=sa, lds_a=sa.shape[1],
                                     scale_b=sb, lds_b=sb.shape[1])
                _exact(run(dt, A, B, M, N, K, lda, ldb, 1.25, False, sa, sb, kernel_id=kid), ref, M,
                       f"instance {kid} K={K} scaled")
        _log(f"[fp6 K sweep] {dt} instance {kid}: exact")


@pytest.mark.parametrize("dt", DTS)
def test_block_scaled_exact_and_refusals(dt):
    """Scales in 2^0..2^1 on both sides, NaN bytes past the live blocks:
    bit-exact on the instances that apply scales; the others refuse."""
    M, N, K = 300, 520, 1000
    lda, ldb = strides(K)
    A, B = si.packed_operands(M, N, K, dt, 5, 6, lda, ldb, pool=pool(dt))
    sa, _ = scales(M, K, 1)
    sb, _ = scales(N, K, 2)
    ref, _ = oracle.gemm(M, N, K, 0.5, False, A, lda, B, ldb, dt, scale_a=sa, lds_a=sa.shape[1], scale_b=sb,
                         lds_b=sb.shape[1])
    ran = 0
    for kid in [-1] + _instances(dt):
        try:
            D_st = run(dt, A, B, M, N, K, lda, ldb, 0.5, False, sa, sb, ldd=M + 1, kernel_id=kid)
        except tg.TileGemmError as e:
            assert e.code == -9 and kid >= 0 and not tg.kernel_info(kid).block_scales, (kid, e.code)
            continue
        _exact(D_st, ref, M, f"{dt} instance {kid}")
        ran += 1
    assert ran == 1 + sum(tg.kernel_info(k).block_scales for k in _instances(dt))
    # one-sided scales and a NaN scale poisoning exactly its row
    ref, _ = oracle.gemm(M, N, K, 0.5, False, A, lda, B, ldb, dt, scale_b=sb, lds_b=sb.shape[1])
    _exact(run(dt, A, B, M, N, K, lda, ldb, 0.5, False, None, sb), ref, M, f"{dt} scales on B only")
    sa2 = sa.copy()
    sa2[17, 9] = 255
    d = run(dt, A, B, M, N, K, lda, ldb, 0.5, False, sa2, sb)[:, :M].numpy()
    assert np.isnan(d[:, 17]).all() and np.isfinite(np.delete(d, 17, axis=1)).all()


@pytest.mark.parametrize("dt", DTS)
def test_full_range_within_bound(dt):
    """Every code, scales spanning 2^-4..2^4, K = 4099: within the bound, also
    with bf16 D."""
    M, N, K = 777, 555, 4099
    lda, ldb = strides(K)
    A, B = si.packed_operands(M, N, K, dt, 21, 22, lda, ldb)
    sa, _ = scales(M, K, 7, lo=123, hi=131)
    sb, _ = scales(N, K, 8, lo=123, hi=131)
    ref, mag = oracle.gemm(M, N, K, 0.5, True, A, lda, B, ldb, dt, scale_a=sa, lds_a=sa.shape[1], scale_b=sb,
                           lds_b=sb.shape[1])
    ok, r = oracle.check(run(dt, A, B, M, N, K, lda, ldb, 0.5, True, sa, sb)[:, :M].double().numpy(), ref, mag, K)
    assert ok, f"worst ratio {r}"
    D_st = run(dt, A, B, M, N, K, lda, ldb, 0.5, True, sa, sb, out=torch.bfloat16)
    raw = D_st[:, :M].contiguous().view(torch.int16).numpy().view(np.uint16)
    ok, r2 = oracle.check_out(oracle.decode(raw, "bf16"), ref, mag, K, "bf16")
    assert ok, f"bf16 out: worst ratio {r2}"
    ref, mag = oracle.gemm(M, N, K, 0.5, True, A, lda, B, ldb, dt)
    ok, r3 = oracle.check(run(dt, A, B, M, N, K, lda, ldb, 0.5, True)[:, :M].double().numpy(), ref, mag, K)
    assert ok, f"unscaled: worst ratio {r3}"
    _log(f"[fp6 full range] {dt}: worst ratio {r:.3g} (scaled), {r2:.3g} (bf16 D), {r3:.3g} (unscaled)")


@pytest.mark.parametrize("dt", DTS)
def test_block_scaled_rows_on_any_byte(dt):
    """Rows on 3-byte boundaries with block scales: the register-staged
    instances, large and small products, bit-exact."""
    for M, N, K in ((600, 700, 1001), (70, 90, 260)):
        lda, ldb = strides(K, False)
        A, B = si.packed_operands(M, N, K, dt, 3 + K, 4 + K, lda, ldb, pool=pool(dt))
        sa, _ = scales(M, K, 5 + K)
        sb, _ = scales(N, K, 6 + K)
        ref, _ = oracle.gemm(M, N, K, 2.0, True, A, lda, B, ldb, dt, scale_a=sa, lds_a=sa.shape[1], scale_b=sb,
                             lds_b=sb.shape[1])
        _exact(run(dt, A, B, M, N, K, lda, ldb, 2.0, True, sa, sb), ref, M, f"{dt} {M}x{N}x{K} misaligned scaled")


def test_fp6_workload_sampled():
    """The measured 6-bit workload at full size, sampled entries (edges
    included): within the bound (every e2m3 code, K = 8192: the sums are
    exact in fp32 only up to 2^18)."""
    w = si.WORKLOADS["square_8192_e2m3_relu"]
    A_st, B_st = si.workload_operands(w)
    D_st = run(w.dtype, A_st.numpy(), B_st.numpy(), w.M, w.N, w.K, w.lda, w.ldb, w.alpha, w.relu, ldd=w.ldd)
    ms, ns = si.sample_coords(w.M, w.N, 3000, 23)
    ref, mag = oracle.gemm_entries(w.M, w.N, w.K, w.alpha, w.relu, A_st.numpy(), w.lda, B_st.numpy(), w.ldb,
                                   w.dtype, ms, ns)
    d = D_st[torch.from_numpy(ns), torch.from_numpy(ms)].double().numpy()
    ok, r = oracle.check(d, ref, mag, w.K)
    assert ok, f"worst ratio {r}"
    _log(f"[fp6 workload] {w.name}: {ms.size} sampled entries, worst ratio {r:.3g}")


def test_splitk_and_batched():
    """Split-K (K ranges of whole 128-element stages: 96-byte steps) and a
    batch with element strides: exact."""
    dev = torch.device("cuda:0")
    dt = "e2m3"
    M, N, K = 300, 200, 4096 + 64
    lda, ldb = strides(K)
    A, B = si.packed_operands(M, N, K, dt, 31, 32, lda, ldb)
    ref, _ = oracle.gemm(M, N, K, 1.0, False, A, lda, B, ldb, dt)
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    D = si.out_storage(M, N).to(dev)
    ws = torch.empty(tg.splitk_workspace_bytes(M, N, 8), dtype=torch.uint8, device=dev)
    rc = tg.tile_gemm_splitk(M, N, K, 1.0, False, tA.data_ptr(), lda, tB.data_ptr(), ldb, D.data_ptr(), M,
                             tg.E2M3, tg.F32, 8, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, tg.strerror(rc)
    torch.cuda.synchronize()
    _exact(D.cpu(), ref, M, "split-K")
    Mb, Nb, Kb, batch = 130, 140, 300, 3
    lda, ldb = strides(Kb)
    A, B = si.packed_operands(batch * Mb, batch * Nb, Kb, dt, 33, 34, lda, ldb)
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    D = si.out_storage(Mb, batch * Nb).to(dev)
    rc = tg.tile_gemm_batched(Mb, Nb, Kb, 2.0, True, tA.data_ptr(), lda, Mb * lda, tB.data_ptr(), ldb, Nb * ldb,
                              D.data_ptr(), Mb, Nb * Mb, batch, tg.E2M3, tg.F32,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0, tg.strerror(rc)
    torch.cuda.synchronize()
    for b in range(batch):
        ref, _ = oracle.gemm(Mb, Nb, Kb, 2.0, True, A[b * Mb:(b + 1) * Mb], lda, B[b * Nb:(b + 1) * Nb], ldb, dt)
        _exact(D.cpu()[b * Nb:(b + 1) * Nb], ref, Mb, f"batch entry {b}")
