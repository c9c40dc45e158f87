"""Batched products (tile_gemm_batched) against the oracle, on the GPU.

Each product of a batch must equal the oracle's result for its own matrices:
exactly on integer data, within |d - ref| <= 4*K*2^-24*sum|alpha*a*b| + 1e-6 on
random data.  Gaps between consecutive matrices hold NaN (A, B) or a sentinel
(D): no product may read or write outside its own matrices.
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


def stacked(parts, gap_rows, ld, dtype):
    """Stack row-major storages with `gap_rows` NaN rows after each one."""
    rows = [torch.cat([p, torch.full((gap_rows, ld), float("nan")).to(p.dtype)]) for p in parts]
    return torch.cat(rows).to(si.TORCH_DTYPES[dtype])


def run_batched(A_all, B_all, M, N, K, lda, ldb, ldd, sa, sb, sd, batch, alpha, relu, out="f32",
                kernel_id=-1):
    dev = torch.device("cuda:0")
    A, B = A_all.to(dev), B_all.to(dev)
    rows_d = (batch - 1) * sd // ldd + N + 1
    D = si.out_storage(M, rows_d, ldd).to({"f32": torch.float32, "bf16": torch.bfloat16}[out]).to(dev)
    dt = {torch.bfloat16: tg.BF16, torch.float16: tg.F16, torch.float32: tg.F32, torch.float8_e4m3fn: tg.E4M3,
          torch.float8_e5m2: tg.E5M2}[A_all.dtype]
    ot = {"f32": tg.F32, "bf16": tg.BF16}[out]
    rc = tg.tile_gemm_batched(M, N, K, alpha, relu, A.data_ptr(), lda, sa, B.data_ptr(), ldb, sb,
                              D.data_ptr(), ldd, sd, batch, dt, ot, torch.cuda.current_stream().cuda_stream,
                              kernel_id)
    assert rc == 0, tg.strerror(rc)
    torch.cuda.synchronize()
    return D.cpu()


def _matrix(storage, start, rows):
    return storage.reshape(-1)[start:start + rows].clone()


def check_batch(D_all, A_all, B_all, M, N, K, lda, ldb, ldd, sa, sb, sd, batch, alpha, relu, dt,
                exact, out="f32"):
    flatA = A_all.reshape(-1)
    flatB = B_all.reshape(-1)
    flatD = D_all.reshape(-1)
    written = torch.zeros(flatD.numel(), dtype=torch.bool)
    worst = 0.0
    for b in range(batch):
        a = flatA[b * sa: b * sa + M * lda].reshape(M, lda)
        bb = flatB[b * sb: b * sb + N * ldb].reshape(N, ldb)
        ref, mag = oracle.gemm(M, N, K, alpha, relu, si.bits(a), lda, si.bits(bb), ldb, dt)
        dview = flatD[b * sd: b * sd + N * ldd].reshape(N, ldd)[:, :M]
        written.view(-1)[b * sd: b * sd + N * ldd].reshape(N, ldd)[:, :M] = True
        if out == "f32":
            d = dview.double().numpy()
            if exact:
                assert np.array_equal(d, ref), f"product {b}: {int((d != ref).sum())} mismatches"
            else:
                ok, r = oracle.check(d, ref, mag, K)
                assert ok, f"product {b}: worst ratio {r}"
                worst = max(worst, r)
        else:
            raw = dview.contiguous().view(torch.int16).numpy().view(np.uint16)
            d = oracle.decode(raw, out)
            ok, r = oracle.check_out(d, ref, mag, K, out)
            assert ok, f"product {b}: worst ratio {r}"
            worst = max(worst, r)
    rest = flatD[~written]
    sentinel = torch.tensor(si.D_SENTINEL).to(flatD.dtype)
    assert bool((rest == sentinel).all()), "storage outside the products was written"
    return worst


def _strides(info_class, M, N, K, es):
    if info_class == 2:
        lda, ldb = K + 2, K + 4
    elif info_class == 4:
        lda = K + (2 - K) % 8 if es == 2 else K + (1 - K) % 4
        ldb = lda + 8 if es == 2 else lda + 4
    else:
        lda = K + (-K) % (16 // es)
        ldb = lda + 16 // es
    return lda, ldb


@pytest.mark.parametrize("batch", [3, 6, 8])
@pytest.mark.parametrize("kid", unpacked_instances())
def test_every_instance_batched(kid, batch):
    """Products with gaps between them, every instance forced: exact on
    integer data with alpha < 0 and ReLU.  Six and eight products run on the
    grid of products by tiles (eight: each product whole on one XCD), three
    on the other."""
    info = tg.kernel_info(kid)
    dt = dtype_name(info)
    es = ELEM_SIZE[dt]
    M, N, K = info.block_m + 21, info.block_n + 45, 2 * info.block_k + 5
    lda, ldb = strides_for_class(info.load_class, K, es)
    ldd = M + 3
    parts_a, parts_b = [], []
    for b in range(batch):
        a, bb = si.int_operands(M, N, K, dt, seed=700 + 10 * kid + b, lda=lda, ldb=ldb)
        parts_a.append(a.float())
        parts_b.append(bb.float())
    A_all = stacked(parts_a, 1, lda, dt)
    B_all = stacked(parts_b, 2, ldb, dt)
    sa, sb, sd = (M + 1) * lda, (N + 2) * ldb, N * ldd + 40
    _log(f"[batched] instance {kid} ({dt}): {batch} x {M}x{N}x{K}")
    D_all = run_batched(A_all, B_all, M, N, K, lda, ldb, ldd, sa, sb, sd, batch, -1.5, True, kernel_id=kid)
    check_batch(D_all, A_all, B_all, M, N, K, lda, ldb, ldd, sa, sb, sd, batch, -1.5, True, dt, exact=True)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_broadcast_operand(dt):
    """stride 0 reuses one A (or one B) for every product."""
    M, N, K, batch = 300, 200, 130, 5
    A_st, _ = si.int_operands(M, 1, K, dt, seed=11)
    parts_b = [si.int_operands(1, N, K, dt, seed=20 + b)[1].float() for b in range(batch)]
    B_all = stacked(parts_b, 0, K, dt)
    D_all = run_batched(A_st, B_all, M, N, K, K, K, M, 0, N * K, N * M, batch, 2.0, False)
    check_batch(D_all, A_st, B_all, M, N, K, K, K, M, 0, N * K, N * M, batch, 2.0, False, dt, exact=True)
    _, B_st = si.int_operands(1, N, K, dt, seed=12)
    parts_a = [si.int_operands(M, 1, K, dt, seed=40 + b)[0].float() for b in range(batch)]
    A_all = stacked(parts_a, 0, K, dt)
    D_all = run_batched(A_all, B_st, M, N, K, K, K, M, M * K, 0, N * M, batch, 1.0, True)
    check_batch(D_all, A_all, B_st, M, N, K, K, K, M, M * K, 0, N * M, batch, 1.0, True, dt, exact=True)


def test_batched_workload_full_parity():
    """The measured batched workload (16 products of 1024^3 bf16) in full, fp32
    and bf16 outputs."""
    w = si.WORKLOADS["batched_16x1024_bf16"]
    A_all, B_all = si.workload_operands(w)
    sa, sb, sd = w.M * w.lda, w.N * w.ldb, w.N * w.ldd
    for out in ("f32", "bf16"):
        _log(f"[batched workload] {w.name} out {out}")
        D_all = run_batched(A_all, B_all, w.M, w.N, w.K, w.lda, w.ldb, w.ldd, sa, sb, sd, w.batch,
                            w.alpha, w.relu, out=out)
        r = check_batch(D_all, A_all, B_all, w.M, w.N, w.K, w.lda, w.ldb, w.ldd, sa, sb, sd, w.batch,
                        w.alpha, w.relu, w.dtype, exact=False, out=out)
        _log(f"  worst ratio {r:.3g}")


def test_batch_of_one_and_zero():
    """batch = 1 is the plain product (bitwise); batch = 0 touches nothing."""
    M, N, K = 777, 333, 515
    A_st, B_st = si.operands(M, N, K, "bf16", "normal_invsqrtk", 81, 82)
    D1 = run_batched(A_st, B_st, M, N, K, K, K, M, 0, 0, 0, 1, 0.5, True)
    dev = torch.device("cuda:0")
    D2 = si.out_storage(M, N + 1, M).to(dev)
    tg.gemm(A_st.to(dev), B_st.to(dev).t(), D2[:N, :M].t(), 0.5, True)
    torch.cuda.synchronize()
    assert torch.equal(D1, D2.cpu())
    D0 = run_batched(A_st, B_st, M, N, K, K, K, M, M * K, N * K, N * M, 0, 0.5, True)
    assert bool((D0 == si.D_SENTINEL).all())


def test_gemm_batched_views():
    """The torch-view wrapper: 3-D views, an expanded (stride-0) operand."""
    M, N, K, batch = 130, 70, 96, 4
    dev = torch.device("cuda:0")
    A_st, _ = si.int_operands(M, 1, K, "f16", seed=5)
    Bs = [si.int_operands(1, N, K, "f16", seed=6 + b)[1] for b in range(batch)]
    A3 = A_st.to(dev).unsqueeze(0).expand(batch, M, K)
    B3 = torch.stack(Bs).to(dev).transpose(1, 2)           # (batch, K, N), K-contiguous
    D3 = torch.empty(batch, N, M, device=dev).transpose(1, 2)  # (batch, M, N), M-contiguous
    tg.gemm_batched(A3, B3, D3, 1.0, False)
    torch.cuda.synchronize()
    for b in range(batch):
        ref, _ = oracle.gemm(M, N, K, 1.0, False, si.bits(A_st), K, si.bits(Bs[b]), K, "f16")
        assert np.array_equal(D3[b].t().double().cpu().numpy(), ref)
