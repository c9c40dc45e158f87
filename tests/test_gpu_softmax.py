"""Row softmax epilogue (tile_gemm_softmax) against the oracle, on the GPU.

d[m, n] = softmax over n of x[m, :], x = alpha*A@B in fp32.  Bound: each
probability within y*(expm1(2T) + 2^-24*(|x - max| + N + 8)) of the fp64
softmax of the exact logits, T the row's largest fp32 logit bound (plus half
a unit of a 16-bit output format).  D storage outside the output window keeps
its sentinel; repeated calls give the same bits.
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


def run_softmax(A_st, B_st, M, N, K, alpha, ldd=None, out="f32", kernel_id=-1):
    ldd = M if ldd is None else ldd
    dev = torch.device("cuda:0")
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out]
    D = si.out_storage(M, N, ldd).to(odt).to(dev)
    tg.gemm_softmax(A_st.to(dev)[:, :K], B_st.to(dev)[:, :K].t(), D[:, :M].t(), alpha, kernel_id=kernel_id)
    torch.cuda.synchronize()
    return D.cpu()


def check(D_st, A_st, B_st, M, N, K, alpha, dt, out="f32"):
    ref, mag = oracle.gemm(M, N, K, alpha, False, si.bits(A_st), A_st.shape[1], si.bits(B_st),
                           B_st.shape[1], dt)
    if out == "f32":
        d = D_st[:, :M].double().numpy()
    else:
        d = oracle.decode(D_st[:, :M].contiguous().view(torch.int16).numpy().view(np.uint16), out)
    ok, ratio = oracle.check_softmax(d, ref, mag, K, out)
    assert ok, f"worst |d-y|/bound = {ratio}"
    sentinel = torch.tensor(si.D_SENTINEL).to(D_st.dtype)
    assert bool((D_st[:, M:] == sentinel).all()), "D padding was written"
    return ratio


@pytest.mark.parametrize("N", [1, 5, 64, 100, 128, 129, 200, 256])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_fused_softmax(dt, N):
    """One tile spans N: the softmax runs in the GEMM's epilogue."""
    M, K = 300, 200
    A_st, B_st = si.operands(M, N, K, dt, "normal_invsqrtk", 70 + N, 80 + N)
    D_st = run_softmax(A_st, B_st, M, N, K, 4.0, ldd=M + 3)
    r = check(D_st, A_st, B_st, M, N, K, 4.0, dt)
    _log(f"[softmax fused] {dt} N={N}: worst ratio {r:.3g}")


@pytest.mark.parametrize("N", [64, 128, 129, 300])
def test_fp32_softmax(N):
    """fp32 operands: fused up to N = 128, two passes beyond."""
    M, K = 260, 150
    A_st, B_st = si.operands(M, N, K, "f32", "uniform_pm1", 90 + N, 91 + N)
    D_st = run_softmax(A_st, B_st, M, N, K, 0.5, ldd=M + 1)
    check(D_st, A_st, B_st, M, N, K, 0.5, "f32")


@pytest.mark.parametrize("N", [257, 1000])
def test_two_pass_softmax(N):
    """N beyond one tile: logits into fp32 D, then the row softmax in place;
    a 16-bit output is refused for these shapes."""
    M, K = 513, 333
    A_st, B_st = si.operands(M, N, K, "bf16", "normal_invsqrtk", 100 + N, 101 + N)
    D_st = run_softmax(A_st, B_st, M, N, K, 3.0, ldd=M + 2)
    check(D_st, A_st, B_st, M, N, K, 3.0, "bf16")
    with pytest.raises(tg.TileGemmError) as e:
        run_softmax(A_st, B_st, M, N, K, 3.0, out="bf16")
    assert e.value.code == -1


@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_fused_softmax_low_precision_output(out):
    M, N, K = 777, 256, 512
    A_st, B_st = si.operands(M, N, K, "bf16", "normal_invsqrtk", 110, 111)
    D_st = run_softmax(A_st, B_st, M, N, K, 2.0, out=out)
    check(D_st, A_st, B_st, M, N, K, 2.0, "bf16", out=out)


def _softmax_instances():
    ids = []
    for k in unpacked_instances():
        info = tg.kernel_info(k)
        dt = dtype_name(info)
        M, N, K = 2 * info.block_m + 7, info.block_n - 3, 2 * info.block_k + 5
        lda, _ = strides_for_class(info.load_class, K, ELEM_SIZE[dt])
        try:
            tg.query_plan(M, N, K, info.dtype, 0x7F0000000000, lda, 0x7F4000000000, lda, 0x7F8000000000, M, k)
        except tg.TileGemmError:
            continue
        ids.append(k)
    return ids


@pytest.mark.parametrize("kid", _softmax_instances())
def test_every_softmax_instance(kid):
    """Every instance, forced into the softmax epilogue when it accepts the
    call (instances without one answer TG_ERR_PLAN)."""
    info = tg.kernel_info(kid)
    dt = dtype_name(info)
    M, N, K = 2 * info.block_m + 7, info.block_n - 3, 2 * info.block_k + 5
    A_st, B_st = si.operands(M, N, K, dt, "normal_invsqrtk", 120 + kid, 130 + kid)
    try:
        D_st = run_softmax(A_st, B_st, M, N, K, 2.0, ldd=M + 4, kernel_id=kid)
    except tg.TileGemmError as e:
        assert e.code == -9
        return
    _log(f"[softmax] instance {kid} ({dt} {info.block_m}x{info.block_n}): {M}x{N}x{K}")
    check(D_st, A_st, B_st, M, N, K, 2.0, dt)


def test_softmax_repeatable_and_extreme_logits():
    """Same bits on every call; logits with a wide range (alpha 64) stay finite
    and within the bound."""
    M, N, K = 640, 192, 256
    A_st, B_st = si.operands(M, N, K, "bf16", "normal_invsqrtk", 140, 141)
    a = run_softmax(A_st, B_st, M, N, K, 1.0)
    b = run_softmax(A_st, B_st, M, N, K, 1.0)
    assert torch.equal(a, b)
    D_st = run_softmax(A_st, B_st, M, N, K, 64.0)
    assert bool(torch.isfinite(D_st[:, :M]).all())
    check(D_st, A_st, B_st, M, N, K, 64.0, "bf16")
