"""Pins for the oracle: what the pages and the mathematics fix, independent of
the oracle's own formula.

Each pin is a function ``pin_*(lib) -> None`` that raises AssertionError when
the oracle library ``lib`` is wrong, so the same pins run against the real
oracle (must pass) and against copies of its source with planted mistakes
(each must be caught by at least one pin; see ``test_planted_mistakes``).

Pins used:
  * decoders against the IEEE/bfloat16 format definitions (golden table) and
    against numpy's float16 and torch's bfloat16 conversions for every bit
    pattern;
  * identity and permutation B: the product reduces to a scaled column copy
    of A (closed form);
  * rank-1 operands: a[m,k] = u_m w_k, b[k,n] = w_k v_n gives
    alpha u_m v_n sum_k w_k^2 (closed form);
  * small-integer operands: exact against numpy's int64 matmul;
  * tiny shapes: within fp64 rounding of the exact rational result
    (Python fractions), and against numpy's float64 matmul;
  * invariants: zero-padding K does not change the result (cuTile.jl
    tutorial, "Sizes that are not a multiple of the tile shape"), NaN in
    the stride padding never reaches the result, the alpha-then-clamp order of
    the scalar epilogue (Tylo.jl manual, "Walk through GEMM", section 5),
    sampled entries equal the full result, K = 0 gives zeros;
  * the 4- and 6-bit formats (e2m1, e2m3, e3m2): every normal code against
    torch's float8_e4m3fn decoding of the same sign, exponent and fraction
    re-biased into e4m3 (every such value is an e4m3 value), zero and
    subnormal codes and hand-packed byte strings against a golden table
    written from the MX format definitions, and packed products (odd K,
    padded strides, block scales) against numpy on values unpacked with
    numpy's own bit unpacking;
  * the 16-bit output encoder (round to nearest, ties to even): every finite
    bf16/fp16 value encodes to itself, fp16 agrees with numpy's float64 ->
    float16 conversion and bf16 with torch's float32 -> bfloat16 conversion
    (on values exact in float32, midpoints included), and the format
    boundaries (overflow to infinity, subnormals) follow the definitions.
"""
from __future__ import annotations

import itertools
import re
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

GOLDEN = Path(__file__).resolve().parent / "golden" / "decode_table.txt"


def _bits(t):
    return si.bits(t)


def _full(lib, M, N, K, alpha, relu, A, lda, B, ldb, dt, threads=4):
    return oracle.gemm(M, N, K, alpha, relu, A, lda, B, ldb, dt, threads=threads, lib=lib)


def _exact_values(t: torch.Tensor) -> np.ndarray:
    """Decoded values through torch's own conversion (independent of the oracle)."""
    return t.to(torch.float64).numpy()


# --------------------------------------------------------------------------- pins

def pin_decode_golden(lib):
    for line in GOLDEN.read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        dt, hexbits, num, den = line.split()
        want = Fraction(int(num), int(den))
        got = oracle.decode(np.array([int(hexbits, 16)], dtype=np.uint16), dt, lib=lib)[0]
        assert Fraction(got) == want, (dt, hexbits, got, float(want))
        if int(hexbits, 16) == 0x8000:
            assert np.signbit(got)


def pin_decode_all_patterns(lib):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = oracle.decode(pats, "f16", lib=lib)
    want16 = pats.view(np.float16).astype(np.float64)
    nan = np.isnan(want16)
    assert np.array_equal(np.isnan(f16), nan)
    assert np.array_equal(f16[~nan], want16[~nan])
    bf = oracle.decode(pats, "bf16", lib=lib)
    wantbf = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nanb = np.isnan(wantbf)
    assert np.array_equal(np.isnan(bf), nanb)
    assert np.array_equal(bf[~nanb], wantbf[~nanb])
    f32 = np.array([0.0, -1.5, 3.0e-39, 1.0e30, 1.0 / 3.0], dtype=np.float32)
    assert np.array_equal(oracle.decode(f32, "f32", lib=lib), f32.astype(np.float64))


def pin_permutation(lib):
    """B[k, n] = [k == pi(n)] makes D[:, n] = relu(alpha * A[:, pi(n)]) exactly."""
    g = torch.Generator().manual_seed(11)
    for dt, (M, N, K), alpha, relu in [("bf16", (37, 29, 41), 1.5, True),
                                       ("f16", (20, 33, 33), -2.0, True),
                                       ("f32", (31, 17, 23), 0.5, False),
                                       ("bf16", (16, 40, 40), 1.0, False)]:
        pi = torch.randint(0, K, (N,), generator=g) if N > K else torch.randperm(K, generator=g)[:N]
        A, _ = si.operands(M, 1, K, dt, "uniform_pm1", 5, 6, lda=K + 3)
        Bst = torch.zeros(N, K, dtype=si.TORCH_DTYPES[dt])
        Bst[torch.arange(N), pi] = 1
        ref, mag = _full(lib, M, N, K, alpha, relu, _bits(A), K + 3, _bits(Bst), K, dt)
        a = _exact_values(A[:, :K])
        want = np.float64(np.float32(alpha)) * a[:, pi.numpy()].T  # (N, M)
        if relu:
            want = np.maximum(want, 0.0)
        assert np.array_equal(ref, want), dt
        assert np.array_equal(mag, np.abs(np.float64(np.float32(alpha)) * a[:, pi.numpy()].T))


def pin_identity(lib):
    M = K = N = 48
    A, _ = si.operands(M, 1, K, "bf16", "uniform_pm1", 7, 8)
    eye = torch.eye(K, dtype=torch.bfloat16)
    ref, _ = _full(lib, M, N, K, 1.0, False, _bits(A), K, _bits(eye), K, "bf16")
    assert np.array_equal(ref, _exact_values(A).T)


def pin_rank1(lib):
    """a[m,k] = u_m w_k, b[k,n] = w_k v_n: D = relu(alpha u_m v_n sum w_k^2)."""
    g = torch.Generator().manual_seed(12)
    for dt, (M, N, K), alpha, relu in [("bf16", (13, 19, 57), 0.5, True),
                                       ("f16", (24, 9, 31), -1.5, True),
                                       ("f32", (7, 30, 64), 2.0, False)]:
        u = torch.randint(-2, 3, (M,), generator=g).double()
        v = torch.randint(-2, 3, (N,), generator=g).double()
        w = torch.randint(-3, 4, (K,), generator=g).double()
        A = (u[:, None] * w[None, :]).to(si.TORCH_DTYPES[dt])
        Bst = (v[:, None] * w[None, :]).to(si.TORCH_DTYPES[dt])
        ref, mag = _full(lib, M, N, K, alpha, relu, _bits(A), K, _bits(Bst), K, dt)
        al = float(np.float32(alpha))
        want = al * np.outer(v.numpy(), u.numpy()) * float((w * w).sum())
        if relu:
            want = np.maximum(want, 0.0)
        assert np.array_equal(ref, want), dt
        assert np.array_equal(mag, abs(al) * np.abs(np.outer(v.numpy(), u.numpy())) * float((w * w).sum()))


def pin_small_integers(lib):
    """Integer operands: exact against numpy's int64 matmul, with padded strides."""
    for dt, (M, N, K), (pa, pb) in [("bf16", (65, 97, 73), (0, 0)), ("f16", (40, 31, 130), (5, 2)),
                                    ("f32", (33, 50, 77), (3, 9)), ("bf16", (1, 1, 1), (0, 0))]:
        A, B = si.int_operands(M, N, K, dt, seed=M * N + K, lda=K + pa, ldb=K + pb)
        ai = A[:, :K].to(torch.float64).numpy().astype(np.int64)
        bi = B[:, :K].to(torch.float64).numpy().astype(np.int64)
        for alpha, relu in [(1.0, False), (2.0, True), (-0.5, True)]:
            ref, mag = _full(lib, M, N, K, alpha, relu, _bits(A), K + pa, _bits(B), K + pb, dt)
            s = (bi @ ai.T).astype(np.float64)           # (N, M): S[m, n] at [n, m]
            want = alpha * s
            if relu:
                want = np.maximum(want, 0.0)
            assert np.array_equal(ref, want), (dt, M, N, K, alpha)
            assert np.array_equal(mag, abs(alpha) * (np.abs(bi) @ np.abs(ai).T).astype(np.float64))


def pin_tiny_rational(lib):
    """Every (M, N, K) in [1..4]^3: within fp64 rounding of the exact rational result."""
    for dt in ("bf16", "f16", "f32"):
        for M, N, K in itertools.product(range(1, 5), repeat=3):
            A, B = si.operands(M, N, K, dt, "uniform_pm1", 100 + M, 200 + N * 7 + K)
            alpha = 1.25
            ref, mag = _full(lib, M, N, K, alpha, True, _bits(A), K, _bits(B), K, dt, threads=1)
            av = _exact_values(A)
            bv = _exact_values(B)
            for m in range(M):
                for n in range(N):
                    s = sum(Fraction(av[m, k]) * Fraction(bv[n, k]) for k in range(K))
                    t = sum(abs(Fraction(av[m, k]) * Fraction(bv[n, k])) for k in range(K))
                    exact = max(Fraction(alpha) * s, Fraction(0))
                    bound = (K + 1) * Fraction(1, 2 ** 52) * abs(Fraction(alpha)) * t
                    assert abs(Fraction(ref[n, m]) - exact) <= bound, (dt, M, N, K, m, n)
                    assert abs(Fraction(mag[n, m]) - abs(Fraction(alpha)) * t) <= bound
    # and a library matmul in fp64 on a bigger random case
    M, N, K = 23, 17, 301
    A, B = si.operands(M, N, K, "f16", "normal_invsqrtk", 1, 2)
    ref, mag = _full(lib, M, N, K, 1.0, False, _bits(A), K, _bits(B), K, "f16")
    want = (_exact_values(A) @ _exact_values(B).T).T
    assert np.all(np.abs(ref - want) <= 1e-13 * (mag + 1e-300))


def pin_zero_padded_k(lib):
    """Appending zero columns along K (and zero padding) leaves the result unchanged."""
    M, N, K, extra = 30, 21, 45, 19
    A, B = si.operands(M, N, K, "bf16", "uniform_pm1", 31, 32, lda=K + extra, ldb=K + extra, pad=0.0)
    ref_a, _ = _full(lib, M, N, K, 1.5, True, _bits(A), K + extra, _bits(B), K + extra, "bf16")
    ref_b, _ = _full(lib, M, N, K + extra, 1.5, True, _bits(A), K + extra, _bits(B), K + extra, "bf16")
    assert np.array_equal(ref_a, ref_b)


def pin_nan_padding_unread(lib):
    M, N, K = 19, 26, 37
    A, B = si.operands(M, N, K, "f16", "uniform_pm1", 41, 42, lda=K + 8, ldb=K + 5)
    assert torch.isnan(A[:, K:].float()).all() and torch.isnan(B[:, K:].float()).all()
    ref, mag = _full(lib, M, N, K, 1.0, False, _bits(A), K + 8, _bits(B), K + 5, "f16")
    Ac, Bc = A[:, :K].contiguous(), B[:, :K].contiguous()
    ref_c, mag_c = _full(lib, M, N, K, 1.0, False, _bits(Ac), K, _bits(Bc), K, "f16")
    assert np.isfinite(ref).all()
    assert np.array_equal(ref, ref_c) and np.array_equal(mag, mag_c)


def pin_alpha_then_relu(lib):
    """relu(alpha * S): a negative alpha flips which entries survive."""
    A = torch.tensor([[1.0, 2.0], [-3.0, 0.5]], dtype=torch.bfloat16)   # a[m, k]
    B = torch.tensor([[1.0, 1.0], [2.0, -1.0]], dtype=torch.bfloat16)   # b[k, n] at [n, k]
    # S[m,n]: S[0,0]=3, S[0,1]=0, S[1,0]=-2.5, S[1,1]=-6.5
    ref, _ = _full(lib, 2, 2, 2, -2.0, True, _bits(A), 2, _bits(B), 2, "bf16")
    assert np.array_equal(ref, np.array([[0.0, 5.0], [0.0, 13.0]]))
    ref, _ = _full(lib, 2, 2, 2, 2.0, True, _bits(A), 2, _bits(B), 2, "bf16")
    assert np.array_equal(ref, np.array([[6.0, 0.0], [0.0, 0.0]]))
    ref, _ = _full(lib, 2, 2, 2, -2.0, False, _bits(A), 2, _bits(B), 2, "bf16")
    assert np.array_equal(ref, np.array([[-6.0, 5.0], [0.0, 13.0]]))


def pin_entries_and_column_ranges(lib):
    M, N, K = 70, 45, 66
    A, B = si.operands(M, N, K, "bf16", "uniform_pm1", 51, 52, lda=K + 2, ldb=K + 6)
    ref, mag = _full(lib, M, N, K, 0.75, True, _bits(A), K + 2, _bits(B), K + 6, "bf16")
    ms, ns = si.sample_coords(M, N, 300, seed=3)
    er, em = oracle.gemm_entries(M, N, K, 0.75, True, _bits(A), K + 2, _bits(B), K + 6, "bf16",
                                 ms, ns, threads=3, lib=lib)
    assert np.array_equal(er, ref[ns, ms]) and np.array_equal(em, mag[ns, ms])
    part, _ = oracle.gemm(M, N, K, 0.75, True, _bits(A), K + 2, _bits(B), K + 6, "bf16",
                          n0=10, n1=23, threads=2, lib=lib)
    assert np.array_equal(part, ref[10:23])


def pin_degenerate(lib):
    A = np.zeros((5, 1), dtype=np.uint16)
    B = np.zeros((4, 1), dtype=np.uint16)
    ref, mag = _full(lib, 5, 4, 0, 3.0, False, A, 1, B, 1, "bf16")
    assert ref.shape == (4, 5) and not ref.any() and not mag.any()
    ref, _ = _full(lib, 0, 4, 3, 1.0, False, np.zeros(0, np.uint16), 3, np.zeros(12, np.uint16), 3, "bf16")
    assert ref.shape == (4, 0)
    with pytest.raises(ValueError):
        _full(lib, 2, 2, 3, 1.0, False, np.zeros(6, np.uint16), 2, np.zeros(6, np.uint16), 3, "bf16")


def _encode(lib, x, dt):
    return oracle.encode(np.asarray(x, dtype=np.float64), dt, lib=lib)


def pin_encode_roundtrip(lib):
    """Every finite value of each format encodes to its own bits (signed zeros too)."""
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        bits = np.arange(1 << 16, dtype=np.uint16)
        vals = torch.from_numpy(bits.view(np.int16).copy()).view(tdt).to(torch.float64).numpy()
        fin = np.isfinite(vals)
        assert np.array_equal(_encode(lib, vals[fin], dt), bits[fin]), dt


def _neighbour_midpoints(tdt):
    """Midpoints between consecutive positive finite values of a 16-bit format,
    and points a quarter-spacing on either side of them."""
    bits = np.arange(0x0000, 0x7C00 if tdt == torch.float16 else 0x7F80, dtype=np.int16)
    v = torch.from_numpy(bits).view(tdt).to(torch.float64).numpy()
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2
    q = (hi - lo) / 4
    return np.concatenate([mid, mid - q, mid + q, -mid])


def pin_encode_f16_vs_numpy(lib):
    """fp16 rounding of fp64 values agrees with numpy's float64 -> float16 cast."""
    rng = np.random.default_rng(7)
    x = np.concatenate([_neighbour_midpoints(torch.float16),
                        rng.standard_normal(20000) * np.exp2(rng.integers(-30, 18, 20000)),
                        [65504.0, 65519.999, 65520.0, 70000.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0001,
                         3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25]])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(_encode(lib, x, "f16"), want)


def pin_encode_bf16_vs_torch(lib):
    """bf16 rounding agrees with torch's float32 -> bfloat16 cast on values that
    are exact in float32 (midpoints between bf16 neighbours have 9 significant
    bits, so they are)."""
    rng = np.random.default_rng(8)
    mids = _neighbour_midpoints(torch.bfloat16)
    mids = mids[np.isfinite(mids.astype(np.float32)) & (mids.astype(np.float32).astype(np.float64) == mids)]
    x = np.concatenate([mids, rng.standard_normal(20000).astype(np.float32).astype(np.float64)])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(_encode(lib, x, "bf16"), want)


def pin_encode_golden(lib):
    """Boundary cases read off the format definitions."""
    cases = {
        "f16": [(65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (-1e6, 0xFC00),
                (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (1.5 * 2.0 ** -24, 0x0002),
                (2.0 ** -14, 0x0400), (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02)],
        "bf16": [(1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82), (2.0 ** -133, 0x0001),
                 (2.0 ** -134, 0x0000), (2.0 ** -126, 0x0080), (3.0e38, 0x7F62), (3.4e38, 0x7F80),
                 (-2.5, 0xC020)],
    }
    for dt, pairs in cases.items():
        got = _encode(lib, [v for v, _ in pairs], dt)
        assert [int(g) for g in got] == [b for _, b in pairs], (dt, [hex(int(g)) for g in got])


def pin_fp8_decode_vs_torch(lib):
    """Every code of e4m3, e5m2 and the e8m0 block scale decodes to torch's
    value for float8_e4m3fn, float8_e5m2 and float8_e8m0fnu (NaN codes alike)."""
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes)
    for dt, tdt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        got = oracle.decode(codes, dt, lib=lib)
        want = t.view(tdt).double().numpy()
        assert np.array_equal(got, want, equal_nan=True), dt
    got = oracle.decode_scale(codes, lib=lib)
    want = t.view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(got, want, equal_nan=True)
    # golden values read off the format definitions
    g = oracle.decode(np.array([0x7E, 0x08, 0x01, 0xFE], dtype=np.uint8), "e4m3", lib=lib)
    assert list(g) == [448.0, 2.0 ** -6, 2.0 ** -9, -448.0]
    g = oracle.decode(np.array([0x7B, 0x04, 0x01, 0x7C], dtype=np.uint8), "e5m2", lib=lib)
    assert list(g) == [57344.0, 2.0 ** -14, 2.0 ** -16, np.inf]


def _fp8_values(codes, dt):
    tdt = torch.float8_e4m3fn if dt == "e4m3" else torch.float8_e5m2
    return torch.from_numpy(np.ascontiguousarray(codes)).view(tdt).double().numpy()


def pin_fp8_gemm_brute_force(lib):
    """8-bit products, with and without block scales, against values decoded
    by torch and summed by numpy.  Unscaled, every value and sum is exact in
    fp64 (e4m3 codes are multiples of 2^-9 below 512, e5m2 codes come from a
    narrow exponent range), so the results must be equal; with scales
    (2^-7..2^7) the sums may round, and the two summation orders must agree
    within 2^-50 of the summed magnitudes."""
    rng = np.random.default_rng(11)
    M, N, K = 5, 6, 70
    for dt in ("e4m3", "e5m2"):
        if dt == "e4m3":
            pool = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
        else:
            pool = np.array([c for c in range(256) if 10 <= ((c >> 2) & 31) <= 20], dtype=np.uint8)
        lda, ldb = K + 3, K + 1
        A = rng.choice(pool, size=(M, lda)).astype(np.uint8)
        B = rng.choice(pool, size=(N, ldb)).astype(np.uint8)
        a, b = _fp8_values(A[:, :K], dt), _fp8_values(B[:, :K], dt)
        ref, mag = oracle.gemm(M, N, K, 0.75, False, A, lda, B, ldb, dt, lib=lib)
        want = 0.75 * (a @ b.T)
        assert np.array_equal(ref, want.T), dt
        assert np.array_equal(mag, (0.75 * (np.abs(a) @ np.abs(b).T)).T), dt
        # block scales: 3 blocks of 32 cover K = 70
        lds_a, lds_b = 4, 5
        sa = rng.integers(120, 135, size=(M, lds_a)).astype(np.uint8)
        sb = rng.integers(120, 135, size=(N, lds_b)).astype(np.uint8)
        blk = np.arange(K) // 32
        a_s = a * np.exp2(sa[:, blk].astype(np.float64) - 127)
        b_s = b * np.exp2(sb[:, blk].astype(np.float64) - 127)
        ref, mag = oracle.gemm(M, N, K, 0.75, True, A, lda, B, ldb, dt, lib=lib, scale_a=sa, lds_a=lds_a,
                               scale_b=sb, lds_b=lds_b)
        want = np.maximum(0.75 * (a_s @ b_s.T), 0).T
        assert np.all(np.abs(ref - want) <= 2.0 ** -50 * (0.75 * (np.abs(a_s) @ np.abs(b_s).T)).T), dt
        assert np.array_equal(mag, (0.75 * (np.abs(a_s) @ np.abs(b_s).T)).T) or \
            np.allclose(mag, (0.75 * (np.abs(a_s) @ np.abs(b_s).T)).T, rtol=2.0 ** -50, atol=0), dt
        ms, ns = np.array([0, 4, 2]), np.array([5, 0, 3])
        e, _ = oracle.gemm_entries(M, N, K, 0.75, True, A, lda, B, ldb, dt, ms, ns, lib=lib, scale_a=sa,
                                   lds_a=lds_a, scale_b=sb, lds_b=lds_b)
        assert np.array_equal(e, ref[ns, ms]), dt
        # a NaN scale poisons exactly the row it scales
        sa2 = sa.copy()
        sa2[2, 1] = 255
        ref2, _ = oracle.gemm(M, N, K, 0.75, False, A, lda, B, ldb, dt, lib=lib, scale_a=sa2, lds_a=lds_a)
        assert np.isnan(ref2[:, 2]).all() and np.isfinite(np.delete(ref2, 2, axis=1)).all()


# ------------------------------------------------------------- 4- and 6-bit formats

# bits per element, exponent bits, fraction bits, exponent bias (MX FP4/FP6 element formats)
_NARROW = {"e2m1": (4, 2, 1, 1), "e2m3": (6, 2, 3, 1), "e3m2": (6, 3, 2, 3)}


def _narrow_golden():
    codes: dict = {dt: {} for dt in _NARROW}
    packed = []
    for line in (GOLDEN.parent / "mx_narrow_codes.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        kind, dt, hx, rest = line.split(None, 3)
        if kind == "code":
            num, den = rest.split()
            codes[dt][int(hx, 16)] = Fraction(int(num), int(den))
        else:
            vals = [Fraction(int(a), int(b)) for a, b in (v.split("/") for v in rest.split(","))]
            packed.append((dt, bytes.fromhex(hx), vals))
    return codes, packed


def _narrow_table(dt) -> np.ndarray:
    """The value of every code of a 4- or 6-bit format, without the oracle:
    normal codes become the e4m3 bit pattern with the same sign, exponent
    (re-biased from the format's bias to 7) and fraction (left-aligned in the
    3 fraction bits) and are decoded by torch's float8_e4m3fn; zero and
    subnormal codes come from the golden table (a negative code is the
    negation of its positive twin)."""
    w, eb, mb, bias = _NARROW[dt]
    golden = _narrow_golden()[0][dt]
    out = np.empty(1 << w)
    for c in range(1 << w):
        sign, e, m = c >> (w - 1), (c >> mb) & ((1 << eb) - 1), c & ((1 << mb) - 1)
        if e == 0:
            v = float(golden[c & ((1 << (w - 1)) - 1)])
            out[c] = -v if sign else v
        else:
            bits = (sign << 7) | ((e - bias + 7) << 3) | (m << (3 - mb))
            out[c] = torch.tensor([bits], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
    return out


def _pack(codes: np.ndarray, w: int) -> np.ndarray:
    """Pack w-bit codes (last axis) into bytes, little-endian bit order, with
    numpy's bit packing."""
    codes = np.asarray(codes, dtype=np.uint8)
    bits = np.unpackbits(codes[..., None], axis=-1, bitorder="little")[..., :w]
    flat = bits.reshape(*codes.shape[:-1], codes.shape[-1] * w)
    return np.packbits(flat, axis=-1, bitorder="little")


def _unpack(storage: np.ndarray, w: int, count: int) -> np.ndarray:
    """Codes of the first `count` w-bit elements of each row of packed bytes."""
    bits = np.unpackbits(np.asarray(storage, dtype=np.uint8), axis=-1, bitorder="little")
    bits = bits[..., : count * w].reshape(*storage.shape[:-1], count, w)
    return (bits * (1 << np.arange(w))).sum(axis=-1).astype(np.int64)


def pin_narrow_decode(lib):
    """Every code of e2m1, e2m3 and e3m2 decodes to the value of the
    torch-based table, and the golden rows hold exactly."""
    golden, _ = _narrow_golden()
    for dt, (w, _, _, _) in _NARROW.items():
        table = _narrow_table(dt)
        codes = np.arange(1 << w, dtype=np.uint8)
        got = oracle.decode(_pack(codes, w), dt, lib=lib, count=1 << w)
        assert np.array_equal(got, table), dt
        for c, v in golden[dt].items():
            assert Fraction(float(got[c])) == v, (dt, hex(c), got[c], v)
        assert table.max() == {"e2m1": 6.0, "e2m3": 7.5, "e3m2": 28.0}[dt]


def pin_narrow_packing_golden(lib):
    """Hand-packed byte strings decode element by element to the listed
    values (fp4 nibble order, fp6 elements straddling bytes)."""
    _, packed = _narrow_golden()
    for dt, raw, vals in packed:
        got = oracle.decode(np.frombuffer(raw, dtype=np.uint8), dt, lib=lib, count=len(vals))
        assert [Fraction(float(g)) for g in got] == vals, (dt, raw.hex(), list(got))


def pin_narrow_gemm_brute_force(lib):
    """Packed 4- and 6-bit products against numpy on values unpacked by
    numpy and looked up in the torch-based table: exact without scales (every
    value and sum is a small multiple of 2^-4, exact in fp64), within 2^-50 of
    the summed magnitudes with block scales; padding codes past K are large
    and would show if read."""
    rng = np.random.default_rng(17)
    M, N = 5, 6
    for dt, (w, _, _, _) in _NARROW.items():
        K = 69 if w == 4 else 70
        lda, ldb = (72, 76) if w == 4 else (72, 80)   # whole bytes per row
        top = (1 << (w - 1)) - 1                        # the largest positive code
        A = np.full((M, lda), top, dtype=np.uint8)
        B = np.full((N, ldb), top, dtype=np.uint8)
        A[:, :K] = rng.integers(0, 1 << w, size=(M, K))
        B[:, :K] = rng.integers(0, 1 << w, size=(N, K))
        pa, pb = _pack(A, w), _pack(B, w)
        table = _narrow_table(dt)
        a = table[_unpack(pa, w, K)]
        b = table[_unpack(pb, w, K)]
        ref, mag = oracle.gemm(M, N, K, 0.75, False, pa.ravel(), lda, pb.ravel(), ldb, dt, lib=lib)
        assert np.array_equal(ref, (0.75 * (a @ b.T)).T), dt
        assert np.array_equal(mag, (0.75 * (np.abs(a) @ np.abs(b).T)).T), dt
        lds_a, lds_b = 3, 4
        sa = rng.integers(120, 135, size=(M, lds_a)).astype(np.uint8)
        sb = rng.integers(120, 135, size=(N, lds_b)).astype(np.uint8)
        blk = np.arange(K) // 32
        a_s = a * np.exp2(sa[:, blk].astype(np.float64) - 127)
        b_s = b * np.exp2(sb[:, blk].astype(np.float64) - 127)
        ref, _ = oracle.gemm(M, N, K, 0.75, True, pa.ravel(), lda, pb.ravel(), ldb, dt, lib=lib, scale_a=sa,
                             lds_a=lds_a, scale_b=sb, lds_b=lds_b)
        want = np.maximum(0.75 * (a_s @ b_s.T), 0).T
        assert np.all(np.abs(ref - want) <= 2.0 ** -50 * (0.75 * (np.abs(a_s) @ np.abs(b_s).T)).T), dt
        ms, ns = np.array([0, 4, 2]), np.array([5, 0, 3])
        e, _ = oracle.gemm_entries(M, N, K, 0.75, True, pa.ravel(), lda, pb.ravel(), ldb, dt, ms, ns, lib=lib,
                                   scale_a=sa, lds_a=lds_a, scale_b=sb, lds_b=lds_b)
        assert np.array_equal(e, ref[ns, ms]), dt


PINS = [pin_decode_golden, pin_decode_all_patterns, pin_permutation, pin_identity, pin_rank1,
        pin_small_integers, pin_tiny_rational, pin_zero_padded_k, pin_nan_padding_unread,
        pin_alpha_then_relu, pin_entries_and_column_ranges, pin_degenerate,
        pin_encode_roundtrip, pin_encode_f16_vs_numpy, pin_encode_bf16_vs_torch, pin_encode_golden,
        pin_fp8_decode_vs_torch, pin_fp8_gemm_brute_force,
        pin_narrow_decode, pin_narrow_packing_golden, pin_narrow_gemm_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle._load())


# ------------------------------------------------------------- planted mistakes

# Each mutation plants a plausible mistake in a copy of the oracle's C source;
# at least one pin must catch every one of them.
MUTATIONS = {
    "drop_last_k": ("for (int64_t k = 0; k < K; ++k) {\n        double p", "for (int64_t k = 0; k + 1 < K; ++k) {\n        double p"),
    "relu_before_alpha": ("double r = alpha * s;\n    if (relu && r < 0.0) r = 0.0;", "double r = s;\n    if (relu && r < 0.0) r = 0.0;\n    r *= alpha;"),
    "b_transposed": ("scaled_at(j->B, j->dtype, n * j->ldb, k, j->sb", "scaled_at(j->B, j->dtype, k * j->ldb, n, j->sb"),
    "a_stride_is_k": ("scaled_at(A, dtype, m * lda, k, sa", "scaled_at(A, dtype, m * K, k, sa"),
    "e4m3_bias_8": ("expo - 10);", "expo - 11);"),
    "e4m3_no_nan": ("if (expo == 15 && frac == 7)", "if (0)"),
    "e5m2_subnormal_scale": ("ldexp((double)frac, -16)", "ldexp((double)frac, -15)"),
    "scale_block_16": ("scales[scale_off + k / 32]", "scales[scale_off + k / 16]"),
    "scale_b_dropped": ("p.sb = sb; p.lds_b = lds_b;\n    int64_t cols", "p.lds_b = lds_b;\n    int64_t cols"),
    "e8m0_bias_128": ("(int)e - 127", "(int)e - 128"),
    "e2m1_bias_2": ("ldexp((double)(2 + frac), expo - 2)", "ldexp((double)(2 + frac), expo - 3)"),
    "e2m3_fraction_scale": ("ldexp((double)(8 + frac), expo - 4)", "ldexp((double)(8 + frac), expo - 3)"),
    "e3m2_subnormal_scale": ("ldexp((double)frac, -4);", "ldexp((double)frac, -3);"),
    "e2m1_sign_bit": ("int sign = (bits >> 3) & 1;", "int sign = (bits >> 2) & 1;"),
    "fp4_high_nibble_first": ("const int sh = (int)(bit & 7);", "const int sh = (int)((bit & 7) ^ (w == 4 ? 4 : 0));"),
    "fp6_no_straddle": ("if (sh + w > 8) v |=", "if (0) v |="),
    "f16_subnormal_flush": ("v = ldexp((double)frac, -24);", "v = 0.0;"),
    "f16_bias_off_by_one": ("expo - 25", "expo - 24"),
    "bf16_wrong_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "mag_signed": ("t += fabs(p);", "t += p;"),
    "sign_flip": ("s += p;", "s -= p;"),
    "relu_inverted": ("if (relu && r < 0.0) r = 0.0;", "if (relu && r > 0.0) r = 0.0;"),
    "encode_ties_away": ("nearbyint(a / ulp)", "floor(a / ulp + 0.5)"),
    "encode_truncate": ("nearbyint(a / ulp)", "trunc(a / ulp)"),
    "encode_no_subnormal_range": ("if (E < emin) E = emin;", ""),
    "encode_saturate": ("if (v > maxf) return (uint16_t)(sign | exp_all);",
                        "if (v > maxf) return (uint16_t)(sign | (exp_all - (1u << mant_bits)) | ((1u << mant_bits) - 1u));"),
}


def _mutant(tmp_path: Path, name: str):
    src = (Path(oracle.__file__).parent / "ref_gemm.c").read_text()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation {name} no longer matches the oracle source"
    path = tmp_path / f"mutant_{name}.c"
    path.write_text(src.replace(old, new))
    return oracle.bind(oracle.compile_source(path, tmp_path / f"libmutant_{name}.so"))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes(tmp_path, name):
    lib = _mutant(tmp_path, name)
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"


def test_out_tolerance_admits_rounded_fp32_results():
    """The low-precision bound admits the nearest bf16/fp16 value of a genuine
    fp32 accumulation, and rejects the same result one output unit off."""
    M, N, K = 16, 16, 1024
    A, B = si.operands(M, N, K, "bf16", "normal_invsqrtk", 63, 64)
    ref, mag = oracle.gemm(M, N, K, 0.5, False, _bits(A), K, _bits(B), K, "bf16")
    a32, b32 = A.float().numpy(), B.float().numpy()
    acc = np.zeros((N, M), dtype=np.float32)
    for k in range(K):
        acc += np.outer(b32[:, k], a32[:, k]).astype(np.float32)
    v = np.float32(0.5) * acc
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        d = torch.from_numpy(v).to(tdt).to(torch.float64).numpy()
        ok, ratio = oracle.check_out(d, ref, mag, K, dt)
        assert ok and ratio <= 1.0, (dt, ratio)
    # exact products far above the fp32 bound: the nearest output value passes,
    # its neighbour one unit up does not
    M, N, K = 16, 16, 4
    a = torch.tensor([[10.0 + m] * K for m in range(M)], dtype=torch.bfloat16)
    b = torch.tensor([[25.0 + n] * K for n in range(N)], dtype=torch.bfloat16)
    ref, mag = oracle.gemm(M, N, K, 1.0, False, _bits(a), K, _bits(b), K, "bf16")
    assert ref.min() >= 1000 and ref.max() < 4096
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        near = torch.from_numpy(ref.astype(np.float32)).to(tdt)
        ok, _ = oracle.check_out(near.to(torch.float64).numpy(), ref, mag, K, dt)
        assert ok, dt
        up = (near.view(torch.int16) + 1).view(tdt).to(torch.float64).numpy()
        moved = up != near.to(torch.float64).numpy()
        assert moved.all()
        ok, _ = oracle.check_out(np.where(ref % 3 == 0, up, near.to(torch.float64).numpy()), ref, mag, K, dt)
        assert not ok, dt


def test_tolerance_bound_holds_for_fp32_accumulation():
    """The acceptance bound admits a genuine fp32 accumulation of the same products
    (sequential fp32 sum in numpy) and rejects a result missing one K-stage."""
    M, N, K = 16, 16, 2048
    A, B = si.operands(M, N, K, "bf16", "normal_invsqrtk", 61, 62)
    ref, mag = oracle.gemm(M, N, K, 0.5, False, _bits(A), K, _bits(B), K, "bf16")
    a32 = A.float().numpy()
    b32 = B.float().numpy()
    acc = np.zeros((N, M), dtype=np.float32)
    for k in range(K):
        acc += np.outer(b32[:, k], a32[:, k]).astype(np.float32)
    d = np.float32(0.5) * acc
    ok, ratio = oracle.check(d, ref, mag, K)
    assert ok and ratio < 0.25, ratio
    # all ones: dropping one 64-wide K stage changes every entry by 64
    ones = np.full((M, K), 0x3F80, dtype=np.uint16)
    ref1, mag1 = oracle.gemm(M, N, K, 1.0, False, ones, K, ones[:N], K, "bf16")
    ok, _ = oracle.check(ref1 - 64.0, ref1, mag1, K)
    assert not ok


def test_softmax_reference():
    """The row softmax of the oracle: probabilities sum to one and are
    nonnegative, a constant added to a row changes nothing, equal logits give
    exactly 1/N, zero B gives uniform rows through the GEMM, and the result
    matches scipy's softmax."""
    from scipy.special import softmax as scipy_softmax

    rng = np.random.default_rng(3)
    x = rng.standard_normal((37, 11)) * 5          # (N, M): 37 columns n, 11 rows m
    y = oracle.softmax_rows(x)
    assert np.all(y >= 0) and np.allclose(y.sum(axis=0), 1.0, rtol=0, atol=1e-15)
    assert np.allclose(oracle.softmax_rows(x + rng.standard_normal((1, 11)) * 100), y, rtol=1e-12, atol=0)
    assert np.allclose(y, scipy_softmax(x, axis=0), rtol=1e-13, atol=0)
    assert np.array_equal(oracle.softmax_rows(np.full((8, 3), 2.5)), np.full((8, 3), 0.125))
    A = torch.ones(5, 7, dtype=torch.bfloat16)
    B = torch.zeros(16, 7, dtype=torch.bfloat16)
    ref, mag = oracle.gemm(5, 16, 7, 3.0, False, _bits(A), 7, _bits(B), 7, "bf16")
    assert np.array_equal(oracle.softmax_rows(ref), np.full((16, 5), 1.0 / 16))


def test_softmax_tolerance_admits_fp32_evaluation():
    """The softmax bound admits a float32 evaluation of the softmax of float32
    logits (a genuine fp32 accumulation) and rejects probabilities off by 1 %."""
    M, N, K = 16, 200, 512
    A, B = si.operands(M, N, K, "bf16", "normal_invsqrtk", 65, 66)
    ref, mag = oracle.gemm(M, N, K, 4.0, False, _bits(A), K, _bits(B), K, "bf16")
    a32, b32 = A.float().numpy(), B.float().numpy()
    acc = np.zeros((N, M), dtype=np.float32)
    for k in range(K):
        acc += np.outer(b32[:, k], a32[:, k]).astype(np.float32)
    x = np.float32(4.0) * acc
    e = np.exp(x - x.max(axis=0, keepdims=True))
    d = e / e.sum(axis=0, keepdims=True, dtype=np.float32)
    ok, ratio = oracle.check_softmax(d, ref, mag, K)
    assert ok and ratio < 0.5, ratio
    ok, _ = oracle.check_softmax(d * 1.01, ref, mag, K)
    assert not ok
