"""Seeded synthetic inputs for the tiled dense GEMM, shared by the tests, the
smoke check and the benchmark.

This module only draws numbers and lays them out in storage; it holds none of
the product's arithmetic, so both the GPU path and the oracle can consume its
output without sharing any computation.

Storage conventions (Tylo.jl manual, "Walk through GEMM", section 2): A is
logically (M,K) and stored K-contiguous, so its storage is a row-major
(M, lda) array whose first K columns hold A; B is logically (K,N) and stored
K-contiguous, so its storage is a row-major (N, ldb) array whose first K
columns hold B transposed; D is logically (M,N) stored M-contiguous, i.e. a
row-major (N, ldd) array whose first M columns hold D transposed.  Padding
columns of A and B are filled with NaN by default so that any read of them
shows up in the result.

Distributions are drawn in fp32 with a seeded torch CPU generator and then
rounded to the operand type (round-to-nearest-even, torch's cast); the rounded
values are the ground truth.  "normal(0, 1/sqrt(K))" is read as standard
deviation 1/sqrt(K).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

TORCH_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32,
                "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
# packed operand types: bits per element (element i of a stored array holds
# bits [w*i, w*i + w) of the bytes read as a little-endian bit string)
PACKED_BITS = {"e2m1": 4, "e2m3": 6, "e3m2": 6}
D_SENTINEL = -7777.0  # value planted in D storage that the product must never write


@dataclass(frozen=True)
class Workload:
    """One GEMM workload: shapes, strides, operand type, distribution, epilogue."""
    name: str
    M: int
    N: int
    K: int
    dtype: str            # operand type of A and B: "bf16", "f16", "f32", "e4m3" or "e2m1"
    dist: str             # "uniform_pm1", "uniform_01", "normal_invsqrtk" or (packed types) "codes"
    alpha: float
    relu: bool
    lda: int
    ldb: int
    ldd: int
    seed_a: int
    seed_b: int
    notes: str = field(default="", compare=False)
    batch: int = 1        # independent products, stored back to back (one launch)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch


def _w(name, M, N, K, dtype, dist, alpha, relu, seed_base, pad_ab=0, pad_d=0, notes="", batch=1):
    return Workload(name, M, N, K, dtype, dist, alpha, relu,
                    lda=K + pad_ab, ldb=K + pad_ab, ldd=M + pad_d,
                    seed_a=seed_base + 1, seed_b=seed_base + 2, notes=notes, batch=batch)


# The five measured/parity workloads, in order; the large square comes in both
# 16-bit operand types.
WORKLOADS = {
    "tiny_bounded_65x97x73_bf16": _w("tiny_bounded_65x97x73_bf16", 65, 97, 73, "bf16",
                                     "uniform_pm1", 1.5, True, 1000,
                                     notes="bounded tile: every edge ragged, K tail of 9"),
    "full_tile_1024_bf16": _w("full_tile_1024_bf16", 1024, 1024, 1024, "bf16",
                              "uniform_pm1", 1.0, False, 2000),
    "fp32_2048": _w("fp32_2048", 2048, 2048, 2048, "f32", "uniform_01", 1.0, False, 3000),
    "square_8192_bf16_relu": _w("square_8192_bf16_relu", 8192, 8192, 8192, "bf16",
                                "normal_invsqrtk", 0.5, True, 4000),
    "square_8192_f16_relu": _w("square_8192_f16_relu", 8192, 8192, 8192, "f16",
                               "normal_invsqrtk", 0.5, True, 4010),
    "ragged_strided_12289x5003x4099_bf16": _w("ragged_strided_12289x5003x4099_bf16",
                                              12289, 5003, 4099, "bf16", "uniform_pm1",
                                              2.0, True, 5000, pad_ab=8, pad_d=16,
                                              notes="lda=ldb=K+8, ldd=M+16"),
    # few output tiles and a long K: the shape split-K is for
    "tall_k_512x512x16384_bf16": _w("tall_k_512x512x16384_bf16", 512, 512, 16384, "bf16", "normal_invsqrtk",
                                    1.0, True, 7000),
    # a row softmax over N fused into the epilogue (one 256-wide tile spans N)
    "softmax_65536x256x4096_bf16": _w("softmax_65536x256x4096_bf16", 65536, 256, 4096, "bf16",
                                      "normal_invsqrtk", 1.0, False, 8000,
                                      notes="measured with tile_gemm_softmax"),
    # 8-bit operands (the block-scaled 8-bit matmul the cuTile tutorial's
    # closing section points to, here without scales): uniform values in
    # [-1, 1) rounded to e4m3, alpha 2^-13 keeps D near unit scale
    "square_8192_e4m3_relu": _w("square_8192_e4m3_relu", 8192, 8192, 8192, "e4m3", "uniform_pm1",
                                2.0 ** -13, True, 9000),
    # batched products (the batched GEMM of the cuTile tutorial's closing
    # section): 16 independent 1024^3 products, matrices stored back to back
    "batched_16x1024_bf16": _w("batched_16x1024_bf16", 1024, 1024, 1024, "bf16", "uniform_pm1",
                               1.0, True, 6000, batch=16,
                               notes="16 products; A (16*M, lda), B (16*N, ldb), D (16*N, ldd) storages"),
    # 4-bit operands (the block-scaled FP4 matmul of the cuTile tutorial's
    # closing section, here without scales): every e2m1 code equally likely,
    # alpha 2^-10 keeps D near unit scale
    "square_8192_e2m1_relu": _w("square_8192_e2m1_relu", 8192, 8192, 8192, "e2m1", "codes", 2.0 ** -10, True,
                                9500, notes="packed two per byte; A (M, lda/2), B (N, ldb/2) byte storages"),
    # 6-bit operands (MX FP6, E2M3), every code equally likely
    "square_8192_e2m3_relu": _w("square_8192_e2m3_relu", 8192, 8192, 8192, "e2m3", "codes", 2.0 ** -10, True,
                                9600, notes="packed four per three bytes; A (M, 3*lda/4), B (N, 3*ldb/4) bytes"),
}


def _draw(rows: int, cols: int, dist: str, K: int, gen: torch.Generator) -> torch.Tensor:
    if dist == "uniform_pm1":
        return torch.rand(rows, cols, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    if dist == "uniform_01":
        return torch.rand(rows, cols, generator=gen, dtype=torch.float32)
    if dist == "normal_invsqrtk":
        return torch.randn(rows, cols, generator=gen, dtype=torch.float32) * (1.0 / math.sqrt(max(K, 1)))
    raise ValueError(f"unknown distribution {dist!r}")


def _stored(rows: int, K: int, ld: int, values: torch.Tensor, dtype: str, pad: float) -> torch.Tensor:
    st = torch.full((rows, ld), pad, dtype=torch.float32).to(TORCH_DTYPES[dtype])
    if rows and K:
        st[:, :K] = values.to(TORCH_DTYPES[dtype])
    return st


def operands(M, N, K, dtype, dist, seed_a, seed_b, lda=None, ldb=None, pad=float("nan")):
    """Seeded storage for A ((M, lda) row-major) and B ((N, ldb) row-major), torch CPU."""
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ga = torch.Generator().manual_seed(int(seed_a))
    gb = torch.Generator().manual_seed(int(seed_b))
    a = _draw(M, K, dist, K, ga)
    b = _draw(N, K, dist, K, gb)
    return _stored(M, K, lda, a, dtype, pad), _stored(N, K, ldb, b, dtype, pad)


def workload_operands(w: Workload, pad=float("nan")):
    """A and B storages; a batched workload stacks its matrices: A is
    (batch*M, lda), matrix b in rows b*M .. b*M+M-1 (B likewise with N).
    Packed types give uint8 byte storages (see ``packed_operands``)."""
    if w.dtype in PACKED_BITS:
        a, b = packed_operands(w.batch * w.M, w.batch * w.N, w.K, w.dtype, w.seed_a, w.seed_b, w.lda, w.ldb)
        return torch.from_numpy(a), torch.from_numpy(b)
    if w.batch == 1:
        return operands(w.M, w.N, w.K, w.dtype, w.dist, w.seed_a, w.seed_b, w.lda, w.ldb, pad)
    ga = torch.Generator().manual_seed(int(w.seed_a))
    gb = torch.Generator().manual_seed(int(w.seed_b))
    a = _draw(w.batch * w.M, w.K, w.dist, w.K, ga)
    b = _draw(w.batch * w.N, w.K, w.dist, w.K, gb)
    return (_stored(w.batch * w.M, w.K, w.lda, a, w.dtype, pad),
            _stored(w.batch * w.N, w.K, w.ldb, b, w.dtype, pad))


def int_operands(M, N, K, dtype, seed, lda=None, ldb=None, lo=-3, hi=3, pad=float("nan")):
    """Seeded integer-valued storage (values in [lo, hi]) for A and B, torch CPU."""
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    g = torch.Generator().manual_seed(int(seed))
    a = torch.randint(lo, hi + 1, (M, K), generator=g).to(torch.float32)
    b = torch.randint(lo, hi + 1, (N, K), generator=g).to(torch.float32)
    return _stored(M, K, lda, a, dtype, pad), _stored(N, K, ldb, b, dtype, pad)


def pack_codes(codes: np.ndarray, w: int) -> np.ndarray:
    """Pack w-bit codes along the last axis into bytes: element i at bits
    [w*i, w*i + w) of the little-endian bit string (the last axis times w
    must be a multiple of 8)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    if (codes.shape[-1] * w) % 8:
        raise ValueError("rows must fill whole bytes")
    bitarr = np.unpackbits(codes[..., None], axis=-1, bitorder="little")[..., :w]
    flat = bitarr.reshape(*codes.shape[:-1], codes.shape[-1] * w)
    return np.packbits(flat, axis=-1, bitorder="little")


def packed_storage(rows: int, K: int, ld: int, dtype: str, seed: int, pool=None, pad_code=None) -> np.ndarray:
    """Seeded packed storage of a (rows, ld)-element operand: codes drawn
    uniformly from `pool` (default every code) for k < K and `pad_code`
    (default the largest positive code, so a read of the padding shows)
    beyond; (rows, ld*w/8) uint8."""
    w = PACKED_BITS[dtype]
    g = np.random.default_rng(int(seed))
    top = (1 << (w - 1)) - 1
    codes = np.full((rows, ld), top if pad_code is None else pad_code, dtype=np.uint8)
    if pool is None:
        codes[:, :K] = g.integers(0, 1 << w, size=(rows, K), dtype=np.uint8)
    else:
        codes[:, :K] = g.choice(np.asarray(pool, dtype=np.uint8), size=(rows, K))
    return pack_codes(codes, w)


def packed_operands(M, N, K, dtype, seed_a, seed_b, lda=None, ldb=None, pool=None, pad_code=None):
    """Seeded packed storages for A ((M, lda*w/8) bytes) and B ((N, ldb*w/8)
    bytes), numpy uint8."""
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    return (packed_storage(M, K, lda, dtype, seed_a, pool, pad_code),
            packed_storage(N, K, ldb, dtype, seed_b, pool, pad_code))


def block_scales(rows: int, K: int, seed: int, lo: int = 124, hi: int = 130, pad: int = 0,
                 dtype: str = "e4m3", fill: int = 127) -> np.ndarray:
    """Seeded block-scale exponents: (rows, lds) uint8 with lds =
    4*ceil(K/128) + pad for 8- and 6-bit operands (whole dwords per 128-k
    stage) or 16*ceil(K/512) + pad for 4-bit ones (16-byte pieces per two
    256-k stages), exponents in [lo, hi] for the ceil(K/32) live blocks and
    `fill` elsewhere."""
    nblk = -(-K // 32)
    lds = (16 * -(-K // 512) if dtype == "e2m1" else 4 * -(-K // 128)) + pad
    g = np.random.default_rng(int(seed))
    s = np.full((rows, max(lds, 4)), fill, dtype=np.uint8)
    s[:, :nblk] = g.integers(lo, hi + 1, size=(rows, nblk), dtype=np.uint8)
    return s


def out_storage(M, N, ldd=None, sentinel=D_SENTINEL) -> torch.Tensor:
    """D storage: row-major (N, ldd) fp32 pre-filled with a sentinel."""
    ldd = M if ldd is None else ldd
    return torch.full((N, ldd), sentinel, dtype=torch.float32)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU tensor as numpy: uint16 for bf16/fp16, float32 for
    fp32, uint8 for the 8-bit formats and for packed byte storages."""
    t = t.contiguous()
    if t.dtype == torch.uint8:
        return t.numpy()
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.view(torch.uint8).numpy()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported storage dtype {t.dtype}")


def sample_coords(M, N, count, seed, include_edges=True):
    """Seeded sample of output coordinates; optionally every entry of the last
    row band and column band plus the four corners, so ragged edges are
    always covered."""
    g = np.random.default_rng(int(seed))
    ms = g.integers(0, M, size=count, dtype=np.int64)
    ns = g.integers(0, N, size=count, dtype=np.int64)
    if include_edges and M and N:
        em = np.concatenate([np.full(N, M - 1), np.arange(M), [0, 0, M - 1, M - 1]]).astype(np.int64)
        en = np.concatenate([np.arange(N), np.full(M, N - 1), [0, N - 1, 0, N - 1]]).astype(np.int64)
        ms = np.concatenate([ms, em])
        ns = np.concatenate([ns, en])
    return ms, ns
