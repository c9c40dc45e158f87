"""Oracle for the tiled dense GEMM (+ReLU): plain fp64 CPU reference.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  It shares no code with the GPU
library (``dense_tiled_gemm_tile_amd``) and neither imports the other; the
product path never falls back to it.

The arithmetic lives in ``ref_gemm.c`` (plain C, built with gcc -O2, no
fast-math): for every requested (m, n) it forms the fp64 sum over k < K of the
decoded a[m,k] * b[k,n] in ascending k, then alpha times that sum, clamped at
zero when ReLU is on (Tylo.jl manual, "Walk through GEMM", opening paragraph and
section 5; cuTile.jl tutorial "Matrix Multiplication", Step 3).  Alongside it
returns mag[m,n] = sum over k of |alpha * a[m,k] * b[k,n]|, the magnitude that the
fp32 acceptance bound is stated in.

Storage follows the Tylo manual, section 2: A is (M,K) stored K-contiguous with
leading stride lda (element m*lda + k), B is (K,N) stored K-contiguous with
leading stride ldb (element k + n*ldb).  Arrays passed here are the raw storage:
``uint16`` bit patterns for bf16/fp16, ``float32`` for fp32, ``uint8`` for the
8-bit formats e4m3/e5m2 and for the packed bytes of the 4-bit (e2m1) and 6-bit
(e2m3, e3m2) formats, which may all carry block scales (``ref_gemm.c`` states
the formats, the packing and the scale reading).  Leading strides and element
counts are in elements for every format.

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed
forms, exact integer and rational arithmetic, and library decoders.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

BF16, F16, F32, E4M3, E5M2, E2M1, E2M3, E3M2 = 1, 2, 3, 4, 5, 6, 7, 8
_DTYPES = {"bf16": BF16, "f16": F16, "f32": F32, "e4m3": E4M3, "e5m2": E5M2,
           "e2m1": E2M1, "e2m3": E2M3, "e3m2": E3M2}
# bits per element; the 4- and 6-bit formats are packed (ref_gemm.c states how)
_BITS = {BF16: 16, F16: 16, F32: 32, E4M3: 8, E5M2: 8, E2M1: 4, E2M3: 6, E3M2: 6}

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "ref_gemm.c"
_LIB = _HERE / "_build" / "libgemm_oracle.so"
_lib = None

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def compile_source(src: Path, out: Path) -> Path:
    """Compile an oracle C source file into a shared library with gcc -O2."""
    out.parent.mkdir(parents=True, exist_ok=True)
    tmp = out.with_name(out.name + ".tmp")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-o", str(tmp), str(src), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> Path:
    """Compile the C oracle (always recompiles)."""
    return compile_source(_SRC, _LIB)


def bind(path) -> ctypes.CDLL:
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(str(path))
    lib.oracle_gemm.argtypes = [_i64, _i64, _i64, ctypes.c_float, ctypes.c_int,
                                _ptr, _i64, _ptr, _i64, ctypes.c_int,
                                _i64, _i64, _ptr, _ptr, _i64, ctypes.c_int]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_entries.argtypes = [_i64, _i64, _i64, ctypes.c_float, ctypes.c_int,
                                        _ptr, _i64, _ptr, _i64, ctypes.c_int,
                                        _i64, _ptr, _ptr, _ptr, _ptr, ctypes.c_int]
    lib.oracle_gemm_entries.restype = ctypes.c_int
    lib.oracle_gemm_scaled.argtypes = [_i64, _i64, _i64, ctypes.c_float, ctypes.c_int,
                                       _ptr, _i64, _ptr, _i64, ctypes.c_int, _ptr, _i64, _ptr, _i64,
                                       _i64, _i64, _ptr, _ptr, _i64, ctypes.c_int]
    lib.oracle_gemm_scaled.restype = ctypes.c_int
    lib.oracle_gemm_entries_scaled.argtypes = [_i64, _i64, _i64, ctypes.c_float, ctypes.c_int,
                                               _ptr, _i64, _ptr, _i64, ctypes.c_int, _ptr, _i64, _ptr, _i64,
                                               _i64, _ptr, _ptr, _ptr, _ptr, ctypes.c_int]
    lib.oracle_gemm_entries_scaled.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [_ptr, ctypes.c_int, _i64, _ptr]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_encode.argtypes = [_ptr, ctypes.c_int, _i64, _ptr]
    lib.oracle_encode.restype = ctypes.c_int
    for name in ("oracle_decode_bf16", "oracle_decode_f16"):
        getattr(lib, name).argtypes = [ctypes.c_uint16]
        getattr(lib, name).restype = ctypes.c_double
    for name in ("oracle_decode_e4m3", "oracle_decode_e5m2", "oracle_decode_e8m0"):
        getattr(lib, name).argtypes = [ctypes.c_uint8]
        getattr(lib, name).restype = ctypes.c_double
    return lib


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build()
        _lib = bind(_LIB)
    return _lib


def affinity_cores() -> int:
    """Cores in the process's CPU affinity mask."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_quota() -> float | None:
    """CPUs the process's cgroup grants (cpu.max quota / period), or None."""
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        return None if quota == "max" else int(quota) / int(period)
    except (OSError, ValueError):
        return None


def default_threads() -> int:
    """Host threads the oracle uses: one per core of the affinity mask, no
    more than the cgroup's CPU quota grants."""
    n = affinity_cores()
    q = cpu_quota()
    if q is not None:
        n = min(n, max(1, int(q)))
    return max(1, n)


def _code(dtype) -> int:
    return _DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def bits(dtype) -> int:
    """Bits per stored element of a dtype."""
    return _BITS[_code(dtype)]


def _storage(arr: np.ndarray, dtype: int) -> np.ndarray:
    want = np.float32 if dtype == F32 else np.uint8 if _BITS[dtype] <= 8 else np.uint16
    arr = np.ascontiguousarray(arr)
    if arr.dtype != want:
        raise TypeError(f"storage for dtype {dtype} must be {np.dtype(want)}, got {arr.dtype}")
    return arr


def decode(bits: np.ndarray, dtype, lib=None, count=None) -> np.ndarray:
    """Decode raw storage (uint16 for bf16/fp16, float32 for fp32, uint8 for
    e4m3/e5m2 and for packed e2m1/e2m3/e3m2) to fp64.  Packed storage decodes
    to a flat array of ``count`` elements (default: every whole element the
    bytes hold); other storage keeps its shape."""
    dt = _code(dtype)
    src = _storage(np.asarray(bits), dt)
    if _BITS[dt] < 8:
        n = src.size * 8 // _BITS[dt] if count is None else int(count)
        if n < 0 or n * _BITS[dt] > src.size * 8:
            raise ValueError("count exceeds the packed storage")
        out = np.empty(n, dtype=np.float64)
    else:
        out = np.empty(src.shape, dtype=np.float64)
    rc = (lib or _load()).oracle_decode(src.ctypes.data, dt, out.size, out.ctypes.data)
    if rc:
        raise ValueError(f"oracle_decode failed ({rc})")
    return out


def encode(values: np.ndarray, dtype, lib=None) -> np.ndarray:
    """Round fp64 values to bf16 or fp16 (nearest, ties to even); uint16 bits."""
    dt = _code(dtype)
    src = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(src.shape, dtype=np.uint16)
    rc = (lib or _load()).oracle_encode(src.ctypes.data, dt, src.size, out.ctypes.data)
    if rc:
        raise ValueError(f"oracle_encode failed ({rc})")
    return out


def _scales(sc, lds):
    if sc is None:
        return None, 0
    arr = np.ascontiguousarray(np.asarray(sc), dtype=np.uint8)
    return arr, int(lds)


def decode_scale(bits, lib=None) -> np.ndarray:
    """Block-scale exponents (uint8) to their values 2^(e - 127) (e = 255: NaN)."""
    lib = lib or _load()
    return np.array([lib.oracle_decode_e8m0(int(b)) for b in np.asarray(bits, dtype=np.uint8).ravel()],
                    dtype=np.float64).reshape(np.shape(bits))


def gemm(M, N, K, alpha, relu, A, lda, B, ldb, dtype, n0=0, n1=None, threads=None, lib=None,
         scale_a=None, lds_a=0, scale_b=None, lds_b=0):
    """Columns n0..n1-1 of the oracle result.

    A is the raw storage of A (at least (M-1)*lda + K elements, row-major
    (M, lda) is the usual shape), B likewise for B ((N, ldb)).  For the
    8-, 6- and 4-bit formats, scale_a / scale_b are optional block-scale exponents
    (uint8, byte m*lds_a + k//32 for A row m, n*lds_b + k//32 for B column n).
    Returns ``(ref, mag)``, both float64 arrays of shape (n1 - n0, M): row j
    holds output column n0 + j, i.e. the M-contiguous storage of the result.
    """
    dt = _code(dtype)
    n1 = N if n1 is None else n1
    a = _storage(np.asarray(A), dt)
    b = _storage(np.asarray(B), dt)
    sa, lds_a = _scales(scale_a, lds_a)
    sb, lds_b = _scales(scale_b, lds_b)
    cols = max(0, n1 - n0)
    ref = np.zeros((cols, M), dtype=np.float64)
    mag = np.zeros((cols, M), dtype=np.float64)
    rc = (lib or _load()).oracle_gemm_scaled(M, N, K, float(alpha), int(bool(relu)),
                                    a.ctypes.data if a.size else None, lda,
                                    b.ctypes.data if b.size else None, ldb, dt,
                                    sa.ctypes.data if sa is not None and sa.size else None, lds_a,
                                    sb.ctypes.data if sb is not None and sb.size else None, lds_b,
                                    n0, n1, ref.ctypes.data, mag.ctypes.data, max(M, 1),
                                    threads or default_threads())
    if rc:
        raise ValueError(f"oracle_gemm failed ({rc})")
    return ref, mag


def gemm_entries(M, N, K, alpha, relu, A, lda, B, ldb, dtype, ms, ns, threads=None, lib=None,
                 scale_a=None, lds_a=0, scale_b=None, lds_b=0):
    """Oracle result at the sampled coordinates (ms[i], ns[i]); returns (ref, mag)."""
    dt = _code(dtype)
    a = _storage(np.asarray(A), dt)
    b = _storage(np.asarray(B), dt)
    sa, lds_a = _scales(scale_a, lds_a)
    sb, lds_b = _scales(scale_b, lds_b)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape:
        raise ValueError("ms and ns must have the same shape")
    ref = np.zeros(ms.shape, dtype=np.float64)
    mag = np.zeros(ms.shape, dtype=np.float64)
    rc = (lib or _load()).oracle_gemm_entries_scaled(M, N, K, float(alpha), int(bool(relu)),
                                            a.ctypes.data if a.size else None, lda,
                                            b.ctypes.data if b.size else None, ldb, dt,
                                            sa.ctypes.data if sa is not None and sa.size else None, lds_a,
                                            sb.ctypes.data if sb is not None and sb.size else None, lds_b,
                                            ms.size, ms.ctypes.data, ns.ctypes.data,
                                            ref.ctypes.data, mag.ctypes.data,
                                            threads or default_threads())
    if rc:
        raise ValueError(f"oracle_gemm_entries failed ({rc})")
    return ref, mag


def tolerance(K: int, mag: np.ndarray) -> np.ndarray:
    """Acceptance bound for an fp32-accumulated result: 4*K*2^-24*mag + 1e-6.

    A K-term fp32 sum carries at most about K unit roundoffs (2^-24) of the
    summed magnitudes; the factor 4 is slack for the summation tree and the
    alpha scaling, and 1e-6 is an absolute floor for results near zero.
    """
    return 4.0 * K * 2.0 ** -24 * np.asarray(mag, dtype=np.float64) + 1e-6


# significant bits and smallest normal exponent of the 16-bit output formats
_FORMAT = {BF16: (8, -126), F16: (11, -14)}


def out_tolerance(K: int, mag: np.ndarray, ref: np.ndarray, out_dtype) -> np.ndarray:
    """Bound for a result rounded to a 16-bit output format: the fp32 bound plus
    half a unit in the last place of the output format at |ref| + that bound
    (the stored value is the nearest format value to an fp32 result within the
    fp32 bound of ref)."""
    p, emin = _FORMAT[_code(out_dtype)]
    tol = tolerance(K, mag)
    x = np.abs(np.asarray(ref, dtype=np.float64)) + tol
    _, e = np.frexp(x)
    E = np.maximum(e - 1, emin)
    return tol + 0.5 * np.ldexp(1.0, E - (p - 1))


def check_out(d: np.ndarray, ref: np.ndarray, mag: np.ndarray, K: int, out_dtype):
    """check() for a bf16/fp16 output (d decoded to fp64)."""
    d = np.asarray(d, dtype=np.float64)
    err = np.abs(d - ref)
    tol = out_tolerance(K, mag, ref, out_dtype)
    ratio = float(np.max(err / tol)) if err.size else 0.0
    ok = bool(np.all(err <= tol)) and not bool(np.any(np.isnan(d)))
    return ok, ratio


def check(d: np.ndarray, ref: np.ndarray, mag: np.ndarray, K: int):
    """Return (ok, worst_ratio): |d - ref| <= tolerance elementwise, and max |d-ref|/tol."""
    d = np.asarray(d, dtype=np.float64)
    err = np.abs(d - ref)
    tol = tolerance(K, mag)
    ratio = float(np.max(err / tol)) if err.size else 0.0
    ok = bool(np.all(err <= tol)) and not bool(np.any(np.isnan(d)))
    return ok, ratio


def softmax_rows(ref: np.ndarray) -> np.ndarray:
    """Softmax over n for every row m of the logits ``ref`` = alpha*S (fp64,
    shape (N, M) as returned by ``gemm`` with relu off): y = exp(x - max_n x) /
    sum_n exp(x - max_n x) (the row-wise epilogue of the Tylo.jl manual,
    "Walk through GEMM", section 5).  numpy's exp and sum serve as the steps."""
    x = np.asarray(ref, dtype=np.float64)
    e = np.exp(x - x.max(axis=0, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def softmax_tolerance(K: int, mag: np.ndarray, ref: np.ndarray, out_dtype="f32") -> np.ndarray:
    """Bound for a softmax computed from fp32 logits.

    Logits within T of the exact ones (T = the row's largest fp32 bound) move
    each probability by at most a factor exp(+-2T); evaluating in fp32 adds
    about one rounding of (x - max) relative to its magnitude inside exp, and
    about N + 8 roundings for the sum, the exponential and the division.  A
    16-bit output adds half a unit of its format."""
    x = np.asarray(ref, dtype=np.float64)
    y = softmax_rows(x)
    T = tolerance(K, mag).max(axis=0, keepdims=True)
    N = x.shape[0]
    rel = np.expm1(2.0 * T) + 2.0 ** -24 * (np.abs(x - x.max(axis=0, keepdims=True)) + N + 8)
    tol = y * rel + 1e-37
    if _code(out_dtype) != F32:
        p, emin = _FORMAT[_code(out_dtype)]
        _, e = np.frexp(y + tol)
        tol = tol + 0.5 * np.ldexp(1.0, np.maximum(e - 1, emin) - (p - 1))
    return tol


def check_softmax(d: np.ndarray, ref: np.ndarray, mag: np.ndarray, K: int, out_dtype="f32"):
    """Return (ok, worst_ratio) of a GPU softmax d (fp64, shape (N, M))."""
    d = np.asarray(d, dtype=np.float64)
    y = softmax_rows(ref)
    tol = softmax_tolerance(K, mag, ref, out_dtype)
    err = np.abs(d - y)
    ratio = float(np.max(err / tol)) if err.size else 0.0
    ok = bool(np.all(err <= tol)) and not bool(np.any(np.isnan(d)))
    return ok, ratio
