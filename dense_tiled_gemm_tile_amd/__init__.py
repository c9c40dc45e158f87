"""Python binding of the tile_gemm C ABI (``include/tile_gemm.h``).

Argument marshalling only: every step of the GEMM runs in the HIP library
``_lib/libtile_gemm.so``; PyTorch supplies device memory and the stream.  If
the library is missing this module raises instead of computing anything on
another path.

Storage conventions (Tylo.jl manual, "Walk through GEMM", section 2): A is
logically (M,K) stored K-contiguous, B is logically (K,N) stored
K-contiguous, D is logically (M,N) stored M-contiguous, fp32 (or bf16/fp16
through ``tile_gemm_out``).  ``gemm`` takes
torch views with exactly those logical shapes and unit strides along K (A, B)
and along M (D), e.g. ``A = A_st[:, :K]``, ``B = B_st[:, :K].t()``,
``D = D_st[:, :M].t()`` for row-major storages A_st (M, lda), B_st (N, ldb),
D_st (N, ldd).  Packed 4-bit operands come as ``torch.float4_e2m1fn_x2``
views (two elements per storage element, low nibble first): A (M, K/2) with
unit stride along K, B (K/2, N) likewise, so K is even there; the raw entry
points take any K and strides in elements (6-bit operands have no torch
type and go through them).
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "_lib" / "libtile_gemm.so"
HEADER_PATH = _PKG.parent / "include" / "tile_gemm.h"

BF16, F16, F32, E4M3, E5M2, E2M1, E2M3, E3M2 = 1, 2, 3, 4, 5, 6, 7, 8
DTYPE_CODES = {"bf16": BF16, "f16": F16, "f32": F32, "e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1, "e2m3": E2M3,
               "e3m2": E3M2}

TG_OK = 0
STATUS = {0: "TG_OK", -1: "TG_ERR_DIMS", -2: "TG_ERR_LD", -3: "TG_ERR_NULL", -4: "TG_ERR_ALIGN",
          -5: "TG_ERR_DTYPE", -6: "TG_ERR_ALIAS", -7: "TG_ERR_LAUNCH", -8: "TG_ERR_DEVICE",
          -9: "TG_ERR_PLAN", -10: "TG_ERR_WORKSPACE"}


class TileGemmError(RuntimeError):
    """A tile_gemm entry point returned a nonzero status."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class PlanInfo(ctypes.Structure):
    """Mirror of ``tile_gemm_plan_info``."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "kernel_id", "dtype", "block_m", "block_n", "block_k", "waves_m", "waves_n",
        "wave_tile_m", "wave_tile_n", "threads", "stages", "lds_bytes", "acc_per_lane",
        "load_class", "group_m", "staged", "k_slices", "block_scales")] + [
        ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64), ("grid", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_i64, _ptr, _int, _f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_SIGNATURES = {
    "tile_gemm": (_int, [_i64, _i64, _i64, _f32, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _ptr]),
    "tile_gemm_ex": (_int, [_i64, _i64, _i64, _f32, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _ptr, _int]),
    "tile_gemm_out": (_int, [_i64, _i64, _i64, _f32, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int,
                             _ptr, _int]),
    "tile_gemm_query_plan": (_int, [_i64, _i64, _i64, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64,
                                    ctypes.POINTER(PlanInfo)]),
    "tile_gemm_batched": (_int, [_i64, _i64, _i64, _f32, _int, _ptr, _i64, _i64, _ptr, _i64, _i64, _ptr, _i64,
                                 _i64, _i64, _int, _int, _ptr, _int]),
    "tile_gemm_query_plan_batched": (_int, [_i64, _i64, _i64, _int, _ptr, _i64, _i64, _ptr, _i64, _i64, _ptr,
                                            _i64, _i64, _i64, _int, _int, ctypes.POINTER(PlanInfo)]),
    "tile_gemm_splitk": (_int, [_i64, _i64, _i64, _f32, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int, _int,
                                _ptr, _i64, _ptr, _int]),
    "tile_gemm_splitk_workspace_bytes": (_i64, [_i64, _i64, _int]),
    "tile_gemm_splitk_noalloc": (_int, [_i64, _i64, _i64, _f32, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int,
                                        _int, _ptr, _int]),
    "tile_gemm_staged": (_int, [_i64, _i64, _i64, _f32, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int, _ptr,
                                _i64, _ptr, _int]),
    "tile_gemm_staged_workspace_bytes": (_i64, [_i64, _i64, _i64, _int]),
    "tile_gemm_scaled": (_int, [_i64, _i64, _i64, _f32, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr,
                                _i64, _int, _int, _ptr, _int]),
    "tile_gemm_softmax": (_int, [_i64, _i64, _i64, _f32, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int, _ptr, _int]),
    "tile_gemm_query_plan_out": (_int, [_i64, _i64, _i64, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int,
                                        ctypes.POINTER(PlanInfo)]),
    "tile_gemm_query_plan_softmax": (_int, [_i64, _i64, _i64, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int,
                                            ctypes.POINTER(PlanInfo)]),
    "tile_gemm_query_plan_scaled": (_int, [_i64, _i64, _i64, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64,
                                           _ptr, _i64, _int, _int, ctypes.POINTER(PlanInfo)]),
    "tile_gemm_query_plan_staged": (_int, [_i64, _i64, _i64, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _ptr,
                                           _i64, _int, ctypes.POINTER(PlanInfo)]),
    "tile_gemm_kernel_count": (_int, []),
    "tile_gemm_kernel_info": (_int, [_int, ctypes.POINTER(PlanInfo)]),
    "tile_gemm_strerror": (ctypes.c_char_p, [_int]),
    "tile_gemm_abi_version": (_int, []),
}

_lib = None


def load_library() -> ctypes.CDLL:
    """Load the in-tree HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m dense_tiled_gemm_tile_amd.build`")
        lib = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/tile_gemm.h."""
    text = re.sub(r"/\*.*?\*/", "", HEADER_PATH.read_text(), flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tile_gemm\w*)\s*\(", text, flags=re.M)


def strerror(code: int) -> str:
    return load_library().tile_gemm_strerror(code).decode()


def _check(code: int) -> int:
    if code != TG_OK:
        raise TileGemmError(code, strerror(code))
    return code


# ---------------------------------------------------------------- raw entry points

def tile_gemm(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, stream=None) -> int:
    """Raw C call; pointers and the stream are integers (device addresses / hipStream_t)."""
    return load_library().tile_gemm(M, N, K, alpha, int(bool(relu)), A, lda, B, ldb, D, ldd,
                                     dtype, stream)


def tile_gemm_ex(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, stream=None, kernel_id=-1) -> int:
    return load_library().tile_gemm_ex(M, N, K, alpha, int(bool(relu)), A, lda, B, ldb, D, ldd,
                                       dtype, stream, kernel_id)


def tile_gemm_out(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, out_dtype, stream=None,
                  kernel_id=-1) -> int:
    return load_library().tile_gemm_out(M, N, K, alpha, int(bool(relu)), A, lda, B, ldb, D, ldd,
                                        dtype, out_dtype, stream, kernel_id)


def tile_gemm_batched(M, N, K, alpha, relu, A, lda, stride_a, B, ldb, stride_b, D, ldd, stride_d, batch,
                      dtype, out_dtype=F32, stream=None, kernel_id=-1) -> int:
    return load_library().tile_gemm_batched(M, N, K, alpha, int(bool(relu)), A, lda, stride_a, B, ldb,
                                            stride_b, D, ldd, stride_d, batch, dtype, out_dtype, stream,
                                            kernel_id)


def tile_gemm_splitk(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, out_dtype, splits, workspace,
                     workspace_bytes, stream=None, kernel_id=-1) -> int:
    return load_library().tile_gemm_splitk(M, N, K, alpha, int(bool(relu)), A, lda, B, ldb, D, ldd, dtype,
                                           out_dtype, splits, workspace, workspace_bytes, stream, kernel_id)


def tile_gemm_splitk_noalloc(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, out_dtype, splits, stream=None,
                             kernel_id=-1) -> int:
    return load_library().tile_gemm_splitk_noalloc(M, N, K, alpha, int(bool(relu)), A, lda, B, ldb, D, ldd, dtype,
                                                   out_dtype, splits, stream, kernel_id)


def tile_gemm_softmax(M, N, K, alpha, A, lda, B, ldb, D, ldd, dtype, out_dtype=F32, stream=None,
                      kernel_id=-1) -> int:
    return load_library().tile_gemm_softmax(M, N, K, alpha, A, lda, B, ldb, D, ldd, dtype, out_dtype, stream,
                                            kernel_id)


def splitk_workspace_bytes(M, N, splits) -> int:
    return load_library().tile_gemm_splitk_workspace_bytes(M, N, splits)


def tile_gemm_staged(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, out_dtype, workspace, workspace_bytes,
                     stream=None, mode=-1) -> int:
    return load_library().tile_gemm_staged(M, N, K, alpha, int(bool(relu)), A, lda, B, ldb, D, ldd, dtype,
                                           out_dtype, workspace, workspace_bytes, stream, mode)


def tile_gemm_scaled(M, N, K, alpha, relu, A, lda, scale_a, lds_a, B, ldb, scale_b, lds_b, D, ldd, dtype,
                     out_dtype=F32, stream=None, kernel_id=-1) -> int:
    return load_library().tile_gemm_scaled(M, N, K, alpha, int(bool(relu)), A, lda, scale_a, lds_a, B, ldb, scale_b,
                                           lds_b, D, ldd, dtype, out_dtype, stream, kernel_id)


def staged_workspace_bytes(M, N, K, dtype) -> int:
    return load_library().tile_gemm_staged_workspace_bytes(M, N, K, dtype)


def query_plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, kernel_id=-1, out_dtype=F32) -> PlanInfo:
    """Host-only plan query; raises TileGemmError on invalid arguments."""
    info = PlanInfo()
    if out_dtype == F32 and kernel_id == -1:
        rc = load_library().tile_gemm_query_plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, ctypes.byref(info))
    else:
        rc = load_library().tile_gemm_query_plan_out(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype,
                                                     kernel_id, ctypes.byref(info))
    _check(rc)
    return info


def query_plan_softmax(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype=F32, kernel_id=-1) -> PlanInfo:
    """Host-only plan of a tile_gemm_softmax call (kernel_id -1: two launches)."""
    info = PlanInfo()
    _check(load_library().tile_gemm_query_plan_softmax(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype, kernel_id,
                                                       ctypes.byref(info)))
    return info


def query_plan_scaled(M, N, K, dtype, A, lda, scale_a, lds_a, B, ldb, scale_b, lds_b, D, ldd, out_dtype=F32,
                      kernel_id=-1) -> PlanInfo:
    """Host-only plan of a tile_gemm_scaled call."""
    info = PlanInfo()
    _check(load_library().tile_gemm_query_plan_scaled(M, N, K, dtype, A, lda, scale_a, lds_a, B, ldb, scale_b, lds_b,
                                                      D, ldd, out_dtype, kernel_id, ctypes.byref(info)))
    return info


def query_plan_staged(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype=F32, workspace=None, workspace_bytes=0,
                      mode=-1) -> PlanInfo:
    """Host-only plan of a tile_gemm_staged call (staged = 1 when the copy runs)."""
    info = PlanInfo()
    _check(load_library().tile_gemm_query_plan_staged(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype, workspace,
                                                      workspace_bytes, mode, ctypes.byref(info)))
    return info


def kernel_count() -> int:
    return load_library().tile_gemm_kernel_count()


def kernel_info(kernel_id: int) -> PlanInfo:
    info = PlanInfo()
    _check(load_library().tile_gemm_kernel_info(kernel_id, ctypes.byref(info)))
    return info


def abi_version() -> int:
    return load_library().tile_gemm_abi_version()


# ---------------------------------------------------------------- torch views

def _operand_args(A, B, D):
    import torch

    codes = {torch.bfloat16: BF16, torch.float16: F16, torch.float32: F32,
             torch.float8_e4m3fn: E4M3, torch.float8_e5m2: E5M2, torch.float4_e2m1fn_x2: E2M1}
    out_codes = (BF16, F16, F32)
    if A.dim() != 2 or B.dim() != 2 or D.dim() != 2:
        raise ValueError("A, B and D must be 2-D views")
    M, K = A.shape
    K2, N = B.shape
    if A.dtype == torch.float4_e2m1fn_x2 and B.dtype == A.dtype:
        # two elements per storage element: sizes and strides in elements
        M, N, K, lda, ldb, ldd, dt, ot = _operand_args_checked(A, B, D, M, N, K, K2, codes, out_codes)
        return M, N, 2 * K, 2 * lda, 2 * ldb, ldd, dt, ot
    return _operand_args_checked(A, B, D, M, N, K, K2, codes, out_codes)


def _operand_args_checked(A, B, D, M, N, K, K2, codes, out_codes):
    if K2 != K or tuple(D.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, D {tuple(D.shape)}")
    if A.dtype != B.dtype or A.dtype not in codes:
        raise TypeError(f"A and B must share a dtype in {list(codes)}; got {A.dtype}, {B.dtype}")
    if D.dtype not in codes or codes[D.dtype] not in out_codes:
        raise TypeError(f"D must be float32, bfloat16 or float16; got {D.dtype}")
    if not (A.is_cuda and B.is_cuda and D.is_cuda):
        raise ValueError("A, B and D must be device tensors")
    if (K > 1 and A.stride(1) != 1) or (K > 1 and B.stride(0) != 1) or (M > 1 and D.stride(0) != 1):
        raise ValueError("A must be K-contiguous, B K-contiguous and D M-contiguous")
    lda = A.stride(0) if (M > 1 and K > 0) else max(K, 1)
    ldb = B.stride(1) if (N > 1 and K > 0) else max(K, 1)
    ldd = D.stride(1) if N > 1 else max(M, 1)
    return M, N, K, lda, ldb, ldd, codes[A.dtype], codes[D.dtype]


def bound_gemm(A, B, D, alpha: float = 1.0, relu: bool = False, stream=None, kernel_id: int = -1):
    """A no-argument callable that enqueues the same call as ``gemm`` with the
    arguments marshalled once (for tight launch loops: each call is then one
    foreign call into the library).  The views must stay alive and unchanged
    while the callable is used, and D's device must be the current device
    when it is called; it raises TileGemmError on a failed call."""
    import torch

    M, N, K, lda, ldb, ldd, dt, ot = _operand_args(A, B, D)
    if stream is None:
        stream = torch.cuda.current_stream(D.device)
    lib = load_library()
    if ot == F32:
        fn = lib.tile_gemm_ex
        args = (M, N, K, float(alpha), int(bool(relu)), A.data_ptr(), lda, B.data_ptr(), ldb, D.data_ptr(), ldd, dt,
                stream.cuda_stream, kernel_id)
    else:
        fn = lib.tile_gemm_out
        args = (M, N, K, float(alpha), int(bool(relu)), A.data_ptr(), lda, B.data_ptr(), ldb, D.data_ptr(), ldd, dt,
                ot, stream.cuda_stream, kernel_id)

    def call():
        rc = fn(*args)
        if rc != TG_OK:
            raise TileGemmError(rc, strerror(rc))

    return call


def gemm(A, B, D, alpha: float = 1.0, relu: bool = False, stream=None, kernel_id: int = -1):
    """D = alpha*A@B (+ReLU) on the GPU through the C ABI; returns D.

    A: (M,K) view with stride (lda, 1); B: (K,N) view with stride (1, ldb);
    D: (M,N) view with stride (1, ldd), float32 (tile_gemm_ex) or
    bfloat16/float16 (tile_gemm_out: fp32 epilogue rounded on the way out).
    The kernel is enqueued on `stream` (a torch.cuda.Stream, default: the
    current stream of D's device).
    """
    import torch

    M, N, K, lda, ldb, ldd, dt, ot = _operand_args(A, B, D)
    if stream is None:
        stream = torch.cuda.current_stream(D.device)
    with torch.cuda.device(D.device):
        if ot == F32:
            rc = tile_gemm_ex(M, N, K, float(alpha), relu, A.data_ptr(), lda, B.data_ptr(), ldb,
                              D.data_ptr(), ldd, dt, stream.cuda_stream, kernel_id)
        else:
            rc = tile_gemm_out(M, N, K, float(alpha), relu, A.data_ptr(), lda, B.data_ptr(), ldb,
                               D.data_ptr(), ldd, dt, ot, stream.cuda_stream, kernel_id)
        _check(rc)
    return D


def _batched_args(A, B, D):
    if A.dim() != 3 or B.dim() != 3 or D.dim() != 3:
        raise ValueError("A, B and D must be 3-D (batch, rows, cols) views")
    batch = D.shape[0]
    if A.shape[0] != batch or B.shape[0] != batch:
        raise ValueError(f"batch mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, D {tuple(D.shape)}")
    M, N, K, lda, ldb, ldd, dt, ot = _operand_args(A[0] if batch else A.new_empty(A.shape[1:]),
                                                   B[0] if batch else B.new_empty(B.shape[1:]),
                                                   D[0] if batch else D.new_empty(D.shape[1:]))
    sa, sb, sd = (A.stride(0), B.stride(0), D.stride(0)) if batch > 1 else (0, 0, 0)
    return M, N, K, lda, ldb, ldd, sa, sb, sd, batch, dt, ot


def plan_for_batched(A, B, D, kernel_id: int = -1) -> PlanInfo:
    """The plan ``gemm_batched`` would launch (grid counts every product)."""
    M, N, K, lda, ldb, ldd, sa, sb, sd, batch, dt, ot = _batched_args(A, B, D)
    info = PlanInfo()
    _check(load_library().tile_gemm_query_plan_batched(M, N, K, dt, A.data_ptr(), lda, sa, B.data_ptr(), ldb,
                                                       sb, D.data_ptr(), ldd, sd, batch, ot, kernel_id,
                                                       ctypes.byref(info)))
    return info


def gemm_batched(A, B, D, alpha: float = 1.0, relu: bool = False, stream=None, kernel_id: int = -1):
    """D[b] = alpha*A[b]@B[b] (+ReLU) for every b, in one launch; returns D.

    A: (batch, M, K) view with strides (stride_a, lda, 1); B: (batch, K, N) with
    strides (stride_b, 1, ldb); D: (batch, M, N) with strides (stride_d, 1, ldd),
    float32, bfloat16 or float16.  A batch stride of 0 (``expand``) reuses one
    operand for every product.
    """
    import torch

    M, N, K, lda, ldb, ldd, sa, sb, sd, batch, dt, ot = _batched_args(A, B, D)
    if stream is None:
        stream = torch.cuda.current_stream(D.device)
    with torch.cuda.device(D.device):
        _check(tile_gemm_batched(M, N, K, float(alpha), relu, A.data_ptr(), lda, sa, B.data_ptr(), ldb, sb,
                                 D.data_ptr(), ldd, sd, batch, dt, ot, stream.cuda_stream, kernel_id))
    return D


def gemm_splitk(A, B, D, alpha: float = 1.0, relu: bool = False, splits: int = 0, workspace=None,
                stream=None, kernel_id: int = -1):
    """As ``gemm``, with K split into `splits` ranges whose fp32 partial
    products are summed in split order before the epilogue (splits = 0: the
    library's automatic choice, within the workspace).  `workspace` is a
    device tensor of at least ``splitk_workspace_bytes(M, N, splits)`` bytes
    (allocated here through torch when omitted; the library itself allocates
    nothing)."""
    import torch

    M, N, K, lda, ldb, ldd, dt, ot = _operand_args(A, B, D)
    need = splitk_workspace_bytes(M, N, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=D.device)
    if stream is None:
        stream = torch.cuda.current_stream(D.device)
    with torch.cuda.device(D.device):
        _check(tile_gemm_splitk(M, N, K, float(alpha), relu, A.data_ptr(), lda, B.data_ptr(), ldb, D.data_ptr(),
                                ldd, dt, ot, splits, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), stream.cuda_stream, kernel_id))
    return D


def gemm_scaled(A, B, D, scale_a=None, scale_b=None, alpha: float = 1.0, relu: bool = False, stream=None,
                kernel_id: int = -1):
    """As ``gemm`` for 8-bit operands (torch.float8_e4m3fn / float8_e5m2 views)
    with block scales: scale_a a (M, lds_a) uint8 view (row stride lds_a,
    element [m, j] the exponent of k-block j of A row m), scale_b (N, lds_b)
    likewise for B's columns; either may be None."""
    import torch

    M, N, K, lda, ldb, ldd, dt, ot = _operand_args(A, B, D)

    def sc(t, rows):
        if t is None:
            return None, 0
        if t.dtype != torch.uint8 or t.dim() != 2 or t.shape[0] != rows or (rows > 1 and t.stride(1) != 1):
            raise ValueError("scales must be a (rows, lds) uint8 view with unit column stride")
        return t.data_ptr(), (t.stride(0) if rows > 1 else t.shape[1])

    pa, la = sc(scale_a, M)
    pb, lb = sc(scale_b, N)
    if stream is None:
        stream = torch.cuda.current_stream(D.device)
    with torch.cuda.device(D.device):
        _check(tile_gemm_scaled(M, N, K, float(alpha), relu, A.data_ptr(), lda, pa, la, B.data_ptr(), ldb, pb, lb,
                                D.data_ptr(), ldd, dt, ot, stream.cuda_stream, kernel_id))
    return D


def gemm_staged(A, B, D, alpha: float = 1.0, relu: bool = False, workspace=None, mode: int = 1, stream=None):
    """As ``gemm``, through tile_gemm_staged: A and B are first copied into
    16-byte aligned rows padded with zeros to whole K stages (mode 1: always;
    -1: when the plan says it pays; 0: never).  `workspace` is a device tensor
    of at least ``staged_workspace_bytes(M, N, K, dtype)`` bytes (allocated
    here through torch when omitted)."""
    import torch

    M, N, K, lda, ldb, ldd, dt, ot = _operand_args(A, B, D)
    if workspace is None:
        workspace = torch.empty(max(staged_workspace_bytes(M, N, K, dt), 256), dtype=torch.uint8, device=D.device)
    if stream is None:
        stream = torch.cuda.current_stream(D.device)
    with torch.cuda.device(D.device):
        _check(tile_gemm_staged(M, N, K, float(alpha), relu, A.data_ptr(), lda, B.data_ptr(), ldb, D.data_ptr(), ldd,
                                dt, ot, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                stream.cuda_stream, mode))
    return D


def gemm_softmax(A, B, D, alpha: float = 1.0, stream=None, kernel_id: int = -1):
    """D[m, :] = softmax over n of alpha*A@B (row m), through tile_gemm_softmax."""
    import torch

    M, N, K, lda, ldb, ldd, dt, ot = _operand_args(A, B, D)
    if stream is None:
        stream = torch.cuda.current_stream(D.device)
    with torch.cuda.device(D.device):
        _check(tile_gemm_softmax(M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb, D.data_ptr(), ldd,
                                 dt, ot, stream.cuda_stream, kernel_id))
    return D


def plan_for(A, B, D, kernel_id: int = -1) -> PlanInfo:
    """The plan ``gemm`` would launch for these views (the plan does not depend
    on the output type)."""
    M, N, K, lda, ldb, ldd, dt, ot = _operand_args(A, B, D)
    return query_plan(M, N, K, dt, A.data_ptr(), lda, B.data_ptr(), ldb, D.data_ptr(), ldd, kernel_id, ot)
