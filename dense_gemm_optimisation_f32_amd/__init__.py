"""Python binding of libmi355gemm.so: row-major GEMM on one MI355X.

The functions take the same arguments as the C ABI in
``include/mi355gemm.h`` and only marshal them (the ``_ex`` forms add the
transA/transB flags of C = alpha*op(A)op(B) + beta*C): every step of the computation
runs in the library's HIP kernels.  Operands may be torch CUDA tensors (their
``data_ptr()`` is passed; dtype, device and storage extent are checked first so
that a wrong buffer is refused on the host instead of faulting the GPU) or raw
integer device addresses (passed as they are).  ``stream`` may be None (torch's
current stream), a ``torch.cuda.Stream`` or a raw ``hipStream_t`` integer.

If the library is not built, importing works but every call raises
``GemmLibraryMissing``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["gemm_f32", "gemm_f16_f32acc", "gemm_batched_f16_f32acc",
           "gemm_f32_ex", "gemm_f16_f32acc_ex", "gemm_batched_f16_f32acc_ex",
           "gemm_bf16_f32acc", "gemm_batched_bf16_f32acc", "gemm_bf16_f32acc_ex", "gemm_batched_bf16_f32acc_ex",
           "gemm_f16_f32acc_noalloc", "status_string",
           "GemmError", "GemmLibraryMissing", "LIB_PATH", "load_library", "EXPORTS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmi355gemm.so")
EXPORTS = ("gemm_f32", "gemm_f16_f32acc", "gemm_batched_f16_f32acc",
           "gemm_f32_ex", "gemm_f16_f32acc_ex", "gemm_batched_f16_f32acc_ex",
           "gemm_bf16_f32acc", "gemm_batched_bf16_f32acc", "gemm_bf16_f32acc_ex", "gemm_batched_bf16_f32acc_ex",
           "gemm_f16_f32acc_noalloc", "gemm_status_string")

_lib = None


class GemmError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")


class GemmLibraryMissing(RuntimeError):
    """libmi355gemm.so has not been built (run dense_gemm_optimisation_f32_amd.build)."""


def load_library(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle of the library."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise GemmLibraryMissing(f"{path} is missing; build it with "
                                 "`python -m dense_gemm_optimisation_f32_amd.build`")
    lib = ctypes.CDLL(path)
    i, f, vp, ll = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_longlong
    lib.gemm_f32.argtypes = [i, i, i, f, vp, i, vp, i, f, vp, i, vp]
    lib.gemm_f32.restype = i
    lib.gemm_f16_f32acc.argtypes = [i, i, i, f, vp, i, vp, i, f, vp, i, vp]
    lib.gemm_f16_f32acc.restype = i
    lib.gemm_batched_f16_f32acc.argtypes = [i, i, i, f, vp, i, ll, vp, i, ll, f, vp, i, ll, i, vp]
    lib.gemm_batched_f16_f32acc.restype = i
    lib.gemm_f32_ex.argtypes = [i, i] + lib.gemm_f32.argtypes
    lib.gemm_f32_ex.restype = i
    lib.gemm_f16_f32acc_ex.argtypes = [i, i] + lib.gemm_f16_f32acc.argtypes
    lib.gemm_f16_f32acc_ex.restype = i
    lib.gemm_batched_f16_f32acc_ex.argtypes = [i, i] + lib.gemm_batched_f16_f32acc.argtypes
    lib.gemm_batched_f16_f32acc_ex.restype = i
    for name, base in (("gemm_bf16_f32acc", lib.gemm_f16_f32acc),
                       ("gemm_batched_bf16_f32acc", lib.gemm_batched_f16_f32acc),
                       ("gemm_bf16_f32acc_ex", lib.gemm_f16_f32acc_ex),
                       ("gemm_batched_bf16_f32acc_ex", lib.gemm_batched_f16_f32acc_ex)):
        fn = getattr(lib, name)
        fn.argtypes = base.argtypes
        fn.restype = i
    lib.gemm_f16_f32acc_noalloc.argtypes = lib.gemm_f16_f32acc.argtypes
    lib.gemm_f16_f32acc_noalloc.restype = i
    lib.gemm_status_string.argtypes = [i]
    lib.gemm_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().gemm_status_string(int(status)).decode()


def _extent(rows: int, cols: int, ld: int) -> int:
    return 0 if rows <= 0 or cols <= 0 else (rows - 1) * ld + cols


def _is_tensor(x) -> bool:
    return type(x).__module__.startswith("torch") and hasattr(x, "data_ptr")


def _ptr(x, name: str, dtype_name: str | None, need: int):
    """Device address of an operand, checking torch tensors against the extent read or written."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if _is_tensor(x):
        if x.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA tensor, got device {x.device}")
        if dtype_name is not None and str(x.dtype) != dtype_name:
            raise TypeError(f"{name} must have dtype {dtype_name}, got {x.dtype}")
        if need > 0:
            st = x.untyped_storage()
            avail = (st.nbytes() - (x.data_ptr() - st.data_ptr())) // x.element_size()
            if avail < need:
                raise ValueError(f"{name} holds {avail} elements from its start; the call needs {need}")
        return x.data_ptr()
    raise TypeError(f"{name}: expected a torch tensor or an integer device address, got {type(x)}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _needs(M, N, K, alpha, lda, ldb, ldc, batch=1, sA=0, sB=0, sC=0, transA=0, transB=0):
    reads_ab = K > 0 and alpha != 0 and M > 0 and N > 0
    nb = max(batch - 1, 0)
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    na = _extent(a_rows, a_cols, lda) + nb * sA if reads_ab else 0
    nbb = _extent(b_rows, b_cols, ldb) + nb * sB if reads_ab else 0
    nc = _extent(M, N, ldc) + nb * sC if batch > 0 else 0
    return na, nbb, nc


def gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> None:
    """C <- alpha*A*B + beta*C, fp32 (see gemm_f32 in include/mi355gemm.h)."""
    lib = load_library()
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc)
    rc = lib.gemm_f32(M, N, K, alpha, _ptr(A, "A", "torch.float32", na), lda,
                      _ptr(B, "B", "torch.float32", nb), ldb, beta,
                      _ptr(C, "C", "torch.float32", nc), ldc, _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_f32")


def gemm_f16_f32acc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> None:
    """C <- alpha*A*B + beta*C with fp16 A, B and fp32 accumulation and C."""
    lib = load_library()
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc)
    rc = lib.gemm_f16_f32acc(M, N, K, alpha, _ptr(A, "A", "torch.float16", na), lda,
                             _ptr(B, "B", "torch.float16", nb), ldb, beta,
                             _ptr(C, "C", "torch.float32", nc), ldc, _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_f16_f32acc")


def gemm_f16_f32acc_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> None:
    """gemm_f16_f32acc for callers that cannot allocate: its K split keeps its partial tiles in one
    static buffer per GPU (calls that overlap on one GPU must not be made)."""
    lib = load_library()
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc)
    rc = lib.gemm_f16_f32acc_noalloc(M, N, K, alpha, _ptr(A, "A", "torch.float16", na), lda,
                                     _ptr(B, "B", "torch.float16", nb), ldb, beta,
                                     _ptr(C, "C", "torch.float32", nc), ldc, _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_f16_f32acc_noalloc")


def gemm_batched_f16_f32acc(M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC,
                            batch_count, stream=None) -> None:
    """Strided-batched form of gemm_f16_f32acc (member b at A + b*strideA etc.)."""
    lib = load_library()
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc, batch_count, strideA, strideB, strideC)
    rc = lib.gemm_batched_f16_f32acc(M, N, K, alpha, _ptr(A, "A", "torch.float16", na), lda, strideA,
                                     _ptr(B, "B", "torch.float16", nb), ldb, strideB, beta,
                                     _ptr(C, "C", "torch.float32", nc), ldc, strideC, batch_count,
                                     _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_batched_f16_f32acc")


def gemm_f32_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> None:
    """C <- alpha*op(A)*op(B) + beta*C, fp32; transA: A stored K x M, transB: B stored N x K."""
    lib = load_library()
    tA, tB = int(transA), int(transB)   # values other than 0/1 are refused by the library
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc, transA=tA, transB=tB)
    rc = lib.gemm_f32_ex(tA, tB, M, N, K, alpha, _ptr(A, "A", "torch.float32", na), lda,
                         _ptr(B, "B", "torch.float32", nb), ldb, beta,
                         _ptr(C, "C", "torch.float32", nc), ldc, _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_f32_ex")


def gemm_f16_f32acc_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> None:
    """gemm_f16_f32acc with op(A)/op(B) (see gemm_f32_ex)."""
    lib = load_library()
    tA, tB = int(transA), int(transB)   # values other than 0/1 are refused by the library
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc, transA=tA, transB=tB)
    rc = lib.gemm_f16_f32acc_ex(tA, tB, M, N, K, alpha, _ptr(A, "A", "torch.float16", na), lda,
                                _ptr(B, "B", "torch.float16", nb), ldb, beta,
                                _ptr(C, "C", "torch.float32", nc), ldc, _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_f16_f32acc_ex")


def gemm_batched_f16_f32acc_ex(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                               strideC, batch_count, stream=None) -> None:
    """gemm_batched_f16_f32acc with op(A)/op(B) (see gemm_f32_ex)."""
    lib = load_library()
    tA, tB = int(transA), int(transB)   # values other than 0/1 are refused by the library
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc, batch_count, strideA, strideB, strideC, tA, tB)
    rc = lib.gemm_batched_f16_f32acc_ex(tA, tB, M, N, K, alpha, _ptr(A, "A", "torch.float16", na), lda, strideA,
                                        _ptr(B, "B", "torch.float16", nb), ldb, strideB, beta,
                                        _ptr(C, "C", "torch.float32", nc), ldc, strideC, batch_count,
                                        _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_batched_f16_f32acc_ex")


def gemm_bf16_f32acc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> None:
    """C <- alpha*A*B + beta*C with bf16 A, B and fp32 accumulation and C."""
    lib = load_library()
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc)
    rc = lib.gemm_bf16_f32acc(M, N, K, alpha, _ptr(A, "A", "torch.bfloat16", na), lda,
                              _ptr(B, "B", "torch.bfloat16", nb), ldb, beta,
                              _ptr(C, "C", "torch.float32", nc), ldc, _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_bf16_f32acc")


def gemm_batched_bf16_f32acc(M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC,
                             batch_count, stream=None) -> None:
    """Strided-batched form of gemm_bf16_f32acc."""
    lib = load_library()
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc, batch_count, strideA, strideB, strideC)
    rc = lib.gemm_batched_bf16_f32acc(M, N, K, alpha, _ptr(A, "A", "torch.bfloat16", na), lda, strideA,
                                      _ptr(B, "B", "torch.bfloat16", nb), ldb, strideB, beta,
                                      _ptr(C, "C", "torch.float32", nc), ldc, strideC, batch_count,
                                      _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_batched_bf16_f32acc")


def gemm_bf16_f32acc_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> None:
    """gemm_bf16_f32acc with op(A)/op(B) (see gemm_f32_ex)."""
    lib = load_library()
    tA, tB = int(transA), int(transB)   # values other than 0/1 are refused by the library
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc, transA=tA, transB=tB)
    rc = lib.gemm_bf16_f32acc_ex(tA, tB, M, N, K, alpha, _ptr(A, "A", "torch.bfloat16", na), lda,
                                 _ptr(B, "B", "torch.bfloat16", nb), ldb, beta,
                                 _ptr(C, "C", "torch.float32", nc), ldc, _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_bf16_f32acc_ex")


def gemm_batched_bf16_f32acc_ex(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                                strideC, batch_count, stream=None) -> None:
    """gemm_batched_bf16_f32acc with op(A)/op(B) (see gemm_f32_ex)."""
    lib = load_library()
    tA, tB = int(transA), int(transB)   # values other than 0/1 are refused by the library
    na, nb, nc = _needs(M, N, K, alpha, lda, ldb, ldc, batch_count, strideA, strideB, strideC, tA, tB)
    rc = lib.gemm_batched_bf16_f32acc_ex(tA, tB, M, N, K, alpha, _ptr(A, "A", "torch.bfloat16", na), lda,
                                         strideA, _ptr(B, "B", "torch.bfloat16", nb), ldb, strideB, beta,
                                         _ptr(C, "C", "torch.float32", nc), ldc, strideC, batch_count,
                                         _stream(stream))
    if rc != 0:
        raise GemmError(rc, "gemm_batched_bf16_f32acc_ex")
