"""CPU oracle for row-major GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library.

``gemm_ref`` wraps ``gemm_oracle.c`` (a plain fp64 triple loop, see that file's
header for the definition it follows and the page passages it cites).
``normalized_error`` is the acceptance measure

    e = max_ij |C_ij - ref_ij| / bound_ij,   bound_ij = |alpha| sum_k |a_ik||b_kj| + |beta||c_ij|

where an element with bound_ij == 0 must equal ref_ij exactly (it counts as
infinite error otherwise).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O3", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-std=c11"]

_libs: dict = {}


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    _libs.pop(out, None)
    return out


def _load(path: str = LIB):
    lib = _libs.get(path)
    if lib is None:
        if not os.path.exists(path) and path == LIB:
            build()
        lib = ctypes.CDLL(path)
        fn = lib.oracle_gemm
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                       ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong,
                       ctypes.c_double, ctypes.c_void_p, ctypes.c_longlong,
                       ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        _libs[path] = lib
    return lib


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when set and by 16 (a GPU host's per-GPU CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, min(n, 16))


def _as_f32(x) -> np.ndarray:
    """Flat float32 view of an operand buffer; float16 values widen exactly."""
    a = np.ascontiguousarray(np.asarray(x).reshape(-1))
    if a.dtype == np.float16:
        return a.astype(np.float32)
    if a.dtype != np.float32:
        raise TypeError(f"operands must be float32 or float16 buffers, got {a.dtype}")
    return a


def widen_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) as the float32 values they denote.

    A bfloat16 is the upper half of an IEEE binary32 (sign, the same 8-bit
    exponent, 7 fraction bits), so the value is exactly the binary32 whose upper
    16 bits are the pattern and whose lower 16 bits are zero.  The MindNotes
    'GEMM' page names bf16 beside fp16 as an input format of its mixed-precision
    interface (section "Batched execution and mixed precision").
    """
    b = np.ascontiguousarray(np.asarray(bits).reshape(-1))
    if b.dtype != np.uint16:
        raise TypeError(f"bfloat16 operands are uint16 bit patterns, got {b.dtype}")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def gemm_ref(M: int, N: int, K: int, alpha: float, A, lda: int, B, ldb: int,
             beta: float, C, ldc: int, rows=None, threads: int | None = None,
             lib_path: str = LIB, transA: bool = False, transB: bool = False, bf16: bool = False):
    """(ref, bound) as float64 arrays of shape (len(rows) or M, N).

    ``A``, ``B``, ``C`` are flat row-major buffers (see ``seeded_inputs.matrix``);
    ``C`` may be None when ``beta == 0``.  ``rows`` selects output rows.
    ``transA`` / ``transB``: A is stored K x M / B is stored N x K (op = transpose).
    ``bf16``: A and B are bfloat16 bit patterns, widened exactly (``widen_bf16``).
    """
    lib = _load(lib_path)
    conv = widen_bf16 if bf16 else _as_f32
    a = conv(A) if M * K > 0 else np.zeros(1, np.float32)
    b = conv(B) if K * N > 0 else np.zeros(1, np.float32)
    c = _as_f32(C) if C is not None else None
    if rows is None:
        rows_arr = None
        nrows = M
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        nrows = int(rows_arr.size)
    ref = np.zeros((nrows, N), dtype=np.float64)
    bound = np.zeros((nrows, N), dtype=np.float64)
    rc = lib.oracle_gemm(
        int(bool(transA)), int(bool(transB)), M, N, K, float(np.float32(alpha)),
        a.ctypes.data, lda, b.ctypes.data, ldb,
        float(np.float32(beta)), c.ctypes.data if c is not None else None, ldc,
        rows_arr.ctypes.data if rows_arr is not None else None, nrows,
        ref.ctypes.data, bound.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_gemm rejected its arguments (status {rc})")
    return ref, bound


def gemm_ref_batched(M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                     strideC, batch, rows=None, threads=None, lib_path: str = LIB,
                     transA: bool = False, transB: bool = False, bf16: bool = False):
    """Strided-batched form: member b uses A + b*strideA, B + b*strideB, C + b*strideC.

    (MindNotes 'GEMM' page, section "Batched execution and mixed precision":
    a batch is a set of independent same-shape GEMMs a fixed stride apart.)
    Returns (ref, bound) of shape (batch, rows, N).
    """
    a = np.asarray(A).reshape(-1)
    b = np.asarray(B).reshape(-1)
    c = None if C is None else np.asarray(C).reshape(-1)
    refs, bounds = [], []
    for i in range(batch):
        ar, ac = (K, M) if transA else (M, K)
        br, bc = (N, K) if transB else (K, N)
        ai = a[i * strideA: i * strideA + (ar - 1) * lda + ac] if M * K else a
        bi = b[i * strideB: i * strideB + (br - 1) * ldb + bc] if K * N else b
        ci = None if c is None else c[i * strideC: i * strideC + (M - 1) * ldc + N]
        r, bd = gemm_ref(M, N, K, alpha, ai, lda, bi, ldb, beta, ci, ldc, rows, threads, lib_path,
                         transA, transB, bf16)
        refs.append(r)
        bounds.append(bd)
    return np.stack(refs), np.stack(bounds)


def normalized_error(Cgpu, ref, bound) -> float:
    """max |C - ref| / bound; elements with zero bound must match exactly."""
    C = np.asarray(Cgpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    if C.shape != ref.shape:
        raise ValueError(f"shape mismatch {C.shape} vs {ref.shape}")
    if C.size == 0:
        return 0.0
    if not np.all(np.isfinite(C)):
        return float("inf")
    diff = np.abs(C - ref)
    zero = bound == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(zero, 0.0, diff / np.where(zero, 1.0, bound))
    return float(e.max())


def logical(buf, rows: int, cols: int, ld: int) -> np.ndarray:
    """The rows x cols logical matrix held in a flat row-major buffer with stride ld."""
    b = np.asarray(buf).reshape(-1)
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols), dtype=b.dtype)
    return np.lib.stride_tricks.as_strided(b, shape=(rows, cols),
                                           strides=(ld * b.itemsize, b.itemsize)).copy()
