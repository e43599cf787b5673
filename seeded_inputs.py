"""Seeded synthetic inputs for GEMM problems.

This module only draws numbers and lays them out in memory.  It holds none of
the GEMM arithmetic: the oracle (under ``oracle/``) and the HIP library both
receive exactly the buffers made here, and neither imports the other.

Generator: splitmix64 (Sebastiano Vigna's public-domain 64-bit mixer).  It is
counter based -- output i depends only on ``seed + (i+1)*0x9E3779B97F4A7C15`` --
so a whole stream is produced with vectorised numpy uint64 arithmetic, and a C
or C++ program can reproduce it bit for bit from the published definition.

Value recipes (each entry of the logical matrix, filled row-major):

* ``"pm1"``   -- uniform on [-1, 1): x = (u >> 40) / 2**23 - 1.  Every value is a
  multiple of 2**-23 with magnitude < 1, hence exactly representable in fp32.
* ``"01"``    -- uniform on [0, 1): x = (u >> 40) / 2**24 (the all-positive
  distribution the MindNotes 'GEMM' page's benchmark harness fills with).
* ``"int4"``  -- integers uniform on [-4, 4]: x = ((u >> 32) * 9 >> 32) - 4.

fp16 operands are the fp32 draw rounded to binary16 with round-to-nearest-even
(numpy's ``astype(float16)``), so both sides see the same rounded values.
bf16 operands (``dtype="bf16"``) are the fp32 draw rounded to bfloat16 with
round-to-nearest-even, held as uint16 bit patterns (numpy has no bfloat16).

Seeds: matrix A of batch b uses ``seed + 0 + 3*b``, B uses ``seed + 1 + 3*b`` and
C uses ``seed + 2 + 3*b``.  Padding elements of a leading dimension larger than
the logical width hold NaN, so any read of a pad poisons the result.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

KINDS = ("pm1", "01", "int4")


def splitmix64(seed: int, n: int) -> np.ndarray:
    """Return the first ``n`` outputs of splitmix64 started from ``seed``."""
    with np.errstate(over="ignore"):
        i = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def draw(seed: int, n: int, kind: str = "pm1") -> np.ndarray:
    """``n`` float32 values of the given recipe (see module docstring)."""
    u = splitmix64(seed, n)
    if kind == "pm1":
        return ((u >> np.uint64(40)).astype(np.float64) / 2.0**23 - 1.0).astype(np.float32)
    if kind == "01":
        return ((u >> np.uint64(40)).astype(np.float64) / 2.0**24).astype(np.float32)
    if kind == "int4":
        hi = u >> np.uint64(32)
        with np.errstate(over="ignore"):
            v = (hi * np.uint64(9)) >> np.uint64(32)
        return (v.astype(np.int64) - 4).astype(np.float32)
    raise ValueError(f"unknown value recipe {kind!r}")


BF16 = "bf16"
_BF16_NAN = np.uint16(0x7FC0)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as uint16
    bit patterns (the upper half of the rounded binary32).  NaN maps to 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)
    r[np.isnan(x)] = _BF16_NAN
    return r


def matrix(seed: int, rows: int, cols: int, ld: int | None = None, kind: str = "pm1",
           dtype=np.float32) -> np.ndarray:
    """A row-major ``rows x cols`` matrix in a flat buffer of ``rows*ld`` elements.

    Element (r, c) sits at index ``r*ld + c``; the ``ld - cols`` pad elements at
    the end of each row are NaN.  ``dtype`` is float32, float16 or ``"bf16"``
    (the float16 and bfloat16 values are the float32 draw rounded to nearest
    even; bfloat16 ones are returned as uint16 bit patterns).
    """
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("leading dimension smaller than the row width")
    vals = draw(seed, rows * cols, kind).reshape(rows, cols)
    if isinstance(dtype, str) and dtype == BF16:
        buf = np.full((rows, ld), _BF16_NAN, dtype=np.uint16)
        buf[:, :cols] = to_bf16_bits(vals)
        return buf.reshape(-1)
    if dtype == np.float16:
        vals = vals.astype(np.float16)
    elif dtype != np.float32:
        raise ValueError("dtype must be float32, float16 or 'bf16'")
    buf = np.full((rows, ld), np.nan, dtype=vals.dtype)
    buf[:, :cols] = vals
    return buf.reshape(-1)


def gemm_problem(M: int, N: int, K: int, *, lda: int | None = None, ldb: int | None = None,
                 ldc: int | None = None, in_dtype=np.float32, kind: str = "pm1",
                 c_kind: str | None = None, seed: int = 42, batch: int = 0,
                 with_c: bool = True, transA: bool = False, transB: bool = False) -> dict:
    """Operands of one GEMM C = alpha*op(A)*op(B) + beta*C (row-major, see :func:`matrix`).

    Returns a dict with flat buffers ``A`` and ``B`` in ``in_dtype`` (float32,
    float16, or ``"bf16"`` for bfloat16 bit patterns) and ``C``
    (M x N, ldc, float32), plus the shape, leading dimensions and flags.  A is
    stored M x K, or K x M when ``transA``; B is stored K x N, or N x K when
    ``transB`` (the draw fills the stored matrix row by row either way).
    ``batch`` selects the seed offset of one member of a batch.
    ``with_c=False`` leaves ``C`` as None (for beta = 0, where C is never read).
    """
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    lda = max(a_cols, 1) if lda is None else lda
    ldb = max(b_cols, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    c_kind = kind if c_kind is None else c_kind
    base = seed + 3 * batch
    return {
        "M": M, "N": N, "K": K, "lda": lda, "ldb": ldb, "ldc": ldc,
        "transA": bool(transA), "transB": bool(transB),
        "A": matrix(base + 0, a_rows, a_cols, lda, kind, in_dtype),
        "B": matrix(base + 1, b_rows, b_cols, ldb, kind, in_dtype),
        "C": matrix(base + 2, M, N, ldc, c_kind, np.float32) if with_c else None,
    }


def logical_transpose(buf: np.ndarray, rows: int, cols: int, ld: int | None = None) -> np.ndarray:
    """The same values stored the other way round: a ``rows x cols`` matrix
    (flat, leading dimension ``ld``) as a flat ``cols x rows`` buffer with
    leading dimension ``rows``.  A pure relayout, no arithmetic."""
    ld = cols if ld is None else ld
    m = np.asarray(buf)[: rows * ld].reshape(rows, ld)[:, :cols]
    return np.ascontiguousarray(m.T).reshape(-1)


def sample_rows(seed: int, M: int, n: int = 64) -> np.ndarray:
    """``n`` distinct sorted row indices of an M-row matrix, always holding 0 and M-1."""
    if M <= n:
        return np.arange(M, dtype=np.int32)
    u = splitmix64(seed ^ 0x5EED, 8 * n)
    picks = {0, M - 1}
    for v in u:
        if len(picks) >= n:
            break
        picks.add(int(v % np.uint64(M)))
    return np.array(sorted(picks), dtype=np.int32)
