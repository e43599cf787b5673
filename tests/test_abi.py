"""C-ABI checks that need no GPU: the library loads, exports every function
include/mi355gemm.h declares, rejects bad arguments with the documented status
codes before any HIP call, and treats empty problems as no-ops."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import dense_gemm_optimisation_f32_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355gemm.h")

OK, ESIZE, ELD, ENULL, ELAUNCH, EALIGN, EOP, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 0x10000          # a non-NULL, 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dg.LIB_PATH):
        pytest.fail("libmi355gemm.so is not built; run python -m dense_gemm_optimisation_f32_amd.build")
    return dg.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(dg.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, f"{n} declared in mi355gemm.h but not exported"
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for code in (OK, ESIZE, ELD, ENULL, EALIGN, ELAUNCH, EOP, ESCRATCH):
        s = dg.status_string(code)
        assert s and s != "unknown status"
    assert dg.status_string(12345) == "unknown status"


def f32(lib, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    return lib.gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)


def f16(lib, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    return lib.gemm_f16_f32acc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)


def bf16(lib, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    return lib.gemm_bf16_f32acc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)


def bat(lib, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, nb):
    return lib.gemm_batched_f16_f32acc(M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, nb, None)


def batbf(lib, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, nb):
    return lib.gemm_batched_bf16_f32acc(M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, nb, None)


@pytest.mark.parametrize("fn", [f32, f16, bf16])
def test_argument_errors(lib, fn):
    # negative sizes
    assert fn(lib, -1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4) == ESIZE
    assert fn(lib, 4, -1, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4) == ESIZE
    assert fn(lib, 4, 4, -1, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4) == ESIZE
    # leading dimensions below the logical width (or below 1)
    assert fn(lib, 4, 5, 6, 1.0, FAKE, 5, FAKE, 5, 0.0, FAKE, 5) == ELD      # lda < K
    assert fn(lib, 4, 5, 6, 1.0, FAKE, 6, FAKE, 4, 0.0, FAKE, 5) == ELD      # ldb < N
    assert fn(lib, 4, 5, 6, 1.0, FAKE, 6, FAKE, 5, 0.0, FAKE, 4) == ELD      # ldc < N
    assert fn(lib, 4, 5, 0, 1.0, FAKE, 0, FAKE, 5, 0.0, FAKE, 5) == ELD      # lda < 1
    # NULL operands that would be read or written
    assert fn(lib, 4, 5, 6, 1.0, None, 6, FAKE, 5, 0.0, FAKE, 5) == ENULL
    assert fn(lib, 4, 5, 6, 1.0, FAKE, 6, None, 5, 0.0, FAKE, 5) == ENULL
    assert fn(lib, 4, 5, 6, 1.0, FAKE, 6, FAKE, 5, 0.0, None, 5) == ENULL
    assert fn(lib, 4, 5, 0, 1.0, None, 1, None, 5, 1.0, None, 5) == ENULL    # K = 0 still writes C
    # misaligned pointers
    assert fn(lib, 4, 5, 6, 1.0, FAKE, 6, FAKE, 5, 0.0, FAKE + 2, 5) == EALIGN
    assert fn(lib, 4, 5, 6, 1.0, FAKE + 1, 6, FAKE, 5, 0.0, FAKE, 5) == EALIGN


def test_f32_alignment_is_four_bytes(lib):
    assert f32(lib, 4, 5, 6, 1.0, FAKE + 2, 6, FAKE, 5, 0.0, FAKE, 5) == EALIGN
    assert f32(lib, 4, 5, 6, 1.0, FAKE, 6, FAKE + 2, 5, 0.0, FAKE, 5) == EALIGN


@pytest.mark.parametrize("bat", [bat, batbf])
def test_batched_argument_errors(lib, bat):
    M, N, K = 4, 5, 6
    assert bat(lib, M, N, K, 1.0, FAKE, K, M * K, FAKE, N, K * N, 0.0, FAKE, N, M * N, -1) == ESIZE
    assert bat(lib, M, N, K, 1.0, FAKE, K, -1, FAKE, N, K * N, 0.0, FAKE, N, M * N, 2) == ELD
    assert bat(lib, M, N, K, 1.0, FAKE, K, M * K, FAKE, N, -1, 0.0, FAKE, N, M * N, 2) == ELD
    assert bat(lib, M, N, K, 1.0, FAKE, K, M * K, FAKE, N, K * N, 0.0, FAKE, N, -1, 2) == ELD
    # C members would overlap
    assert bat(lib, M, N, K, 1.0, FAKE, K, M * K, FAKE, N, K * N, 0.0, FAKE, N, M * N - 1, 2) == ELD
    # a single member needs no C stride; operand strides may be 0 (shared operand)
    assert bat(lib, 0, N, K, 1.0, FAKE, K, 0, FAKE, N, 0, 0.0, FAKE, N, 0, 2) == OK
    # batch extent overflow
    assert bat(lib, M, N, K, 1.0, FAKE, K, 2**62, FAKE, N, K * N, 0.0, FAKE, N, M * N, 3) == ESIZE


def test_empty_problems_are_noops(lib):
    # No HIP call happens for these, so they succeed without a GPU.
    for fn in (f32, f16, bf16):
        assert fn(lib, 0, 5, 6, 1.0, None, 6, None, 5, 0.0, None, 5) == OK
        assert fn(lib, 4, 0, 6, 1.0, None, 6, None, 1, 0.0, None, 1) == OK
    assert bat(lib, 4, 5, 6, 1.0, None, 6, 0, None, 5, 0, 0.0, None, 5, 0, 0) == OK
    assert batbf(lib, 4, 5, 6, 1.0, None, 6, 0, None, 5, 0, 0.0, None, 5, 0, 0) == OK


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    a = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError):
        dg.gemm_f32(4, 4, 4, 1.0, a, 4, a, 4, 0.0, a, 4, stream=0)


def test_binding_reports_status_as_exception():
    with pytest.raises(dg.GemmError) as e:
        dg.gemm_f32(-1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, stream=0)
    assert e.value.status == ESIZE


def f32x(lib, tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    return lib.gemm_f32_ex(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)


def f16x(lib, tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    return lib.gemm_f16_f32acc_ex(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)


def bf16x(lib, tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    return lib.gemm_bf16_f32acc_ex(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)


@pytest.mark.parametrize("fn", [f32x, f16x, bf16x])
def test_transposed_leading_dimensions(lib, fn):
    M, N, K = 4, 5, 6
    # flags other than 0 / 1, checked first
    assert fn(lib, 2, 0, M, N, K, 1.0, FAKE, K, FAKE, N, 0.0, FAKE, N) == EOP
    assert fn(lib, 0, -1, M, N, K, 1.0, FAKE, K, FAKE, N, 0.0, FAKE, N) == EOP
    assert fn(lib, 2, 0, -1, N, K, 1.0, FAKE, K, FAKE, N, 0.0, FAKE, N) == EOP
    # A stored K x M needs lda >= M (not K); B stored N x K needs ldb >= K (not N)
    assert fn(lib, 1, 0, M, N, K, 1.0, FAKE, M - 1, FAKE, N, 0.0, FAKE, N) == ELD
    assert fn(lib, 0, 1, M, N, K, 1.0, FAKE, K, FAKE, K - 1, 0.0, FAKE, N) == ELD
    assert fn(lib, 1, 1, M, N, K, 1.0, FAKE, M, FAKE, K - 1, 0.0, FAKE, N) == ELD
    # the transposed widths are accepted even where the untransposed check would fail
    assert fn(lib, 1, 0, 0, N, K, 1.0, FAKE, 1, FAKE, N, 0.0, FAKE, N) == OK         # M = 0: no-op
    assert fn(lib, 1, 1, M, 0, K, 1.0, FAKE, M, FAKE, K, 0.0, FAKE, 1) == OK         # N = 0: no-op
    # misaligned pointer with transposed storage still refused
    assert fn(lib, 1, 1, M, N, K, 1.0, FAKE + 1, M, FAKE, K, 0.0, FAKE, N) == EALIGN
    # NULL operand still refused
    assert fn(lib, 1, 0, M, N, K, 1.0, None, M, FAKE, N, 0.0, FAKE, N) == ENULL


@pytest.mark.parametrize("name", ["gemm_batched_f16_f32acc_ex", "gemm_batched_bf16_f32acc_ex"])
def test_batched_transposed_errors(lib, name):
    M, N, K = 4, 5, 6
    bx = getattr(lib, name)
    assert bx(3, 0, M, N, K, 1.0, FAKE, K, M * K, FAKE, N, K * N, 0.0, FAKE, N, M * N, 2, None) == EOP
    assert bx(1, 0, M, N, K, 1.0, FAKE, M - 1, M * K, FAKE, N, K * N, 0.0, FAKE, N, M * N, 2, None) == ELD
    assert bx(0, 1, M, N, K, 1.0, FAKE, K, M * K, FAKE, N, K * N, 0.0, FAKE, N, M * N, 0, None) == ELD
    assert bx(1, 1, M, N, K, 1.0, FAKE, M, M * K, FAKE, K, K * N, 0.0, FAKE, N, M * N, 0, None) == OK


def test_binding_transposed_extent_check():
    torch = pytest.importorskip("torch")
    a = torch.zeros(16, dtype=torch.float32)
    # the binding refuses CPU tensors before computing anything (no GPU call)
    with pytest.raises(ValueError):
        dg.gemm_f32_ex(1, 1, 4, 4, 4, 1.0, a, 4, a, 4, 0.0, a, 4, stream=0)
    with pytest.raises(dg.GemmError) as e:
        dg.gemm_f32_ex(2, 0, 4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, stream=0)
    assert e.value.status == EOP


def test_grid_too_large_is_refused(lib):
    # ceil(M/32) * ceil(N/32) beyond INT_MAX cannot be one launch's grid: refused
    # before any HIP call (the pointers are never dereferenced)
    big = 2**31 - 1
    assert f32(lib, big, big, 1, 1.0, FAKE, 1, FAKE, big, 0.0, FAKE, big) == ESIZE
    assert f16(lib, big, big, 1, 1.0, FAKE, 1, FAKE, big, 0.0, FAKE, big) == ESIZE
    assert bf16(lib, big, big, 1, 1.0, FAKE, 1, FAKE, big, 0.0, FAKE, big) == ESIZE


def test_binding_checks_bf16_dtype():
    torch = pytest.importorskip("torch")
    h = torch.zeros(16, dtype=torch.float16)
    # the binding refuses a CPU tensor, and checks the dtype of device tensors
    with pytest.raises(ValueError):
        dg.gemm_bf16_f32acc(4, 4, 4, 1.0, h, 4, h, 4, 0.0, h, 4, stream=0)
    with pytest.raises(dg.GemmError) as e:
        dg.gemm_batched_bf16_f32acc_ex(0, 2, 4, 4, 4, 1.0, FAKE, 4, 16, FAKE, 4, 16, 0.0, FAKE, 4, 16, 2, stream=0)
    assert e.value.status == EOP


def test_noalloc_entry_point_checks_arguments_first(lib):
    # the entry point that allocates nothing runs the same checks before any HIP call
    fn = lib.gemm_f16_f32acc_noalloc
    assert fn(-1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, None) == ESIZE
    assert fn(4, 4, 4, 1.0, FAKE, 3, FAKE, 4, 0.0, FAKE, 4, None) == ELD
    assert fn(4, 4, 4, 1.0, None, 4, FAKE, 4, 0.0, FAKE, 4, None) == ENULL
    assert fn(4, 4, 4, 1.0, FAKE + 1, 4, FAKE, 4, 0.0, FAKE, 4, None) == EALIGN
    assert fn(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, None) == OK   # empty: nothing to do
