"""Pins for the CPU oracle (CPU only).

The oracle is checked against things other than itself: closed forms of the
GEMM definition (identity, permutation, all-ones, rank-1 operands), the
alpha/beta quick-return semantics, the leading-dimension and row-major/
transpose worked examples of the MindNotes 'GEMM' page (fixtures under
tests/golden/), exact rational arithmetic on tiny shapes, and fp64 rounding
bounds.  The last test plants a set of plausible mistakes in a copy of the
oracle's C source and checks that every one of them is caught by some pin.
"""
from __future__ import annotations

import itertools
import json
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALPHAS_BETAS = [(1.0, 0.0), (1.5, -0.5), (-1.0, 1.0), (0.0, 1.5), (1.0, -0.5)]


def _ref(p, alpha, beta, lib, **kw):
    return oracle.gemm_ref(p["M"], p["N"], p["K"], alpha, p["A"], p["lda"], p["B"], p["ldb"],
                           beta, p["C"], p["ldc"], lib_path=lib, **kw)


def _L(buf, r, c, ld):
    return oracle.logical(buf, r, c, ld).astype(np.float64)


def _exact(A, B, C, alpha, beta):
    """Exact rational alpha*A*B + beta*C and bound, from Python Fractions."""
    M, K = A.shape
    N = B.shape[1]
    fa, fb = Fraction(float(np.float32(alpha))), Fraction(float(np.float32(beta)))
    ref = [[None] * N for _ in range(M)]
    bnd = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = sum((Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)), Fraction(0))
            t = sum((abs(Fraction(float(A[i, k])) * Fraction(float(B[k, j]))) for k in range(K)), Fraction(0))
            c = Fraction(float(C[i, j])) if beta != 0 else Fraction(0)
            ref[i][j] = fa * s + fb * c
            bnd[i][j] = abs(fa) * t + abs(fb) * abs(c)
    return ref, bnd


# --------------------------------------------------------------------------- pins
# Each pin takes the path of a built oracle library and raises AssertionError
# when that oracle disagrees with what the definition fixes.

def pin_identity(lib):
    """A = I (M = K): ref = alpha*B + beta*C exactly, also with padded lda/ldb/ldc."""
    for n, N, pad in [(5, 7, 0), (17, 9, 3), (64, 33, 1)]:
        p = si.gemm_problem(n, N, n, lda=n + pad, ldb=N + pad, ldc=N + 2 * pad, seed=7)
        A = np.full(n * (n + pad), np.nan, np.float32).reshape(n, n + pad)
        A[:, :n] = np.eye(n, dtype=np.float32)
        p["A"] = A.reshape(-1)
        for alpha, beta in ALPHAS_BETAS:
            ref, bound = _ref(p, alpha, beta, lib)
            B = _L(p["B"], n, N, p["ldb"])
            C = _L(p["C"], n, N, p["ldc"])
            want = np.float64(np.float32(alpha)) * B + (np.float64(np.float32(beta)) * C if beta else 0.0)
            assert np.array_equal(ref, want), f"identity n={n} alpha={alpha} beta={beta}"
            wb = abs(np.float64(np.float32(alpha))) * np.abs(B) + (abs(beta) * np.abs(C) if beta else 0.0)
            assert np.array_equal(bound, wb)


def pin_permutation(lib):
    """A = P_pi picks rows of B; B = P_sigma permutes columns of A (pi, sigma not involutions)."""
    M, K, N = 6, 6, 5
    pi = [2, 0, 1, 5, 3, 4]          # row i of A has its 1 in column pi[i]
    p = si.gemm_problem(M, N, K, seed=11)
    A = np.zeros((M, K), np.float32)
    A[np.arange(M), pi] = 1
    p["A"] = A.reshape(-1)
    ref, _ = _ref(p, 1.0, 0.0, lib)
    B = _L(p["B"], K, N, N)
    for i in range(M):
        assert np.array_equal(ref[i], B[pi[i]]), f"row {i} should be row {pi[i]} of B"
    # B = P_sigma (K x N): column j of the product is column sigma^-1(j) of A.
    K2, N2 = 5, 5
    sigma = [1, 2, 3, 4, 0]          # B[k][sigma[k]] = 1
    q = si.gemm_problem(7, N2, K2, seed=12)
    Bp = np.zeros((K2, N2), np.float32)
    Bp[np.arange(K2), sigma] = 1
    q["B"] = Bp.reshape(-1)
    ref2, _ = _ref(q, 1.0, 0.0, lib)
    A2 = _L(q["A"], 7, K2, K2)
    for k in range(K2):
        assert np.array_equal(ref2[:, sigma[k]], A2[:, k])


def pin_closed_forms(lib):
    """All-ones operands, rank-1 operands, alpha = 0, K = 0 and beta = 0 with NaN C."""
    M, N, K = 9, 11, 13
    p = si.gemm_problem(M, N, K, seed=13)
    C = _L(p["C"], M, N, N)
    p1 = dict(p, A=np.ones(M * K, np.float32), B=np.ones(K * N, np.float32))
    for alpha, beta in ALPHAS_BETAS:
        ref, bound = _ref(p1, alpha, beta, lib)
        want = np.float64(alpha) * K + (np.float64(beta) * C if beta else 0.0)
        assert np.array_equal(ref, np.broadcast_to(want, (M, N)))
    # rank-1: a_ik = u_i, b_kj = v_j (small integers: every sum exact)
    u = np.arange(-4, M - 4, dtype=np.float32)
    v = np.arange(N, dtype=np.float32) - 5
    pr = dict(p, A=np.repeat(u, K), B=np.tile(v, K))
    ref, bound = _ref(pr, 1.5, -0.5, lib)
    want = 1.5 * K * np.outer(u, v) - 0.5 * C
    assert np.array_equal(ref, want)
    assert np.array_equal(bound, 1.5 * K * np.abs(np.outer(u, v)) + 0.5 * np.abs(C))
    # alpha = 0: A and B are not read (NaN operands), ref = beta*C
    pn = dict(p, A=np.full(M * K, np.nan, np.float32), B=np.full(K * N, np.nan, np.float32))
    ref, bound = _ref(pn, 0.0, -0.5, lib)
    assert np.array_equal(ref, -0.5 * C)
    # K = 0: ref = beta*C
    pk = dict(p, K=0, lda=1)
    ref, _ = _ref(pk, 1.5, 1.5, lib)
    assert np.array_equal(ref, 1.5 * C)
    # beta = 0: C is not read
    pc = dict(p, C=np.full(M * N, np.nan, np.float32))
    ref, bound = _ref(pc, 1.0, 0.0, lib)
    assert np.all(np.isfinite(ref)) and np.all(np.isfinite(bound))


def pin_brute_force_exact(lib):
    """Every shape in {1..6}^3 plus a few larger ones, small-integer entries: exact equality
    with rational arithmetic (every intermediate is an integer or half-integer far below 2**53)."""
    shapes = list(itertools.product(range(1, 7), repeat=3)) + [(7, 5, 3), (17, 9, 33)]
    for t, (M, N, K) in enumerate(shapes):
        alpha, beta = ALPHAS_BETAS[t % len(ALPHAS_BETAS)]
        p = si.gemm_problem(M, N, K, kind="int4", seed=100 + t)
        ref, bound = _ref(p, alpha, beta, lib)
        A, B, C = _L(p["A"], M, K, K), _L(p["B"], K, N, N), _L(p["C"], M, N, N)
        er, eb = _exact(A, B, C, alpha, beta)
        for i in range(M):
            for j in range(N):
                assert Fraction(ref[i, j]) == er[i][j], f"shape {(M, N, K)} ({i},{j})"
                assert Fraction(bound[i, j]) == eb[i][j]


def pin_fp64_rounding_bound(lib):
    """Random fp32 entries: |ref - exact| <= (K+2) * 2**-53 * bound (recursive summation bound)."""
    for t, (M, N, K) in enumerate([(3, 4, 5), (8, 8, 64), (5, 3, 200)]):
        p = si.gemm_problem(M, N, K, ldb=N + 1, seed=300 + t)
        ref, bound = _ref(p, 1.5, -0.5, lib)
        A, B, C = _L(p["A"], M, K, K), _L(p["B"], K, N, N + 1), _L(p["C"], M, N, N)
        er, eb = _exact(A, B, C, 1.5, -0.5)
        tol = (K + 2) * 2.0**-53
        for i in range(M):
            for j in range(N):
                assert abs(Fraction(ref[i, j]) - er[i][j]) <= Fraction(tol) * eb[i][j]
                assert abs(Fraction(bound[i, j]) - eb[i][j]) <= Fraction(tol) * eb[i][j]


def pin_lda_worked_example(lib):
    """The padded 2x3 matrix of the MindNotes leading-dimension example gives the same
    product with lda = 4 as the compact copy with lda = 3 (pads are NaN, so a read shows)."""
    g = json.load(open(os.path.join(GOLDEN, "lda_worked_example.json")))
    compact = np.array(g["compact"]["memory"], np.float32)
    padded = np.array([np.nan if v == "pad" else v for v in g["padded"]["memory"]], np.float32)
    assert np.array_equal(oracle.logical(padded, 2, 3, g["padded"]["ld"]), np.array(g["A_logical"], np.float32))
    Bm = si.matrix(5, 3, 4, 6, kind="int4")        # B 3x4 stored with ldb = 6
    Cm = si.matrix(6, 2, 4, 5, kind="int4")        # C 2x4 stored with ldc = 5
    r1, b1 = oracle.gemm_ref(2, 4, 3, 1.5, compact, 3, Bm, 6, -0.5, Cm, 5, lib_path=lib)
    r2, b2 = oracle.gemm_ref(2, 4, 3, 1.5, padded, 4, Bm, 6, -0.5, Cm, 5, lib_path=lib)
    assert np.array_equal(r1, r2) and np.array_equal(b1, b2)
    A = np.array(g["A_logical"], np.float64)
    want = 1.5 * A @ _L(Bm, 3, 4, 6) - 0.5 * _L(Cm, 2, 4, 5)
    assert np.array_equal(r1, want)


def pin_transpose_invariant(lib):
    """(A B)^T = B^T A^T: oracle(B^T, A^T)^T equals oracle(A, B) bit for bit (same products,
    same k order); at the MindNotes example's 2x3x4 shape the transposed result, read
    column-major, is C in row-major order."""
    g = json.load(open(os.path.join(GOLDEN, "row_major_transpose_example.json")))
    for (M, K, N) in [(g["M"], g["K"], g["N"]), (13, 29, 7), (33, 5, 40)]:
        p = si.gemm_problem(M, N, K, seed=400 + M)
        A, B, C = (oracle.logical(p["A"], M, K, K), oracle.logical(p["B"], K, N, N),
                   oracle.logical(p["C"], M, N, N))
        r, b = _ref(p, 1.5, -0.5, lib)
        At, Bt, Ct = (np.ascontiguousarray(x.T) for x in (A, B, C))
        rt, bt = oracle.gemm_ref(N, M, K, 1.5, Bt, K, At, M, -0.5, Ct, M, lib_path=lib)
        assert np.array_equal(r, rt.T) and np.array_equal(b, bt.T)
        # column-major read of the N x M result == row-major C
        assert np.array_equal(rt.reshape(-1, order="F"), r.reshape(-1))


def pin_row_subset_and_threads(lib):
    """Row subsets equal the same rows of the full result; thread count changes nothing."""
    M, N, K = 37, 19, 23
    p = si.gemm_problem(M, N, K, lda=K + 2, seed=500)
    full, fb = _ref(p, 1.5, -0.5, lib, threads=1)
    full8, fb8 = _ref(p, 1.5, -0.5, lib, threads=8)
    assert np.array_equal(full, full8) and np.array_equal(fb, fb8)
    rows = si.sample_rows(3, M, 10)
    sub, sb = _ref(p, 1.5, -0.5, lib, rows=rows)
    assert np.array_equal(sub, full[rows]) and np.array_equal(sb, fb[rows])


def _padded(mat, ld, tail):
    """Row-major copy of ``mat`` with leading dimension ``ld`` and ``tail`` NaN elements after it."""
    r, c = mat.shape
    buf = np.full(r * ld + tail, np.nan, np.float32)
    buf[: r * ld].reshape(r, ld)[:, :c] = mat
    return buf


def pin_op_storage(lib):
    """op(A) = A^T and op(B) = B^T (MindNotes definition C = alpha*op(A)op(B) + beta*C): storing
    the transpose and flagging it gives the same products in the same k order, so all four
    storage combinations agree bit for bit with the plain problem (which the exact brute force
    pins).  Buffers carry a NaN tail, so an index that strays past the stored matrix shows."""
    for (M, N, K) in [(5, 9, 7), (13, 8, 21), (32, 17, 1), (9, 4, 30)]:
        p = si.gemm_problem(M, N, K, seed=600 + M)
        A, B = oracle.logical(p["A"], M, K, K), oracle.logical(p["B"], K, N, N)
        tail = 4 * (M + N + K) * (M + N + K + 8)
        A_n, A_t = _padded(A, K + 2, tail), _padded(np.ascontiguousarray(A.T), M + 3, tail)
        B_n, B_t = _padded(B, N + 1, tail), _padded(np.ascontiguousarray(B.T), K + 5, tail)
        base = None
        for ta, tb in [(False, False), (True, False), (False, True), (True, True)]:
            r, b = oracle.gemm_ref(M, N, K, 1.5, A_t if ta else A_n, M + 3 if ta else K + 2,
                                   B_t if tb else B_n, K + 5 if tb else N + 1, -0.5, p["C"], N,
                                   lib_path=lib, transA=ta, transB=tb)
            if base is None:
                base = (r, b)
            assert np.array_equal(r, base[0]) and np.array_equal(b, base[1]), f"op {ta},{tb} shape {(M, N, K)}"
    # The MindNotes row-major trick with op flags: C^T = op(B')op(A') with B' = B stored K x N
    # read transposed and A' = A stored M x K read transposed gives C^T (N x M).
    M, K, N = 2, 3, 4
    p = si.gemm_problem(M, N, K, kind="int4", seed=77)
    r, _ = oracle.gemm_ref(M, N, K, 1.0, p["A"], K, p["B"], N, 0.0, None, N, lib_path=lib)
    rt, _ = oracle.gemm_ref(N, M, K, 1.0, p["B"], N, p["A"], K, 0.0, None, M, lib_path=lib,
                            transA=True, transB=True)
    assert np.array_equal(rt.T, r)


PINS = [pin_identity, pin_permutation, pin_closed_forms, pin_brute_force_exact,
        pin_fp64_rounding_bound, pin_lda_worked_example, pin_transpose_invariant,
        pin_row_subset_and_threads, pin_op_storage]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.LIB)


def test_bf16_widening_fixed_values():
    """A bfloat16 pattern is the upper half of a binary32 (1 sign, 8 exponent, 7
    fraction bits); the values of a few patterns worked out by hand."""
    cases = {0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3E80: 0.25, 0xC0A0: -5.0,
             0x4049: 3.140625, 0x3F81: 1.0 + 2.0**-7, 0x0000: 0.0, 0x0001: 2.0**-133,
             0x7F7F: (2.0 - 2.0**-7) * 2.0**127}
    got = oracle.widen_bf16(np.array(list(cases), dtype=np.uint16))
    for (bits, want), g in zip(cases.items(), got):
        assert float(g) == want, hex(bits)
    special = oracle.widen_bf16(np.array([0x8000, 0x7F80, 0xFF80, 0x7FC0], dtype=np.uint16))
    assert special[0] == 0.0 and np.signbit(special[0])
    assert special[1] == np.inf and special[2] == -np.inf and np.isnan(special[3])
    with pytest.raises(TypeError):
        oracle.widen_bf16(np.zeros(4, np.float16))


def test_bf16_inputs_are_round_to_nearest_even():
    """The bf16 input recipe: the fp32 draw rounded to nearest, ties to even, checked
    against torch's float32 -> bfloat16 conversion and two hand-made ties."""
    torch = pytest.importorskip("torch")
    x = si.draw(11, 50000)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(si.to_bf16_bits(x), want)
    ties = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8)], dtype=np.float32)
    assert si.to_bf16_bits(ties).tolist() == [0x3F80, 0x3F82, 0xBF80]
    buf = si.matrix(3, 4, 5, 7, "pm1", "bf16")   # pads are NaN patterns
    assert buf.dtype == np.uint16 and np.isnan(oracle.widen_bf16(buf).reshape(4, 7)[:, 5:]).all()


def test_bf16_problem_is_the_problem_of_the_values_it_denotes():
    """On bf16 operands the oracle computes exactly what it computes on the float32
    values the patterns denote (widened here by torch, not by the oracle), in all four
    storage combinations; and on small-integer bf16 entries it equals exact rational
    arithmetic."""
    torch = pytest.importorskip("torch")

    def torch_widen(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()

    for t, (tA, tB) in enumerate(itertools.product((False, True), repeat=2)):
        M, N, K = 7, 5, 19
        p = si.gemm_problem(M, N, K, in_dtype="bf16", seed=500 + t, transA=tA, transB=tB,
                            lda=(M if tA else K) + 2, ldb=(K if tB else N) + 1)
        r16, b16 = oracle.gemm_ref(M, N, K, 1.5, p["A"], p["lda"], p["B"], p["ldb"], -0.5, p["C"],
                                   p["ldc"], transA=tA, transB=tB, bf16=True)
        r32, b32 = oracle.gemm_ref(M, N, K, 1.5, torch_widen(p["A"]), p["lda"], torch_widen(p["B"]),
                                   p["ldb"], -0.5, p["C"], p["ldc"], transA=tA, transB=tB)
        assert np.array_equal(r16, r32) and np.array_equal(b16, b32)
    for t, (M, N, K) in enumerate([(3, 4, 5), (6, 2, 9), (5, 5, 16)]):
        p = si.gemm_problem(M, N, K, in_dtype="bf16", kind="int4", seed=600 + t)
        ref, bound = oracle.gemm_ref(M, N, K, 1.5, p["A"], K, p["B"], N, -0.5, p["C"], N, bf16=True)
        # the int4 draws are exact in bf16, so the float32 draws are the values the patterns denote
        A = si.matrix(600 + t, M, K, K, "int4").reshape(M, K).astype(np.float64)
        B = si.matrix(601 + t, K, N, N, "int4").reshape(K, N).astype(np.float64)
        C = si.matrix(602 + t, M, N, N, "int4").reshape(M, N).astype(np.float64)
        er, eb = _exact(A, B, C, 1.5, -0.5)
        for i in range(M):
            for j in range(N):
                assert Fraction(ref[i, j]) == er[i][j] and Fraction(bound[i, j]) == eb[i][j]


def test_rejects_bad_arguments():
    p = si.gemm_problem(4, 4, 4)
    with pytest.raises(ValueError):
        oracle.gemm_ref(4, 4, 4, 1.0, p["A"], 3, p["B"], 4, 0.0, None, 4)   # lda < K
    with pytest.raises(ValueError):
        oracle.gemm_ref(-1, 4, 4, 1.0, p["A"], 4, p["B"], 4, 0.0, None, 4)
    with pytest.raises(ValueError):
        oracle.gemm_ref(4, 4, 4, 1.0, p["A"], 4, p["B"], 4, 0.0, None, 4, rows=[4])
    with pytest.raises(ValueError):   # A stored transposed (K x M) needs lda >= M
        oracle.gemm_ref(5, 4, 3, 1.0, np.zeros(40, np.float32), 4, p["B"], 4, 0.0, None, 4, transA=True)
    with pytest.raises(ValueError):   # B stored transposed (N x K) needs ldb >= K
        oracle.gemm_ref(4, 3, 5, 1.0, np.zeros(40, np.float32), 5, np.zeros(40, np.float32), 4, 0.0, None, 3,
                        transB=True)


def test_normalized_error():
    ref = np.array([[1.0, 0.0]])
    bound = np.array([[2.0, 0.0]])
    assert oracle.normalized_error(np.array([[1.0, 0.0]]), ref, bound) == 0.0
    assert oracle.normalized_error(np.array([[1.5, 0.0]]), ref, bound) == 0.25
    assert oracle.normalized_error(np.array([[1.0, 1e-30]]), ref, bound) == float("inf")
    assert oracle.normalized_error(np.array([[np.nan, 0.0]]), ref, bound) == float("inf")


def test_batched_members_are_independent_problems():
    M, N, K, nb = 5, 6, 7, 3
    probs = [si.gemm_problem(M, N, K, seed=42, batch=b) for b in range(nb)]
    A = np.concatenate([q["A"] for q in probs]).astype(np.float16)
    B = np.concatenate([q["B"] for q in probs]).astype(np.float16)
    C = np.concatenate([q["C"] for q in probs])
    r, bd = oracle.gemm_ref_batched(M, N, K, 1.0, A, K, M * K, B, N, K * N, 1.0, C, N, M * N, nb)
    for b, q in enumerate(probs):
        r1, b1 = oracle.gemm_ref(M, N, K, 1.0, q["A"].astype(np.float16), K,
                                 q["B"].astype(np.float16), N, 1.0, q["C"], N)
        assert np.array_equal(r[b], r1) and np.array_equal(bd[b], b1)


# ------------------------------------------------------------------ planted mistakes
# Each entry replaces one fragment of the oracle's C source.  Every mutant stays
# in bounds for every shape the pins use, so a mutant can only give wrong values.
MUTANTS = {
    "drop_last_k": ("for (int k = 0; k < jb->K; ++k)", "for (int k = 0; k < jb->K - 1; ++k)"),
    "skip_first_k": ("for (int k = 0; k < jb->K; ++k)", "for (int k = (jb->K > 1); k < jb->K; ++k)"),
    "beta_sign": ("ref[j] = ab + jb->beta * c;", "ref[j] = ab - jb->beta * c;"),
    "beta_term_dropped": ("ref[j] = ab + jb->beta * c;", "ref[j] = ab;"),
    "alpha_on_c": ("ref[j] = ab + jb->beta * c;", "ref[j] = ab + jb->alpha * c;"),
    "alpha_dropped": ("double ab = jb->alpha != 0.0 ? jb->alpha * acc[j] : 0.0;",
                      "double ab = jb->alpha != 0.0 ? acc[j] : 0.0;"),
    "b_rows_reversed": ("(double)jb->B[(size_t)k * (size_t)jb->ldb + (size_t)j]",
                        "(double)jb->B[(size_t)(jb->K - 1 - k) * (size_t)jb->ldb + (size_t)j]"),
    "a_index_shifted": ("(double)jb->A[(size_t)i * (size_t)jb->lda + (size_t)k]",
                        "(double)jb->A[(size_t)i * (size_t)jb->lda + (size_t)((k + 1) % jb->K)]"),
    "b_column_shifted": ("(double)jb->B[(size_t)k * (size_t)jb->ldb + (size_t)j]",
                         "(double)jb->B[(size_t)k * (size_t)jb->ldb + (size_t)((j + 1) % N)]"),
    "bound_signed": ("acc_abs[j] += a_abs * fabs(b);", "acc_abs[j] += a_abs * b;"),
    "c_read_when_beta_zero": ("if (jb->beta != 0.0) {\n            const double c",
                              "if (crow) {\n            const double c"),
    "a_stride_ignores_lda": ("(double)jb->A[(size_t)i * (size_t)jb->lda + (size_t)k]",
                             "(double)jb->A[(size_t)i * (size_t)jb->K + (size_t)k]"),
    "c_stride_ignores_ldc": ("jb->C + (size_t)i * (size_t)jb->ldc", "jb->C + (size_t)i * (size_t)jb->N"),
    "float_accumulator": ("acc[j] += a * b;", "acc[j] = (double)(float)(acc[j] + a * b);"),
    "transA_ignored": ("const double a = jb->transA ?", "const double a = 0 ?"),
    "transB_ignored": ("const double b = jb->transB ?", "const double b = 0 ?"),
    "transposed_a_ignores_lda": ("(double)jb->A[(size_t)k * (size_t)jb->lda + (size_t)i]",
                                 "(double)jb->A[(size_t)k * (size_t)jb->M + (size_t)i]"),
    "transposed_b_ignores_ldb": ("(double)jb->B[(size_t)j * (size_t)jb->ldb + (size_t)k]",
                                 "(double)jb->B[(size_t)j * (size_t)jb->K + (size_t)k]"),
    "transposed_a_swapped_index": ("(double)jb->A[(size_t)k * (size_t)jb->lda + (size_t)i]",
                                   "(double)jb->A[(size_t)i * (size_t)jb->lda + (size_t)k]"),
}


def test_planted_mistakes_are_caught(tmp_path):
    src = open(oracle.SRC).read()
    survivors = []
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) >= 1, f"mutant {name}: fragment not found in the oracle source"
        msrc = tmp_path / f"{name}.c"
        msrc.write_text(src.replace(old, new, 1))
        lib = str(tmp_path / f"lib{name}.so")
        subprocess.run(["gcc", *oracle.CFLAGS, str(msrc), "-o", lib, "-lm"], check=True)
        caught = False
        for pin in PINS:
            try:
                pin(lib)
            except AssertionError:
                caught = True
                break
        if not caught:
            survivors.append(name)
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
