"""Host-side model of the global addresses the masked direct-to-LDS kernels
read in their slice loads, checked against the smallest allocation a caller may
pass ((K-1)*ld + cols elements for a K-row operand, and so on).

The kernels load every slice as 16-byte chunks (4 floats or 8 halves).  Rows
of a K-contiguous operand past M or N re-read row lim-1; chunks of an
MN-contiguous operand wholly past M or N re-read chunk 0 of their row; a chunk
that straddles M or N is loaded whole, its extra elements reaching only C
entries that are never stored.  Such a chunk reads into the next row, so when
one exists the slices stop before row K-1 and the rest of K is read element by
element.  This file restates that arithmetic (tile sizes, slice depth, clamps,
the slice count) and checks the largest element index each operand's slices
touch.  It runs on the CPU; the GPU parity tests check the results.
"""
import itertools
import random

import pytest

# (kind, BM, BN, BK): the direct-to-LDS tile configurations
CONFIGS = [("f32", 256, 256, 32), ("f32", 128, 128, 32), ("f32", 64, 64, 32),
           ("f16", 256, 256, 64), ("f16", 128, 128, 64), ("f16", 64, 128, 64)]


def takes(kind, BM, BN, tA, tB):
    """Storage combinations a tile is launched for: an fp16 MN-contiguous slice
    needs 128-wide rows (A stored K x M needs BM >= 128, B stored K x N BN >= 128)."""
    return kind != "f16" or ((not tA or BM >= 128) and (tB or BN >= 128))


def max_slice_index(kind, M, N, K, lda, ldb, tA, tB, BM, BN, BK, stop_before_last_row=True):
    """Largest element index that any slice load reads in A and in B."""
    ch = 4 if kind == "f32" else 8
    a_kc, b_kc = not tA, tB
    straddle = ((not a_kc) and M % ch != 0) or ((not b_kc) and N % ch != 0)
    nk = ((K - 1) if (straddle and stop_before_last_row) else K) // BK
    if nk == 0:
        return -1, -1
    t = nk - 1                      # the highest slice touches the highest addresses
    hi = {}
    for name, kc, R, extent, ld, tiles in (("A", a_kc, BM, M, lda, -(-M // BM)), ("B", b_kc, BN, N, ldb, -(-N // BN))):
        best = -1
        for tile in range(tiles):
            first = tile * R
            lim = min(extent - first, R)
            if kc:   # rows first .. first+R-1 (clamped to lim-1), k in the slice
                best = max(best, (first + min(R - 1, lim - 1)) * ld + t * BK + BK - 1)
            else:    # k rows of the slice, chunks along M or N (wholly outside -> chunk 0)
                top = max(c for c in range(R // ch) if not ch * c >= lim) if lim > 0 else 0
                best = max(best, (t * BK + BK - 1) * ld + first + ch * top + ch - 1)
        hi[name] = best
    return hi["A"], hi["B"]


def minimal_sizes(M, N, K, lda, ldb, tA, tB):
    size_a = (K - 1) * lda + M if tA else (M - 1) * lda + K
    size_b = (N - 1) * ldb + K if tB else (K - 1) * ldb + N
    return size_a, size_b


def shapes():
    fixed = [(1500, 1500, 1536), (1500, 1500, 257), (1001, 1003, 1024), (4095, 4093, 256), (9, 13, 64),
             (13, 9, 256), (2050, 2046, 320), (1002, 998, 65), (200, 140, 320), (4100, 4092, 512)]
    rng = random.Random(1)
    rand = [(rng.randint(8, 3000), rng.randint(8, 3000), rng.choice([65, 96, 129, 192, 257, 320, 1000, 1024]))
            for _ in range(120)]
    return fixed + rand


@pytest.mark.parametrize("kind,BM,BN,BK", CONFIGS)
def test_slice_loads_stay_inside_minimal_operands(kind, BM, BN, BK):
    checked = 0
    for (M, N, K), (tA, tB) in itertools.product(shapes(), [(0, 0), (0, 1), (1, 0), (1, 1)]):
        if not takes(kind, BM, BN, tA, tB):
            continue
        for pad in (0, 2, 6) if kind == "f16" else (0, 1, 3):
            lda, ldb = (M if tA else K) + pad, (K if tB else N) + pad
            hi_a, hi_b = max_slice_index(kind, M, N, K, lda, ldb, tA, tB, BM, BN, BK)
            size_a, size_b = minimal_sizes(M, N, K, lda, ldb, tA, tB)
            assert hi_a < size_a and hi_b < size_b, (kind, BM, M, N, K, tA, tB, pad)
            checked += 1
    assert checked > 500


def test_last_row_rule_is_needed():
    # without stopping the slices before row K-1, a straddling chunk in the last
    # row reads past a minimal operand
    hits = 0
    for (kind, BM, BN, BK), (M, N, K) in itertools.product(CONFIGS, shapes()[:10]):
        lda, ldb = M, N            # A stored K x M, B stored K x N, no padding
        hi_a, hi_b = max_slice_index(kind, M, N, K, lda, ldb, 1, 0, BM, BN, BK, stop_before_last_row=False)
        size_a, size_b = minimal_sizes(M, N, K, lda, ldb, 1, 0)
        hits += hi_a >= size_a or hi_b >= size_b
    assert hits > 0
