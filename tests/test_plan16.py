"""Host check of the 16-bit-input GEMM planner (csrc/plan16.h): which kernel,
tile and K split each shape gets, for the shapes the GPU tests rely on to reach
each path, and the structural rules (K split only with scratch, on grids that
leave most CUs idle and have a long K; orientations each tile can take)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR_DIR = os.path.join(ROOT, "dense_gemm_optimisation_f32_amd", "csrc")

PROG = r"""
#include <cstdio>
#include <cstdlib>
#include "plan16.h"
using namespace mi355gemm;
int main(int argc, char **argv) {
    // argv: M N K batch transA transB lda ldb strideA strideB addrA addrB scratch
    Problem16 q;
    q.M = atoi(argv[1]); q.N = atoi(argv[2]); q.K = atoi(argv[3]); q.batch = atoi(argv[4]);
    q.transA = atoi(argv[5]); q.transB = atoi(argv[6]);
    q.lda = atoll(argv[7]); q.ldb = atoll(argv[8]); q.strideA = atoll(argv[9]); q.strideB = atoll(argv[10]);
    q.A = (uintptr_t)atoll(argv[11]); q.B = (uintptr_t)atoll(argv[12]);
    const Plan16 p = plan16(q, atoi(argv[13]) != 0);
    static const char *names[] = {"dma256", "dma128", "dma64x128", "reg128", "reg64"};
    std::printf("%s %d\n", names[(int)p.kernel], p.nsplit);
    return 0;
}
"""


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    d = tmp_path_factory.mktemp("plan16")
    src = d / "p.cpp"
    src.write_text(PROG)
    exe = d / "p"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", HDR_DIR, str(src), "-o", str(exe)], check=True)

    def plan(M, N, K, batch=1, tA=0, tB=0, lda=None, ldb=None, sA=None, sB=None, a=1 << 20, b=1 << 21,
             scratch=True):
        lda = lda if lda is not None else (M if tA else K)
        ldb = ldb if ldb is not None else (K if tB else N)
        sA = sA if sA is not None else (M * K if batch > 1 else 0)
        sB = sB if sB is not None else (K * N if batch > 1 else 0)
        args = [M, N, K, batch, tA, tB, lda, ldb, sA, sB, a, b, int(scratch)]
        out = subprocess.run([str(exe), *map(str, args)], capture_output=True, text=True, check=True).stdout.split()
        return out[0], int(out[1])
    return plan


@pytest.mark.parametrize("shape,want", [
    # the step's HGEMM and the batched configuration: 256x256 tiles, one round
    ((4096, 4096, 4096), ("dma256", 1)),
    ((1024, 1024, 1024, 16), ("dma256", 1)),
    # the 256x256 tiles of the beta epilogue tests: two or three slices, batched
    ((4096, 4096, 128), ("dma256", 1)),
    ((4096, 4096, 192, 1, 1, 1), ("dma256", 1)),
    ((1024, 1024, 320, 12), ("dma256", 1)),
    # HGEMM 2048^3: 256 tiles of 128^2 fill the CUs; no split
    ((2048, 2048, 2048), ("dma128", 1)),
    # one GPU's row share under an 8-way split: 64x128 tiles
    ((512, 4096, 4096), ("dma64x128", 1)),
    # ... which take A stored M x K only: A stored K x M keeps 128x128 tiles
    ((512, 4096, 4096, 1, 1, 0), ("dma128", 1)),
    ((1000, 1000, 2000), ("dma64x128", 1)),
    ((1000, 1000, 2000, 1, 1, 0), ("dma128", 1)),
    # long K on few tiles: K split of the 128x128 tile
    ((512, 512, 8192), ("dma128", 8)),
    ((1024, 1024, 8192), ("dma128", 2)),
    ((768, 768, 4096), ("dma128", 3)),
    ((256, 256, 8192), ("dma128", 8)),
    ((4096, 256, 8192), ("dma128", 2)),
    ((1000, 1000, 5000), ("dma128", 2)),            # 78 slices: ragged tiles and a K tail
    ((300, 200, 6000), ("dma128", 5)),              # 93 slices over 5 splits (18 or 19 each)
    ((500, 1002, 8192), ("dma128", 4)),             # N % 8 != 0, B stored K x N: 127 slices
    ((256, 384, 4096, 3), ("dma128", 4)),           # batched: 18 tiles
    ((512, 768, 5000, 1, 1, 1), ("dma128", 4)),     # both operands stored transposed
    # short K or a full grid: no split
    ((1024, 1024, 2048), ("dma64x128", 1)),
    ((512, 512, 2048), ("dma64x128", 1)),
    ((512, 512, 4096, 8), ("dma64x128", 1)),
    ((1536, 1536, 4096), ("dma128", 1)),
])
def test_plans(planner, shape, want):
    M, N, K, *rest = shape
    batch = rest[0] if rest else 1
    tA = rest[1] if len(rest) > 1 else 0
    tB = rest[2] if len(rest) > 2 else 0
    assert planner(M, N, K, batch, tA, tB) == want


def test_no_split_without_scratch(planner):
    assert planner(512, 512, 8192, scratch=False) == ("dma64x128", 1)
    assert planner(512, 512, 8192, tA=1, scratch=False) == ("dma128", 1)


def test_register_kernel_for_rows_not_dword_aligned(planner):
    # odd fp16 leading dimension: rows only 2-byte aligned
    assert planner(1024, 1024, 8192, lda=8193)[0] in ("reg64", "reg128")
    assert planner(2048, 2048, 2048, ldb=2049) == ("reg128", 1)
    # base 2 bytes past a dword
    assert planner(512, 512, 8192, a=(1 << 20) + 2) == ("reg64", 1)


def test_short_k_below_the_ring(planner):
    # K = 128 is two slices: enough for the 256x256 ring only, which needs a full grid
    assert planner(4096, 4096, 128) == ("dma256", 1)
    assert planner(1024, 1024, 128) == ("reg64", 1)


def test_split_counts_stay_in_range(planner):
    for M, N, K in ((128, 128, 65536), (64, 64, 4096), (130, 70, 100000), (1024, 1024, 65536)):
        kern, s = planner(M, N, K)
        assert kern == "dma128" and 2 <= s <= 8, (M, N, K, s)
        slices = K // 64
        assert slices // s >= 16
