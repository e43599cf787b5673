// plan16.h -- which kernel, tile and K split a 16-bit-input GEMM runs.
//
// Host-only and free of HIP types, so that the choice can be checked on a
// machine without a GPU.  The tile shapes here are those of the kernels in
// hgemm_mfma.hip (which asserts that they agree).
#pragma once

#include <stdint.h>

namespace mi355gemm {

// A direct-to-LDS tile: BM x BN outputs, BK-k slices in a ring of `stages`.
struct TileShape16 {
    int bm, bn, bk, stages;
};
constexpr TileShape16 kDma256{256, 256, 64, 2};
constexpr TileShape16 kDma128{128, 128, 64, 4};
constexpr TileShape16 kDma64x128{64, 128, 64, 4};

// The operands as the planner sees them (element strides, byte addresses).
struct Problem16 {
    int M, N, K, batch;
    int transA, transB;   // A stored K x M, B stored N x K
    long long lda, ldb, strideA, strideB;
    uintptr_t A, B;
};

enum class Kernel16 { Dma256, Dma128, Dma64x128, Reg128, Reg64 };

struct Plan16 {
    Kernel16 kernel;
    int nsplit;   // workgroups sharing each tile's K range (Dma128 only); 1 = no split
};

// An MN-contiguous operand (A stored K x M, B stored K x N) whose M or N is not
// a multiple of eight has a 16-byte chunk that straddles that edge; the kernel
// then leaves the operand's last row of k to the tail it reads from global
// memory.  Whole BK-k slices the direct-to-LDS kernel runs.
inline int dma_slices(const Problem16 &q, const TileShape16 &t)
{
    const bool straddle = (q.transA && q.M % 8 != 0) || (!q.transB && q.N % 8 != 0);
    return (q.K - (straddle ? 1 : 0)) / t.bk;
}

// The direct-to-LDS kernel with tile t applies: 4-byte aligned operand rows
// (16-byte chunks start a multiple of eight halves into a row, so they stay
// dword aligned, which is all the 16-byte loads need), at least `stages` whole
// slices, an MN-contiguous operand at least eight wide where a chunk straddles
// its edge (its overflow then stays in the next row), 32-bit per-lane offsets
// within a slice, and MN-contiguous slices of at least 16 chunks (BM >= 128 for
// A stored K x M, BN >= 128 for B stored K x N).
inline bool dma_fits(const Problem16 &q, const TileShape16 &t)
{
    const bool aligned = q.lda % 2 == 0 && q.ldb % 2 == 0 && q.strideA % 2 == 0 && q.strideB % 2 == 0 &&
                         q.A % 4 == 0 && q.B % 4 == 0;
    const bool shape = dma_slices(q, t) >= t.stages && (!q.transA || q.M % 8 == 0 || q.M >= 8) &&
                       (q.transB || q.N % 8 == 0 || q.N >= 8);
    const long long rows_a = q.transA ? t.bk : t.bm, rows_b = q.transB ? t.bn : t.bk;
    const bool fits = rows_a * q.lda * 2 < (1LL << 31) && rows_b * q.ldb * 2 < (1LL << 31);
    const bool orient = (!q.transA || t.bm >= 128) && (q.transB || t.bn >= 128);
    return aligned && shape && fits && orient;
}

inline long long tile_count(const Problem16 &q, const TileShape16 &t)
{
    return (long long)((q.M + t.bm - 1) / t.bm) * ((q.N + t.bn - 1) / t.bn) * q.batch;
}

// K split of the 128x128 tile for grids that leave most CUs idle and have a
// long K: when the tiles fill at most a quarter of the 256 CUs and K holds at
// least 64 slices, split each tile's K range over s workgroups so that the
// tiles times s fill about half the CUs (s <= 8, each split at least 16
// slices).  The last workgroup of a tile to finish adds the s partial tiles
// (s * 64 KB of reads), which is why fewer, longer splits win over filling
// every CU.  Measured, one MI355X (us, split against the best unsplit tile):
// 512^2 x 8192 19.8 vs 37.1, 1024^2 x 8192 29.3 vs 38.1, 256^2 x 8192 16.6
// vs 30.5, 768^2 x 4096 17.6 vs 19.8, 4096 x 256 x 8192 29.4 vs 34.5.
inline int split_count(const Problem16 &q)
{
    const long long tiles = tile_count(q, kDma128);
    const int slices = dma_slices(q, kDma128);
    if (tiles > 64 || slices < 64) return 1;
    int s = (int)(128 / tiles);
    if (s > 8) s = 8;
    while (s > 1 && slices / s < 16) --s;
    return s;
}

// scratch: memory for a K split's partial tiles can be had for this call.
inline Plan16 plan16(const Problem16 &q, bool scratch)
{
    const bool ok256 = dma_fits(q, kDma256), ok128 = dma_fits(q, kDma128);
    const long long t256 = tile_count(q, kDma256), t128 = tile_count(q, kDma128);
    if (ok128 && scratch) {
        const int s = split_count(q);
        if (s > 1) return {Kernel16::Dma128, s};
    }
    // 64x128 tiles on grids of 128x128 tiles that fill at most a quarter of the
    // CUs, or at most half with K >= 4096 (measured: 512x4096x4096 29.8 -> 26.0
    // us, 1000x1000x2000 16.5 -> 12.9 us; 1024x2048x2048, half filled with
    // K = 2048, 17.0 -> 17.8 us, so it keeps 128x128 tiles)
    if (ok128 && (4 * t128 <= 256 || (2 * t128 <= 256 && q.K >= 4096)) && dma_fits(q, kDma64x128))
        return {Kernel16::Dma64x128, 1};
    // Both direct-to-LDS tiles run one workgroup per CU, so a grid runs in
    // rounds of 256 workgroups.  A 128x128 tile does a quarter of a 256x256
    // tile's work at about 0.6 of its rate (measured), i.e. takes 0.4 of its
    // time: the 256x256 tile wins when 5 * its rounds <= 2 * the 128x128 rounds.
    if (ok256 && ok128) {
        const long long r256 = (t256 + 255) / 256, r128 = (t128 + 255) / 256;
        return {5 * r256 <= 2 * r128 ? Kernel16::Dma256 : Kernel16::Dma128, 1};
    }
    if (ok256 && t256 >= 256) return {Kernel16::Dma256, 1};
    if (ok128) return {Kernel16::Dma128, 1};
    // register-staged kernel: 64x64 tiles when 128x128 ones would not fill the CUs
    return {t128 < 256 ? Kernel16::Reg64 : Kernel16::Reg128, 1};
}

}  // namespace mi355gemm
