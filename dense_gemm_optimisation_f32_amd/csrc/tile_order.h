// tile_order.h -- workgroup-to-tile mapping for the GEMM kernels.
//
// The MindNotes 'GEMM' page (section "thread-block grid swizzling") remaps the
// block index so that blocks running at the same time cover a compact 2D
// neighbourhood of C and share their A rows and B columns in L2.  On MI355X
// the dispatcher deals workgroups out round-robin over 8 XCDs, each with its
// own L2, so the remap here first gathers the workgroups of one XCD
// (linear ids x, x+8, x+16, ...) into one contiguous run of "logical" tile
// numbers, then walks the tiles in groups of GROUP_M tile rows, column by
// column inside a group, so that a run of consecutive logical numbers is a
// GROUP_M-tall block of C.  The mapping is a bijection on [0, tiles_m*tiles_n).
#pragma once

namespace mi355gemm {

constexpr int kNumXcd = 8;
constexpr int kGroupM = 4;

__host__ __device__ inline void tile_coords(int wg, int tiles_m, int tiles_n, int *tm, int *tn)
{
    const int total = tiles_m * tiles_n;
    // XCD-contiguous logical index
    const int xcd = wg % kNumXcd, slot = wg / kNumXcd;
    const int per = total / kNumXcd, extra = total % kNumXcd;
    const int logical = xcd * per + (xcd < extra ? xcd : extra) + slot;
    // grouped order: GROUP_M tile rows at a time, column-major inside a group
    const int per_group = kGroupM * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * kGroupM;
    const int rows = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
    const int in_group = logical - group * per_group;
    *tm = first_m + in_group % rows;
    *tn = in_group / rows;
}

}  // namespace mi355gemm
