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

// wg: blockIdx.x within one batch member's work items; z: blockIdx.z (the
// batch member index within the launch), nbatch: gridDim.z.  A work item is one
// tile, or with a K split over nsplit workgroups, one split of one tile
// (gridDim.x = tiles_m*tiles_n*nsplit).  The dispatcher numbers workgroups
// x-fastest, so the linear id is z*items + wg; the XCD-contiguous remap runs
// over all nbatch*items workgroups of the launch, which gives each XCD whole
// batch members when items*nbatch is a multiple of 8 and items is small (their
// A and B then pass through one L2), keeps the splits of one tile next to each
// other (so they run on one XCD when the count per XCD allows), and reduces to
// the single-problem order when nbatch == nsplit == 1.  Outputs: the batch
// member, the tile of it and the split.  A bijection onto [0, nbatch) x
// [0, tiles_m) x [0, tiles_n) x [0, nsplit).
__host__ __device__ inline void tile_coords_split(int wg, int z, int nbatch, int tiles_m, int tiles_n, int nsplit,
                                                  int *member, int *tm, int *tn, int *split)
{
    const long long tiles = (long long)tiles_m * tiles_n;
    const long long items = tiles * nsplit;
    const long long total = items * nbatch;
    const long long lin = (long long)z * items + wg;
    // XCD-contiguous logical index
    const long long xcd = lin % kNumXcd, slot = lin / kNumXcd;
    const long long per = total / kNumXcd, extra = total % kNumXcd;
    const long long logical = xcd * per + (xcd < extra ? xcd : extra) + slot;
    *member = (int)(logical / items);
    const long long rest = logical - (long long)(*member) * items;
    *split = (int)(rest % nsplit);
    const int t = (int)(rest / nsplit);
    // grouped order: GROUP_M tile rows at a time, column-major inside a group
    const int per_group = kGroupM * tiles_n;
    const int group = t / per_group;
    const int first_m = group * kGroupM;
    const int rows = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
    const int in_group = t - group * per_group;
    *tm = first_m + in_group % rows;
    *tn = in_group / rows;
}

// The same map without a K split (gridDim.x = tiles_m*tiles_n).
__host__ __device__ inline void tile_coords(int wg, int z, int nbatch, int tiles_m, int tiles_n, int *member,
                                            int *tm, int *tn)
{
    int split;
    tile_coords_split(wg, z, nbatch, tiles_m, tiles_n, 1, member, tm, tn, &split);
}

}  // namespace mi355gemm
