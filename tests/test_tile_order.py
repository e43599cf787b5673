"""Host check of the workgroup-to-tile mapping (csrc/tile_order.h): for every grid
shape up to 24 x 24 tiles and up to 5 batch members, the map from (workgroup,
member) ids to (member, tile row, tile column) is a bijection, with whole groups
the tiles one XCD runs form compact blocks of C, and a batch of small problems
gives each XCD whole members."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR_DIR = os.path.join(ROOT, "dense_gemm_optimisation_f32_amd", "csrc")

PROG = r"""
#include <cstdio>
#include <vector>
#include "tile_order.h"
int main() {
    // bijection onto (member, tile row, tile column) for grids up to 24 x 24 tiles and 1..5 members
    for (int nb = 1; nb <= 5; ++nb)
        for (int tm_n = 1; tm_n <= 24; ++tm_n)
            for (int tn_n = 1; tn_n <= 24; ++tn_n) {
                std::vector<int> seen(nb * tm_n * tn_n, 0);
                for (int z = 0; z < nb; ++z)
                    for (int w = 0; w < tm_n * tn_n; ++w) {
                        int mb, tm, tn;
                        mi355gemm::tile_coords(w, z, nb, tm_n, tn_n, &mb, &tm, &tn);
                        if (mb < 0 || mb >= nb || tm < 0 || tm >= tm_n || tn < 0 || tn >= tn_n) {
                            std::printf("range %d %d %d %d %d\n", nb, tm_n, tn_n, z, w); return 1; }
                        if (seen[(mb * tm_n + tm) * tn_n + tn]++) {
                            std::printf("dup %d %d %d %d %d\n", nb, tm_n, tn_n, z, w); return 1; }
                    }
            }
    // one member, 16 x 16 tiles (HGEMM 4096^2 with 256^2 tiles): XCD x runs linear ids x, x+8,
    // ...; they must cover exactly 4 tile rows and 8 tile columns.
    for (int x = 0; x < 8; ++x) {
        int rows[16] = {0}, cols[16] = {0}, nr = 0, nc = 0;
        for (int w = x; w < 256; w += 8) {
            int mb, tm, tn;
            mi355gemm::tile_coords(w, 0, 1, 16, 16, &mb, &tm, &tn);
            if (!rows[tm]++) ++nr;
            if (!cols[tn]++) ++nc;
        }
        if (nr != 4 || nc != 8) { std::printf("xcd %d spans %d rows %d cols\n", x, nr, nc); return 1; }
    }
    // 16 members of 4 x 4 tiles (batched 1024^2 with 256^2 tiles): each XCD runs two whole members
    for (int x = 0; x < 8; ++x) {
        int count[16] = {0}, members = 0;
        for (int lin = x; lin < 256; lin += 8) {
            int mb, tm, tn;
            mi355gemm::tile_coords(lin % 16, lin / 16, 16, 4, 4, &mb, &tm, &tn);
            if (!count[mb]++) ++members;
        }
        for (int m = 0; m < 16; ++m)
            if (count[m] != 0 && count[m] != 16) { std::printf("xcd %d has part of member %d\n", x, m); return 1; }
        if (members != 2) { std::printf("xcd %d runs %d members\n", x, members); return 1; }
    }
    // with a K split: a bijection onto (member, tile, split), and the splits of
    // one tile land on one XCD when the split count divides the items per XCD
    for (int ns = 1; ns <= 4; ++ns)
        for (int nb = 1; nb <= 3; ++nb)
            for (int tm_n = 1; tm_n <= 12; ++tm_n)
                for (int tn_n = 1; tn_n <= 12; ++tn_n) {
                    const int items = tm_n * tn_n * ns;
                    std::vector<int> seen(nb * items, 0), xcd_of(nb * tm_n * tn_n, -1);
                    bool same_xcd = true;
                    for (int z = 0; z < nb; ++z)
                        for (int w = 0; w < items; ++w) {
                            int mb, tm, tn, sp;
                            mi355gemm::tile_coords_split(w, z, nb, tm_n, tn_n, ns, &mb, &tm, &tn, &sp);
                            if (mb < 0 || mb >= nb || tm < 0 || tm >= tm_n || tn < 0 || tn >= tn_n || sp < 0 ||
                                sp >= ns) { std::printf("split range\n"); return 1; }
                            const int tile = (mb * tm_n + tm) * tn_n + tn;
                            if (seen[tile * ns + sp]++) { std::printf("split dup\n"); return 1; }
                            const int x = (z * items + w) % 8;
                            if (xcd_of[tile] < 0) xcd_of[tile] = x;
                            else if (xcd_of[tile] != x) same_xcd = false;
                        }
                    if ((nb * items) % (8 * ns) == 0 && !same_xcd) {
                        std::printf("splits of a tile on two XCDs %d %d %d %d\n", ns, nb, tm_n, tn_n); return 1; }
                }
    std::printf("ok\n");
    return 0;
}
"""


def test_tile_order_is_a_bijection(tmp_path):
    src = tmp_path / "t.cpp"
    src.write_text(PROG)
    exe = tmp_path / "t"
    subprocess.run(["g++", "-std=c++17", "-O1", "-D__host__=", "-D__device__=", "-I", HDR_DIR,
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
