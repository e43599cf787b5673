"""Host check of the workgroup-to-tile mapping (csrc/tile_order.h): for every grid
shape up to 40 x 40 tiles, the map from workgroup id to (tile row, tile column)
is a bijection onto the tile grid, and with whole groups the tiles one XCD runs
form compact blocks of C."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR_DIR = os.path.join(ROOT, "dense_gemm_optimisation_f32_amd", "csrc")

PROG = r"""
#include <cstdio>
#include <vector>
#include "tile_order.h"
int main() {
    for (int tm_n = 1; tm_n <= 40; ++tm_n)
        for (int tn_n = 1; tn_n <= 40; ++tn_n) {
            std::vector<int> seen(tm_n * tn_n, 0);
            for (int w = 0; w < tm_n * tn_n; ++w) {
                int tm, tn;
                mi355gemm::tile_coords(w, tm_n, tn_n, &tm, &tn);
                if (tm < 0 || tm >= tm_n || tn < 0 || tn >= tn_n) { std::printf("range %d %d %d\n", tm_n, tn_n, w); return 1; }
                if (seen[tm * tn_n + tn]++) { std::printf("dup %d %d %d\n", tm_n, tn_n, w); return 1; }
            }
        }
    // 16 x 16 tiles (HGEMM 4096^2 with 256^2 tiles): XCD x runs ids x, x+8, ...; they must
    // cover exactly 4 tile rows and 8 tile columns.
    for (int x = 0; x < 8; ++x) {
        int rows[16] = {0}, cols[16] = {0}, nr = 0, nc = 0;
        for (int w = x; w < 256; w += 8) {
            int tm, tn;
            mi355gemm::tile_coords(w, 16, 16, &tm, &tn);
            if (!rows[tm]++) ++nr;
            if (!cols[tn]++) ++nc;
        }
        if (nr != 4 || nc != 8) { std::printf("xcd %d spans %d rows %d cols\n", x, nr, nc); return 1; }
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
