// hgemm_mfma.hip -- fp16-input, fp32-accumulate row-major GEMM (single and
// strided-batched) on the CDNA4 fp16 matrix cores.
//
// The tiling follows the wave-level hierarchy of the dandandamowang.xyz
// 'GEMM optimisation (2): Tensor Core wmma API' page (sections 4-7: one warp
// owning a grid of MMA tiles, double-buffered shared-memory staging, padding
// against bank conflicts, and the larger 128x128 block tile), rebuilt for
// gfx950 rather than translated:
//   * matrix-core op: v_mfma_f32_32x32x16_f16 (a 32x32 fp32 block, 16 k per op,
//     8 fp16 values of A and of B per lane);
//   * a workgroup of 4 waves in a 2x2 grid; each wave owns a (BM/2) x (BN/2)
//     tile of (BM/64) x (BN/64) MFMA blocks whose accumulators stay in
//     registers for the whole K loop;
//   * A is staged in LDS as [m][k] (K contiguous, 128-byte rows of eight
//     16-byte chunks whose chunk index is XOR-swizzled with bits of the row --
//     the MindNotes page's swizzling idea applied to 16-byte chunks), so an A
//     operand is one 16-byte LDS read per lane;
//   * B is staged in LDS in its own row-major [k][n] layout (rows padded so the
//     four rows a transposed read touches fall in different banks -- the
//     dandandamowang page's padding).  The K-packed B operand is assembled by
//     two ds_read_b64_tr_b16 transposed LDS reads: within each 16-lane group,
//     lane i receives element i%4 of the four-element vectors addressed by
//     lanes i/4, i/4+4, i/4+8 and i/4+12, so lanes pointing at four
//     consecutive n of rows k..k+3 hand each lane one column's four k values;
//   * LDS is double-buffered with one barrier per K step; the next step's
//     global loads are issued before the current step's MFMAs and written to
//     the other buffer after them;
//   * workgroups are mapped to tiles so that the tiles one XCD (one L2) runs
//     form a compact block of C;
//   * epilogue C = alpha*acc + beta*C (C not read when beta == 0).
// Two instantiations per tile shape: MASK = false for problems made of whole
// tiles with 16-byte aligned rows (no bounds checks anywhere), MASK = true for
// everything else (out-of-range elements load as zero, stores are masked).
#include "gemm_internal.h"
#include "tile_order.h"

namespace mi355gemm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;

struct HgemmArgs {
    int M, N, K;
    float alpha, beta;
    const uint16_t *A;
    long long lda, sA;
    const uint16_t *B;
    long long ldb, sB;
    float *C;
    long long ldc, sC;
    int tiles_m, tiles_n;
};

template <int BM_, int BN_>
struct HgCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64, WM = 2, WN = 2, NT = 256;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int CPR = BK / 8;                 // 16-byte chunks per A row
    static constexpr int LDB = BN + 32;                // B row pitch in halves (64-byte pad)
    static constexpr int A_HALVES = BM * BK;
    static constexpr int B_HALVES = BK * LDB;
    static constexpr int BUF_HALVES = A_HALVES + B_HALVES;
    static constexpr int A_LOADS = BM * CPR / NT;      // 16-byte A chunks per thread
    static constexpr int B_LOADS = BK * (BN / 8) / NT; // 16-byte B chunks per thread
    static_assert(BM * CPR % NT == 0 && BK * (BN / 8) % NT == 0, "tile loads must split evenly");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole MFMA blocks");
};

__device__ __forceinline__ int swz(int row, int chunk)
{
    return chunk ^ ((row ^ (row >> 3)) & 7);
}

// Eight fp16 values at p[0..7]; elements at or beyond `valid` read as zero.
__device__ __forceinline__ u32x4 load8_masked(const uint16_t *p, int valid)
{
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (e < valid) ? p[e] : (uint16_t)0;
    u32x4 v;
    v.x = h[0] | ((unsigned)h[1] << 16);
    v.y = h[2] | ((unsigned)h[3] << 16);
    v.z = h[4] | ((unsigned)h[5] << 16);
    v.w = h[6] | ((unsigned)h[7] << 16);
    return v;
}

template <class Cfg, bool MASK, bool VEC>
__global__ __launch_bounds__(256) void hgemm_mfma_kernel(HgemmArgs p)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, CPR = Cfg::CPR, LDB = Cfg::LDB;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Cfg::BUF_HALVES];

    const int tid = threadIdx.x;
    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, &tm, &tn);
    const long long m0 = (long long)tm * BM, n0 = (long long)tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const uint16_t *A = p.A + (long long)blockIdx.z * p.sA;
    const uint16_t *B = p.B + (long long)blockIdx.z * p.sB;
    float *C = p.C + (long long)blockIdx.z * p.sC;
    const long long lda = p.lda, ldb = p.ldb, ldc = p.ldc;

    u32x4 ra[Cfg::A_LOADS], rb[Cfg::B_LOADS];

    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < Cfg::A_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int row = id / CPR, kc = (id % CPR) * 8;
            const long long gm = m0 + row;
            const int gk = k0 + kc;
            const uint16_t *src = A + gm * lda + gk;
            if (!MASK) {
                ra[i] = *reinterpret_cast<const u32x4 *>(src);
            } else if (gm >= M || gk >= K) {
                ra[i] = u32x4{0u, 0u, 0u, 0u};
            } else if (VEC && gk + 8 <= K) {
                ra[i] = *reinterpret_cast<const u32x4 *>(src);
            } else {
                ra[i] = load8_masked(src, K - gk);
            }
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int kr = id / (BN / 8), nc = (id % (BN / 8)) * 8;
            const int gk = k0 + kr;
            const long long gn = n0 + nc;
            const uint16_t *src = B + (long long)gk * ldb + gn;
            if (!MASK) {
                rb[i] = *reinterpret_cast<const u32x4 *>(src);
            } else if (gk >= K || gn >= N) {
                rb[i] = u32x4{0u, 0u, 0u, 0u};
            } else if (VEC && gn + 8 <= N) {
                rb[i] = *reinterpret_cast<const u32x4 *>(src);
            } else {
                rb[i] = load8_masked(src, (int)(N - gn));
            }
        }
    };

    auto store_tiles = [&](int buf) {
        uint16_t *la = lds + buf * Cfg::BUF_HALVES;
        uint16_t *lb = la + Cfg::A_HALVES;
#pragma unroll
        for (int i = 0; i < Cfg::A_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int row = id / CPR, c = id % CPR;
            *reinterpret_cast<u32x4 *>(la + row * BK + 8 * swz(row, c)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int kr = id / (BN / 8), nc = (id % (BN / 8)) * 8;
            *reinterpret_cast<u32x4 *>(lb + kr * LDB + nc) = rb[i];
        }
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int lr = lane & 31, lk = lane >> 5;
    // transposed-read lane roles: group q of 16 lanes, lane j within it
    const int q = lane >> 4, j = lane & 15;
    const int tr_row = 8 * (q >> 1) + (j >> 2);                         // + 16*s + 4*h
    const int tr_col = wn * Cfg::TN + 16 * (q & 1) + 4 * (j & 3);        // + 32*bn

    f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < Cfg::FN; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;

    const int nk = (K + BK - 1) / BK;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const int buf = t & 1;
        if (t + 1 < nk) load_tiles((t + 1) * BK);
        const uint16_t *la = lds + buf * Cfg::BUF_HALVES;
        const uint16_t *lb = la + Cfg::A_HALVES;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int c = 2 * s + lk;   // A chunk: halves 16s + 8*lk .. +7
            half8 a[Cfg::FM], b[Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) {
                const int row = wm * Cfg::TM + 32 * i + lr;
                a[i] = *reinterpret_cast<const half8 *>(la + row * BK + 8 * swz(row, c));
            }
#pragma unroll
            for (int jj = 0; jj < Cfg::FN; ++jj) {
                const uint16_t *base = lb + (16 * s + tr_row) * LDB + tr_col + 32 * jj;
                const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(base));
                const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(base + 4 * LDB));
                const short4v both[2] = {lo, hi};
                b[jj] = __builtin_bit_cast(half8, both);
            }
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int jj = 0; jj < Cfg::FN; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[jj], acc[i][jj], 0, 0, 0);
        }
        if (t + 1 < nk) store_tiles(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: register r of lane l in a 32x32 block is row 8*(r/4)+4*(l/32)+r%4,
    // column l%32.
    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
#pragma unroll
        for (int jj = 0; jj < Cfg::FN; ++jj) {
            const long long col = n0 + wn * Cfg::TN + 32 * jj + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const long long row = m0 + wm * Cfg::TM + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
                if (!MASK || (row < M && col < N)) {
                    float *dst = C + row * ldc + col;
                    float v = alpha * acc[i][jj][r];
                    if (beta != 0.f) v += beta * *dst;
                    *dst = v;
                }
            }
        }
    }
}

using Hg256 = HgCfg<256, 256>;
using Hg128 = HgCfg<128, 128>;

template <class Cfg>
hipError_t launch_cfg(const GemmProblem &q, hipStream_t stream)
{
    HgemmArgs a;
    a.M = q.M; a.N = q.N; a.K = q.K;
    a.alpha = q.alpha; a.beta = q.beta;
    a.A = static_cast<const uint16_t *>(q.A); a.lda = q.lda; a.sA = q.strideA;
    a.B = static_cast<const uint16_t *>(q.B); a.ldb = q.ldb; a.sB = q.strideB;
    a.C = q.C; a.ldc = q.ldc; a.sC = q.strideC;
    a.tiles_m = (q.M + Cfg::BM - 1) / Cfg::BM;
    a.tiles_n = (q.N + Cfg::BN - 1) / Cfg::BN;
    const bool vec = (q.lda % 8 == 0) && (q.ldb % 8 == 0) &&
                     (reinterpret_cast<uintptr_t>(q.A) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(q.B) % 16 == 0) &&
                     (q.strideA % 8 == 0) && (q.strideB % 8 == 0);
    const bool whole = vec && q.M % Cfg::BM == 0 && q.N % Cfg::BN == 0 && q.K % Cfg::BK == 0;
    dim3 grid(a.tiles_m * a.tiles_n, 1, q.batch);
    dim3 block(Cfg::NT);
    if (whole)
        hipLaunchKernelGGL((hgemm_mfma_kernel<Cfg, false, true>), grid, block, 0, stream, a);
    else if (vec)
        hipLaunchKernelGGL((hgemm_mfma_kernel<Cfg, true, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((hgemm_mfma_kernel<Cfg, true, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_hgemm(const GemmProblem &q, hipStream_t stream)
{
    // 256x256 tiles when they give at least one tile per CU, else 128x128.
    const long long t256 = (long long)((q.M + 255) / 256) * ((q.N + 255) / 256) * q.batch;
    if (t256 >= 256) return launch_cfg<Hg256>(q, stream);
    return launch_cfg<Hg128>(q, stream);
}

}  // namespace mi355gemm
