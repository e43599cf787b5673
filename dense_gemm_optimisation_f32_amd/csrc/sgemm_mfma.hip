// sgemm_mfma.hip -- fp32 row-major GEMM on the CDNA4 fp32 matrix cores.
//
// Structure (the hierarchy of the ssxxe.cn V100 SGEMM article, section 3 and
// its kernels of sections 2.1-2.3, and the MindNotes 'GEMM' page's
// register-tiling sections, rebuilt for gfx950):
//   * each workgroup owns one BM x BN tile of C and walks K in BK-wide steps;
//   * each step's A (BM x BK) and B (BK x BN) tiles are read from HBM with
//     coalesced 128-bit loads into registers, then written to LDS; LDS is
//     double-buffered, so the loads of step t+1 are in flight while step t is
//     computed and one barrier per step suffices (the article's section 2.3
//     double buffering);
//   * A is stored transposed in LDS, [k][m] (the pages store A as [BK][BM] so
//     that one k gives consecutive m); B keeps its [k][n] layout;
//   * the 2D register tile of outer products is executed by the matrix core:
//     v_mfma_f32_32x32x2_f32 adds, for a 32x32 block of C held in 16 fp32
//     registers per lane, the outer products of a 32-row column pair of A and a
//     32-column row pair of B.  The four waves of a workgroup form a 2 x 2 grid
//     of 64 x 64 wave tiles (2 x 2 MFMA blocks each).
//   * the epilogue applies C = alpha*acc + beta*C (C not read when beta == 0)
//     with per-element masks, so any M, N, K and leading dimension work;
//     out-of-range A/B elements are loaded as zero.
// Why MFMA and not VALU: fp32 VALU FMA without the packed form reaches half of
// the chip's fp32 rate; the fp32 MFMA path has the full rate.
// Two instantiations per tile shape: MASK = false for problems made of whole
// tiles with 16-byte aligned rows (no bounds checks anywhere), MASK = true for
// everything else.  Workgroups are mapped to tiles XCD by XCD (tile_order.h).
#include "gemm_internal.h"
#include "tile_order.h"

namespace mi355gemm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct SgemmArgs {
    int M, N, K;
    float alpha, beta;
    const float *A;
    long long lda, sA;
    const float *B;
    long long ldb, sB;
    float *C;
    long long ldc, sC;
    int tiles_m, tiles_n;
};

// Tile configuration.  WM x WN waves, each owning a (BM/WM) x (BN/WN) tile made
// of 32 x 32 MFMA blocks.
template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct SgCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;      // wave tile
    static constexpr int FM = TM / 32, FN = TN / 32;      // MFMA blocks per wave
    static constexpr int LDA_S = BM + 2;                  // A^T row pitch in LDS (floats)
    static constexpr int LDB_S = BN + 4;                  // B row pitch in LDS (floats, 16 B multiple)
    static constexpr int A_CPR = BK / 4;                  // float4 chunks per A row
    static constexpr int B_CPR = BN / 4;                  // float4 chunks per B row
    static constexpr int A_LOADS = BM * BK / 4 / NT;
    static constexpr int B_LOADS = BK * BN / 4 / NT;
    static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be whole MFMA blocks");
    static_assert((BM * BK / 4) % NT == 0 && (BK * BN / 4) % NT == 0, "tile loads must split evenly");
    static_assert(BK % 2 == 0, "MFMA consumes k in pairs");
};

template <class Cfg, bool MASK, bool VEC>
__global__ __launch_bounds__(Cfg::NT) void sgemm_mfma_kernel(SgemmArgs p)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr int LDA_S = Cfg::LDA_S, LDB_S = Cfg::LDB_S;
    __shared__ float lds_a[2 * BK * LDA_S];
    __shared__ float lds_b[2 * BK * LDB_S];

    const int tid = threadIdx.x;
    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, &tm, &tn);
    const long long m0 = (long long)tm * BM, n0 = (long long)tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const float *A = p.A + (long long)blockIdx.z * p.sA;
    const float *B = p.B + (long long)blockIdx.z * p.sB;
    float *C = p.C + (long long)blockIdx.z * p.sC;
    const long long lda = p.lda, ldb = p.ldb, ldc = p.ldc;

    float4 ra[Cfg::A_LOADS], rb[Cfg::B_LOADS];

    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < Cfg::A_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int row = id / Cfg::A_CPR, kc = (id % Cfg::A_CPR) * 4;
            const long long gm = m0 + row;
            const int gk = k0 + kc;
            const float *src = A + gm * lda + gk;
            if (!MASK || (VEC && gm < M && gk + 3 < K)) {
                ra[i] = *reinterpret_cast<const float4 *>(src);
            } else {
                const bool rok = gm < M;
                ra[i].x = (rok && gk + 0 < K) ? src[0] : 0.f;
                ra[i].y = (rok && gk + 1 < K) ? src[1] : 0.f;
                ra[i].z = (rok && gk + 2 < K) ? src[2] : 0.f;
                ra[i].w = (rok && gk + 3 < K) ? src[3] : 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int krow = id / Cfg::B_CPR, nc = (id % Cfg::B_CPR) * 4;
            const int gk = k0 + krow;
            const long long gn = n0 + nc;
            const float *src = B + (long long)gk * ldb + gn;
            if (!MASK || (VEC && gk < K && gn + 3 < N)) {
                rb[i] = *reinterpret_cast<const float4 *>(src);
            } else {
                const bool kok = gk < K;
                rb[i].x = (kok && gn + 0 < N) ? src[0] : 0.f;
                rb[i].y = (kok && gn + 1 < N) ? src[1] : 0.f;
                rb[i].z = (kok && gn + 2 < N) ? src[2] : 0.f;
                rb[i].w = (kok && gn + 3 < N) ? src[3] : 0.f;
            }
        }
    };

    auto store_tiles = [&](int buf) {
        float *as = lds_a + buf * (BK * LDA_S);
        float *bs = lds_b + buf * (BK * LDB_S);
#pragma unroll
        for (int i = 0; i < Cfg::A_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int row = id / Cfg::A_CPR, kc = (id % Cfg::A_CPR) * 4;
            as[(kc + 0) * LDA_S + row] = ra[i].x;
            as[(kc + 1) * LDA_S + row] = ra[i].y;
            as[(kc + 2) * LDA_S + row] = ra[i].z;
            as[(kc + 3) * LDA_S + row] = ra[i].w;
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int krow = id / Cfg::B_CPR, nc = (id % Cfg::B_CPR) * 4;
            *reinterpret_cast<float4 *>(&bs[krow * LDB_S + nc]) = rb[i];
        }
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int lr = lane & 31, lk = lane >> 5;

    f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (K + BK - 1) / BK;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const int buf = t & 1;
        if (t + 1 < nk) load_tiles((t + 1) * BK);
        const float *as = lds_a + buf * (BK * LDA_S) + wm * Cfg::TM + lr;
        const float *bs = lds_b + buf * (BK * LDB_S) + wn * Cfg::TN + lr;
#pragma unroll
        for (int s = 0; s < BK / 2; ++s) {
            const int k = 2 * s + lk;
            float a[Cfg::FM], b[Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) a[i] = as[k * LDA_S + 32 * i];
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) b[j] = bs[k * LDB_S + 32 * j];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (t + 1 < nk) store_tiles(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  In a 32x32 MFMA block, register r of lane l holds row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32.
    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) {
            const long long col = n0 + wn * Cfg::TN + 32 * j + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const long long row = m0 + wm * Cfg::TM + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
                if (!MASK || (row < M && col < N)) {
                    float *dst = C + row * ldc + col;
                    float v = alpha * acc[i][j][r];
                    if (beta != 0.f) v += beta * *dst;
                    *dst = v;
                }
            }
        }
    }
}

using SgBig = SgCfg<128, 128, 16, 2, 2>;

template <class Cfg>
hipError_t launch_cfg(const GemmProblem &q, hipStream_t stream)
{
    SgemmArgs a;
    a.M = q.M; a.N = q.N; a.K = q.K;
    a.alpha = q.alpha; a.beta = q.beta;
    a.A = static_cast<const float *>(q.A); a.lda = q.lda; a.sA = q.strideA;
    a.B = static_cast<const float *>(q.B); a.ldb = q.ldb; a.sB = q.strideB;
    a.C = q.C; a.ldc = q.ldc; a.sC = q.strideC;
    a.tiles_m = (q.M + Cfg::BM - 1) / Cfg::BM;
    a.tiles_n = (q.N + Cfg::BN - 1) / Cfg::BN;
    const bool vec = (q.lda % 4 == 0) && (q.ldb % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(q.A) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(q.B) % 16 == 0) &&
                     (q.strideA % 4 == 0) && (q.strideB % 4 == 0);
    const bool whole = vec && q.M % Cfg::BM == 0 && q.N % Cfg::BN == 0 && q.K % Cfg::BK == 0;
    dim3 grid(a.tiles_m * a.tiles_n, 1, q.batch);
    dim3 block(Cfg::NT);
    if (whole)
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, false, true>), grid, block, 0, stream, a);
    else if (vec)
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, true, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, true, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sgemm(const GemmProblem &q, hipStream_t stream)
{
    return launch_cfg<SgBig>(q, stream);
}

}  // namespace mi355gemm
