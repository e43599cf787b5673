// hgemm_mfma.hip -- fp16-input, fp32-accumulate row-major GEMM (single and
// strided-batched) on the CDNA4 fp16 matrix cores.
//
// The tiling follows the wave-level hierarchy of the dandandamowang.xyz
// 'GEMM optimisation (2): Tensor Core wmma API' page (sections 4-7: one warp
// owning a grid of MMA tiles, double-buffered shared-memory staging, padding
// against bank conflicts, and the larger 128x128 block tile), rebuilt for
// gfx950 rather than translated:
//   * matrix-core op: v_mfma_f32_32x32x16_f16 (32x32 fp32 block, 16 k per op,
//     8 fp16 values of A and of B per lane);
//   * workgroup of 4 waves in a 2x2 grid; each wave owns a (BM/2) x (BN/2) tile
//     = (BM/64) x (BN/64) MFMA blocks whose accumulators stay in registers for
//     the whole K loop;
//   * both operands sit in LDS "K-contiguous": A as [m][k], B transposed as
//     [n][k], so every MFMA operand is one 16-byte LDS read per lane.  B arrives
//     row-major ([k][n]); each thread loads an 8(k) x 8(n) block with eight
//     16-byte loads and transposes it in registers before the LDS write;
//   * LDS rows are 128 bytes (BK = 64 halves = eight 16-byte chunks); the chunk
//     index is XOR-swizzled with bits of the row index (the MindNotes page's
//     swizzling idea applied to 16-byte chunks) so that the eight rows a
//     group of lanes reads or writes land in distinct banks;
//   * LDS is double-buffered with one barrier per K step; the next step's
//     global loads are issued before the current step's MFMAs;
//   * epilogue C = alpha*acc + beta*C with per-element masks; out-of-range A/B
//     elements are loaded as zero, so any M, N, K and leading dimension work.
#include "gemm_internal.h"

namespace mi355gemm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
    static constexpr int CPR = BK / 8;                         // 16-byte chunks per LDS row
    static constexpr int A_CHUNKS = BM * CPR;                  // chunks in an A tile
    static constexpr int A_LOADS = A_CHUNKS / NT;
    static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);       // 8x8 blocks in a B tile
    static constexpr int B_LOADS = (B_BLOCKS + NT - 1) / NT;
    static constexpr int LDS_CHUNKS = (BM + BN) * CPR;         // per buffer
    static_assert(A_CHUNKS % NT == 0, "A tile loads must split evenly");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole MFMA blocks");
};

// Chunk swizzle: rows r..r+7 (aligned to 8) get distinct chunks for a fixed
// logical chunk, and so do rows 8 apart.
__device__ __forceinline__ int swz(int row, int chunk)
{
    return chunk ^ ((row ^ (row >> 3)) & 7);
}

__device__ __forceinline__ u32x4 load16(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// Eight fp16 values at p[0..7] (elements at or beyond `valid` read as zero).
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

template <class Cfg, bool VEC>
__global__ __launch_bounds__(256) void hgemm_mfma_kernel(HgemmArgs p)
{
    constexpr int BM = Cfg::BM, BK = Cfg::BK, CPR = Cfg::CPR;
    __shared__ u32x4 lds[2 * Cfg::LDS_CHUNKS];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x;
    const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
    const long long m0 = (long long)tm * BM, n0 = (long long)tn * Cfg::BN;
    const int M = p.M, N = p.N, K = p.K;
    const uint16_t *A = p.A + (long long)blockIdx.z * p.sA;
    const uint16_t *B = p.B + (long long)blockIdx.z * p.sB;
    float *C = p.C + (long long)blockIdx.z * p.sC;
    const long long lda = p.lda, ldb = p.ldb, ldc = p.ldc;

    u32x4 ra[Cfg::A_LOADS];
    u32x4 rb[Cfg::B_LOADS][8];

    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < Cfg::A_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int row = id / CPR, kc = (id % CPR) * 8;
            const long long gm = m0 + row;
            const int gk = k0 + kc;
            const uint16_t *src = A + gm * lda + gk;
            if (gm >= M || gk >= K)
                ra[i] = u32x4{0u, 0u, 0u, 0u};
            else if (VEC && gk + 8 <= K)
                ra[i] = load16(src);
            else
                ra[i] = load8_masked(src, K - gk);
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int kb = id / (Cfg::BN / 8), nb = id % (Cfg::BN / 8);
            const long long gn = n0 + nb * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int gk = k0 + kb * 8 + e;
                const uint16_t *src = B + (long long)gk * ldb + gn;
                if (id >= Cfg::B_BLOCKS || gk >= K || gn >= N)
                    rb[i][e] = u32x4{0u, 0u, 0u, 0u};
                else if (VEC && gn + 8 <= N)
                    rb[i][e] = load16(src);
                else
                    rb[i][e] = load8_masked(src, (int)(N - gn));
            }
        }
    };

    auto store_tiles = [&](int buf) {
        u32x4 *la = lds + buf * Cfg::LDS_CHUNKS;
        u32x4 *lb = la + BM * CPR;
#pragma unroll
        for (int i = 0; i < Cfg::A_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int row = id / CPR, c = id % CPR;
            la[row * CPR + swz(row, c)] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            if (id >= Cfg::B_BLOCKS) continue;
            const int kb = id / (Cfg::BN / 8), nb = id % (Cfg::BN / 8);
            // rb[i][e] holds B[kb*8+e][nb*8 .. nb*8+7] as 4 dwords of 2 halves.
            // Column n = nb*8 + j becomes one chunk: halves k = kb*8 .. kb*8+7.
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                u32x4 w;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const unsigned lo = rb[i][2 * d][j >> 1];
                    const unsigned hi = rb[i][2 * d + 1][j >> 1];
                    w[d] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
                }
                const int n = nb * 8 + j;
                lb[n * CPR + swz(n, kb)] = w;
            }
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
        const u32x4 *la = lds + buf * Cfg::LDS_CHUNKS;
        const u32x4 *lb = la + BM * CPR;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int c = 2 * s + lk;   // logical chunk: halves 16s + 8*lk .. +7
            half8 a[Cfg::FM], b[Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) {
                const int row = wm * Cfg::TM + 32 * i + lr;
                a[i] = __builtin_bit_cast(half8, la[row * CPR + swz(row, c)]);
            }
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) {
                const int n = wn * Cfg::TN + 32 * j + lr;
                b[j] = __builtin_bit_cast(half8, lb[n * CPR + swz(n, c)]);
            }
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
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
        for (int j = 0; j < Cfg::FN; ++j) {
            const long long col = n0 + wn * Cfg::TN + 32 * j + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const long long row = m0 + wm * Cfg::TM + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
                if (row < M && col < N) {
                    float *dst = C + row * ldc + col;
                    float v = alpha * acc[i][j][r];
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
    dim3 grid(a.tiles_m * a.tiles_n, 1, q.batch);
    dim3 block(Cfg::NT);
    if (vec)
        hipLaunchKernelGGL((hgemm_mfma_kernel<Cfg, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((hgemm_mfma_kernel<Cfg, false>), grid, block, 0, stream, a);
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
