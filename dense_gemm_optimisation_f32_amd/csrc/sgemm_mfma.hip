// sgemm_mfma.hip -- fp32 row-major GEMM on the CDNA4 fp32 matrix cores.
//
// The 2D register tile of outer products (the MindNotes 'GEMM' page's
// register-tiling sections; the tile hierarchy of section 3 of the ssxxe.cn
// V100 SGEMM article) is executed by the matrix core: v_mfma_f32_32x32x2_f32
// adds, for a 32x32 block of C held in 16 fp32 registers per lane, the outer
// products of a 32-row column pair of A and a 32-column row pair of B.  Why
// MFMA and not VALU: fp32 VALU FMA without the packed form reaches half of the
// chip's fp32 rate; the fp32 MFMA path has the full rate.
//
// Three kernels; launch_sgemm picks one per problem:
//   * sgemm_dma_kernel -- the main kernel (any leading dimension).  Each
//     K slice of A and B goes from global memory straight into a ring of two
//     or four LDS slots (direct-to-LDS loads: the gfx950 form of the article's
//     section 2.3 double buffering, with no register staging), in 256x256, 128x128 or
//     64x64 tiles; the 64x64 tiles and whole 128x128 tiles split each slice's
//     eight-k steps over K groups of waves and sum their partial tiles in a
//     fixed order.  Ragged M, N and K are handled by clamped slice loads, a K
//     tail read from global memory and masked stores;
//   * sgemm_mfma_kernel -- problems the direct-to-LDS kernel cannot take (K
//     below the ring's slices, or an MN-contiguous operand whose M or N is
//     below eight and not a multiple of four) when there are enough tiles:
//     128x128 tiles read with 16-byte loads into registers and written to a
//     double-buffered LDS (one barrier per step), zero outside the matrix;
//   * sgemm_small_kernel -- grids of fewer than 256 tiles of 128x128 whose
//     64x64 tiles would fill fewer than five eighths of the CUs: the waves of a
//     workgroup split K, and their partial tiles are summed in a fixed order.
// Every kernel applies C = alpha*acc + beta*C (C not read when beta == 0),
// masked where the tile crosses the edge of C, and maps workgroups to tiles XCD
// by XCD (tile_order.h).  Global accesses are 16 bytes wide at any leading
// dimension: multi-dword global loads and stores need only dword alignment on
// CDNA.
//
// Transposed operands (C = alpha*op(A)op(B) + beta*C, the MindNotes 'GEMM'
// page, section "core problem and arithmetic characteristics"): every kernel
// is instantiated for the four storage combinations.  An operand is either
// K-contiguous (A stored M x K, or B stored N x K) or MN-contiguous (A stored
// K x M, or B stored K x N); each kernel reads a tile from global memory in its
// stored orientation, with 16-byte loads along the contiguous dimension, and
// only the LDS placement and the operand reads depend on the orientation.  The
// order in which k terms meet each MFMA is the same for all four.
#include "gemm_internal.h"
#include "tile_order.h"
#include "epilogue.h"

#include <type_traits>

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
    static constexpr int A_LOADS = BM * BK / 4 / NT;
    static constexpr int B_LOADS = BK * BN / 4 / NT;
    static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be whole MFMA blocks");
    static_assert((BM * BK / 4) % NT == 0 && (BK * BN / 4) % NT == 0, "tile loads must split evenly");
    static_assert(BK % 2 == 0, "MFMA consumes k in pairs");
};

// Four consecutive floats (r, c..c+3) of a row-major rows x cols matrix X with
// leading dimension ld, as one 16-byte load (dword alignment suffices for it);
// with MASK, elements outside the matrix read as zero.
template <bool MASK>
__device__ __forceinline__ f32x4_t load4(const float *X, long long ld, long long r, long long c, long long rows,
                                         long long cols)
{
    const float *src = X + r * ld + c;
    if (!MASK || (r < rows && c + 3 < cols)) return *reinterpret_cast<const f32x4_g *>(src);
    const bool rok = r < rows;
    f32x4_t v;
    v.x = (rok && c + 0 < cols) ? src[0] : 0.f;
    v.y = (rok && c + 1 < cols) ? src[1] : 0.f;
    v.z = (rok && c + 2 < cols) ? src[2] : 0.f;
    v.w = (rok && c + 3 < cols) ? src[3] : 0.f;
    return v;
}

// ---------------------------------------------------------------------------
// Register-staged kernel (operands the direct-to-LDS kernel cannot take).
// MASK = false for problems made of whole tiles (no bounds checks anywhere),
// MASK = true for everything else.  TA: A stored K x M; TB: B stored N x K.
// In LDS both operands are kept MN-contiguous ([k][m] and [k][n], the pages'
// [BK][BM] layout of A); a K-contiguous operand is transposed on its way in by
// four scalar LDS writes, an MN-contiguous one is written as 16-byte rows.
template <class Cfg, bool MASK, bool TA, bool TB>
__global__ __launch_bounds__(Cfg::NT) void sgemm_mfma_kernel(SgemmArgs p)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    // LDS row pitches (floats): a multiple of four where rows are written as
    // float4, 2 mod 4 where they are written by transposing scatter (spreads
    // the four scattered k rows over the banks).
    constexpr int LDA_S = TA ? BM + 4 : BM + 2;
    constexpr int LDB_S = TB ? BN + 2 : BN + 4;
    // float4 chunks per row of each tile as stored in global memory
    constexpr int A_CPR = (TA ? BM : BK) / 4;
    constexpr int B_CPR = (TB ? BK : BN) / 4;
    __shared__ __attribute__((aligned(16))) float lds_a[2 * BK * LDA_S];
    __shared__ __attribute__((aligned(16))) float lds_b[2 * BK * LDB_S];

    const int tid = threadIdx.x;
    int mb, tm, tn;   // batch member, tile row, tile column
    tile_coords(blockIdx.x, blockIdx.z, gridDim.z, p.tiles_m, p.tiles_n, &mb, &tm, &tn);
    const long long m0 = (long long)tm * BM, n0 = (long long)tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const float *A = p.A + (long long)mb * p.sA;
    const float *B = p.B + (long long)mb * p.sB;
    float *C = p.C + (long long)mb * p.sC;
    const long long lda = p.lda, ldb = p.ldb, ldc = p.ldc;

    f32x4_t ra[Cfg::A_LOADS], rb[Cfg::B_LOADS];

    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < Cfg::A_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int r = id / A_CPR, c = (id % A_CPR) * 4;
            ra[i] = TA ? load4<MASK>(A, lda, k0 + r, m0 + c, K, M) : load4<MASK>(A, lda, m0 + r, k0 + c, M, K);
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int r = id / B_CPR, c = (id % B_CPR) * 4;
            rb[i] = TB ? load4<MASK>(B, ldb, n0 + r, k0 + c, N, K) : load4<MASK>(B, ldb, k0 + r, n0 + c, K, N);
        }
    };

    auto store_tiles = [&](int buf) {
        float *as = lds_a + buf * (BK * LDA_S);
        float *bs = lds_b + buf * (BK * LDB_S);
#pragma unroll
        for (int i = 0; i < Cfg::A_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int r = id / A_CPR, c = (id % A_CPR) * 4;
            if (TA) {   // r = k, c = m
                *reinterpret_cast<f32x4_t *>(&as[r * LDA_S + c]) = ra[i];
            } else {    // r = m, c = k
                as[(c + 0) * LDA_S + r] = ra[i].x;
                as[(c + 1) * LDA_S + r] = ra[i].y;
                as[(c + 2) * LDA_S + r] = ra[i].z;
                as[(c + 3) * LDA_S + r] = ra[i].w;
            }
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_LOADS; ++i) {
            const int id = i * Cfg::NT + tid;
            const int r = id / B_CPR, c = (id % B_CPR) * 4;
            if (TB) {   // r = n, c = k
                bs[(c + 0) * LDB_S + r] = rb[i].x;
                bs[(c + 1) * LDB_S + r] = rb[i].y;
                bs[(c + 2) * LDB_S + r] = rb[i].z;
                bs[(c + 3) * LDB_S + r] = rb[i].w;
            } else {    // r = k, c = n
                *reinterpret_cast<f32x4_t *>(&bs[r * LDB_S + c]) = rb[i];
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
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(b[j], a[i], acc[i][j], 0, 0, 0);
        }
        if (t + 1 < nk) store_tiles(buf ^ 1);
        __syncthreads();
    }

    // Epilogue (operands were swapped, so each lane holds four consecutive
    // columns of one row per register quad; see epilogue.h).
    const float alpha = p.alpha, beta = p.beta;
    auto epilogue = [&](auto with_c) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) {
            const long long row = m0 + wm * Cfg::TM + 32 * i + lr;
#pragma unroll
            for (int jj = 0; jj < Cfg::FN; ++jj) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const long long col = n0 + wn * Cfg::TN + 32 * jj + 8 * g + 4 * lk;
                    const f32x4_t v = {acc[i][jj][4 * g], acc[i][jj][4 * g + 1], acc[i][jj][4 * g + 2],
                                       acc[i][jj][4 * g + 3]};
                    store_row4<MASK, decltype(with_c)::value>(C, ldc, row, col, v, alpha, beta, M, N);
                }
            }
        }
    };
    if (beta != 0.f)
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

// ---------------------------------------------------------------------------
// Kernel fed by direct-to-LDS loads (global_load_lds_dwordx4: lane l's 16
// bytes land at M0 + 16*l, no register staging, no LDS-write instructions).
// Two LDS slots of BK = 32 k; slice t+2 is fetched while slice t+1 waits and
// slice t is computed, which at fp32-MFMA speed (64 cycles per 32x32x2 op)
// leaves a whole slice of compute to hide the fetch.
//
// Each operand slice is kept in LDS in its stored orientation:
//   * K-contiguous (A stored M x K, B stored N x K): R rows (R = BM or BN) of
//     128 bytes (eight 16-byte chunks of four k); the chunk at physical
//     position p of row r holds logical chunk p ^ ((r ^ r>>3) & 7), so the
//     sixteen rows one LDS cycle serves fall on distinct banks.  A lane reads
//     one whole chunk (four consecutive k of its row) per ds_read_b128: lanes
//     0-31 the chunk 2u, lanes 32-63 the chunk 2u+1.  Element e of that read
//     feeds the e-th MFMA of quad u;
//   * MN-contiguous (A stored K x M, B stored K x N): 32 rows of R floats; the
//     chunk at physical position p of row k holds logical chunk
//     p ^ (8 * ((k >> 2) & 1)), which puts rows k and k+4 (read by the two
//     half-waves of one MFMA operand) on different banks.  The operand of
//     MFMA (u, e) is row 8u+e+4*(lane/32), at the lane's column; where a wave
//     has two or four blocks of that operand their columns interleave, so one
//     8- or 16-byte read serves them all (see the kernel).
// Either way lane l of MFMA (u, e) holds k = 8u + 4*(l/32) + e, so the op's k
// pair is {8u+e, 8u+4+e} -- one fixed reordering of the sum over k for all
// four storage combinations.
// KS > 1: KS groups of WM x WN waves split each slice's eight-k steps (group
// ks takes steps ks, ks + KS, ...) and their partial tiles are summed at the end.
// SLOTS: LDS ring depth (2 or 4 slices in flight).
template <int BM_, int BN_, int WM_, int WN_, int KS_ = 1, int SLOTS_ = 2>
struct SgDmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 32, WM = WM_, WN = WN_, KS = KS_, SLOTS = SLOTS_;
    static_assert(SLOTS == 2 || SLOTS == 4, "ring of two or four slices");
    static constexpr int NW = WM * WN * KS, NT = 64 * NW;
    // Waves per SIMD the register budget must allow: the 64x64 tile's grids can
    // hold two work-groups per CU, which its masked instantiations would
    // otherwise exceed (142 VGPRs against 126 with the bound, no spills)
    static constexpr int WPE = BM * BN <= 64 * 64 ? 4 : 1;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int A_BYTES = BM * BK * 4;
    static constexpr int B_BYTES = BK * BN * 4;
    static constexpr int SLOT_BYTES = A_BYTES + B_BYTES;
    // The upper half of the waves (one per SIMD with eight waves) issues every
    // slice load, so the other waves are never blocked issuing them.
    static constexpr int LW = NW / 2;                        // loading waves
    static constexpr int A_LOADS = A_BYTES / 1024 / LW;      // per loading wave per slice
    static constexpr int B_LOADS = B_BYTES / 1024 / LW;
    static_assert(A_BYTES % (1024 * LW) == 0 && B_BYTES % (1024 * LW) == 0, "slices must split over the loaders");
    static_assert(BM >= 64 && BN >= 64, "MN-contiguous slices need at least 16 chunks per row");
    static_assert(SLOTS * SLOT_BYTES <= 160 * 1024, "LDS slots too large");
    static_assert((BK / 8) % KS == 0 && (KS & (KS - 1)) == 0, "K groups must split the slice's steps");
    // the partial tiles of groups 1 .. KS-1 pass through the LDS of the ring
    static constexpr int PART_BYTES = (KS - 1) * WM * WN * FM * FN * 16 * 64 * 4;
    static constexpr int LDS_BYTES = SLOTS * SLOT_BYTES > PART_BYTES ? SLOTS * SLOT_BYTES : PART_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "partial tiles exceed the LDS");
};

__device__ __forceinline__ int sg_swz_a(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int sg_swz_b(int k) { return 8 * ((k >> 2) & 1); }

// One direct-to-LDS load (16 bytes per lane, the wave's 1 KB contiguous at LDS
// byte lds_addr).  M0 (the LDS destination) is set inside the statement; the
// compiler does not track that clobber, which is safe because these kernels
// give M0 no other use.
__device__ __forceinline__ void sg_dma16(const void *sbase, unsigned voff, unsigned lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory", "m0");
}

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) f32x4v lds_f32x4;
typedef __attribute__((address_space(3))) f32x2v lds_f32x2;
typedef __attribute__((address_space(3))) float lds_f32;

// Byte offset (within one slice of global memory) of the 16-byte chunk that
// lane `lane` of wave load g fetches for an operand slice of R rows or
// columns (see the layouts above), split into a uniform row part, added to the
// base pointer, and a per-lane part.  The per-lane part depends on g only
// through the chunk swizzle: g % 8 for a K-contiguous operand (rows 8g ..
// 8g+7), bit 2 of RPL*g for an MN-contiguous one (rows RPL*g .. RPL*g + RPL-1
// share one swizzle since RPL divides four).
//
// MASK: `lim` is how many of the R rows (K-contiguous) or columns
// (MN-contiguous) lie inside M or N, and a chunk past it re-reads a valid one
// (row lim-1, or chunk 0 of its row), whose products only reach C entries that
// are never stored.  A masked K-contiguous load whose rows reach lim takes its
// whole clamped offset from sg_kc_clamped instead.
template <bool KC, int R>
__device__ __forceinline__ long long sg_row_part(int g, long long ld)
{
    return KC ? 32LL * g * ld : (long long)(256 / R) * g * ld * 4;
}

template <bool KC, int R, bool MASK>
__device__ __forceinline__ unsigned sg_lane_part(int g, int lane, long long ld, int lim)
{
    if (KC) {
        const int l3 = lane >> 3, ch = (lane & 7) ^ l3 ^ (g & 7);   // (r ^ r>>3) & 7 for r = 8g + l3
        return (unsigned)(l3 * ld + 4 * ch) * 4u;
    }
    constexpr int CPR = R / 4, RPL = 256 / R;   // chunks per row, rows per wave load
    int ch = (lane % CPR) ^ sg_swz_b(RPL * g);
    if (MASK && 4 * ch >= lim) ch = 0;
    return (unsigned)((lane / CPR) * ld + 4 * ch) * 4u;
}

// Whole offset of K-contiguous load g with its rows clamped to `lim`: rows
// past it re-read row lim-1.  The lane id is read afresh so that it need not
// stay live across the K loop.
__device__ __forceinline__ unsigned sg_kc_clamped(int g, long long ld, int lim)
{
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int l3 = lane >> 3, r = 8 * g + l3, ch = (lane & 7) ^ l3 ^ (g & 7);
    return (unsigned)((r >= lim ? lim - 1 : r) * ld + 4 * ch) * 4u;
}

// How many distinct per-lane parts the loads g = lw + LW*i (i < LOADS) of one
// loading wave have: the swizzle's period in g (8, or 8/RPL) divided by its gcd
// with LW is the period in i.
template <bool KC, int R, int LOADS, int LW>
constexpr int sg_lane_parts()
{
    const int per_g = KC ? 8 : 8 / (256 / R);
    int a = per_g, b = LW;
    while (b) {
        const int t = a % b;
        a = b;
        b = t;
    }
    return per_g / a < LOADS ? per_g / a : LOADS;
}

// TA: A stored K x M; TB: B stored N x K.  MASK: M and N need not be
// multiples of the tile, nor K of BK (the loads clamp to valid rows and
// columns, the K % BK tail is read straight from global memory after the last
// slice, and stores outside C are skipped); a 16-byte chunk of an
// MN-contiguous operand may straddle M or N (see the slice count below).
template <class Cfg, bool TA, bool TB, bool MASK>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::WPE))) void sgemm_dma_kernel(SgemmArgs p)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr bool A_KC = !TA, B_KC = TB;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[Cfg::LDS_BYTES];
    const unsigned lds0 = (unsigned)(uintptr_t)lds;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    int mb, tm, tn;   // batch member, tile row, tile column
    tile_coords(blockIdx.x, blockIdx.z, gridDim.z, p.tiles_m, p.tiles_n, &mb, &tm, &tn);
    const long long m0 = (long long)tm * BM, n0 = (long long)tn * BN;
    const long long lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    // first element of the tile's slice 0 in each operand
    const char *Ab = reinterpret_cast<const char *>(p.A + (long long)mb * p.sA + (A_KC ? m0 * lda : m0));
    const char *Bb = reinterpret_cast<const char *>(p.B + (long long)mb * p.sB + (B_KC ? n0 * ldb : n0));
    float *C = p.C + (long long)mb * p.sC;
    // bytes between consecutive slices
    const long long stepA = A_KC ? BK * 4 : BK * lda * 4;
    const long long stepB = B_KC ? BK * 4 : BK * ldb * 4;

    const bool loader = uwave >= Cfg::NW - Cfg::LW;
    const int lw = loader ? uwave - (Cfg::NW - Cfg::LW) : 0;   // loader index
    // rows / columns of the tile inside M and N
    const int limA = MASK ? (int)(p.M - m0 < BM ? p.M - m0 : BM) : BM;
    const int limB = MASK ? (int)(p.N - n0 < BN ? p.N - n0 : BN) : BN;
    // Loading wave lw issues loads g = lw + LW*i, so the loaders fetch
    // neighbouring rows, and load g lands at byte 1024*g of the operand's part
    // of the slot.  Load i uses per-lane part i % P.
    constexpr int LW = Cfg::LW;
    //
    // Masked K-contiguous loads clamp rows past the edge.  The 256x256 tile has
    // no registers to spare: it keeps the shared per-lane parts and computes a
    // clamped offset at issue for the loads whose rows reach the edge (tested
    // only in tiles that the edge crosses).  The smaller tiles keep one clamped
    // offset per load and no test in the loop.
    constexpr bool CLAMP_AT_ISSUE = BM * BN >= 256 * 256;
    constexpr bool PER_LOAD_A = MASK && A_KC && !CLAMP_AT_ISSUE, PER_LOAD_B = MASK && B_KC && !CLAMP_AT_ISSUE;
    constexpr int PA = PER_LOAD_A ? Cfg::A_LOADS : sg_lane_parts<A_KC, BM, Cfg::A_LOADS, LW>();
    constexpr int PB = PER_LOAD_B ? Cfg::B_LOADS : sg_lane_parts<B_KC, BN, Cfg::B_LOADS, LW>();
    unsigned offA[PA], offB[PB];
#pragma unroll
    for (int d = 0; d < PA; ++d)
        offA[d] = PER_LOAD_A ? sg_kc_clamped(lw + LW * d, lda, limA)
                             : sg_lane_part<A_KC, BM, MASK>(lw + LW * d, lane, lda, limA);
#pragma unroll
    for (int d = 0; d < PB; ++d)
        offB[d] = PER_LOAD_B ? sg_kc_clamped(lw + LW * d, ldb, limB)
                             : sg_lane_part<B_KC, BN, MASK>(lw + LW * d, lane, ldb, limB);
    // one operand's loads of a slice: base pointer, per-lane offsets, rows or
    // columns inside the tile, and the slot's LDS address for the operand
    auto issue_operand = [&](auto kc, auto rr, auto per_load, auto nloads, auto np, const char *x,
                             const unsigned *off, long long ld, int lim, unsigned dst) {
        constexpr bool KC = decltype(kc)::value;
        constexpr int R = decltype(rr)::value, NL = decltype(nloads)::value, NP = decltype(np)::value;
        if constexpr (decltype(per_load)::value) {
#pragma unroll
            for (int i = 0; i < NL; ++i) sg_dma16(x, off[i], dst + 1024 * (lw + LW * i));
        } else if (MASK && KC && lim < R) {   // an edge tile (wave-uniform): test each load
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int g = lw + LW * i;
                if (8 * g + 8 > lim)
                    sg_dma16(x, sg_kc_clamped(g, ld, lim), dst + 1024 * g);
                else
                    sg_dma16(x + sg_row_part<KC, R>(g, ld), off[i % NP], dst + 1024 * g);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int g = lw + LW * i;
                sg_dma16(x + sg_row_part<KC, R>(g, ld), off[i % NP], dst + 1024 * g);
            }
        }
    };
    auto issue_slice = [&](int kt, int slot) {
        if (!loader) return;
        const char *a = Ab + (long long)kt * stepA;
        const char *b = Bb + (long long)kt * stepB;
        const unsigned sa = lds0 + slot * Cfg::SLOT_BYTES, sb = sa + Cfg::A_BYTES;
        issue_operand(std::bool_constant<A_KC>{}, std::integral_constant<int, BM>{},
                      std::bool_constant<PER_LOAD_A>{}, std::integral_constant<int, Cfg::A_LOADS>{},
                      std::integral_constant<int, PA>{}, a, offA, lda, limA, sa);
        issue_operand(std::bool_constant<B_KC>{}, std::integral_constant<int, BN>{},
                      std::bool_constant<PER_LOAD_B>{}, std::integral_constant<int, Cfg::B_LOADS>{},
                      std::integral_constant<int, PB>{}, b, offB, ldb, limB, sb);
    };

    // Wave uwave owns part mn = uwave % (WM*WN) of the tile and, in K group
    // ks = uwave / (WM*WN), the eight-k steps ks, ks + KS, ... of every slice.
    constexpr int KS = Cfg::KS;
    const int mn = uwave % (Cfg::WM * Cfg::WN), ks = uwave / (Cfg::WM * Cfg::WN);
    const int wm = mn / Cfg::WN, wn = mn % Cfg::WN;
    const int lr = lane & 31, lk = lane >> 5;
    // Rows of the wave's A blocks.  With a K-contiguous A, block i holds rows
    // 32i .. 32i+31 of the wave tile.  With an MN-contiguous A, the rows of
    // IA consecutive blocks interleave (block i of a group holds rows IA*r + i),
    // so that one LDS read of IA consecutive m gives a lane its operand for
    // all IA blocks: four 16-byte reads per step instead of sixteen 4-byte ones.
    // The k order of every MFMA is unchanged.
    constexpr int IA = A_KC ? 1 : (Cfg::FM % 4 == 0 ? 4 : (Cfg::FM % 2 == 0 ? 2 : 1));
    auto arow = [&](int i, int l) { return wm * Cfg::TM + 32 * IA * (i / IA) + IA * l + (i % IA); };
    // Likewise the columns of an MN-contiguous B interleave over pairs of blocks
    // (block j of a pair holds columns 2c + j), read with one 8-byte read per k.
    // The accumulator of MFMA block (i, j) gives a lane four consecutive rows of
    // D = C^T, i.e. columns 2c + j for four consecutive c: across the pair the
    // lane then owns eight consecutive columns, stored as two 16-byte rows.
    constexpr int IB = (B_KC || Cfg::FN % 2 != 0) ? 1 : 2;
    auto bcol = [&](int j, int l) { return wn * Cfg::TN + 32 * IB * (j / IB) + IB * l + (j % IB); };
    // Operand read addresses (bytes within a slot).  K-contiguous: the row and
    // the lane part of its chunk index (logical chunk 2u+lk).  MN-contiguous:
    // row 4*lk (plus 8u+e), logical chunk m/4 of the lane's first m, physical
    // chunk flipped by 8 when lk = 1 (for A, one address per group of IA blocks).
    // The wave's first step ks is folded in: step u = ks + KS*j adds 2*ks to
    // the chunk index (no carry, as KS is a power of two) and 8*ks rows.
    unsigned rowA[Cfg::FM], tA[Cfg::FM], rowB[Cfg::FN], tB[Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
        const int r = arow(i, lr);
        if (A_KC) {
            rowA[i] = (unsigned)(r * BK * 4);
            tA[i] = (unsigned)(lk ^ sg_swz_a(r) ^ (2 * ks));
        } else {
            const int q = r >> 2;
            rowA[i] = (unsigned)((4 * lk + 8 * ks) * BM * 4 + 16 * (q ^ (8 * lk)) + 4 * (r & 3));
            tA[i] = 0;
        }
    }
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
        const int c = bcol(j, lr);
        if (B_KC) {
            rowB[j] = (unsigned)(Cfg::A_BYTES + c * BK * 4);
            tB[j] = (unsigned)(lk ^ sg_swz_a(c) ^ (2 * ks));
        } else {
            const int q = c >> 2;
            rowB[j] = (unsigned)(Cfg::A_BYTES + (4 * lk + 8 * ks) * BN * 4 + 16 * (q ^ (8 * lk)) + 4 * (c & 3));
            tB[j] = 0;
        }
    }

    f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Operand fragments of the wave's j-th eight-k step of a slice (step
    // u = ks + KS*j): element e of fa[i] / fb[j] is the operand of MFMA (u, e)
    // for block i / j.  A K-contiguous fragment is one
    // 16-byte read; an MN-contiguous B fragment is four 4-byte reads, and an
    // MN-contiguous A group of IA blocks four reads of IA floats.
    auto read_frags = [&](int slot, int jstep, f32x4v *fa, f32x4v *fb) {
        const int u = KS * jstep;   // the ks part is in rowA/tA, rowB/tB
        const unsigned base = lds0 + slot * Cfg::SLOT_BYTES;
        if constexpr (A_KC) {
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
                fa[i] = *(const lds_f32x4 *)(uintptr_t)(base + rowA[i] + 16 * (tA[i] ^ (2u * u)));
        } else {
#pragma unroll
            for (int g = 0; g < Cfg::FM; g += IA) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned at = base + rowA[g] + (8 * u + e) * BM * 4;
                    if constexpr (IA == 4) {
                        const f32x4v v = *(const lds_f32x4 *)(uintptr_t)at;
#pragma unroll
                        for (int x = 0; x < 4; ++x) fa[g + x][e] = v[x];
                    } else if constexpr (IA == 2) {
                        const f32x2v v = *(const lds_f32x2 *)(uintptr_t)at;
                        fa[g][e] = v[0];
                        fa[g + 1][e] = v[1];
                    } else {
                        fa[g][e] = *(const lds_f32 *)(uintptr_t)at;
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < Cfg::FN; j += IB) {
            if constexpr (B_KC) {
                fb[j] = *(const lds_f32x4 *)(uintptr_t)(base + rowB[j] + 16 * (tB[j] ^ (2u * u)));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned at = base + rowB[j] + (8 * u + e) * BN * 4;
                    if constexpr (IB == 2) {
                        const f32x2v v = *(const lds_f32x2 *)(uintptr_t)at;
                        fb[j][e] = v[0];
                        fb[j + 1][e] = v[1];
                    } else {
                        fb[j][e] = *(const lds_f32 *)(uintptr_t)at;
                    }
                }
            }
        }
    };
    auto mfmas = [&](const f32x4v *fa, const f32x4v *fb) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[j][e], fa[i][e], acc[i][j], 0, 0, 0);
    };
    // Issue the LDS reads of the next step one after each of this step's first
    // MFMAs, so they have the rest of the step to land.
    constexpr int READS = (A_KC ? Cfg::FM : Cfg::FM / IA * 4) + (B_KC ? Cfg::FN : Cfg::FN / IB * 4);
    constexpr int PAIRS = READS < 4 * Cfg::FM * Cfg::FN ? READS : 4 * Cfg::FM * Cfg::FN;
    auto interleave = [&]() {
#pragma unroll
        for (int r = 0; r < PAIRS; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
    };
    auto lds_barrier = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    constexpr int LOADS = Cfg::A_LOADS + Cfg::B_LOADS;
    static_assert(LOADS < 64, "vmcnt range");

    // Fragments are double-buffered in registers: step u+1's are read while
    // step u's MFMAs run.  Before the last step of slice t, once slice t+1 has
    // landed for every wave (own loads counted down to PENDING outstanding
    // slices, then the barrier) and every wave holds its slice-t fragments, the
    // slot of slice t is refilled with slice t+S and the first fragments of
    // slice t+1 are read.
    constexpr int S = Cfg::SLOTS;
    constexpr int NU = BK / 8, NUW = NU / KS;   // steps per slice, per wave
    // With an odd step count per slice the buffers alternate from slice to
    // slice: slice t starts in buffer (t * NUW) & 1, passed as PAR.
    f32x4v fa[2][Cfg::FM], fb[2][Cfg::FN];
    auto step = [&](int t, auto refill, auto pending, auto par) {
        constexpr int PAR = decltype(par)::value, PEND = LOADS * decltype(pending)::value;
        const int slot = t & (S - 1);
#pragma unroll
        for (int u = 0; u < NUW; ++u) {
            const int cur = (u + PAR) & 1, nxt = cur ^ 1;
            if (u + 1 < NUW) {
                read_frags(slot, u + 1, fa[nxt], fb[nxt]);
            } else {
                // vmcnt(PEND): slice t+1 done for this lane; lgkmcnt(0): this
                // wave's slice-t reads are done
                __builtin_amdgcn_s_waitcnt((PEND & 15) | ((PEND >> 4) << 14) | (7 << 4) | (15 << 8));
                __builtin_amdgcn_s_waitcnt(0xC07F);
                lds_barrier();
                if (decltype(refill)::value) issue_slice(t + S, slot);
                read_frags((t + 1) & (S - 1), 0, fa[nxt], fb[nxt]);
            }
            mfmas(fa[cur], fb[cur]);
            interleave();
        }
    };

    // An MN-contiguous operand whose M or N is not a multiple of four has a
    // chunk that straddles that edge.  Its floats past the edge only reach C
    // entries that are never stored, and in any row but the matrix's last they
    // lie in the next row.  The slices then stop before row K-1 and the K tail
    // below takes the rest, so no slice load reads past the operand.
    const bool straddle = MASK && ((!A_KC && p.M % 4 != 0) || (!B_KC && p.N % 4 != 0));
    const int nk = (p.K - (straddle ? 1 : 0)) / BK;   // whole slices, >= S (checked by the launcher)
    // the last slice: resident, nothing left to fetch
    auto last_slice = [&](auto par) {
        constexpr int PAR = decltype(par)::value;
        const int slot = (nk - 1) & (S - 1);
#pragma unroll
        for (int u = 0; u < NUW; ++u) {
            const int cur = (u + PAR) & 1, nxt = cur ^ 1;
            if (u + 1 < NUW) read_frags(slot, u + 1, fa[nxt], fb[nxt]);
            mfmas(fa[cur], fb[cur]);
        }
    };
    // Prologue: slices 0 .. S-1 in flight, slice 0 resident, its first
    // fragments read.
#pragma unroll
    for (int st = 0; st < S; ++st) issue_slice(st, st);
    constexpr int FIRST = LOADS * (S - 1);
    __builtin_amdgcn_s_waitcnt((FIRST & 15) | ((FIRST >> 4) << 14) | (7 << 4) | (15 << 8));   // slice 0 done
    lds_barrier();
    read_frags(0, 0, fa[0], fb[0]);
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using Steady = std::integral_constant<int, S - 2>;   // slices after t+1 in flight
    // The last S-1 steps issue nothing and drain the ring; p0 is the buffer
    // parity of slice nk-S.
    auto tail = [&](auto p0) {
        constexpr int A0 = decltype(p0)::value, A1 = A0 ^ (NUW & 1);
        const int t0 = nk - S;
        if constexpr (S == 4) {
            step(t0, std::false_type{}, std::integral_constant<int, 2>{}, std::integral_constant<int, A0>{});
            step(t0 + 1, std::false_type{}, std::integral_constant<int, 1>{}, std::integral_constant<int, A1>{});
            step(t0 + 2, std::false_type{}, std::integral_constant<int, 0>{}, std::integral_constant<int, A0>{});
            last_slice(std::integral_constant<int, A1>{});
        } else {
            step(t0, std::false_type{}, std::integral_constant<int, 0>{}, std::integral_constant<int, A0>{});
            last_slice(std::integral_constant<int, A1>{});
        }
    };
    if constexpr (NUW % 2 == 0) {
        for (int t = 0; t + S < nk; ++t) step(t, std::true_type{}, Steady{}, P0{});
        tail(P0{});
    } else {   // slices in pairs, so that each call knows its buffer
        int t = 0;
        for (; t + 1 + S < nk; t += 2) {
            step(t, std::true_type{}, Steady{}, P0{});
            step(t + 1, std::true_type{}, Steady{}, P1{});
        }
        if (t + S < nk) step(t, std::true_type{}, Steady{}, P0{});
        if ((nk - S) & 1)
            tail(P1{});
        else
            tail(P0{});
    }
    // The tail and the epilogue take the lane's row and k half from a lane id
    // read afresh, so that no address derived from it stays live (and spills)
    // across the K loop.
    const int elane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int elr = elane & 31, elk = elane >> 5;
    if constexpr (MASK) {
        // The K % BK tail, after the whole slices (k still ascends): each lane
        // loads its operand quads (four k) straight from global memory, zero
        // for k >= K, rows and columns clamped as for the slices.
        const int K = p.K, k0 = nk * BK;
        if (k0 < K) {
            const float *Am = p.A + (long long)mb * p.sA;
            const float *Bm = p.B + (long long)mb * p.sB;
            long long ar[Cfg::FM], bc[Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) {
                const long long r = m0 + arow(i, elr);
                ar[i] = r < p.M ? r : p.M - 1;
            }
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) {
                const long long c = n0 + bcol(j, elr);
                bc[j] = c < p.N ? c : p.N - 1;
            }
            // four k from kq of a row (stride 1) or a column (stride ld)
            auto quad = [&](const float *x, long long stride, int kq) {
                f32x4v v;
                if (stride == 1 && kq + 3 < K) {
                    const f32x4_g w = *reinterpret_cast<const f32x4_g *>(x);
                    v = f32x4v{w[0], w[1], w[2], w[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = kq + e < K ? x[e * stride] : 0.f;
                }
                return v;
            };
#pragma unroll
            for (int jstep = 0; jstep < NUW; ++jstep) {
                const int u = ks + KS * jstep;   // this wave's steps, as in the slices
                if (k0 + 8 * u >= K) break;
                const int kq = k0 + 8 * u + 4 * elk;   // this lane's quad
                f32x4v qa[Cfg::FM], qb[Cfg::FN];
#pragma unroll
                for (int i = 0; i < Cfg::FM; ++i)
                    qa[i] = A_KC ? quad(Am + ar[i] * lda + kq, 1, kq) : quad(Am + (long long)kq * lda + ar[i], lda, kq);
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    qb[j] = B_KC ? quad(Bm + bc[j] * ldb + kq, 1, kq) : quad(Bm + (long long)kq * ldb + bc[j], ldb, kq);
                mfmas(qa, qb);
            }
        }
    }

    if constexpr (KS > 1) {
        // Groups 1 .. KS-1 hand their partial tiles to group 0 through the LDS
        // of the ring, which no wave reads any more; group 0 adds them in group order
        // (a fixed order, so results are deterministic) and runs the epilogue.
        constexpr int PART = Cfg::WM * Cfg::WN * Cfg::FM * Cfg::FN * 16 * 64;   // floats per group
        lds_barrier();
        lds_f32 *part = (lds_f32 *)(uintptr_t)lds0;
        if (ks > 0) {
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        part[(ks - 1) * PART + (((mn * Cfg::FM + i) * Cfg::FN + j) * 16 + r) * 64 + elane] = acc[i][j][r];
        }
        lds_barrier();
        if (ks > 0) return;
#pragma unroll
        for (int g = 1; g < KS; ++g)
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[i][j][r] += part[(g - 1) * PART + (((mn * Cfg::FM + i) * Cfg::FN + j) * 16 + r) * 64 + elane];
    }

    const float alpha = p.alpha, beta = p.beta;
    auto epilogue = [&](auto with_c) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) {
            const long long row = m0 + arow(i, elr);
            if constexpr (IB == 1) {
#pragma unroll
                for (int jj = 0; jj < Cfg::FN; ++jj) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const long long col = n0 + wn * Cfg::TN + 32 * jj + 8 * g + 4 * elk;
                        const f32x4_t v = {acc[i][jj][4 * g], acc[i][jj][4 * g + 1], acc[i][jj][4 * g + 2],
                                           acc[i][jj][4 * g + 3]};
                        store_row4<MASK, decltype(with_c)::value>(C, ldc, row, col, v, alpha, beta, p.M, p.N);
                    }
                }
            } else {
                // blocks jj, jj+1: columns 2c + 0/1 for c = 8g + 4lk + e, i.e. eight
                // consecutive columns from 16g + 8lk
#pragma unroll
                for (int jj = 0; jj < Cfg::FN; jj += 2) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const long long col = n0 + wn * Cfg::TN + 32 * jj + 16 * g + 8 * elk;
                        const f32x16 &a0 = acc[i][jj], &a1 = acc[i][jj + 1];
                        const f32x4_t lo = {a0[4 * g], a1[4 * g], a0[4 * g + 1], a1[4 * g + 1]};
                        const f32x4_t hi = {a0[4 * g + 2], a1[4 * g + 2], a0[4 * g + 3], a1[4 * g + 3]};
                        store_row4<MASK, decltype(with_c)::value>(C, ldc, row, col, lo, alpha, beta, p.M, p.N);
                        store_row4<MASK, decltype(with_c)::value>(C, ldc, row, col + 4, hi, alpha, beta, p.M, p.N);
                    }
                }
            }
        }
    };
    if (beta != 0.f)
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

// Eight waves, two per SIMD (one wave's MFMAs cover the other's LDS and barrier
// latency): 256x256 tiles as 2 x 4 waves of 128x64, 128x128 tiles as 2 x 4 of
// 64x32.  64x64 tiles serve grids that 128x128 tiles would leave under-filled:
// four K groups of 2 x 1 waves of 32x64, each group taking one eight-k step of
// every slice, so that each SIMD runs two waves with two accumulator chains
// each, and an MN-contiguous B is read for both blocks at once.
using SgDma256 = SgDmaCfg<256, 256, 2, 4>;
using SgDma128 = SgDmaCfg<128, 128, 2, 4>;
// Whole 128x128 tiles: two K groups of 2 x 2 waves of 64x64 (3-6% faster than
// 2 x 4 waves of 64x32 on whole tiles; the masked form of this split needs
// more registers and loses on ragged grids, which keep SgDma128).
using SgDma128K = SgDmaCfg<128, 128, 2, 2, 2>;
using SgDma64 = SgDmaCfg<64, 64, 2, 1, 4>;
// With a four-slice ring (64 KB of LDS, still two work-groups per CU): each
// slice holds only about 0.2 us of MFMA work, so two slots prefetch less than
// a load's latency.  The wave tile pairs the blocks of the MN-contiguous
// operand: 32x64 when B is stored K x N (NN; NT too), 64x32 when only A is
// stored K x M (TT).  Measured 20-30% faster at long K (1024^2 x 4096: NN
// 88 -> 68 us, TT 84 -> 66 us); with both operands MN-contiguous (TN) neither
// layout gained consistently, so TN keeps the two-slot ring.
using SgDma64D = SgDmaCfg<64, 64, 2, 1, 4, 4>;
using SgDma64DT = SgDmaCfg<64, 64, 1, 2, 4, 4>;

// The direct-to-LDS kernel applies: 4-byte aligned operands, at least a ring
// of whole slices of k, an MN-contiguous operand (A stored K x M, B stored K x N)
// at least eight wide where M or N is not a multiple of four, and 32-bit slice
// offsets.
template <class Cfg>
bool sg_dma_ok(const GemmProblem &q)
{
    // 16-byte chunks start a multiple of four floats into a row, so they are
    // dword aligned, which is all the 16-byte loads need
    const bool aligned = (reinterpret_cast<uintptr_t>(q.A) % 4 == 0) && (reinterpret_cast<uintptr_t>(q.B) % 4 == 0);
    // a chunk straddling M or N (see the kernel) needs M or N >= 8, so that its
    // overflow stays in the next row, and one row of K left to the tail
    const bool straddle = (q.transA && q.M % 4 != 0) || (!q.transB && q.N % 4 != 0);
    const bool shape = q.K - (straddle ? 1 : 0) >= Cfg::SLOTS * Cfg::BK && (!q.transA || q.M % 4 == 0 || q.M >= 8) &&
                       (q.transB || q.N % 4 == 0 || q.N >= 8);
    // per-lane offsets within one slice are 32-bit: rows of the slice times ld
    const long long rows_a = q.transA ? Cfg::BK : Cfg::BM, rows_b = q.transB ? Cfg::BN : Cfg::BK;
    const bool fits = rows_a * q.lda * 4 < (1LL << 31) && rows_b * q.ldb * 4 < (1LL << 31);
    return aligned && shape && fits;
}

// Storage combinations as bits: 1 << (2*transA + transB).
constexpr int OP_NN = 1, OP_NT = 2, OP_TN = 4, OP_TT = 8, OP_ALL = 15;

// OPS: the storage combinations instantiated (the caller has checked).
template <class Cfg, bool MASK, int OPS>
void launch_sg_dma_ops(const SgemmArgs &a, dim3 grid, bool tA, bool tB, hipStream_t stream)
{
    const dim3 block(Cfg::NT);
    if constexpr ((OPS & OP_NN) != 0)
        if (!tA && !tB) hipLaunchKernelGGL((sgemm_dma_kernel<Cfg, false, false, MASK>), grid, block, 0, stream, a);
    if constexpr ((OPS & OP_NT) != 0)
        if (!tA && tB) hipLaunchKernelGGL((sgemm_dma_kernel<Cfg, false, true, MASK>), grid, block, 0, stream, a);
    if constexpr ((OPS & OP_TN) != 0)
        if (tA && !tB) hipLaunchKernelGGL((sgemm_dma_kernel<Cfg, true, false, MASK>), grid, block, 0, stream, a);
    if constexpr ((OPS & OP_TT) != 0)
        if (tA && tB) hipLaunchKernelGGL((sgemm_dma_kernel<Cfg, true, true, MASK>), grid, block, 0, stream, a);
}

// WHOLE_ONLY: the caller has checked that the problem is made of whole tiles,
// so only the unmasked kernels are instantiated.  OPS: likewise for the
// storage combinations.
template <class Cfg, bool WHOLE_ONLY = false, int OPS = OP_ALL>
hipError_t launch_sg_dma(const GemmProblem &q, hipStream_t stream)
{
    if ((OPS & (1 << (2 * q.transA + q.transB))) == 0) return hipErrorInvalidValue;
    SgemmArgs a;
    a.M = q.M; a.N = q.N; a.K = q.K;
    a.alpha = q.alpha; a.beta = q.beta;
    a.A = static_cast<const float *>(q.A); a.lda = q.lda; a.sA = q.strideA;
    a.B = static_cast<const float *>(q.B); a.ldb = q.ldb; a.sB = q.strideB;
    a.C = q.C; a.ldc = q.ldc; a.sC = q.strideC;
    a.tiles_m = (q.M + Cfg::BM - 1) / Cfg::BM;
    a.tiles_n = (q.N + Cfg::BN - 1) / Cfg::BN;
    const dim3 grid(a.tiles_m * a.tiles_n, 1, q.batch);
    const bool whole = q.M % Cfg::BM == 0 && q.N % Cfg::BN == 0 && q.K % Cfg::BK == 0;
    if constexpr (WHOLE_ONLY) {
        if (!whole) return hipErrorInvalidValue;
        launch_sg_dma_ops<Cfg, false, OPS>(a, grid, q.transA, q.transB, stream);
    } else if (whole) {
        launch_sg_dma_ops<Cfg, false, OPS>(a, grid, q.transA, q.transB, stream);
    } else {
        launch_sg_dma_ops<Cfg, true, OPS>(a, grid, q.transA, q.transB, stream);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small / under-filled problems: split K inside the workgroup.
//
// When even 128x128 tiles leave most CUs idle (M*N small next to K), one
// workgroup owns a (32*FM) x (32*FN) tile of C and its KW waves split K
// into KW contiguous ranges (multiples of 8).  Each wave streams its
// operands straight from global memory into registers -- A as 16-byte quads
// of four consecutive k of a row (element e of quad u feeds k pair
// {8u+e, 8u+4+e}, as in the whole-tile kernel), B as one float per lane and k
// -- keeping P steps of eight k in flight, and accumulates its partial tile on
// the fp32 MFMA.  The KW partial tiles meet in LDS and are summed in a fixed
// order (wave 0 + wave 1 + ...), so results are deterministic; each wave then
// finishes its share of the tile's register quads through the alpha/beta
// epilogue.  Out-of-range rows, columns and k load as zero.
// A transposed operand changes only the loads: a K-contiguous operand (A
// stored M x K, B stored N x K) is read as 16-byte quads of four k, an
// MN-contiguous one as one float per lane and k (coalesced across the lanes).
template <int FM_, int FN_, int KW_, int P_>
struct SgSmallCfg {
    static constexpr int FM = FM_, FN = FN_, KW = KW_, NT = 64 * KW, P = P_;   // P: steps of 8 k in flight
    static constexpr int TM = 32 * FM, TN = 32 * FN;
    static_assert(KW * FM * FN * 4 * 64 * 16 <= 160 * 1024, "partial tiles exceed LDS");
};

template <class Cfg, bool TA, bool TB>
__global__ __launch_bounds__(Cfg::NT) void sgemm_small_kernel(SgemmArgs p)
{
    constexpr int FM = Cfg::FM, FN = Cfg::FN, KW = Cfg::KW, P = Cfg::P;
    __shared__ f32x4_t part[KW * FM * FN * 4 * 64];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int lr = lane & 31, lk = lane >> 5;
    int mb, tm, tn;   // batch member, tile row, tile column
    tile_coords(blockIdx.x, blockIdx.z, gridDim.z, p.tiles_m, p.tiles_n, &mb, &tm, &tn);
    const long long m0 = (long long)tm * Cfg::TM, n0 = (long long)tn * Cfg::TN;
    const int M = p.M, N = p.N, K = p.K;
    const float *A = p.A + (long long)mb * p.sA;
    const float *B = p.B + (long long)mb * p.sB;
    float *C = p.C + (long long)mb * p.sC;
    const long long lda = p.lda, ldb = p.ldb, ldc = p.ldc;

    // this wave's k range
    const int kc = (((K + KW - 1) / KW) + 7) & ~7;
    const int kb = w * kc;
    const int ke = (kb + kc < K) ? kb + kc : K;

    // Row i of op(A) starts at arow[i] and its k-th element is arow[i][k * sa];
    // column j of op(B) likewise with bcol[j] and sb.
    const long long sa = TA ? lda : 1, sb = TB ? 1 : ldb;
    // Rows and columns past M or N read row or column 0.
    const float *arow[FM];
    const float *bcol[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const long long r = m0 + 32 * i + lr;
        arow[i] = A + (r < M ? r : 0) * (TA ? 1 : lda);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const long long c = n0 + 32 * j + lr;
        bcol[j] = B + (c < N ? c : 0) * (TB ? ldb : 1);
    }

    // Four k of one operand row or column starting at kq, zero for k >= ke
    // (the masked form, for a wave's last partial step of eight k).
    auto quad = [&](const float *x, long long stride, int kq, bool kcontig) {
        f32x4_t v;
        if (kcontig && kq + 3 < ke) {
            v = *reinterpret_cast<const f32x4_g *>(x + kq);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = kq + e < ke ? x[(long long)(kq + e) * stride] : 0.f;
        }
        return v;
    };
    // The same for a whole step (kq + 3 < ke), with no branch: out-of-range
    // rows and columns read row or column 0 instead, and their products reach
    // only entries of C that are never stored.
    auto quad_full = [&](const float *x, long long stride, int kq, bool kcontig) {
        f32x4_t v;
        if (kcontig) {
            v = *reinterpret_cast<const f32x4_g *>(x + kq);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = x[(long long)(kq + e) * stride];
        }
        return v;
    };
    f32x4_t ra[P][FM], rb[P][FN];
    auto load_step = [&](int k, f32x4_t *a, f32x4_t *b) {
        const int kq = k + 4 * lk;   // this lane's k quad starts here
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = quad_full(arow[i], sa, kq, !TA);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = quad_full(bcol[j], sb, kq, TB);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    auto mfmas = [&](const f32x4_t *a, const f32x4_t *b) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(b[j][e], a[i][e], acc[i][j], 0, 0, 0);
    };

    // Whole steps of eight k, P in flight.  The loads are unconditional so the
    // compiler waits only for the step about to be used; a load past the last
    // whole step re-reads that step and is never used.
    const int nfull = (ke > kb) ? (ke - kb) / 8 : 0;
    if (nfull > 0) {
        const int last = kb + 8 * (nfull - 1);
#pragma unroll
        for (int s = 0; s < P; ++s) load_step(min(kb + 8 * s, last), ra[s], rb[s]);
        int s0 = 0;
        for (; s0 + P <= nfull; s0 += P) {
#pragma unroll
            for (int s = 0; s < P; ++s) {
                mfmas(ra[s], rb[s]);
                load_step(min(kb + 8 * (s0 + s + P), last), ra[s], rb[s]);
                __builtin_amdgcn_sched_barrier(0);   // keep each refill right after its step
            }
        }
#pragma unroll
        for (int s = 0; s < P; ++s)
            if (s0 + s < nfull) mfmas(ra[s], rb[s]);
    }
    if (kb + 8 * nfull < ke) {   // the partial step (K not a multiple of 8)
        const int kq = kb + 8 * nfull + 4 * lk;
        f32x4_t a[FM], b[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = quad(arow[i], sa, kq, !TA);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = quad(bcol[j], sb, kq, TB);
        mfmas(a, b);
    }

    // Partial tiles to LDS: quad g of block (i, j) of wave w at
    // part[(((w*FM + i)*FN + j)*4 + g)*64 + lane].
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                part[(((w * FM + i) * FN + j) * 4 + g) * 64 + lane] =
                    f32x4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
    __syncthreads();

    // The FM*FN*4 (block, quad) pairs q = (i*FN + j)*4 + g are shared out
    // round robin: wave w reduces pairs w, w + KW, ... over the KW partial
    // tiles in wave order and writes them.
    const float alpha = p.alpha, beta = p.beta;
    constexpr int PAIRS = FM * FN * 4;
#pragma unroll
    for (int q0 = 0; q0 < PAIRS; q0 += KW) {
        const int q = q0 + w;
        if (PAIRS % KW != 0 && q >= PAIRS) break;
        f32x4_t sum = part[q * 64 + lane];
#pragma unroll
        for (int ww = 1; ww < KW; ++ww) sum += part[(ww * PAIRS + q) * 64 + lane];
        const int b = q >> 2, g = q & 3, i = b / FN, j = b % FN;
        const long long row = m0 + 32 * i + lr;
        const long long col = n0 + 32 * j + 8 * g + 4 * lk;
        if (beta != 0.f)
            store_row4<true, true>(C, ldc, row, col, sum, alpha, beta, M, N);
        else
            store_row4<true, false>(C, ldc, row, col, sum, alpha, beta, M, N);
    }
}


template <class Cfg>
hipError_t launch_small(const GemmProblem &q, hipStream_t stream)
{
    SgemmArgs a;
    a.M = q.M; a.N = q.N; a.K = q.K;
    a.alpha = q.alpha; a.beta = q.beta;
    a.A = static_cast<const float *>(q.A); a.lda = q.lda; a.sA = q.strideA;
    a.B = static_cast<const float *>(q.B); a.ldb = q.ldb; a.sB = q.strideB;
    a.C = q.C; a.ldc = q.ldc; a.sC = q.strideC;
    a.tiles_m = (q.M + Cfg::TM - 1) / Cfg::TM;
    a.tiles_n = (q.N + Cfg::TN - 1) / Cfg::TN;
    const dim3 grid(a.tiles_m * a.tiles_n, 1, q.batch), block(Cfg::NT);
    if (!q.transA && !q.transB)
        hipLaunchKernelGGL((sgemm_small_kernel<Cfg, false, false>), grid, block, 0, stream, a);
    else if (!q.transA)
        hipLaunchKernelGGL((sgemm_small_kernel<Cfg, false, true>), grid, block, 0, stream, a);
    else if (!q.transB)
        hipLaunchKernelGGL((sgemm_small_kernel<Cfg, true, false>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((sgemm_small_kernel<Cfg, true, true>), grid, block, 0, stream, a);
    return hipGetLastError();
}

// eight waves, two per SIMD, so that one wave's loads overlap the other's MFMAs
// Eight waves each.  The 32x32 tile keeps two steps in flight: fewer registers
// (52 against 68) let four work-groups share a CU instead of three.
using SgSmall64 = SgSmallCfg<2, 2, 8, 4>;
using SgSmall32 = SgSmallCfg<1, 1, 8, 2>;

using SgBig = SgCfg<128, 128, 16, 2, 2>;

template <class Cfg, bool TA, bool TB>
void launch_cfg_kernel(const SgemmArgs &a, bool whole, dim3 grid, hipStream_t stream)
{
    const dim3 block(Cfg::NT);
    if (whole)
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, false, TA, TB>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, true, TA, TB>), grid, block, 0, stream, a);
}

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
    const bool whole = q.M % Cfg::BM == 0 && q.N % Cfg::BN == 0 && q.K % Cfg::BK == 0;
    const dim3 grid(a.tiles_m * a.tiles_n, 1, q.batch);
    if (!q.transA && !q.transB)
        launch_cfg_kernel<Cfg, false, false>(a, whole, grid, stream);
    else if (!q.transA)
        launch_cfg_kernel<Cfg, false, true>(a, whole, grid, stream);
    else if (!q.transB)
        launch_cfg_kernel<Cfg, true, false>(a, whole, grid, stream);
    else
        launch_cfg_kernel<Cfg, true, true>(a, whole, grid, stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sgemm(const GemmProblem &q, hipStream_t stream)
{
    // Direct-to-LDS tiles: 256x256 or 128x128 (cost model below), else 64x64
    // while those fill at least five eighths of the CUs (below that the
    // split-K kernel's eight-way K split wins: measured crossover between 144
    // and 196 tiles); the split-K kernel for smaller grids;
    // register-staged 128x128 tiles with bounds checks for operands the
    // direct-to-LDS kernel cannot take.
    //
    // A 256x256 tile takes a CU's whole LDS, so a grid of them runs in rounds
    // of 256 work-groups.  128x128 tiles run two per CU and spread evenly; 1024
    // of them take about 1.05 rounds of 256x256 tiles (measured).  So the
    // 256x256 tile wins when 1024 * its rounds <= 1.05 * the 128x128 tiles.
    const long long t256 = (long long)((q.M + 255) / 256) * ((q.N + 255) / 256) * q.batch;
    const long long t128 = (long long)((q.M + 127) / 128) * ((q.N + 127) / 128) * q.batch;
    const long long t64 = (long long)((q.M + 63) / 64) * ((q.N + 63) / 64) * q.batch;
    if (t128 < 256 && 8 * t64 >= 5 * 256) {
        if (!q.transA && sg_dma_ok<SgDma64D>(q)) return launch_sg_dma<SgDma64D, false, OP_NN | OP_NT>(q, stream);
        if (q.transA && q.transB && sg_dma_ok<SgDma64DT>(q)) return launch_sg_dma<SgDma64DT, false, OP_TT>(q, stream);
        if (sg_dma_ok<SgDma64>(q)) return launch_sg_dma<SgDma64>(q, stream);
    }
    if (t128 < 256) {
        // fewer 128x128 tiles than CUs: split K inside smaller workgroup tiles
        if (t64 >= 256) return launch_small<SgSmall64>(q, stream);
        return launch_small<SgSmall32>(q, stream);
    }
    const long long r256 = (t256 + 255) / 256;
    if (20 * 1024 * r256 <= 21 * t128 && sg_dma_ok<SgDma256>(q)) return launch_sg_dma<SgDma256>(q, stream);
    if (q.M % 128 == 0 && q.N % 128 == 0 && q.K % 32 == 0 && sg_dma_ok<SgDma128K>(q))
        return launch_sg_dma<SgDma128K, true, OP_ALL>(q, stream);
    if (sg_dma_ok<SgDma128>(q)) return launch_sg_dma<SgDma128>(q, stream);
    return launch_cfg<SgBig>(q, stream);
}

}  // namespace mi355gemm
