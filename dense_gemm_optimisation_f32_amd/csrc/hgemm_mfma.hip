// hgemm_mfma.hip -- 16-bit-input, fp32-accumulate row-major GEMM (single and
// strided-batched) on the CDNA4 matrix cores: IEEE binary16 inputs (fp16 MFMA)
// and, through the same kernels, bfloat16 inputs (bf16 MFMA), the two input
// formats of the MindNotes 'GEMM' page's mixed-precision interface (section
// "Batched execution and mixed precision").
//
// The tiling follows the wave-level hierarchy of the dandandamowang.xyz
// 'GEMM optimisation (2): Tensor Core wmma API' page (sections 4-7: one warp
// owning a grid of MMA tiles, double-buffered shared-memory staging, padding
// against bank conflicts, and the larger 128x128 block tile), rebuilt for
// gfx950 rather than translated:
//   * matrix-core op: v_mfma_f32_32x32x16_f16 (a 32x32 fp32 block, 16 k per op,
//     8 fp16 values of A and of B per lane); each wave owns a grid of such
//     blocks whose accumulators stay in registers for the whole K loop;
//   * a K-contiguous operand tile (A stored M x K, B stored N x K) sits in LDS
//     as rows of 16-byte chunks whose chunk index is XOR-swizzled with bits of
//     the row (the MindNotes page's swizzling idea applied to 16-byte chunks),
//     so an operand fragment is one 16-byte LDS read per lane;
//   * an MN-contiguous tile (A stored K x M, B stored K x N) keeps its [k][mn]
//     layout, swizzled or padded so that the rows one transposed read touches
//     fall in different banks (the dandandamowang page's padding), and the
//     K-packed fragment is assembled by two ds_read_b64_tr_b16 transposed LDS
//     reads: within each 16-lane group, lane i receives element i%4 of the
//     four-element vectors addressed by lanes i/4, i/4+4, i/4+8 and i/4+12, so
//     lanes pointing at four consecutive n of rows k..k+3 hand each lane one
//     column's four k values;
//   * both reads hand lane l the same eight k (8*(l/32) .. +7 of the 16-k
//     substep), so the four storage combinations (C = alpha*op(A)op(B) +
//     beta*C, the MindNotes 'GEMM' page, section "core problem and arithmetic
//     characteristics") add the same products in the same order;
//   * workgroups are mapped to tiles so that the tiles one XCD (one L2) runs
//     form a compact block of C;
//   * epilogue C = alpha*acc + beta*C (C not read when beta == 0).
//
// Two kernels; launch_hgemm (binary16) and launch_bgemm (bfloat16) pick one
// per problem:
//   * hgemm_dma_kernel -- operands whose rows start 4-byte aligned.  K slices
//     go from global memory straight into an LDS ring (direct-to-LDS loads, the
//     gfx950 form of the page's asynchronous double buffering): 256x256 tiles
//     with two slots of 64 k, or 128x128 or 64x128 tiles with four.  Ragged M, N and K
//     are handled by clamped slice loads, a K tail read from global memory and
//     masked stores.  Whole tiles with beta != 0 run an instantiation whose
//     epilogue reads and writes C by rows of the wave tile, one block row
//     ahead (on 256x256 tiles, block row 1 goes straight into the LDS slot
//     that the K loop has finished with);
//   * hgemm_mfma_kernel -- everything else: 128x128 (64x64 for small grids)
//     tiles of four waves in a 2 x 2 grid, read into registers with 16-byte
//     loads (row starts 4-byte aligned: CDNA's multi-dword global loads need
//     only dword alignment), with a 16-byte and a dword load joined by a
//     funnel shift (rows starting at an odd half), or, at the matrix's edge,
//     with element loads, and written to a double-buffered
//     LDS with one barrier per K step.  MASK = false for whole tiles, true
//     otherwise (out-of-range elements load as zero, stores are masked).
#include "gemm_internal.h"
#include "tile_order.h"
#include "epilogue.h"
#include "plan16.h"

#include <type_traits>

namespace mi355gemm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// One 32x32x16 matrix-core op on eight 16-bit values of B and of A per lane:
// IEEE binary16 (BF = false) or bfloat16 (BF = true).  The kernels only move
// 16-bit payloads (half8 is their carrier type); the format matters here alone.
// Products of either format are exact in fp32, and the sum is accumulated in
// fp32 in both.
template <bool BF>
__device__ __forceinline__ f32x16 mfma16(half8 b, half8 a, f32x16 c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// 16 bytes in global memory at dword (not 16-byte) alignment: multi-dword
// global loads need only dword alignment on CDNA
typedef unsigned int u32x4_g __attribute__((ext_vector_type(4), aligned(4)));
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
    // K split over workgroups (direct-to-LDS kernel only): nsplit workgroups
    // share each tile, split s taking whole slices [s*q + min(s, r), ...) of the
    // nk slices (q = nk / nsplit, r = nk % nsplit) and the last split the K
    // tail; their partial tiles meet in ws_part and the last to finish (counted
    // in ws_count) adds them in split order and runs the epilogue.  nsplit = 1:
    // no split, ws_* unused.
    int nsplit;
    unsigned *ws_count;   // one counter per (member, tile), zero between launches
    float *ws_part;       // nsplit partial tiles per (member, tile)
};

template <int BM_, int BN_>
struct HgCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64, WM = 2, WN = 2, NT = 256;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole MFMA blocks");
};

// One operand tile of the register-staged kernel: R rows or columns of the
// output (BM for A, BN for B) by BK k.  KC: stored K-contiguous, kept in LDS
// as R rows of BK halves with swizzled 16-byte chunks; otherwise stored
// MN-contiguous, kept as BK rows of R halves plus a 64-byte pad.
template <bool KC, int R, int BK, int NT>
struct HgTile {
    static constexpr bool KCONTIG = KC;
    static constexpr int ROWS = KC ? R : BK;         // rows as stored
    static constexpr int COLS = KC ? BK : R;         // contiguous halves per stored row
    static constexpr int CPR = COLS / 8;             // 16-byte chunks per stored row
    static constexpr int LOADS = ROWS * CPR / NT;    // 16-byte chunks per thread
    static constexpr int PITCH = KC ? BK : R + 32;   // LDS row pitch (halves)
    static constexpr int HALVES = ROWS * PITCH;
    static_assert((ROWS * CPR) % NT == 0, "tile loads must split evenly");
    static_assert(!KC || BK == 64, "K-contiguous LDS rows are eight 16-byte chunks");
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

// Eight halves at p, which may start 2 bytes past a dword: a 16-byte load from
// the dword holding p[0] and a 4-byte load of the dword holding p[7], joined by
// a funnel shift of 0 or 16 bits.  Every dword read holds one of the eight
// halves, so no load leaves the words the matrix occupies.
__device__ __forceinline__ u32x4 load8_words(const uint16_t *p)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const unsigned sh = (unsigned)(a & 2) * 8;
    const unsigned *w = reinterpret_cast<const unsigned *>(a & ~(uintptr_t)3);
    const u32x4 lo = *reinterpret_cast<const u32x4_g *>(w);
    const unsigned hi = w[sh ? 4 : 3];
    return u32x4{__builtin_amdgcn_alignbit(lo.y, lo.x, sh), __builtin_amdgcn_alignbit(lo.z, lo.y, sh),
                 __builtin_amdgcn_alignbit(lo.w, lo.z, sh), __builtin_amdgcn_alignbit(hi, lo.w, sh)};
}

// Eight consecutive halves (r, c..c+7) of a row-major rows x cols matrix X;
// with MASK, elements outside it read as zero.  VEC: row starts are 4-byte
// aligned, so eight halves inside the matrix are one 16-byte load; otherwise
// they are two dword-aligned loads and a shift.
template <bool MASK, bool VEC>
__device__ __forceinline__ u32x4 load8(const uint16_t *X, long long ld, long long r, long long c, long long rows,
                                       long long cols)
{
    const uint16_t *src = X + r * ld + c;
    if (!MASK) return *reinterpret_cast<const u32x4_g *>(src);
    if (r >= rows || c >= cols) return u32x4{0u, 0u, 0u, 0u};
    if (c + 8 <= cols) return VEC ? *reinterpret_cast<const u32x4_g *>(src) : load8_words(src);
    return load8_masked(src, (int)(cols - c));
}

// TA: A stored K x M; TB: B stored N x K.
template <class Cfg, bool BF, bool MASK, bool VEC, bool TA, bool TB>
__global__ __launch_bounds__(256) void hgemm_mfma_kernel(HgemmArgs p)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::NT;
    using TileA = HgTile<!TA, BM, BK, NT>;
    using TileB = HgTile<TB, BN, BK, NT>;
    constexpr int BUF_HALVES = TileA::HALVES + TileB::HALVES;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BUF_HALVES];

    const int tid = threadIdx.x;
    int mb, tm, tn;   // batch member, tile row, tile column
    tile_coords(blockIdx.x, blockIdx.z, gridDim.z, p.tiles_m, p.tiles_n, &mb, &tm, &tn);
    const long long m0 = (long long)tm * BM, n0 = (long long)tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const uint16_t *A = p.A + (long long)mb * p.sA;
    const uint16_t *B = p.B + (long long)mb * p.sB;
    float *C = p.C + (long long)mb * p.sC;
    const long long lda = p.lda, ldb = p.ldb, ldc = p.ldc;

    u32x4 ra[TileA::LOADS], rb[TileB::LOADS];

    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < TileA::LOADS; ++i) {
            const int id = i * NT + tid;
            const int r = id / TileA::CPR, c = (id % TileA::CPR) * 8;
            ra[i] = TA ? load8<MASK, VEC>(A, lda, k0 + r, m0 + c, K, M) : load8<MASK, VEC>(A, lda, m0 + r, k0 + c, M, K);
        }
#pragma unroll
        for (int i = 0; i < TileB::LOADS; ++i) {
            const int id = i * NT + tid;
            const int r = id / TileB::CPR, c = (id % TileB::CPR) * 8;
            rb[i] = TB ? load8<MASK, VEC>(B, ldb, n0 + r, k0 + c, N, K) : load8<MASK, VEC>(B, ldb, k0 + r, n0 + c, K, N);
        }
    };

    // K-contiguous rows go to swizzled chunks, MN-contiguous rows to padded rows.
    auto store_one = [&](auto tile, uint16_t *dst, int i, const u32x4 &v) {
        using T = decltype(tile);
        const int id = i * NT + tid;
        const int r = id / T::CPR, c = id % T::CPR;
        if constexpr (T::KCONTIG)
            *reinterpret_cast<u32x4 *>(dst + r * BK + 8 * swz(r, c)) = v;
        else
            *reinterpret_cast<u32x4 *>(dst + r * T::PITCH + 8 * c) = v;
    };
    auto store_tiles = [&](int buf) {
        uint16_t *la = lds + buf * BUF_HALVES;
        uint16_t *lb = la + TileA::HALVES;
#pragma unroll
        for (int i = 0; i < TileA::LOADS; ++i) store_one(TileA{}, la, i, ra[i]);
#pragma unroll
        for (int i = 0; i < TileB::LOADS; ++i) store_one(TileB{}, lb, i, rb[i]);
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int lr = lane & 31, lk = lane >> 5;
    // transposed-read lane roles: group q of 16 lanes, lane j within it
    const int q = lane >> 4, j = lane & 15;
    const int tr_row = 8 * (q >> 1) + (j >> 2);   // + 16*s + 4*h
    const int tr_col = 16 * (q & 1) + 4 * (j & 3);  // + wave offset + 32*block

    f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < Cfg::FN; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;

    // Fragment of 32 output rows (or columns) starting at `first`, for the
    // 16-wide k substep s: lane l gets row/column first + l%32 and the eight k
    // 16s + 8*(l/32) .. +7.
    auto read_frag = [&](auto tile, const uint16_t *base, int first, int s) -> half8 {
        using T = decltype(tile);
        if constexpr (T::KCONTIG) {
            const int row = first + lr;
            return *reinterpret_cast<const half8 *>(base + row * BK + 8 * swz(row, 2 * s + lk));
        } else {
            const uint16_t *at = base + (16 * s + tr_row) * T::PITCH + first + tr_col;
            const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(at));
            const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(at + 4 * T::PITCH));
            const short4v both[2] = {lo, hi};
            return __builtin_bit_cast(half8, both);
        }
    };
    // Operand fragments of one 16-wide k substep, double-buffered in registers:
    // the fragments of substep s+1 are read from LDS while the MFMAs of
    // substep s run.
    half8 fa[2][Cfg::FM], fb[2][Cfg::FN];
    auto read_frags = [&](int buf, int s, half8 *a, half8 *b) {
        const uint16_t *la = lds + buf * BUF_HALVES;
        const uint16_t *lb = la + TileA::HALVES;
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) a[i] = read_frag(TileA{}, la, wm * Cfg::TM + 32 * i, s);
#pragma unroll
        for (int jj = 0; jj < Cfg::FN; ++jj) b[jj] = read_frag(TileB{}, lb, wn * Cfg::TN + 32 * jj, s);
    };
    auto mfmas = [&](const half8 *a, const half8 *b) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < Cfg::FN; ++jj)
                acc[i][jj] = mfma16<BF>(b[jj], a[i], acc[i][jj]);
    };

    constexpr int NS = BK / 16;   // k substeps per K step
    const int nk = (K + BK - 1) / BK;
    // Prologue: tile 0 into LDS buffer 0, tile 1 on its way into registers,
    // fragments of substep 0 in registers.
    load_tiles(0);
    store_tiles(0);
    if (nk > 1) load_tiles(BK);
    __syncthreads();
    read_frags(0, 0, fa[0], fb[0]);

    // Step t computes tile t from LDS buffer t%2.  Registers hold tile t+1;
    // they are written to the other buffer during step t (that buffer was last
    // read in step t-1, before its closing barrier) and refilled with tile t+2.
    for (int t = 0; t < nk; ++t) {
        const int buf = t & 1;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int cur = s & 1, nxt = cur ^ 1;
            if (s + 1 < NS) {
                read_frags(buf, s + 1, fa[nxt], fb[nxt]);
                if (s + 2 == NS && t + 1 < nk) {
                    store_tiles(buf ^ 1);
                    if (t + 2 < nk) load_tiles((t + 2) * BK);
                }
            } else if (t + 1 < nk) {
                __syncthreads();
                read_frags(buf ^ 1, 0, fa[nxt], fb[nxt]);
            }
            mfmas(fa[cur], fb[cur]);
        }
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
// Whole-tile kernel fed by direct-to-LDS loads.
//
// gfx950's global_load_lds_dwordx4 moves 16 bytes per lane from global memory
// straight into LDS, lane l's bytes landing at M0 + 16*l, with no trip through
// vector registers and no LDS-write instruction.  The K loop keeps a ring of
// STAGES slices of BK k in LDS and fetches slice t+STAGES while slice t is
// computed.  Because a wave's load fills 1 KB of LDS contiguously, the
// swizzled layouts are produced by choosing, per lane, which global chunk to
// fetch for the LDS position the lane owns.  Each operand slice keeps its
// stored orientation:
//   * K-contiguous (A stored M x K, B stored N x K): R rows (R = BM or BN) of
//     BK halves (four or eight 16-byte k chunks); the chunk at physical
//     position p of row r holds logical chunk p ^ swz_a(r); one ds_read_b128
//     per lane and fragment;
//   * MN-contiguous (A stored K x M, B stored K x N): BK rows of R halves; the
//     chunk at physical position p of row k holds logical chunk p ^ swz_b(k);
//     two ds_read_b64_tr_b16 per lane and fragment.
// swz_a keeps the rows one LDS cycle serves on distinct banks for the 16-byte
// reads; swz_b does the same for the four rows a transposed read touches
// (measured conflict-free on gfx950 for 128- and 256-byte windows).
// The workgroup runs WM x WN waves; with eight waves two share each SIMD, so
// one wave's MFMAs cover the other's LDS latency.
// Requires M % BM == 0, N % BN == 0, K % BK == 0, K >= STAGES*BK, 16-byte
// aligned rows and byte offsets within a slice below 2^31.
template <int BM_, int BN_, int STAGES_, int WM_, int WN_, int BK_, bool SPLITS_ = false>
struct HgDmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WM = WM_, WN = WN_;
    static constexpr bool SPLITS = SPLITS_;   // also built with a K split over workgroups
    static constexpr int NW = WM * WN, NT = 64 * NW;
    static constexpr int A_CPR = BK / 8;                        // 16-byte chunks per A row
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int A_BYTES = BM * BK * 2;                 // one A slice
    static constexpr int B_BYTES = BK * BN * 2;                 // one B slice
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // A 1 KB direct-to-LDS load occupies the CU's vector-memory path for about
    // 16 cycles, and a wave blocked on issuing loads cannot issue MFMAs.  With
    // a two-slot ring the upper half of the waves (one per SIMD) issues every
    // load, right after the barrier that frees a slot, and the other wave on
    // each SIMD keeps the matrix core busy meanwhile.  With three or more
    // slots (STAGGER) every wave loads a share: the lower half right after the
    // barrier, the upper half two substeps before the next one, into the slot
    // that the previous barrier freed, so the two waves of a SIMD block on
    // their loads at different times.
    static constexpr bool STAGGER = STAGES >= 3;
    static constexpr int LW = STAGGER ? NW : NW / 2;            // loading waves
    static constexpr int A_LOADS = A_BYTES / 1024 / LW;         // per loading wave per slice
    static constexpr int B_LOADS = B_BYTES / 1024 / LW;
    static_assert(A_BYTES % (1024 * LW) == 0 && B_BYTES % (1024 * LW) == 0, "slices must split over the loaders");
    static_assert(A_CPR == 4 || A_CPR == 8, "K-contiguous rows of 64 or 128 bytes");
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS ring too large");
};

// A chunk swizzle.  64-byte rows (four chunks): rows that one LDS cycle
// serves get distinct (row, chunk) bank groups.  128-byte rows (eight chunks):
// the chunk is XORed with row bits 0-2 and 3-4, which keeps any aligned 16
// rows on distinct banks and is unchanged by the 32-row steps between the
// MFMA blocks of a wave.
template <int CPR>
__device__ __forceinline__ int swz_a(int r)
{
    return CPR == 8 ? ((r & 7) ^ ((r >> 3) & 3)) : (((r >> 1) ^ (r >> 3)) & 3);
}
__device__ __forceinline__ int swz_b(int k)
{
    // rows k..k+3 of an aligned group of four map to XOR patterns 0, 6, 10, 12
    return (0xCA60 >> (4 * (k & 3))) & 15;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) half8 lds_half8;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4;

__device__ __forceinline__ lds_void *lds_ptr(unsigned byte)
{
    return (lds_void *)(uintptr_t)byte;
}

// One direct-to-LDS load: every lane fetches 16 bytes at sbase + voff and the
// wave's 1 KB lands contiguously at LDS byte lds_addr (lane l at +16*l).  It is
// issued through inline asm so that the compiler neither reorders LDS accesses
// around it (memory clobber) nor adds its own conservative vmcnt(0) before
// every later LDS read: completion is tracked explicitly with wait_vmcnt.  M0
// (the LDS destination) is set inside the statement; the compiler does not
// track that clobber, which is safe because these kernels give M0 no other use.
__device__ __forceinline__ void dma16(const void *sbase, unsigned voff, unsigned lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory", "m0");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Per-lane byte offset (within one slice of global memory) of the 16-byte
// chunk that lane `lane` of wave load g fetches for an operand slice of R rows
// or columns and BK k; see the layouts above.  With CLAMP, `lim` is how many
// of the R rows (K-contiguous) or columns (MN-contiguous) lie inside M or N:
// a chunk past it re-reads a valid one (row lim-1, or chunk 0 of its row),
// whose products only reach C entries that are never stored.
template <bool KC, int R, int BK, bool CLAMP>
__device__ __forceinline__ unsigned dma_offset(int g, int lane, long long ld, int lim)
{
    if (KC) {
        constexpr int CPR = BK / 8;
        const int r = (64 / CPR) * g + lane / CPR;
        const int rr = (CLAMP && r >= lim) ? lim - 1 : r;
        return (unsigned)(rr * ld + 8 * ((lane % CPR) ^ swz_a<CPR>(r))) * 2u;
    }
    constexpr int CPR = R / 8, RPL = 64 / CPR;   // chunks per row, rows per wave load
    const int k = RPL * g + lane / CPR;
    int ch = (lane % CPR) ^ swz_b(k);
    if (CLAMP && 8 * ch >= lim) ch = 0;
    return (unsigned)(k * ld + 8 * ch) * 2u;
}

// Fragment read address (bytes within a slot, substep 0, MFMA block 0) for the
// lane; KC: the rows start at `first`, MN-contiguous: the columns do.
// K-contiguous fragments of substep s and block i add 16*(s-chunk XOR) and
// i*32 rows; MN-contiguous ones add 16*s rows and 32*i columns.
template <bool KC, int R, int BK>
__device__ __forceinline__ unsigned frag_offset(int first, int lane, int s)
{
    const int lr = lane & 31, lk = lane >> 5, q = lane >> 4, j = lane & 15;
    if (KC) {
        const int r = first + lr;
        return (unsigned)(r * BK * 2 + 16 * ((2 * s + lk) ^ swz_a<BK / 8>(r)));
    }
    const int kq = 8 * (q >> 1) + (j >> 2);     // row within a 16-row substep (plus 4*h)
    const int n = first + 16 * (q & 1) + 4 * (j & 3);
    return (unsigned)(kq * R * 2 + 16 * ((n >> 3) ^ swz_b(kq)) + 2 * (n & 7));
}

// TA: A stored K x M; TB: B stored N x K.  MASK: M and N need not be
// multiples of the tile, nor K of BK (the loads clamp to valid rows and
// columns, the K % BK tail is read straight from global memory after the last
// slice, and stores outside C are skipped); a 16-byte chunk of an
// MN-contiguous operand may straddle M or N (see the slice count below).
template <class Cfg, bool BF, bool TA, bool TB, bool MASK, bool SPLIT, bool CROWS>
__global__ __launch_bounds__(Cfg::NT) void hgemm_dma_kernel(HgemmArgs p)
{
    static_assert(!CROWS || !MASK, "the epilogue by rows is for whole tiles");
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, S = Cfg::STAGES;
    constexpr bool A_KC = !TA, B_KC = TB;
    static_assert((A_KC || BM >= 128) && (B_KC || BN >= 128), "MN-contiguous slices need 16 chunks per row");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[S * Cfg::STAGE_BYTES];
    const unsigned lds0 = (unsigned)(uintptr_t)lds;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nsplit = SPLIT ? p.nsplit : 1;
    int mb, tm, tn, sp;   // batch member, tile row, tile column, K split
    tile_coords_split(blockIdx.x, blockIdx.z, gridDim.z, p.tiles_m, p.tiles_n, nsplit, &mb, &tm, &tn, &sp);
    const long long m0 = (long long)tm * BM, n0 = (long long)tn * BN;
    const long long lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    // An MN-contiguous operand whose M or N is not a multiple of eight has a
    // chunk that straddles that edge.  Its halves past the edge only reach C
    // entries that are never stored, and in any row but the matrix's last they
    // lie in the next row.  The slices then stop before row K-1 and the K tail
    // below takes the rest, so no slice load reads past the operand.
    const bool straddle = MASK && ((!A_KC && p.M % 8 != 0) || (!B_KC && p.N % 8 != 0));
    const int nk_all = (p.K - (straddle ? 1 : 0)) / BK;   // whole slices of the problem
    // this workgroup's slices [s_begin, s_begin + nk), nk >= S (checked by the launcher)
    const int q_split = nk_all / nsplit, r_split = nk_all % nsplit;
    const int s_begin = sp * q_split + (sp < r_split ? sp : r_split);
    const int nk = q_split + (sp < r_split ? 1 : 0);
    const bool last_split = sp == nsplit - 1;
    // first element of the workgroup's first slice in each operand, and the
    // bytes between consecutive slices
    const long long stepA = A_KC ? BK * 2 : BK * lda * 2;
    const long long stepB = B_KC ? BK * 2 : BK * ldb * 2;
    const char *Ab = reinterpret_cast<const char *>(p.A + (long long)mb * p.sA + (A_KC ? m0 * lda : m0)) +
                     (long long)s_begin * stepA;
    const char *Bb = reinterpret_cast<const char *>(p.B + (long long)mb * p.sB + (B_KC ? n0 * ldb : n0)) +
                     (long long)s_begin * stepB;
    float *C = p.C + (long long)mb * p.sC;

    // Loading waves are NW-LW .. NW-1; loader index lw numbers their 1 KB
    // pieces of each slice.
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const bool loader = uwave >= Cfg::NW - Cfg::LW;
    const int lw = loader ? uwave - (Cfg::NW - Cfg::LW) : 0;
    // rows / columns of the tile inside M and N
    const int limA = MASK ? (int)(p.M - m0 < BM ? p.M - m0 : BM) : BM;
    const int limB = MASK ? (int)(p.N - n0 < BN ? p.N - n0 : BN) : BN;
    unsigned offA[Cfg::A_LOADS], offB[Cfg::B_LOADS];
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i)
        offA[i] = dma_offset<A_KC, BM, BK, MASK>(lw * Cfg::A_LOADS + i, lane, lda, limA);
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i)
        offB[i] = dma_offset<B_KC, BN, BK, MASK>(lw * Cfg::B_LOADS + i, lane, ldb, limB);
    auto issue_slice = [&](int kt, int slot) {
        if (!loader) return;
        const char *a = Ab + (long long)kt * stepA;
        const char *b = Bb + (long long)kt * stepB;
        const unsigned la = lds0 + slot * Cfg::A_BYTES + lw * Cfg::A_LOADS * 1024;
        const unsigned lb = lds0 + S * Cfg::A_BYTES + slot * Cfg::B_BYTES + lw * Cfg::B_LOADS * 1024;
#pragma unroll
        for (int i = 0; i < Cfg::A_LOADS; ++i) dma16(a, offA[i], la + 1024 * i);
#pragma unroll
        for (int i = 0; i < Cfg::B_LOADS; ++i) dma16(b, offB[i], lb + 1024 * i);
    };
    // vector-memory ops per slice per loading lane (the other waves have none
    // outstanding, so their waits on this count return at once)
    constexpr int LOADS = Cfg::A_LOADS + Cfg::B_LOADS;

    // Fragment read addresses (bytes, without the slot base): per substep for a
    // K-contiguous operand (blocks are 32 rows apart, which the swizzle
    // ignores), per block for an MN-contiguous one (substeps are 16 rows
    // apart, which the swizzle ignores too).
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int lr = lane & 31, lk = lane >> 5;
    constexpr int NS = BK / 16;
    constexpr int NFA = A_KC ? NS : Cfg::FM, NFB = B_KC ? NS : Cfg::FN;
    unsigned fragA[NFA], fragB[NFB];
#pragma unroll
    for (int x = 0; x < NFA; ++x)
        fragA[x] = A_KC ? frag_offset<true, BM, BK>(wm * Cfg::TM, lane, x)
                        : frag_offset<false, BM, BK>(wm * Cfg::TM + 32 * x, lane, 0);
#pragma unroll
    for (int x = 0; x < NFB; ++x)
        fragB[x] = S * Cfg::A_BYTES + (B_KC ? frag_offset<true, BN, BK>(wn * Cfg::TN, lane, x)
                                        : frag_offset<false, BN, BK>(wn * Cfg::TN + 32 * x, lane, 0));

    f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < Cfg::FN; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;

    // Fragment x (MFMA block) of substep s of an operand with R rows/columns.
    auto frag = [&](auto kc, auto rr, unsigned base, const unsigned *off, int x, int s) -> half8 {
        constexpr int R = decltype(rr)::value;
        if constexpr (decltype(kc)::value) {
            return *(const lds_half8 *)(uintptr_t)(base + off[s] + x * 32 * BK * 2);
        } else {
            const unsigned at = base + off[x] + 16 * s * R * 2;
            const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(uintptr_t)at);
            const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(uintptr_t)(at + 4 * R * 2));
            const short4v both[2] = {lo, hi};
            return __builtin_bit_cast(half8, both);
        }
    };
    half8 fa[2][Cfg::FM], fb[2][Cfg::FN];
    // LDS ring layout: the S slots of A, then the S slots of B, so that with the
    // slot known at compile time every fragment read is a register offset fixed
    // for the whole loop plus an immediate below 64 KB (slot, block, substep).
    auto read_frags = [&](int slot, int s, half8 *a, half8 *b) {
        const unsigned base_a = lds0 + slot * Cfg::A_BYTES, base_b = lds0 + slot * Cfg::B_BYTES;
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
            a[i] = frag(std::bool_constant<A_KC>{}, std::integral_constant<int, BM>{}, base_a, fragA, i, s);
#pragma unroll
        for (int jj = 0; jj < Cfg::FN; ++jj)
            b[jj] = frag(std::bool_constant<B_KC>{}, std::integral_constant<int, BN>{}, base_b, fragB, jj, s);
    };
    auto mfmas = [&](const half8 *a, const half8 *b) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < Cfg::FN; ++jj)
                acc[i][jj] = mfma16<BF>(b[jj], a[i], acc[i][jj]);
    };
    auto lds_barrier = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    // Interleave each substep's MFMAs one-for-one with the LDS reads of the
    // next substep's fragments.
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < Cfg::FM * Cfg::FN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        }
    };
    // One step on slice t (slot t % S).  The fragments of substep sub+1 are read
    // while substep sub is computed; before the last substep, once slice t+1 is
    // resident for every wave (this lane's loads counted down to PENDING
    // outstanding slices, then the barrier) and every wave holds its slice-t
    // fragments, slot t % S is refilled with slice t+S and the first fragments
    // of slice t+1 are read while the last substep of slice t is computed.
    // Staggered refills: the upper half of the waves loads its share of slice
    // t-1+S during substep NS-2 of step t (t >= 1).  The count of outstanding
    // slices at each wait is the same for both halves.
    const bool late = Cfg::STAGGER && uwave >= Cfg::NW / 2;
    static_assert(!Cfg::STAGGER || NS >= 2, "staggered refills need two substeps per slice");
    // slot_of(t): the ring slot of slice t, t % S; where the caller knows it at
    // compile time (the unrolled steady loop below) it passes it as a constant,
    // so every fragment read of the step addresses LDS with a fixed offset from
    // registers computed once, instead of adding the slot base per read.
    auto step_in = [&](int t, auto pending, auto refill, bool late_refill, auto slot_c) {
        constexpr int SC = decltype(slot_c)::value;   // < 0: not known at compile time
        const int slot = SC >= 0 ? SC : t % S;
        const int next = SC >= 0 ? (SC + 1) % S : (t + 1) % S;
        const int prev = SC >= 0 ? (SC + S - 1) % S : (t - 1 + S) % S;
#pragma unroll
        for (int sub = 0; sub < NS; ++sub) {
            const int cur = sub & 1, nxt = cur ^ 1;
            if (sub + 1 < NS) {
                read_frags(slot, sub + 1, fa[nxt], fb[nxt]);
                if (Cfg::STAGGER && sub == NS - 2 && late && late_refill) issue_slice(t - 1 + S, prev);
            } else {
                wait_vmcnt<LOADS * decltype(pending)::value>();
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's slice-t reads are done
                lds_barrier();
                if (decltype(refill)::value && !late) issue_slice(t + S, slot);
                read_frags(next, 0, fa[nxt], fb[nxt]);
            }
            mfmas(fa[cur], fb[cur]);
            interleave();
        }
    };
    auto step = [&](int t, auto pending, auto refill, bool late_refill) {
        step_in(t, pending, refill, late_refill, std::integral_constant<int, -1>{});
    };

    // Prologue: slices 0..S-1 in flight; slice 0 resident; substep 0 fragments read.
#pragma unroll
    for (int st = 0; st < S; ++st) issue_slice(st, st);
    wait_vmcnt<LOADS * (S - 1)>();
    lds_barrier();
    read_frags(0, 0, fa[0], fb[0]);

    // Steady state: slices up to t+S-1 issued, slice t+1 needed.
    // (unrolled over the S slots, so each step's slot is a compile-time constant;
    // not for the 64-row tile, whose four-way unrolled loop measured slower:
    // 512x4096x4096 25.0 -> 26.2 us)
    {
        int t = 0;
        constexpr bool UNROLL = Cfg::BM >= 128 && !MASK && B_KC == false;
        for (; UNROLL && t + S - 1 + S < nk; t += S) {
            [&]<int... I>(std::integer_sequence<int, I...>) {
                (step_in(t + I, std::integral_constant<int, S - 2>{}, std::true_type{}, t + I >= 1,
                         std::integral_constant<int, I>{}),
                 ...);
            }(std::make_integer_sequence<int, S>{});
        }
        for (; t + S < nk; ++t) step(t, std::integral_constant<int, S - 2>{}, std::true_type{}, t >= 1);
    }
    // Tail: no more slices to issue; the outstanding count drains to zero
    // (with staggered refills, the upper waves still issue their share of the
    // last slice during the first of these steps).
    const int t0 = nk - S;
    static_assert(S >= 2 && S <= 4, "ring of two to four slices");
    step(t0, std::integral_constant<int, S - 2>{}, std::false_type{}, t0 >= 1);
    if constexpr (S >= 3) step(t0 + 1, std::integral_constant<int, S - 3>{}, std::false_type{}, false);
    if constexpr (S >= 4) step(t0 + 2, std::integral_constant<int, S - 4>{}, std::false_type{}, false);
    // CROWS (whole tiles, beta != 0): the epilogue runs by rows (below), C read
    // and written in row segments of the wave tile, one 32-row block row
    // ahead.  Where the workgroup is the only one on its tile (no K split),
    // the first block row's read is issued here, so that it is in flight
    // during the last slice's MFMAs.  In the row layout lane l covers columns
    // 4*(l % LPR) .. +3 of row (l / LPR) + RPI*q of a block row, q = 0 .. NQ-1.
    const float alpha = p.alpha, beta = p.beta;
    auto col_of = [&](int jj, int g) -> long long { return n0 + wn * Cfg::TN + 32 * jj + 8 * g + 4 * lk; };
    constexpr int PITCH = Cfg::TN + 4;   // floats per staged row (the pad spreads 32 rows over the banks)
    constexpr int LPR = Cfg::TN / 4, RPI = 64 / LPR, NQ = 32 / RPI;
    static_assert(NQ == Cfg::FN * 4, "a block row holds as many quads in either layout");
    f32x4_t cb[NQ];
    auto read_row = [&](int i, f32x4_t *dst) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int r = q * RPI + lane / LPR, c = 4 * (lane % LPR);
            dst[q] = load_row4<MASK>(C, ldc, m0 + wm * Cfg::TM + 32 * i + r, n0 + wn * Cfg::TN + c, p.M, p.N);
        }
    };
    constexpr bool early_c = CROWS && !SPLIT;
    if constexpr (early_c) read_row(0, cb);
    // CDMA: the 256x256 tile (two slots of 64 KB; eight waves, each with four
    // block rows of 32 x 64 floats, 8 KB apiece).  Slot s splits into eight
    // 8 KB wave areas: waves 0-3 in its A part, waves 4-7 in its B part.  The
    // slot of slice nk-2 is free once every wave is past the K loop's last
    // barrier (in the step on slice nk-2, after every wave's reads of that
    // slice): C block row 1 of each wave tile is loaded into the wave's area
    // there now, straight from global memory (eight direct-to-LDS loads, lane
    // l covering columns 4*(l%16) .. +3 of row 4j + l/16), so that it arrives
    // during the last slice's MFMAs together with block row 0's register read.
    constexpr bool CDMA = early_c && S == 2 && Cfg::NW == 8 && Cfg::FM == 4 && Cfg::TN == 64 &&
                          Cfg::A_BYTES == 8 * 4096 && Cfg::B_BYTES == 8 * 4096;
    auto wave_area = [&](int slot) -> unsigned {
        return uwave < 4 ? lds0 + slot * Cfg::A_BYTES + uwave * 8192
                         : lds0 + S * Cfg::A_BYTES + slot * Cfg::B_BYTES + (uwave - 4) * 8192;
    };
    if constexpr (CDMA) {
        const int uwm = uwave / Cfg::WN, uwn = uwave % Cfg::WN;
        const unsigned dst = wave_area((nk - 2) % S);
        const float *row1 = C + (m0 + uwm * Cfg::TM + 32) * ldc + n0 + uwn * Cfg::TN;
        const unsigned voff = (unsigned)(((lane >> 4) * ldc + 4 * (lane & 15)) * 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) dma16(row1 + 4 * j * ldc, voff, dst + 1024 * j);
    }
    {   // last slice: everything is resident
        const int slot = (nk - 1) % S;
#pragma unroll
        for (int sub = 0; sub < NS; ++sub) {
            const int cur = sub & 1, nxt = cur ^ 1;
            if (sub + 1 < NS) read_frags(slot, sub + 1, fa[nxt], fb[nxt]);
            mfmas(fa[cur], fb[cur]);
        }
    }
    if constexpr (MASK) {
        // The K % BK tail, after the whole slices (k still ascends): each lane
        // loads its eight k of each operand fragment straight from global
        // memory, zero for k >= K, rows and columns clamped as for the slices.
        const int K = p.K, k0 = (s_begin + nk) * BK;
        if (last_split && k0 < K) {
            const uint16_t *Am = p.A + (long long)mb * p.sA;
            const uint16_t *Bm = p.B + (long long)mb * p.sB;
            long long ar[Cfg::FM], bc[Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) {
                const long long r = m0 + wm * Cfg::TM + 32 * i + lr;
                ar[i] = r < p.M ? r : p.M - 1;
            }
#pragma unroll
            for (int jj = 0; jj < Cfg::FN; ++jj) {
                const long long c = n0 + wn * Cfg::TN + 32 * jj + lr;
                bc[jj] = c < p.N ? c : p.N - 1;
            }
            // eight k from kq of a row (stride 1) or a column (stride ld)
            auto eight = [&](const uint16_t *x, long long stride, int kq) -> half8 {
                if (stride == 1 && kq + 7 < K) return __builtin_bit_cast(half8, *reinterpret_cast<const u32x4_g *>(x));
                uint16_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = kq + e < K ? x[e * stride] : (uint16_t)0;
                return __builtin_bit_cast(half8, h);
            };
#pragma unroll
            for (int sub = 0; sub < NS; ++sub) {
                if (k0 + 16 * sub >= K) break;
                const int kq = k0 + 16 * sub + 8 * lk;   // this lane's eight k
                half8 ta[Cfg::FM], tb[Cfg::FN];
#pragma unroll
                for (int i = 0; i < Cfg::FM; ++i)
                    ta[i] = A_KC ? eight(Am + ar[i] * lda + kq, 1, kq) : eight(Am + (long long)kq * lda + ar[i], lda, kq);
#pragma unroll
                for (int jj = 0; jj < Cfg::FN; ++jj)
                    tb[jj] = B_KC ? eight(Bm + bc[jj] * ldb + kq, 1, kq) : eight(Bm + (long long)kq * ldb + bc[jj], ldb, kq);
                mfmas(ta, tb);
            }
        }
    }

    if constexpr (SPLIT) {
        // K split: publish this workgroup's partial tile, count the arrival, and
        // let the last of the tile's nsplit workgroups add the partials in split
        // order -- a fixed order, so the bits do not depend on which finishes
        // last -- and run the epilogue.  No workgroup waits for another.
        //
        // Visibility across XCDs: the partials are written and read with
        // device-scope accesses (relaxed atomic stores and loads at agent scope,
        // which go through to the device's point of coherence instead of staying
        // in one XCD's L2), each wave waits for its stores to complete before the
        // barrier that precedes the arrival count, and the partials are read only
        // after the count has shown the workgroup to be last.  Nothing else
        // crosses workgroups, so no L2-wide write-back or invalidation is needed.
        //
        // Layout per (member, tile, split): per wave and accumulator register,
        // the 64 lanes' values side by side, so each lane reads back exactly the
        // entries it holds and every access is a full 256-byte row.
        constexpr int NR = Cfg::FM * Cfg::FN * 16;   // accumulator registers per lane
        const long long tile_id = ((long long)mb * p.tiles_m + tm) * p.tiles_n + tn;
        const long long tiles_all = (long long)gridDim.z * p.tiles_m * p.tiles_n;
        auto part = [&](int s) -> float * {
            return p.ws_part + ((s * tiles_all + tile_id) * Cfg::NW + wave) * NR * 64 + lane;
        };
        auto reg = [&](int r) -> float { return acc[r / 16 / Cfg::FN][(r / 16) % Cfg::FN][r % 16]; };
        auto set_reg = [&](int r, float v) { acc[r / 16 / Cfg::FN][(r / 16) % Cfg::FN][r % 16] = v; };
        {
            float *mine = part(sp);
#pragma unroll
            for (int r = 0; r < NR; ++r) __hip_atomic_store(mine + r * 64, reg(r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __shared__ unsigned arrived;
        __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores are complete
        __syncthreads();
        if (tid == 0)
            arrived = __hip_atomic_fetch_add(p.ws_count + tile_id, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrived != (unsigned)(nsplit - 1)) return;
        if (tid == 0) __hip_atomic_store(p.ws_count + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        auto load = [&](const float *q, int r) {
            return __hip_atomic_load(q + r * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        if (nsplit == 2) {
            // p0 + p1: IEEE addition is commutative, so either workgroup gets the same sum
            const float *other = part(1 - sp);
            float o[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) o[r] = load(other, r);
#pragma unroll
            for (int r = 0; r < NR; ++r) set_reg(r, reg(r) + o[r]);
        } else {
            // ((p0 + p1) + p2) + ...: every partial, this workgroup's included,
            // read back in split order
            const float *first = part(0);
#pragma unroll
            for (int r = 0; r < NR; ++r) set_reg(r, load(first, r));
            for (int s = 1; s < nsplit; ++s) {
                const float *ps = part(s);
                float o[NR];
#pragma unroll
                for (int r = 0; r < NR; ++r) o[r] = load(ps, r);
#pragma unroll
                for (int r = 0; r < NR; ++r) set_reg(r, reg(r) + o[r]);
            }
        }
    }

    auto quad = [&](int i, int jj, int g) -> f32x4_t {
        return {acc[i][jj][4 * g], acc[i][jj][4 * g + 1], acc[i][jj][4 * g + 2], acc[i][jj][4 * g + 3]};
    };
    if constexpr (!CROWS) {
        // Straight from the accumulators (beta == 0, or tiles at the edge of C,
        // whose masked reads need the registers that a read-ahead would take;
        // a separate instantiation keeps the beta == 0 kernels free of the
        // by-rows code and its registers).
        auto plain = [&](auto with_c) {
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) {
                const long long row = m0 + wm * Cfg::TM + 32 * i + lr;
#pragma unroll
                for (int jj = 0; jj < Cfg::FN; ++jj)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        store_row4<MASK, decltype(with_c)::value>(C, ldc, row, col_of(jj, g), quad(i, jj, g), alpha,
                                                                  beta, p.M, p.N);
            }
        };
        if (beta != 0.f)
            plain(std::true_type{});
        else
            plain(std::false_type{});
    } else {
        // By rows.  Straight from the accumulators a 16-byte access covers four
        // columns of each of 32 rows, 32 bytes per row and cache line; here
        // each wave passes a block row through a private LDS area (the ring is
        // free once every wave is past the barrier) and reads C and writes it
        // back in whole row segments of its tile (TN/4 lanes per row, 128 or
        // 256 contiguous bytes).  C is read one block row ahead: the reads of
        // block row i+1 are issued as soon as block row i is combined, before
        // its stores, so they are in flight while block row i is stored and
        // block row i+1 staged, and each wait covers one read latency instead
        // of one per block row behind the previous stores (the vector-memory
        // counter counts stores too).
        if constexpr (!early_c) read_row(0, cb);
        static_assert(Cfg::NW * 32 * PITCH * 4 <= S * Cfg::STAGE_BYTES, "staging area exceeds the ring");
        lds_barrier();
        if constexpr (CDMA) {
            // Staging in the wave's area of the last slice's slot: rows of 256
            // bytes, 16-byte chunk k of row r at chunk k ^ (r % 16), so that the
            // 16 lanes of a quarter-wave hit 16 different chunks when writing (one
            // column chunk of 16 rows) and reading back (the 16 chunks of a row).
            // Order of the four block rows: 0 from registers (read before the last
            // slice), 1 from LDS, 2 and 3 from registers, each read issued while
            // the block row before it is stored.
            const unsigned stage = wave_area((nk - 1) % S), cdat = wave_area((nk - 2) % S);
            auto stage_row = [&](int i) {
#pragma unroll
                for (int jj = 0; jj < Cfg::FN; ++jj)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int k = 8 * jj + 2 * g + lk;
                        *(lds_f32x4 *)(uintptr_t)(stage + lr * 256 + ((k ^ (lr & 15)) * 16)) = quad(i, jj, g);
                    }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            };
            auto staged = [&](int q) -> f32x4_t {
                const int r = 4 * q + (lane >> 4), c = lane & 15;
                return *(const lds_f32x4 *)(uintptr_t)(stage + r * 256 + ((c ^ (r & 15)) * 16));
            };
            auto store_row = [&](int i, const f32x4_t *v) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    store_row4_v(C, ldc, m0 + wm * Cfg::TM + 32 * i + 4 * q + (lane >> 4), n0 + wn * Cfg::TN + 4 * (lane & 15),
                                 v[q]);
            };
            f32x4_t v[8];
            stage_row(0);
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = fma_row4(staged(q), cb[q], alpha, beta);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            read_row(2, cb);
            store_row(0, v);
            // block row 1: its direct-to-LDS loads precede only the 8 reads and the
            // 8 stores just issued (the count is kept in order, stores included)
            stage_row(1);
            wait_vmcnt<16>();
#pragma unroll
            for (int q = 0; q < 8; ++q)
                v[q] = fma_row4(staged(q), *(const lds_f32x4 *)(uintptr_t)(cdat + (4 * q + (lane >> 4)) * 256 + (lane & 15) * 16),
                                alpha, beta);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            store_row(1, v);
            stage_row(2);
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = fma_row4(staged(q), cb[q], alpha, beta);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            read_row(3, cb);
            store_row(2, v);
            stage_row(3);
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = fma_row4(staged(q), cb[q], alpha, beta);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            store_row(3, v);
        } else {
            const unsigned stage = lds0 + wave * 32 * PITCH * 4;
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) {
#pragma unroll
                for (int jj = 0; jj < Cfg::FN; ++jj)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *(lds_f32x4 *)(uintptr_t)(stage + (lr * PITCH + 32 * jj + 8 * g + 4 * lk) * 4) = quad(i, jj, g);
                // a wave's LDS accesses complete in order; this orders the compiler's too
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                f32x4_t v[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int r = q * RPI + lane / LPR, c = 4 * (lane % LPR);
                    v[q] = fma_row4(*(const lds_f32x4 *)(uintptr_t)(stage + (r * PITCH + c) * 4), cb[q], alpha, beta);
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (i + 1 < Cfg::FM) read_row(i + 1, cb);
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int r = q * RPI + lane / LPR, c = 4 * (lane % LPR);
                    store_row4_v(C, ldc, m0 + wm * Cfg::TM + 32 * i + r, n0 + wn * Cfg::TN + c, v[q]);
                }
            }
        }
    }
}

using Hg128 = HgCfg<128, 128>;
using Hg64 = HgCfg<64, 64>;   // for grids that 128x128 tiles would leave under-filled

template <class Cfg, bool BF, bool TA, bool TB>
void launch_cfg_kernel(const HgemmArgs &a, bool whole, bool vec, dim3 grid, hipStream_t stream)
{
    const dim3 block(Cfg::NT);
    if (whole)
        hipLaunchKernelGGL((hgemm_mfma_kernel<Cfg, BF, false, true, TA, TB>), grid, block, 0, stream, a);
    else if (vec)
        hipLaunchKernelGGL((hgemm_mfma_kernel<Cfg, BF, true, true, TA, TB>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((hgemm_mfma_kernel<Cfg, BF, true, false, TA, TB>), grid, block, 0, stream, a);
}

template <class Cfg, bool BF>
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
    a.nsplit = 1; a.ws_count = nullptr; a.ws_part = nullptr;
    // 16-byte loads need 4-byte aligned row starts (column offsets are
    // multiples of eight halves)
    const bool vec = (q.lda % 2 == 0) && (q.ldb % 2 == 0) &&
                     (reinterpret_cast<uintptr_t>(q.A) % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(q.B) % 4 == 0) &&
                     (q.strideA % 2 == 0) && (q.strideB % 2 == 0);
    const bool whole = vec && q.M % Cfg::BM == 0 && q.N % Cfg::BN == 0 && q.K % Cfg::BK == 0;
    const dim3 grid(a.tiles_m * a.tiles_n, 1, q.batch);
    if (!q.transA && !q.transB)
        launch_cfg_kernel<Cfg, BF, false, false>(a, whole, vec, grid, stream);
    else if (!q.transA)
        launch_cfg_kernel<Cfg, BF, false, true>(a, whole, vec, grid, stream);
    else if (!q.transB)
        launch_cfg_kernel<Cfg, BF, true, false>(a, whole, vec, grid, stream);
    else
        launch_cfg_kernel<Cfg, BF, true, true>(a, whole, vec, grid, stream);
    return hipGetLastError();
}

}  // namespace

// 256x256 tile, 8 waves (2 x 4) of 128x64, BK = 64, two LDS slots of 64 KB.
using HgDma256 = HgDmaCfg<256, 256, 2, 2, 4, 64>;
// 128x128 tile, 8 waves (2 x 4) of 64x32, BK = 64, four slots of 32 KB: for
// grids that 256x256 tiles would leave under-filled.
using HgDma128 = HgDmaCfg<128, 128, 4, 2, 4, 64, true>;
// 64x128 tile, 8 waves (2 x 4) of 32x32, four slots of 24 KB: for grids that
// 128x128 tiles leave at most half filled.  Its A slice is 64 wide, so it takes
// only A stored M x K (B either way).
using HgDma64x128 = HgDmaCfg<64, 128, 4, 2, 4, 64>;

// Storage combinations a tile can take: an MN-contiguous slice needs rows of
// at least 16 chunks, i.e. BM >= 128 for A stored K x M and BN >= 128 for B
// stored K x N.
template <class Cfg>
constexpr bool dma_orientation_ok(bool tA, bool tB)
{
    return (!tA || Cfg::BM >= 128) && (tB || Cfg::BN >= 128);
}

template <class Cfg, bool BF, bool MASK, bool SPLIT, bool CROWS = false>
void launch_dma_ops(const HgemmArgs &a, dim3 grid, bool tA, bool tB, hipStream_t stream)
{
    const dim3 block(Cfg::NT);
    if (!tA && !tB) {
        if constexpr (dma_orientation_ok<Cfg>(false, false))
            hipLaunchKernelGGL((hgemm_dma_kernel<Cfg, BF, false, false, MASK, SPLIT, CROWS>), grid, block, 0, stream, a);
    } else if (!tA) {
        if constexpr (dma_orientation_ok<Cfg>(false, true))
            hipLaunchKernelGGL((hgemm_dma_kernel<Cfg, BF, false, true, MASK, SPLIT, CROWS>), grid, block, 0, stream, a);
    } else if (!tB) {
        if constexpr (dma_orientation_ok<Cfg>(true, false))
            hipLaunchKernelGGL((hgemm_dma_kernel<Cfg, BF, true, false, MASK, SPLIT, CROWS>), grid, block, 0, stream, a);
    } else {
        if constexpr (dma_orientation_ok<Cfg>(true, true))
            hipLaunchKernelGGL((hgemm_dma_kernel<Cfg, BF, true, true, MASK, SPLIT, CROWS>), grid, block, 0, stream, a);
    }
}

// Bytes of scratch a K split over nsplit workgroups per tile needs: the tile
// counters, then nsplit fp32 partial tiles per (member, tile).
template <class Cfg>
size_t split_bytes(const GemmProblem &q, int nsplit)
{
    const long long tiles = (long long)((q.M + Cfg::BM - 1) / Cfg::BM) * ((q.N + Cfg::BN - 1) / Cfg::BN) * q.batch;
    return kCounterBytes + (size_t)nsplit * tiles * Cfg::BM * Cfg::BN * sizeof(float);
}

// A K split over nsplit workgroups per tile applies: scratch given, one
// counter per (member, tile), and every split at least STAGES whole slices (the
// ring is filled before the first wait, so fewer would load past the split's
// range -- and, for the last split, past K).
template <class Cfg>
bool split_ok(const GemmProblem &q, int nsplit, const void *ws)
{
    const long long tiles = (long long)((q.M + Cfg::BM - 1) / Cfg::BM) * ((q.N + Cfg::BN - 1) / Cfg::BN) * q.batch;
    const bool straddle = (q.transA && q.M % 8 != 0) || (!q.transB && q.N % 8 != 0);
    const int slices = (q.K - (straddle ? 1 : 0)) / Cfg::BK;
    return ws != nullptr && tiles <= (long long)(kCounterBytes / sizeof(unsigned)) && slices / nsplit >= Cfg::STAGES;
}


// ws: scratch of split_bytes<Cfg>(q, nsplit) bytes when nsplit > 1.
template <class Cfg, bool BF>
hipError_t launch_dma(const GemmProblem &q, hipStream_t stream, int nsplit = 1, void *ws = nullptr)
{
    // a storage combination the tile cannot take launches nothing below: refuse
    // it here so that the caller sees an error instead of an unwritten C
    if (!dma_orientation_ok<Cfg>(q.transA, q.transB)) return hipErrorInvalidValue;
    if (nsplit > 1 && !split_ok<Cfg>(q, nsplit, ws)) return hipErrorInvalidValue;
    HgemmArgs a;
    a.M = q.M; a.N = q.N; a.K = q.K;
    a.alpha = q.alpha; a.beta = q.beta;
    a.A = static_cast<const uint16_t *>(q.A); a.lda = q.lda; a.sA = q.strideA;
    a.B = static_cast<const uint16_t *>(q.B); a.ldb = q.ldb; a.sB = q.strideB;
    a.C = q.C; a.ldc = q.ldc; a.sC = q.strideC;
    a.tiles_m = (q.M + Cfg::BM - 1) / Cfg::BM;
    a.tiles_n = (q.N + Cfg::BN - 1) / Cfg::BN;
    a.nsplit = nsplit;
    a.ws_count = static_cast<unsigned *>(ws);
    a.ws_part = ws ? reinterpret_cast<float *>(static_cast<char *>(ws) + kCounterBytes) : nullptr;
    const dim3 grid(a.tiles_m * a.tiles_n * nsplit, 1, q.batch);
    const bool whole = q.M % Cfg::BM == 0 && q.N % Cfg::BN == 0 && q.K % Cfg::BK == 0;
    const bool by_rows = q.beta != 0.f;   // epilogue by rows for whole tiles that read C
    if (nsplit > 1) {
        if constexpr (Cfg::SPLITS) {
            if (whole && by_rows)
                launch_dma_ops<Cfg, BF, false, true, true>(a, grid, q.transA, q.transB, stream);
            else if (whole)
                launch_dma_ops<Cfg, BF, false, true>(a, grid, q.transA, q.transB, stream);
            else
                launch_dma_ops<Cfg, BF, true, true>(a, grid, q.transA, q.transB, stream);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (whole && by_rows) {
        launch_dma_ops<Cfg, BF, false, false, true>(a, grid, q.transA, q.transB, stream);
    } else if (whole) {
        launch_dma_ops<Cfg, BF, false, false>(a, grid, q.transA, q.transB, stream);
    } else {
        launch_dma_ops<Cfg, BF, true, false>(a, grid, q.transA, q.transB, stream);
    }
    return hipGetLastError();
}

template <class Cfg>
constexpr bool same_shape(const TileShape16 &t)
{
    return Cfg::BM == t.bm && Cfg::BN == t.bn && Cfg::BK == t.bk && Cfg::STAGES == t.stages;
}
static_assert(same_shape<HgDma256>(kDma256) && same_shape<HgDma128>(kDma128) && same_shape<HgDma64x128>(kDma64x128),
              "plan16.h describes the tiles built here");

Problem16 planner_view(const GemmProblem &q)
{
    Problem16 v;
    v.M = q.M; v.N = q.N; v.K = q.K; v.batch = q.batch;
    v.transA = q.transA; v.transB = q.transB;
    v.lda = q.lda; v.ldb = q.ldb; v.strideA = q.strideA; v.strideB = q.strideB;
    v.A = reinterpret_cast<uintptr_t>(q.A); v.B = reinterpret_cast<uintptr_t>(q.B);
    return v;
}

template <bool BF>
hipError_t launch_gemm16(const GemmProblem &q, hipStream_t stream)
{
    const Problem16 v = planner_view(q);
    Plan16 plan = plan16(v, true);
    void *ws = nullptr;
    if (plan.nsplit > 1) {
        ws = q.scratch.acquire(split_bytes<HgDma128>(q, plan.nsplit), stream);
        if (ws == nullptr) plan = plan16(v, false);   // no scratch to be had: a plan that needs none
    }
    switch (plan.kernel) {
    case Kernel16::Dma256: return launch_dma<HgDma256, BF>(q, stream);
    case Kernel16::Dma128: return launch_dma<HgDma128, BF>(q, stream, plan.nsplit, ws);
    case Kernel16::Dma64x128: return launch_dma<HgDma64x128, BF>(q, stream);
    case Kernel16::Reg64: return launch_cfg<Hg64, BF>(q, stream);
    case Kernel16::Reg128: return launch_cfg<Hg128, BF>(q, stream);
    }
    return hipErrorInvalidValue;
}

size_t gemm16_scratch_bytes(const GemmProblem &q)
{
    if (q.M <= 0 || q.N <= 0 || q.batch <= 0 || q.K <= 0 || q.alpha == 0.f) return 0;
    const Plan16 plan = plan16(planner_view(q), true);
    return plan.nsplit > 1 ? split_bytes<HgDma128>(q, plan.nsplit) : 0;
}

hipError_t launch_hgemm(const GemmProblem &q, hipStream_t stream)
{
    return launch_gemm16<false>(q, stream);
}

hipError_t launch_bgemm(const GemmProblem &q, hipStream_t stream)
{
    return launch_gemm16<true>(q, stream);
}

}  // namespace mi355gemm
