// epilogue.h -- the alpha/beta epilogue shared by the GEMM kernels.
//
// The kernels issue their MFMAs with the B fragment as the first operand and
// the A fragment as the second, so a 32x32 accumulator block holds the
// transposed product: register r of lane l is C[row l%32][col 8*(r/4) +
// 4*(l/32) + r%4] of the block.  Registers 4g..4g+3 are therefore four
// consecutive columns of one row, written with one 16-byte store.  Multi-dword
// global accesses need only dword alignment on CDNA, so the 16-byte store is
// used for any fp32 C (every float is 4-byte aligned).
#pragma once

#include <hip/hip_runtime.h>

namespace mi355gemm {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
// four consecutive floats in global memory at dword (not 16-byte) alignment
typedef float f32x4_g __attribute__((ext_vector_type(4), aligned(4)));

// C[row][col..col+3] = alpha*acc + beta*C (beta term only when WITH_C), as
// fma(beta, c, alpha*acc) written out: left to the compiler, the contraction
// of alpha*acc + beta*c may come out either way round in different kernels,
// and the storage orientations of one product must give the same bits.
// MASK: rows >= M and columns >= N are skipped (a row whose four columns are
// all inside is still written with one 16-byte access).
template <bool MASK, bool WITH_C>
__device__ __forceinline__ void store_row4(float *C, long long ldc, long long row, long long col,
                                           f32x4_t acc, float alpha, float beta, int M, int N)
{
    if (MASK && row >= M) return;
    float *dst = C + row * ldc + col;
    if (!MASK || col + 3 < N) {
        f32x4_t v = alpha * acc;
        if (WITH_C) {
            const f32x4_t c = *reinterpret_cast<const f32x4_g *>(dst);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(beta, c[e], v[e]);
        }
        *reinterpret_cast<f32x4_g *>(dst) = v;
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (MASK && col + e >= N) break;
        float v = alpha * acc[e];
        if (WITH_C) v = __builtin_fmaf(beta, dst[e], v);
        dst[e] = v;
    }
}

// The beta term split from the store, so that a kernel can read C ahead of
// the stores that use it: four consecutive floats of C at (row, col..col+3),
// with MASK rows >= M and columns >= N reading as zero (they are never stored).
template <bool MASK>
__device__ __forceinline__ f32x4_t load_row4(const float *C, long long ldc, long long row, long long col, int M, int N)
{
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
    if (MASK && row >= M) return c;
    const float *src = C + row * ldc + col;
    if (!MASK || col + 3 < N) return *reinterpret_cast<const f32x4_g *>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (col + e < N) c[e] = src[e];
    return c;
}

// For whole tiles that read C ahead of the stores: alpha*acc + beta*c for c
// read by load_row4, the same fma(beta, c, alpha*acc) as store_row4, so either
// path gives the same bits; and the 16-byte store of the result.
__device__ __forceinline__ f32x4_t fma_row4(f32x4_t acc, f32x4_t c, float alpha, float beta)
{
    f32x4_t v = alpha * acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(beta, c[e], v[e]);
    return v;
}
__device__ __forceinline__ void store_row4_v(float *C, long long ldc, long long row, long long col, f32x4_t v)
{
    *reinterpret_cast<f32x4_g *>(C + row * ldc + col) = v;
}

}  // namespace mi355gemm
