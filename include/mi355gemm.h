/*
 * mi355gemm.h -- row-major GEMM on one AMD Instinct MI355X (gfx950), C ABI.
 *
 * Every entry point computes, for row-major matrices,
 *
 *     C <- alpha * A * B + beta * C,      A: M x K,  B: K x N,  C: M x N
 *
 * which is the general matrix multiply C = alpha*op(A)op(B) + beta*C of the
 * MindNotes 'GEMM' page (section "core problem and arithmetic
 * characteristics") with op the identity.  That page's "cuBLAS engineering
 * interface" sections fix the other parts of the interface used here: a
 * leading dimension is the distance in elements between the starts of two
 * consecutive rows and may exceed the logical width (section "Leading
 * Dimension (lda, ldb, ldc)"); a strided batch is a set of same-shape GEMMs
 * placed a fixed element stride apart and run by one call, and mixed precision
 * means fp16 inputs with fp32 accumulation (section "Batched execution and
 * mixed precision").  Unlike cuBLAS the storage is row-major, there is no
 * handle, and alpha/beta are host values passed by value.
 *
 * Layout: element (i,k) of A is A[i*lda + k], (k,j) of B is B[k*ldb + j],
 * (i,j) of C is C[i*ldc + j].  Batched member b starts at A + b*strideA,
 * B + b*strideB, C + b*strideC (strides in elements).
 *
 * Ownership: A, B and C are device pointers owned by the caller.  The library
 * allocates no memory, keeps no state besides its loaded kernels, and never
 * synchronises: each call enqueues its kernels on `stream` (0 = the null
 * stream) and returns.  C must not overlap A or B, and batched C members must
 * not overlap one another.
 *
 * Semantics the pages leave open, taken from the BLAS reference:
 *   - beta == 0: C is written without being read (it may hold NaN);
 *   - K == 0 or alpha == 0: C <- beta*C (C <- 0 when beta == 0 too); A and B
 *     are not read;
 *   - M == 0, N == 0 or batch_count == 0: nothing is done.
 *
 * Errors: every entry point returns an int status.  Arguments are checked
 * before any HIP call; on an error nothing is enqueued.  Codes 0 to -4 are the
 * BLAS-style set (size, leading dimension or stride, NULL pointer, launch
 * refused); -5 and -6 report the two conditions that set has no code for (an
 * element-misaligned pointer, a transpose flag other than 0 or 1).
 */
#ifndef MI355GEMM_H
#define MI355GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t; /* the HIP runtime's stream handle */

enum {
    GEMM_OK = 0,
    GEMM_ERR_SIZE = -1,      /* M, N, K or batch_count negative, an extent overflows 64 bits, or
                                ceil(M/32)*ceil(N/32) exceeds INT_MAX (one launch's grid) */
    GEMM_ERR_LD = -2,        /* lda < max(1,K), ldb < max(1,N) (with transA: lda < max(1,M); with
                                transB: ldb < max(1,K)), ldc < max(1,N), negative stride, or
                                strideC smaller than one C member when batch_count > 1 */
    GEMM_ERR_NULL = -3,      /* NULL pointer for an operand that the call would read or write */
    GEMM_ERR_LAUNCH = -4,    /* the HIP runtime refused a kernel launch (hipGetLastError) */
    GEMM_ERR_ALIGN = -5,     /* pointer not aligned to its element size */
    GEMM_ERR_OP = -6,        /* transA or transB is neither 0 nor 1 */
    GEMM_ERR_SCRATCH = -7    /* gemm_f16_f32acc_noalloc only: the call needs more scratch than
                                the library's static buffer holds */
};

/*
 * gemm_f32 -- SGEMM: fp32 A, B, C; fp32 multiply-add.
 *   M, N, K    : logical sizes (>= 0).
 *   alpha, beta: fp32 scalars.
 *   A, lda     : device fp32, M x K row-major, lda >= max(1,K).
 *   B, ldb     : device fp32, K x N row-major, ldb >= max(1,N).
 *   C, ldc     : device fp32, M x N row-major, ldc >= max(1,N); read only when beta != 0.
 *   stream     : HIP stream the kernels are enqueued on.
 * Results agree with the fp64 definition to a normalized error
 * |C - ref| / (|alpha| sum_k |a_ik||b_kj| + |beta||c_ij|) <= 1e-5 and are
 * bit-identical from call to call for the same arguments.
 */
int gemm_f32(int M, int N, int K, float alpha,
             const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, hipStream_t stream);

/*
 * gemm_f16_f32acc -- HGEMM: A and B hold IEEE binary16 values (bit patterns in
 * uint16_t), products are formed exactly and accumulated in fp32; alpha, beta
 * and C are fp32.  Arguments as for gemm_f32.
 */
int gemm_f16_f32acc(int M, int N, int K, float alpha,
                    const uint16_t *A, int lda, const uint16_t *B, int ldb,
                    float beta, float *C, int ldc, hipStream_t stream);

/*
 * gemm_batched_f16_f32acc -- batch_count independent HGEMMs of one shape.
 *   strideA, strideB, strideC: element distance between consecutive members
 *   (>= 0; strideA/strideB may be 0 to reuse one operand; strideC must be at
 *   least (M-1)*ldc + N when batch_count > 1).
 * Other arguments as for gemm_f16_f32acc; batch_count >= 0.
 */
int gemm_batched_f16_f32acc(int M, int N, int K, float alpha,
                            const uint16_t *A, int lda, long long strideA,
                            const uint16_t *B, int ldb, long long strideB,
                            float beta, float *C, int ldc, long long strideC,
                            int batch_count, hipStream_t stream);

/*
 * The _ex forms compute C <- alpha*op(A)*op(B) + beta*C, op(X) = X or X^T, the
 * general form of the MindNotes page's definition (section "core problem and
 * arithmetic characteristics").  op(A) is M x K and op(B) is K x N:
 *   transA = 0: A is stored M x K, element (i,k) at A[i*lda + k], lda >= max(1,K);
 *   transA = 1: A is stored K x M, element (i,k) at A[k*lda + i], lda >= max(1,M);
 *   transB = 0: B is stored K x N, element (k,j) at B[k*ldb + j], ldb >= max(1,N);
 *   transB = 1: B is stored N x K, element (k,j) at B[j*ldb + k], ldb >= max(1,K).
 * C is always M x N row-major.  Flags other than 0 or 1 return GEMM_ERR_OP.
 * Everything else is as for the entry points above (which are the _ex forms
 * with transA = transB = 0).
 */
int gemm_f32_ex(int transA, int transB, int M, int N, int K, float alpha,
                const float *A, int lda, const float *B, int ldb,
                float beta, float *C, int ldc, hipStream_t stream);

int gemm_f16_f32acc_ex(int transA, int transB, int M, int N, int K, float alpha,
                       const uint16_t *A, int lda, const uint16_t *B, int ldb,
                       float beta, float *C, int ldc, hipStream_t stream);

int gemm_batched_f16_f32acc_ex(int transA, int transB, int M, int N, int K, float alpha,
                               const uint16_t *A, int lda, long long strideA,
                               const uint16_t *B, int ldb, long long strideB,
                               float beta, float *C, int ldc, long long strideC,
                               int batch_count, hipStream_t stream);

/*
 * bfloat16 inputs.  The MindNotes page's mixed-precision interface (section
 * "Batched execution and mixed precision") takes either fp16 or bf16 inputs
 * with fp32 accumulation.  These four entry points are the bf16 forms of
 * gemm_f16_f32acc, gemm_batched_f16_f32acc, gemm_f16_f32acc_ex and
 * gemm_batched_f16_f32acc_ex, in that order: A and B hold bfloat16 values (the
 * upper 16 bits of an IEEE binary32, as uint16_t bit patterns), products are
 * formed exactly and accumulated in fp32; alpha, beta and C are fp32.
 * Arguments, layout, ownership, status codes and the accuracy statement are
 * as for the fp16 forms.
 */
int gemm_bf16_f32acc(int M, int N, int K, float alpha,
                     const uint16_t *A, int lda, const uint16_t *B, int ldb,
                     float beta, float *C, int ldc, hipStream_t stream);

int gemm_batched_bf16_f32acc(int M, int N, int K, float alpha,
                             const uint16_t *A, int lda, long long strideA,
                             const uint16_t *B, int ldb, long long strideB,
                             float beta, float *C, int ldc, long long strideC,
                             int batch_count, hipStream_t stream);

int gemm_bf16_f32acc_ex(int transA, int transB, int M, int N, int K, float alpha,
                        const uint16_t *A, int lda, const uint16_t *B, int ldb,
                        float beta, float *C, int ldc, hipStream_t stream);

int gemm_batched_bf16_f32acc_ex(int transA, int transB, int M, int N, int K, float alpha,
                                const uint16_t *A, int lda, long long strideA,
                                const uint16_t *B, int ldb, long long strideB,
                                float beta, float *C, int ldc, long long strideC,
                                int batch_count, hipStream_t stream);

/*
 * gemm_f16_f32acc_noalloc -- gemm_f16_f32acc for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and status codes, plus
 * GEMM_ERR_SCRATCH.  Where gemm_f16_f32acc splits a tile's K range over several
 * workgroups it keeps the partial tiles and counters in scratch that the
 * library allocates per (device, stream) on first need; this form uses instead
 * one static device buffer per GPU, 8.25 MiB (256 KiB of tile counters and 128
 * fp32 partial tiles of 128 x 128), which covers every split the library makes,
 * and calls no allocating routine.  That buffer is shared by every call of this
 * entry point on the GPU and keeps the last call's contents: calls that overlap
 * on one GPU (different streams, or graphs replayed concurrently) race and must
 * not be made.  A call that would need more scratch returns GEMM_ERR_SCRATCH
 * and enqueues nothing.
 */
int gemm_f16_f32acc_noalloc(int M, int N, int K, float alpha,
                            const uint16_t *A, int lda, const uint16_t *B, int ldb,
                            float beta, float *C, int ldc, hipStream_t stream);

/* gemm_status_string -- a static, NUL-terminated description of a status code. */
const char *gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MI355GEMM_H */
