// gemm_internal.h -- kernel launchers shared between the C-ABI layer and the
// kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355gemm {

// One (possibly batched) row-major GEMM after argument checking.  Offsets are
// 64-bit; strides are in elements.
struct GemmProblem {
    int transA, transB;   // A stored K x M / B stored N x K
    int M, N, K, batch;
    float alpha, beta;
    const void *A;
    long long lda, strideA;
    const void *B;
    long long ldb, strideB;
    float *C;
    long long ldc, strideC;
};

// fp32 SGEMM on fp32 MFMA (K > 0, alpha != 0, M, N > 0; any transA/transB).
hipError_t launch_sgemm(const GemmProblem &p, hipStream_t stream);
// fp16-input, fp32-accumulate GEMM on fp16 MFMA (same preconditions).
hipError_t launch_hgemm(const GemmProblem &p, hipStream_t stream);
// bf16-input, fp32-accumulate GEMM on bf16 MFMA (same kernels and preconditions).
hipError_t launch_bgemm(const GemmProblem &p, hipStream_t stream);
// C <- beta*C (or 0 when beta == 0) for the K == 0 / alpha == 0 cases.
hipError_t launch_scale_c(const GemmProblem &p, hipStream_t stream);

}  // namespace mi355gemm
