// gemm_internal.h -- kernel launchers shared between the C-ABI layer and the
// kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355gemm {

// Scratch device memory a launcher may use for one call (the partial tiles and
// tile counters of a K split over workgroups).  get(ctx, bytes, stream) returns
// at least `bytes` bytes, 256-byte aligned, whose first kCounterBytes bytes are
// zero, or nullptr when no such memory can be had (the launcher then takes a
// plan that needs none).  Every kernel that uses the counters leaves them zero.
// The memory is not used by another call that can overlap this one.
constexpr size_t kCounterBytes = 256 * 1024;   // 65536 tile counters
struct Scratch {
    void *(*get)(void *ctx, size_t bytes, hipStream_t stream) = nullptr;
    void *ctx = nullptr;
    void *acquire(size_t bytes, hipStream_t stream) const { return get ? get(ctx, bytes, stream) : nullptr; }
};

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
    Scratch scratch;      // where a K split may keep its partial tiles
};

// fp32 SGEMM on fp32 MFMA (K > 0, alpha != 0, M, N > 0; any transA/transB).
hipError_t launch_sgemm(const GemmProblem &p, hipStream_t stream);
// fp16-input, fp32-accumulate GEMM on fp16 MFMA (same preconditions).
hipError_t launch_hgemm(const GemmProblem &p, hipStream_t stream);
// bf16-input, fp32-accumulate GEMM on bf16 MFMA (same kernels and preconditions).
hipError_t launch_bgemm(const GemmProblem &p, hipStream_t stream);
// Scratch bytes the fp16/bf16 launchers will ask p.scratch for (0: none).
size_t gemm16_scratch_bytes(const GemmProblem &p);
// C <- beta*C (or 0 when beta == 0) for the K == 0 / alpha == 0 cases.
hipError_t launch_scale_c(const GemmProblem &p, hipStream_t stream);

}  // namespace mi355gemm
