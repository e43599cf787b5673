// scale_c.hip -- C <- beta*C for the GEMM cases with no product term (K == 0
// or alpha == 0).  With beta == 0, C is set to zero without being read, as in
// the BLAS reference semantics.
#include "gemm_internal.h"

namespace mi355gemm {
namespace {

__global__ __launch_bounds__(256) void scale_c_kernel(int M, int N, float beta, float *C, long long ldc,
                                                      long long sC)
{
    float *c = C + (long long)blockIdx.z * sC;
    const long long total = (long long)M * N;
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const long long i = e / N, j = e - i * N;
        float *dst = c + i * ldc + j;
        *dst = (beta != 0.f) ? beta * *dst : 0.f;
    }
}

}  // namespace

hipError_t launch_scale_c(const GemmProblem &q, hipStream_t stream)
{
    const long long total = (long long)q.M * q.N;
    long long blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(scale_c_kernel, dim3((unsigned)blocks, 1, q.batch), dim3(256), 0, stream, q.M, q.N,
                       q.beta, q.C, q.ldc, q.strideC);
    return hipGetLastError();
}

}  // namespace mi355gemm
