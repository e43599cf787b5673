// gemm_api.cpp -- the exported C ABI (include/mi355gemm.h): argument checks,
// the BLAS-style quick returns, and dispatch to the kernel launchers.
// Argument checks run before any HIP call, so they work on a host with no GPU.
#include <limits.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/mi355gemm.h"
#include "gemm_internal.h"

namespace {

using mi355gemm::GemmProblem;

// Scratch for K splits, one buffer per (device, stream): calls on one stream
// run one after another, so they can share it, and calls on different streams
// never do.  A buffer is allocated (and its counters cleared on the stream) the
// first time a call on that stream needs more than it holds; the one it
// replaces may still be in use by work queued on the stream, so it is kept
// until the process ends.  Nothing is allocated while the stream is being
// captured into a graph: the call then gets no scratch and runs a plan that
// needs none.
constexpr size_t kScratchMin = 16u << 20;
constexpr size_t kScratchMax = 512u << 20;

struct StreamScratch {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_scratch_mutex;
std::map<std::pair<int, hipStream_t>, StreamScratch> g_scratch;
std::vector<void *> g_scratch_retired;

void *stream_scratch(void *, size_t bytes, hipStream_t stream)
{
    if (bytes > kScratchMax) return nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    StreamScratch &e = g_scratch[{dev, stream}];
    if (e.bytes >= bytes) return e.ptr;
    hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &status) != hipSuccess || status != hipStreamCaptureStatusNone) return nullptr;
    size_t want = bytes < kScratchMin ? kScratchMin : bytes;
    want = (want + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
    void *p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (hipMemsetAsync(p, 0, mi355gemm::kCounterBytes, stream) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(p);
        return nullptr;
    }
    if (e.ptr) g_scratch_retired.push_back(e.ptr);
    e.ptr = p;
    e.bytes = want;
    return p;
}

constexpr int kMaxGridZ = 65535;  // batch members per launch

bool misaligned(const void *p, uintptr_t align)
{
    return p != nullptr && (reinterpret_cast<uintptr_t>(p) % align) != 0;
}

// Overflow-checked (rows-1)*ld + cols, the element extent of a row-major matrix.
bool extent(long long rows, long long cols, long long ld, long long *out)
{
    if (rows == 0 || cols == 0) {
        *out = 0;
        return true;
    }
    if ((rows - 1) > 0 && ld > (LLONG_MAX - cols) / (rows - 1)) return false;
    *out = (rows - 1) * ld + cols;
    return true;
}

int check(const GemmProblem &p, size_t elem_in)
{
    if ((p.transA != 0 && p.transA != 1) || (p.transB != 0 && p.transB != 1)) return GEMM_ERR_OP;
    if (p.M < 0 || p.N < 0 || p.K < 0 || p.batch < 0) return GEMM_ERR_SIZE;
    // stored shapes: A is M x K (or K x M), B is K x N (or N x K)
    const long long a_rows = p.transA ? p.K : p.M, a_cols = p.transA ? p.M : p.K;
    const long long b_rows = p.transB ? p.N : p.K, b_cols = p.transB ? p.K : p.N;
    const long long N1 = p.N > 1 ? p.N : 1;
    if (p.lda < (a_cols > 1 ? a_cols : 1) || p.ldb < (b_cols > 1 ? b_cols : 1) || p.ldc < N1) return GEMM_ERR_LD;
    if (p.strideA < 0 || p.strideB < 0 || p.strideC < 0) return GEMM_ERR_LD;
    long long ea, eb, ec;
    if (!extent(a_rows, a_cols, p.lda, &ea) || !extent(b_rows, b_cols, p.ldb, &eb) || !extent(p.M, p.N, p.ldc, &ec))
        return GEMM_ERR_SIZE;
    if (p.batch > 1 && ec > 0 && p.strideC < ec) return GEMM_ERR_LD;
    if (p.batch > 1) {
        const long long nb = p.batch - 1;
        if ((p.strideA > 0 && nb > (LLONG_MAX - ea) / p.strideA) ||
            (p.strideB > 0 && nb > (LLONG_MAX - eb) / p.strideB) ||
            (p.strideC > 0 && nb > (LLONG_MAX - ec) / p.strideC))
            return GEMM_ERR_SIZE;
    }
    if (p.M == 0 || p.N == 0 || p.batch == 0) return GEMM_OK;
    // one workgroup per tile of at least 32 x 32: the grid must fit a launch
    if (((long long)p.M + 31) / 32 * (((long long)p.N + 31) / 32) > INT_MAX) return GEMM_ERR_SIZE;
    const bool reads_ab = p.K > 0 && p.alpha != 0.f;
    if (!p.C) return GEMM_ERR_NULL;
    if (reads_ab && (!p.A || !p.B)) return GEMM_ERR_NULL;
    if (misaligned(p.C, sizeof(float))) return GEMM_ERR_ALIGN;
    if (reads_ab && (misaligned(p.A, elem_in) || misaligned(p.B, elem_in))) return GEMM_ERR_ALIGN;
    return GEMM_OK;
}

template <class Launch>
int run(GemmProblem p, size_t elem_in, hipStream_t stream, Launch launch)
{
    const int rc = check(p, elem_in);
    if (rc != GEMM_OK) return rc;
    if (p.M == 0 || p.N == 0 || p.batch == 0) return GEMM_OK;
    const bool product = p.K > 0 && p.alpha != 0.f;
    const int total = p.batch;
    for (int b0 = 0; b0 < total; b0 += kMaxGridZ) {
        GemmProblem q = p;
        q.batch = (total - b0) < kMaxGridZ ? (total - b0) : kMaxGridZ;
        q.C = p.C + (long long)b0 * p.strideC;
        if (product) {
            q.A = static_cast<const char *>(p.A) + (long long)b0 * p.strideA * (long long)elem_in;
            q.B = static_cast<const char *>(p.B) + (long long)b0 * p.strideB * (long long)elem_in;
        }
        const hipError_t e = product ? launch(q, stream) : mi355gemm::launch_scale_c(q, stream);
        if (e != hipSuccess) return GEMM_ERR_LAUNCH;
    }
    return GEMM_OK;
}

// ---- scratch of the entry point that allocates nothing
//
// One file-scope array per GPU holds the K split's tile counters and partial
// tiles for gemm_f16_f32acc_noalloc.  Its size covers every K split the
// planner makes (at most 128 workgroups of 128 x 128 fp32 partial tiles, see
// plan16.h), so no call is refused today; the check stays for any plan that
// would need more.  In host code `noalloc_scratch` names a host-side stand-in:
// the device address comes from hipGetSymbolAddress, once per device, and only
// that address is passed to kernels.
constexpr size_t kNoallocScratchBytes = mi355gemm::kCounterBytes + (size_t)128 * 128 * 128 * sizeof(float);
__device__ __align__(256) unsigned char noalloc_scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mutex;
void *g_noalloc_ptr[kMaxDevices];

// The device address of this GPU's array (the current device), looked up on
// the first call on the device.  The array is zero when the library is loaded
// and every kernel leaves its counters zero; the first call also clears them on
// its stream unless that stream is being captured into a graph.
void *noalloc_scratch_setup(hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_noalloc_mutex);
    if (g_noalloc_ptr[dev]) return g_noalloc_ptr[dev];
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &status) == hipSuccess && status == hipStreamCaptureStatusNone) {
        if (hipMemsetAsync(ptr, 0, mi355gemm::kCounterBytes, stream) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
    }
    g_noalloc_ptr[dev] = ptr;
    return ptr;
}

void *noalloc_scratch_get(void *ctx, size_t bytes, hipStream_t)
{
    return bytes <= kNoallocScratchBytes ? ctx : nullptr;
}

GemmProblem make(int tA, int tB, int M, int N, int K, float alpha, const void *A, int lda, long long sA,
                 const void *B, int ldb, long long sB, float beta, float *C, int ldc, long long sC, int batch)
{
    GemmProblem p;
    p.scratch.get = stream_scratch;
    p.transA = tA; p.transB = tB;
    p.M = M; p.N = N; p.K = K; p.batch = batch;
    p.alpha = alpha; p.beta = beta;
    p.A = A; p.lda = lda; p.strideA = sA;
    p.B = B; p.ldb = ldb; p.strideB = sB;
    p.C = C; p.ldc = ldc; p.strideC = sC;
    return p;
}

}  // namespace

extern "C" {

int gemm_f32_ex(int transA, int transB, int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                int ldb, float beta, float *C, int ldc, hipStream_t stream)
{
    return run(make(transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1), sizeof(float),
               stream, mi355gemm::launch_sgemm);
}

int gemm_f16_f32acc_ex(int transA, int transB, int M, int N, int K, float alpha, const uint16_t *A, int lda,
                       const uint16_t *B, int ldb, float beta, float *C, int ldc, hipStream_t stream)
{
    return run(make(transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1), sizeof(uint16_t),
               stream, mi355gemm::launch_hgemm);
}

int gemm_batched_f16_f32acc_ex(int transA, int transB, int M, int N, int K, float alpha, const uint16_t *A, int lda,
                               long long strideA, const uint16_t *B, int ldb, long long strideB, float beta, float *C,
                               int ldc, long long strideC, int batch_count, hipStream_t stream)
{
    return run(make(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC,
                    batch_count),
               sizeof(uint16_t), stream, mi355gemm::launch_hgemm);
}

int gemm_bf16_f32acc_ex(int transA, int transB, int M, int N, int K, float alpha, const uint16_t *A, int lda,
                        const uint16_t *B, int ldb, float beta, float *C, int ldc, hipStream_t stream)
{
    return run(make(transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1), sizeof(uint16_t),
               stream, mi355gemm::launch_bgemm);
}

int gemm_batched_bf16_f32acc_ex(int transA, int transB, int M, int N, int K, float alpha, const uint16_t *A,
                                int lda, long long strideA, const uint16_t *B, int ldb, long long strideB,
                                float beta, float *C, int ldc, long long strideC, int batch_count,
                                hipStream_t stream)
{
    return run(make(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC,
                    batch_count),
               sizeof(uint16_t), stream, mi355gemm::launch_bgemm);
}

int gemm_f32(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb, float beta,
             float *C, int ldc, hipStream_t stream)
{
    return gemm_f32_ex(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16_f32acc(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B, int ldb,
                    float beta, float *C, int ldc, hipStream_t stream)
{
    return gemm_f16_f32acc_ex(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_batched_f16_f32acc(int M, int N, int K, float alpha, const uint16_t *A, int lda, long long strideA,
                            const uint16_t *B, int ldb, long long strideB, float beta, float *C, int ldc,
                            long long strideC, int batch_count, hipStream_t stream)
{
    return gemm_batched_f16_f32acc_ex(0, 0, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC,
                                      batch_count, stream);
}

int gemm_f16_f32acc_noalloc(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
                            int ldb, float beta, float *C, int ldc, hipStream_t stream)
{
    GemmProblem p = make(0, 0, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1);
    const int rc = check(p, sizeof(uint16_t));
    if (rc != GEMM_OK) return rc;
    if (M == 0 || N == 0) return GEMM_OK;
    if (mi355gemm::gemm16_scratch_bytes(p) > kNoallocScratchBytes) return GEMM_ERR_SCRATCH;
    void *ptr = noalloc_scratch_setup(stream);
    if (ptr == nullptr) return GEMM_ERR_LAUNCH;
    p.scratch.get = noalloc_scratch_get;
    p.scratch.ctx = ptr;
    return run(p, sizeof(uint16_t), stream, mi355gemm::launch_hgemm);
}

int gemm_bf16_f32acc(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B, int ldb,
                     float beta, float *C, int ldc, hipStream_t stream)
{
    return gemm_bf16_f32acc_ex(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_batched_bf16_f32acc(int M, int N, int K, float alpha, const uint16_t *A, int lda, long long strideA,
                             const uint16_t *B, int ldb, long long strideB, float beta, float *C, int ldc,
                             long long strideC, int batch_count, hipStream_t stream)
{
    return gemm_batched_bf16_f32acc_ex(0, 0, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                                       strideC, batch_count, stream);
}

const char *gemm_status_string(int status)
{
    switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_SIZE: return "invalid size: M, N, K or batch_count negative, or an extent overflows";
    case GEMM_ERR_LD: return "invalid leading dimension or batch stride";
    case GEMM_ERR_NULL: return "NULL pointer for an operand the call reads or writes";
    case GEMM_ERR_ALIGN: return "pointer not aligned to its element size";
    case GEMM_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case GEMM_ERR_OP: return "transpose flag is neither 0 nor 1";
    case GEMM_ERR_SCRATCH: return "the call needs more scratch than the static buffer of the no-allocation entry point holds";
    default: return "unknown status";
    }
}

}  // extern "C"
