// gemm_noalloc.hip -- the entry point that allocates nothing.
//
// gemm_run_noalloc is gemm_run_ws with the workspace taken from a fixed
// array in device memory that the library owns (`scratch`, kScratchBytes),
// for callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc).  The stream-K and split-k configs
// are the only ones that use a workspace: the stream-K arrival counters and
// partial tiles, the split-k partial tiles, live in it.  Each GPU holds its own copy of the array, from the library's first
// use on that GPU until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory; its
// device address on a GPU comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is ever passed to
// a kernel.
#include "mi355_gemm.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "gemm_plan.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // GEMM_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == GEMM_NOALLOC_SCRATCH_BYTES, "header and library disagree");

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];

// Device address of `scratch` on device `dev` (looked up on first use).
int scratch_on(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_HIP;
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return GEMM_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return GEMM_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return GEMM_ERR_HIP;
        if (e != hipSuccess || !p) return GEMM_ERR_HIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return GEMM_OK;
}

// Zero n 16-byte words (the arrival counters) on the caller's stream: a
// kernel rather than hipMemsetAsync, so the call can also be captured.
__global__ void __launch_bounds__(256) zero_words(uint4* p, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" int gemm_run_noalloc(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                                int dtype, const void* A, const void* B, void* C, int64_t lda, int64_t ldb,
                                int64_t ldc, void* stream, int config_id)
{
    int config = -1;
    uint64_t need = 0, count_bytes = 0;
    const int st = mg::plan_ws(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, kScratchBytes,
                               config_id < 0 ? -1 : config_id, &config, &need, &count_bytes);
    if (st != GEMM_OK) return st;
    if (need > kScratchBytes) return GEMM_ERR_SCRATCH_LIMIT;
    if (need == 0)   // nothing launched, or a config without a workspace
        return gemm_run_ws(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, nullptr, 0, stream,
                           config);
    int dev = -1;
    const hipError_t de = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (de != hipSuccess) return GEMM_ERR_HIP;
    void* ws = nullptr;
    const int sst = scratch_on(dev, &ws);
    if (sst != GEMM_OK) return sst;
    // The counters must be zero at launch.  Every completed call leaves them
    // so; clearing them here does not depend on that.
    int words = (int)(count_bytes / 16);
    uint4* counters = (uint4*)ws;
    void* args[] = {&counters, &words};
    if (words > 0 && hipLaunchKernel((const void*)&zero_words, dim3((words + 255) / 256), dim3(256), args, 0,
                                     (hipStream_t)stream) != hipSuccess)
        return GEMM_ERR_HIP;
    return gemm_run_ws(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, ws, kScratchBytes,
                       stream, config);
}
