// gemm_probe.hip -- measurement probes behind include/mi355_gemm_probe.h.
//
// Not part of the GEMM path: two small kernels that measure the ceilings the
// GEMM kernels are measured against on this part.
//
//  * mfma_probe: nothing but MFMAs on operands held in registers.  Each wave
//    keeps 8 A and 8 B operand sets and 8 independent accumulators; with
//    `rotate` every MFMA takes a different (A, B) pair, so the operand bits
//    change from one MFMA to the next as they do in a GEMM on random data,
//    otherwise every MFMA reuses set 0.  The rate it reaches is the MFMA
//    throughput the chip sustains under its power limit for that data.
//  * hbm_probe: streams rows of a matrix from HBM into an LDS ring with the
//    same direct-to-LDS loads, waits and barrier as the GEMM main loop, in
//    segments of SEG bytes per row per step, 32 KB per stage, 3 stages: the
//    read rate an operand laid out that way can reach.
#include "mi355_gemm.h"
#include "mi355_gemm_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int SHAPE>
struct Mfma;
template <>
struct Mfma<GEMM_PROBE_F16_16x16x32> {
    typedef f32x4 Acc;
    static constexpr double kFlops = 16.0 * 16 * 32 * 2;
    __device__ static Acc step(i32x4 a, i32x4 b, Acc c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <>
struct Mfma<GEMM_PROBE_F16_32x32x16> {
    typedef f32x16 Acc;
    static constexpr double kFlops = 32.0 * 32 * 16 * 2;
    __device__ static Acc step(i32x4 a, i32x4 b, Acc c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <>
struct Mfma<GEMM_PROBE_BF16_16x16x32> {
    typedef f32x4 Acc;
    static constexpr double kFlops = 16.0 * 16 * 32 * 2;
    __device__ static Acc step(i32x4 a, i32x4 b, Acc c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
// 64 MFMAs per iteration per wave: accumulator j takes A set (j + t) mod 8
// and B set (3j + t) mod 8 at step t (all 64 pairs once), or set 0 and 0.
template <int SHAPE, bool ROT>
__global__ void __launch_bounds__(256) mfma_probe(const i32x4* ops, int64_t iters, float* sink)
{
    using M = Mfma<SHAPE>;
    const int lane = threadIdx.x & 63;
    i32x4 a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        a[s] = ops[s * 64 + lane];
        b[s] = ops[(8 + s) * 64 + lane];
    }
    typename M::Acc acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = typename M::Acc{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = M::step(a[ROT ? (j + t) % 8 : 0], b[ROT ? (3 * j + t) % 8 : 0], acc[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xf00);
}

constexpr int kStageBytes = 32768, kStages = 3, kWaves = 8;

// Workgroup w streams rows [w * RPW, (w + 1) * RPW) of the matrix, SEG bytes
// of each row per step.
template <int SEG>
__global__ void __launch_bounds__(kWaves * 64) hbm_probe(const char* A, int64_t row_bytes, float* sink)
{
    constexpr int RPW = kStageBytes / SEG;
    constexpr int IPW = kStageBytes / 1024 / kWaves;          // 1 KB loads per wave per step
    __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageBytes];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nsteps = (int)(row_bytes / SEG);
    int voff[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
        const int slot = (wave * IPW + j) * 64 + lane;
        voff[j] = (int)((slot / (SEG / 16)) * row_bytes) + (slot % (SEG / 16)) * 16;
    }
    const uint64_t base = (uint64_t)(A + (int64_t)blockIdx.x * RPW * row_bytes);
    const uint64_t extent = (uint64_t)RPW * row_bytes;
    auto issue = [&](int step, bool live) {
        const uint64_t addr = base + (uint64_t)step * SEG;
        const uint64_t rem = live ? extent - (uint64_t)step * SEG : 0;
        i32x4 rs;
        rs[0] = (int)(uint32_t)addr;
        rs[1] = (int)((uint32_t)(addr >> 32) & 0xffffu);
        rs[2] = (int)(uint32_t)(rem > 0xffffffffull ? 0xffffffffull : rem);
        rs[3] = 0x00020000;
        const uint32_t l0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(lds + (step % kStages) * kStageBytes) +
                            (uint32_t)(wave * IPW * 1024);
#pragma unroll
        for (int j = 0; j < IPW; ++j)
            asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :
                         : "s"(__builtin_amdgcn_readfirstlane(l0 + j * 1024)), "v"(voff[j]), "s"(rs)
                         : "memory", "m0");
    };
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s, s < nsteps);
    float acc = 0.f;
    for (int t = 0; t < nsteps; ++t) {
        wait_vm<IPW * (kStages - 2)>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        acc += ((const float*)(lds + (t % kStages) * kStageBytes))[threadIdx.x];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        issue(t + kStages - 1, t + kStages - 1 < nsteps);
    }
    wait_vm<0>();
    sink[blockIdx.x * kWaves * 64 + threadIdx.x] = acc;
}

template <int SHAPE>
hipError_t launch_mfma(bool rot, const void* ops, int64_t iters, int grid, float* sink, hipStream_t s)
{
    const i32x4* o = (const i32x4*)ops;
    void* args[] = {&o, &iters, &sink};
    const void* fn = rot ? (const void*)&mfma_probe<SHAPE, true> : (const void*)&mfma_probe<SHAPE, false>;
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, s);
}

template <int SEG>
hipError_t launch_hbm(const void* A, int64_t rows, int64_t row_bytes, float* sink, hipStream_t s)
{
    const char* a = (const char*)A;
    void* args[] = {&a, &row_bytes, &sink};
    return hipLaunchKernel((const void*)&hbm_probe<SEG>, dim3((unsigned)(rows / (kStageBytes / SEG))),
                           dim3(kWaves * 64), args, 0, s);
}

}  // namespace

extern "C" {

double gemm_probe_mfma_flops(int shape)
{
    switch (shape) {
    case GEMM_PROBE_F16_16x16x32: return Mfma<GEMM_PROBE_F16_16x16x32>::kFlops;
    case GEMM_PROBE_F16_32x32x16: return Mfma<GEMM_PROBE_F16_32x32x16>::kFlops;
    case GEMM_PROBE_BF16_16x16x32: return Mfma<GEMM_PROBE_BF16_16x16x32>::kFlops;
    default: return 0.0;
    }
}

int gemm_probe_mfma(int shape, int rotate, const void* operands, int64_t iters, int grid, float* sink, void* stream)
{
    if (gemm_probe_mfma_flops(shape) == 0.0 || iters < 0 || grid < 1 || grid > (1 << 20)) return GEMM_ERR_BAD_SHAPE;
    if (!operands || !sink) return GEMM_ERR_NULL_PTR;
    if (((uintptr_t)operands & 15) || ((uintptr_t)sink & 3)) return GEMM_ERR_MISALIGNED;
    hipError_t e;
    const bool rot = rotate != 0;
    hipStream_t s = (hipStream_t)stream;
    switch (shape) {
    case GEMM_PROBE_F16_16x16x32: e = launch_mfma<GEMM_PROBE_F16_16x16x32>(rot, operands, iters, grid, sink, s); break;
    case GEMM_PROBE_F16_32x32x16: e = launch_mfma<GEMM_PROBE_F16_32x32x16>(rot, operands, iters, grid, sink, s); break;
    default: e = launch_mfma<GEMM_PROBE_BF16_16x16x32>(rot, operands, iters, grid, sink, s); break;
    }
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int gemm_probe_hbm_read(const void* A, int64_t rows, int64_t row_bytes, int seg_bytes, float* sink, void* stream)
{
    if (seg_bytes != 128 && seg_bytes != 256 && seg_bytes != 512 && seg_bytes != 1024) return GEMM_ERR_BAD_SHAPE;
    const int64_t rpw = kStageBytes / seg_bytes;
    if (rows <= 0 || rows % rpw != 0 || rows / rpw > (1 << 24)) return GEMM_ERR_BAD_SHAPE;
    if (row_bytes < seg_bytes || row_bytes % seg_bytes != 0 || row_bytes * rpw >= ((int64_t)1 << 31))
        return GEMM_ERR_BAD_LD;
    if (!A || !sink) return GEMM_ERR_NULL_PTR;
    if (((uintptr_t)A & 15) || ((uintptr_t)sink & 3)) return GEMM_ERR_MISALIGNED;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (seg_bytes) {
    case 128: e = launch_hbm<128>(A, rows, row_bytes, sink, s); break;
    case 256: e = launch_hbm<256>(A, rows, row_bytes, sink, s); break;
    case 512: e = launch_hbm<512>(A, rows, row_bytes, sink, s); break;
    default: e = launch_hbm<1024>(A, rows, row_bytes, sink, s); break;
    }
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

}  // extern "C"
