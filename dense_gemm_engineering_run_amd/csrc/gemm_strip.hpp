// gemm_strip.hpp -- the last few columns (or rows) of C, when they are all
// that lies past a multiple of the tile.
//
// A tiled kernel spends a whole tile column on a last column of C that is 1
// to 4 wide: the same MFMAs and operand traffic as a full column of tiles,
// and on a grid just past a whole number of waves (fp32 4095 x 2049 x 1028 on
// 128 x 128 tiles: 544 tiles for 512 workgroup slots) a partial wave more.
// The launch path therefore runs the tiled kernel on the full tiles only and
// this kernel on the strip: C[i][s0 + j] = sum_k L[i][k] * S[j][k] for the r
// <= kStripMax rows j of the short operand S (B's last rows for a column
// strip, A's for a row strip) and every row i of the long operand L (A, or B
// for a row strip).  Its time is that of reading L once.
//
// Workgroup: 16 rows of L, 256 threads.  K is taken in chunks of KC = 512 E
// elements (E per 16 bytes; 2048 fp32 or 4096 16-bit values, one chunk for
// most K): each thread has all 32 of its 16-byte loads of L for the chunk in
// flight, while the chunk of S (r x KC, as fp32) is staged
// in LDS; then fp32 FMAs in ascending k per thread and a fixed reduction
// order, so results are deterministic.
//  * L k-contiguous: 16 threads per row, thread l takes k = (l + 16 c) E ..
//    + E - 1; the 16 partial sums of a row are added by lane shuffles.
//  * L row-contiguous (element i of row k at k * ld + i): a 16-byte load
//    holds E consecutive rows at one k; thread t takes row group t mod (16/E)
//    and k = t / (16/E) + 16 E c; the partial sums go through LDS and are
//    added in k order.
// Elements k >= K are zeroed in both operands (the ld padding of L may hold
// anything, NaN included).  Operands are 16-byte aligned with ld * element
// size a multiple of 16 (the non-scalar configs' condition), so every 16-byte
// load of an element below K stays inside its row's padding.
#pragma once

#include "gemm_kernel.hpp"

namespace mg {

template <In TI>
__device__ __forceinline__ float strip_elem(const char* base, int64_t idx)
{
    if constexpr (TI == In::F32) {
        return ((const float*)base)[idx];
    } else if constexpr (TI == In::F16) {
        return (float)((const _Float16*)base)[idx];
    } else {
        const uint32_t u = ((const uint16_t*)base)[idx];
        return __uint_as_float(u << 16);
    }
}

// Element e of a 16-byte chunk as fp32.
template <In TI>
__device__ __forceinline__ float chunk_elem(const i32x4& v, int e)
{
    if constexpr (TI == In::F32) {
        return __int_as_float(v[e]);
    } else {
        const uint32_t w = (uint32_t)v[e / 2];
        const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xffffu);
        if constexpr (TI == In::F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
        else return __uint_as_float(h << 16);
    }
}

template <In TI, Out TO, bool LK, bool SK, bool ROWS>
__global__ void __launch_bounds__(256)
gemm_strip_kernel(Params p)
{
    constexpr int ES = TI == In::F32 ? 4 : 2, E = 16 / ES;
    constexpr int RL = 16, NT = 256, NC = 32, KC = NC * 16 * E;   // rows per workgroup, loads per thread per chunk
    __shared__ float s_lds[kStripMax][KC];
    __shared__ float red[LK ? 1 : (NT / (RL / E))][RL][kStripMax];

    select_batch(p);
    const char* L = ROWS ? p.B : p.A;
    const int64_t ldl = ROWS ? p.ldb : p.lda;
    const int nl = ROWS ? p.N : p.M;
    const char* S = ROWS ? p.A : p.B;
    const int64_t ldsh = ROWS ? p.lda : p.ldb;
    const int s0 = p.strip0, r = (ROWS ? p.M : p.N) - s0;
    const int tid = threadIdx.x, i0 = blockIdx.x * RL;

    float acc[LK ? 1 : E][kStripMax];
#pragma unroll
    for (int e = 0; e < (LK ? 1 : E); ++e)
#pragma unroll
        for (int j = 0; j < kStripMax; ++j) acc[e][j] = 0.f;

    // This thread's part of a chunk of L.
    constexpr int GR = RL / E;                 // row groups per k (row-contiguous L)
    const int row = LK ? i0 + tid / 16 : i0 + (tid % GR) * E;
    const int kl = LK ? tid % 16 : tid / GR;
    const bool row_ok = row < nl;

    for (int k0 = 0; k0 < p.K; k0 += KC) {
        i32x4 v[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int k = LK ? k0 + (kl + 16 * c) * E : k0 + kl + 16 * E * c;
            v[c] = i32x4{0, 0, 0, 0};
            if (row_ok && k < p.K) {
                const int64_t idx = LK ? (int64_t)row * ldl + k : (int64_t)k * ldl + row;
                v[c] = *(const i32x4*)(L + idx * ES);
            }
        }
        // The chunk of S, all loads in flight before the LDS writes; element q
        // of the chunk is (j, kk) with the contiguous index fastest across
        // threads (kk for k-contiguous S, j otherwise).
        constexpr int QN = kStripMax * KC / NT;
        float sv[QN];
#pragma unroll
        for (int u = 0; u < QN; ++u) {
            const int q = tid + u * NT;
            const int j = SK ? q / KC : q % kStripMax, kk = SK ? q % KC : q / kStripMax, k = k0 + kk;
            sv[u] = 0.f;
            if (j < r && k < p.K)
                sv[u] = strip_elem<TI>(S, SK ? (int64_t)(s0 + j) * ldsh + k : (int64_t)k * ldsh + s0 + j);
        }
        __syncthreads();   // the previous chunk's S is no longer read
#pragma unroll
        for (int u = 0; u < QN; ++u) {
            const int q = tid + u * NT;
            const int j = SK ? q / KC : q % kStripMax, kk = SK ? q % KC : q / kStripMax;
            s_lds[j][kk] = sv[u];
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if constexpr (LK) {
                const int kk = (kl + 16 * c) * E;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = k0 + kk + e < p.K ? chunk_elem<TI>(v[c], e) : 0.f;
#pragma unroll
                    for (int j = 0; j < kStripMax; ++j) acc[0][j] = __builtin_fmaf(x, s_lds[j][kk + e], acc[0][j]);
                }
            } else {
                const int kk = kl + 16 * E * c;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = k0 + kk < p.K ? chunk_elem<TI>(v[c], e) : 0.f;
#pragma unroll
                    for (int j = 0; j < kStripMax; ++j) acc[e][j] = __builtin_fmaf(x, s_lds[j][kk], acc[e][j]);
                }
            }
        }
    }

    auto store = [&](int i, int j, float x) {
        const int m = ROWS ? s0 + j : i, n = ROWS ? i : s0 + j;
        if (p.epi) store_epi<TO>(p, m, n, x);
        else store_out<TO>(p.C, p.c_trans ? (int64_t)n * p.ldc + m : (int64_t)m * p.ldc + n, x);
    };
    if constexpr (LK) {
        // The 16 lanes of a row are 16 consecutive lanes of one wave.
#pragma unroll
        for (int j = 0; j < kStripMax; ++j)
#pragma unroll
            for (int o = 8; o >= 1; o /= 2) acc[0][j] += __shfl_xor(acc[0][j], o, 16);
        if (kl == 0 && row_ok) {
#pragma unroll
            for (int j = 0; j < kStripMax; ++j)
                if (j < r) store(row, j, acc[0][j]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
            for (int j = 0; j < kStripMax; ++j) red[kl][(tid % GR) * E + e][j] = acc[e][j];
        __syncthreads();
        if (tid < RL * kStripMax) {
            const int rr = tid / kStripMax, j = tid % kStripMax, i = i0 + rr;
            if (i < nl && j < r) {
                float x = red[0][rr][j];
                for (int t = 1; t < NT / GR; ++t) x += red[t][rr][j];
                store(i, j, x);
            }
        }
    }
}

// Launch of the strip of canonical layout `layout` (A k|m x B k|n as for the
// tile configs): rows = false for C's last columns [p.strip0, p.N), true for
// its last rows [p.strip0, p.M) over columns [0, p.N).
template <In TI, Out TO>
struct StripInst {
    template <bool LK, bool SK, bool ROWS>
    static hipError_t go(const Params& p, hipStream_t s)
    {
        Params copy = p;
        void* args[] = {&copy};
        const int nl = ROWS ? p.N : p.M;
        return hipLaunchKernel((const void*)&gemm_strip_kernel<TI, TO, LK, SK, ROWS>,
                               dim3((unsigned)((nl + 15) / 16), (unsigned)p.batch), dim3(256), args, 0, s);
    }
    template <bool ROWS>
    static hipError_t go_rows(bool ak, bool bk, const Params& p, hipStream_t s)
    {
        const bool lk = ROWS ? bk : ak, sk = ROWS ? ak : bk;
        if (lk) return sk ? go<true, true, ROWS>(p, s) : go<true, false, ROWS>(p, s);
        return sk ? go<false, true, ROWS>(p, s) : go<false, false, ROWS>(p, s);
    }
    static hipError_t launch(int layout, bool rows, const Params& p, hipStream_t s)
    {
        const bool ak = layout < 2, bk = (layout & 1) == 0;
        return rows ? go_rows<true>(ak, bk, p, s) : go_rows<false>(ak, bk, p, s);
    }
};

}  // namespace mg
