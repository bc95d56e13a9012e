// gemm_kernel.hpp -- gfx950 (CDNA4) MFMA GEMM kernel template.
//
// Computes C[m][n] = sum_k A[m][k] * B[n][k] with C row-major ("n"-major);
// the host turns an m-major C into this form by computing C^T = B * A^T.
// The operation, the M x K / N x K / M x N shapes and the k/m/n "major"
// storage options are those of the CuTe DSL Ampere SGEMM example (module
// docstring); the block tile / wave tile hierarchy is that of the CK Tile
// practice GEMM README ("PracticeGemmShape Configuration").  The design below
// is for CDNA4, not a translation of either page:
//
//  * Workgroup = WM x WN waves of 64 lanes; block tile BM x BN x BK; each wave
//    owns a (BM/WM) x (BN/WN) sub-tile made of MI x MI MFMA tiles (MI = 32 or
//    16).  fp32 inputs use v_mfma_f32_32x32x2_f32 / 16x16x4_f32; fp16 and
//    bf16 use the gfx950 K-doubled v_mfma_f32_32x32x16_* / 16x16x32_*.
//    Accumulation is fp32.
//  * HBM -> LDS: every lane issues 128-bit buffer loads (buffer resource
//    bounds checking returns zero outside the operand's extent).  Operands
//    whose contiguous index is k are copied chunk by chunk; operands whose
//    contiguous index is m (or n) are loaded as CE x CE blocks and transposed
//    in registers, so LDS always holds k-contiguous rows and one MFMA inner
//    loop serves all four layouts.
//  * LDS: a ring of STAGES (2) buffers of [BM][BK] + [BN][BK]; 16-byte chunks
//    are XOR-swizzled by row so that the 128-bit writes and the 128-bit
//    fragment reads of a quarter-wave hit distinct banks of gfx950's 256-byte
//    bank window (the SGEMM example pads rows for the same purpose).
//  * Registers: the global loads of tile t+2 are issued while tile t is
//    consumed and land in VGPRs that are written to LDS after the MFMAs of
//    tile t+1's predecessor finish (one tile in flight per operand); the MFMA
//    fragments of k-group g+1 are read from LDS while those of g are used.
//  * fp32 operands: a lane reads 4 consecutive k of its row with one 128-bit
//    LDS read and feeds them to 4 successive MFMAs; A and B use the same
//    relabelling of k, so each element's sum is unchanged up to rounding
//    order (the SGEMM example permutes its thread layout for vectorised
//    shared-memory reads in the same spirit).
//  * Edges: rows past M/N read zeros or padding that only reach C elements
//    which are never stored; the partial last k-tile of a k-contiguous operand
//    is masked to exact zeros in registers (both operands, so NaN padding
//    cannot leak); C stores are predicated on m < M and n < N.
//  * Workgroup -> tile: workgroups are dispatched round-robin over the 8 XCDs,
//    so the linear id is remapped to give each XCD a contiguous range of the
//    tile order, and that order walks groups of `group_m` tile rows column by
//    column (L2 reuse inside one XCD).  grid.y indexes the entries of a
//    strided batch.
//  * Operands that are not 16-byte aligned use the same kernel with VEC =
//    false: each 16-byte chunk is loaded element by element.
//  * Epilogue: the plain store writes each accumulator; with the elementwise
//    epilogue (act(alpha * acc + beta * C_old + bias)) the tile goes through
//    LDS in bands and out as 4-wide runs (store_tile_via_lds).
//
// This header also holds what the other kernels share: Params, the buffer
// helpers, the swizzle, the epilogue helpers and the tile raster.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum class In : int { F32 = 0, F16 = 1, BF16 = 2 };
enum class Out : int { F32 = 0, F16 = 1, BF16 = 2 };

// Kernel arguments, already canonicalised to C n-major.
struct Params {
    const char* A;        // bytes
    const char* B;
    char* C;
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;          // tile rows per raster group
    int batch;            // number of batch entries (grid.y)
    int64_t lda, ldb, ldc;  // elements
    uint64_t a_bytes;     // readable extent of A / B in bytes (one batch entry)
    uint64_t b_bytes;
    int64_t sA, sB, sC;   // batch strides in bytes (grid.y = batch index)
    // Stream-K schedule (persistent kernels only; see gemm_f32dma.hpp).
    int grid;             // persistent workgroups (0: one workgroup per tile)
    int sk_first;         // tiles [0, sk_first) are data-parallel, the rest stream-K
    int sk_wgs;           // workgroups sharing the stream-K k-iterations
    int sk_base, sk_rem;  // k-iterations per workgroup: sk_base, +1 for the first sk_rem
    float* sk_part;       // 2 partial tiles per stream-K workgroup
    int* sk_count;        // one arrival counter per stream-K tile, zero between calls
    // Elementwise epilogue (store_epi); epi == 0 stores the accumulator as is.
    int epi;
    float alpha, beta;    // C = act(alpha * acc + beta * C_old + bias)
    const float* bias;    // fp32, indexed by column n (by row m when bias_rows), or null
    int bias_rows;
    int act;              // Act
    int c_vec;            // C and ldc allow 16-byte stores (else element stores only)
    int strip0;           // strip kernel: first column (or row) of C that it computes
    int c_trans;          // C stored transposed: element (m, n) at n * ldc + m (no epilogue)
    int split;            // split-k configs: k-ranges per tile (partial tiles in sk_part)
};

// Point A, B, C at this workgroup's batch entry.
__device__ __forceinline__ void select_batch(Params& p)
{
    const int64_t l = blockIdx.y;
    p.A += l * p.sA;
    p.B += l * p.sB;
    p.C += l * p.sC;
}

// Third dword of a buffer resource on gfx9-family parts: 32-bit data format,
// raw (unswizzled) addressing.
constexpr int kBufferFlags = 0x00020000;
// Cache-policy operand of buffer loads and stores: sc1, device (agent) scope.
constexpr int kDeviceCoherent = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, uint64_t bytes)
{
    uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, kBufferFlags);
}

__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// The 16 bytes at `off` as one 128-bit load (VEC), or element by element:
// the SGEMM example falls back to scalar copies when an operand is not
// 16-byte aligned, and so do the kernels instantiated with VEC = false (each
// element then only needs its natural alignment; out-of-range elements read 0).
template <int ES, bool VEC>
__device__ __forceinline__ i32x4 load_chunk(__amdgpu_buffer_rsrc_t r, int off)
{
    if constexpr (VEC) {
        return buf_load16(r, off);
    } else if constexpr (ES == 4) {
        i32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * e, 0, 0);
        return v;
    } else {
        i32x4 v;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * d, 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * d + 2, 0, 0);
            v[d] = (int)(lo | (hi << 16));
        }
        return v;
    }
}

// LDS bank window of gfx950: 64 banks x 4 bytes = 256 bytes = 16 chunks of
// 16 B (measured: 128-bit reads of 16 lanes from 16 distinct chunk positions of
// a 256-byte window complete without conflict; 8 positions in 128 bytes do not).
constexpr int kBankWindowChunks = 16;

// Physical 16-byte chunk of logical chunk c in LDS row `row` (rows of CPR
// chunks).  Rows shorter than the bank window share it; the XOR term gives the
// rows that share a window position different chunks, so that the 16 lanes of a
// quarter-wave reading the same logical chunk of 16 consecutive rows (MFMA
// fragment reads) and the lanes writing consecutive chunks of a row both hit 16
// distinct positions.
template <int CPR, bool SWZ>
__device__ __forceinline__ int swz_chunk(int row, int c)
{
    if constexpr (!SWZ) {
        return c;
    } else {
        constexpr int RPW = CPR >= kBankWindowChunks ? 1 : kBankWindowChunks / CPR;
        constexpr int XM = CPR >= kBankWindowChunks ? kBankWindowChunks : CPR;
        return c ^ ((row / RPW) % XM);
    }
}

// Masks the elements k >= K of a 16-byte chunk starting at element k0.
template <In TI>
__device__ __forceinline__ i32x4 mask_k(i32x4 v, int k0, int K)
{
    if constexpr (TI == In::F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (k0 + e >= K) v[e] = 0;
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t m = (k0 + 2 * d < K ? 0x0000ffffu : 0u) | (k0 + 2 * d + 1 < K ? 0xffff0000u : 0u);
            v[d] = (int)((uint32_t)v[d] & m);
        }
    }
    return v;
}

// Operand tile loader: ROWS x BK tile of an operand into LDS rows of BK.
// KMAJ: the operand's contiguous index is k.
template <In TI, int ROWS, int BK, int NT, bool KMAJ, bool SWZ, bool VEC = true>
struct TileLoader {
    static constexpr int ES = TI == In::F32 ? 4 : 2;   // element bytes
    static constexpr int CE = 16 / ES;                  // elements per chunk
    static constexpr int CPR = BK / CE;                 // chunks per LDS row
    static constexpr int RB = BK * ES;                  // LDS row bytes
    static constexpr int CHUNKS = ROWS * CPR;
    static_assert(BK % CE == 0, "BK must be a multiple of the chunk");
    static_assert(ROWS % CE == 0, "rows must be a multiple of the chunk");
    // k-contiguous: one chunk per load; m-contiguous: CE x CE blocks.
    static constexpr int UNITS = KMAJ ? CHUNKS : CHUNKS / CE;
    static constexpr int PER = (UNITS + NT - 1) / NT;
    static constexpr int REGS = KMAJ ? PER : PER * CE;  // i32x4 per thread
    static constexpr bool FULL = UNITS % NT == 0;

    i32x4 r[REGS];
    int voff[PER];

    // Precompute the per-thread byte offsets relative to the tile origin.
    __device__ __forceinline__ void init(int tid, int64_t ld)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int id = i * NT + tid;
            if (KMAJ) {
                int row = id / CPR, c = id % CPR;
                voff[i] = (int)(row * ld * ES) + c * 16;
            } else {
                int kg = id % CPR, mc = id / CPR;
                voff[i] = (int)(kg * CE * ld * ES) + mc * 16;
            }
        }
        (void)ld;
    }

    // Issue the loads of the tile whose origin is (row0, k0).
    __device__ __forceinline__ void load(const char* base, uint64_t bytes, int64_t ld, int row0,
                                         int k0, int tid)
    {
        int64_t origin = KMAJ ? ((int64_t)row0 * ld + k0) * ES : ((int64_t)k0 * ld + row0) * ES;
        uint64_t rem = (uint64_t)origin < bytes ? bytes - (uint64_t)origin : 0;
        __amdgpu_buffer_rsrc_t rs = make_rsrc(base + origin, rem);
        int ldb = (int)(ld * ES);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (FULL || i * NT + tid < UNITS) {
                if (KMAJ) {
                    r[i] = load_chunk<ES, VEC>(rs, voff[i]);
                } else {
#pragma unroll
                    for (int j = 0; j < CE; ++j) r[i * CE + j] = load_chunk<ES, VEC>(rs, voff[i] + j * ldb);
                }
            }
        }
    }

    // Zero k >= K in the loaded chunks (k-contiguous operands only; rows
    // k >= K of an m-contiguous operand lie outside its extent and read 0).
    __device__ __forceinline__ void mask(int k0, int K, int tid)
    {
        if constexpr (KMAJ) {
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                int id = i * NT + tid;
                int c = id % CPR;
                r[i] = mask_k<TI>(r[i], k0 + c * CE, K);
            }
        }
    }

    // Write the registers to LDS (k-contiguous rows, swizzled chunks).
    __device__ __forceinline__ void store(char* lds, int tid)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int id = i * NT + tid;
            if (!(FULL || id < UNITS)) continue;
            if (KMAJ) {
                int row = id / CPR, c = id % CPR;
                *(i32x4*)(lds + row * RB + swz_chunk<CPR, SWZ>(row, c) * 16) = r[i];
            } else {
                int kg = id % CPR, mc = id / CPR;
                // r[i*CE + j] holds k = kg*CE + j for m = mc*CE .. mc*CE+CE-1.
#pragma unroll
                for (int e = 0; e < CE; ++e) {
                    i32x4 o;
                    if constexpr (ES == 4) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) o[j] = r[i * CE + j][e];
                    } else {
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            uint32_t lo = (uint32_t)r[i * CE + 2 * d][e >> 1];
                            uint32_t hi = (uint32_t)r[i * CE + 2 * d + 1][e >> 1];
                            if (e & 1) o[d] = (int)((lo >> 16) | (hi & 0xffff0000u));
                            else o[d] = (int)((lo & 0xffffu) | (hi << 16));
                        }
                    }
                    int row = mc * CE + e;
                    *(i32x4*)(lds + row * RB + swz_chunk<CPR, SWZ>(row, kg) * 16) = o;
                }
            }
        }
    }
};

template <In TI, int MI>
__device__ __forceinline__ void mfma_step(const i32x4& a, const i32x4& b, f32x16& acc)
{
    if constexpr (TI == In::F32) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a[0]), __int_as_float(b[0]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a[1]), __int_as_float(b[1]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a[2]), __int_as_float(b[2]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a[3]), __int_as_float(b[3]), acc, 0, 0, 0);
    } else if constexpr (TI == In::F16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
}

template <In TI, int MI>
__device__ __forceinline__ void mfma_step(const i32x4& a, const i32x4& b, f32x4& acc)
{
    if constexpr (TI == In::F32) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[0]), __int_as_float(b[0]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[1]), __int_as_float(b[1]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[2]), __int_as_float(b[2]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[3]), __int_as_float(b[3]), acc, 0, 0, 0);
    } else if constexpr (TI == In::F16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
}

// One fp32 MFMA (k = 2 for 32x32, k = 4 for 16x16) on raw 32-bit operands.
template <int MI>
__device__ __forceinline__ void mfma_f32_one(int a, int b, f32x16& acc)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a), __int_as_float(b), acc, 0, 0, 0);
}
template <int MI>
__device__ __forceinline__ void mfma_f32_one(int a, int b, f32x4& acc)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a), __int_as_float(b), acc, 0, 0, 0);
}

template <Out TO>
__device__ __forceinline__ void store_out(char* C, int64_t idx, float v)
{
    if constexpr (TO == Out::F32) {
        ((float*)C)[idx] = v;
    } else if constexpr (TO == Out::F16) {
        ((_Float16*)C)[idx] = (_Float16)v;                       // round to nearest even
    } else {
        ((uint16_t*)C)[idx] = __builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest even
    }
}

template <Out TO>
__device__ __forceinline__ float load_out(const char* C, int64_t idx)
{
    if constexpr (TO == Out::F32) {
        return ((const float*)C)[idx];
    } else if constexpr (TO == Out::F16) {
        return (float)((const _Float16*)C)[idx];
    } else {
        return (float)__builtin_bit_cast(__bf16, ((const uint16_t*)C)[idx]);
    }
}

// Activations of the epilogue.
enum Act : int { kActNone = 0, kActRelu = 1, kActGelu = 2 };

// erf(x) for the GELU epilogue, inline (a library call in an unrolled
// epilogue would make the accumulators live across calls and spill them):
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26,
// |error| <= 1.5e-7:  erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^{-x^2},
// t = 1 / (1 + p x) for x >= 0, and erf(-x) = -erf(x).
__device__ __forceinline__ float erf_as(float x)
{
    const float ax = __builtin_fabsf(x);
    const float t = 1.f / (1.f + 0.3275911f * ax);
    const float poly = t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f +
                                                t * (-1.453152027f + t * 1.061405429f))));
    const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.44269504088896341f);   // e^{-x^2}
    const float y = 1.f - poly * e;
    return x < 0.f ? -y : y;
}

// Store output element (m, n) of the canonical C through the elementwise
// epilogue (kernels call this only when p.epi is set, from a loop of its own,
// so that the plain store path keeps its code).  The SGEMM example applies
// its epilogue_op to the accumulator fragment right before the store, and CK
// Tile's kernel has an Epilogue stage after the GEMM.  In fp32:
//   v = act(alpha * acc + beta * C_old + bias)     (C_old read only if beta != 0)
// relu(x) = (x < 0 ? 0 : x), which keeps NaN; gelu(x) = x/2 * (1 + erf(x / sqrt 2)),
// with erf_as above (GELU values within about 1e-7 |x| of the exact ones).
template <Out TO>
__device__ __forceinline__ float epi_value(const Params& p, int m, int n, float v)
{
    float t = p.alpha * v;
    if (p.beta != 0.f) t = __builtin_fmaf(p.beta, load_out<TO>(p.C, (int64_t)m * p.ldc + n), t);
    if (p.bias) t += p.bias[p.bias_rows ? m : n];
    if (p.act == kActRelu) t = t < 0.f ? 0.f : t;
    else if (p.act == kActGelu) t = 0.5f * t * (1.f + erf_as(t * 0.70710678118654752f));
    return t;
}

template <Out TO>
__device__ __forceinline__ void store_epi(const Params& p, int m, int n, float v)
{
    store_out<TO>(p.C, (int64_t)m * p.ldc + n, epi_value<TO>(p, m, n, v));
}

// Store 4 consecutive outputs (m, n .. n+3) of the canonical C, given in fp32:
// through the elementwise epilogue when p.epi is set, then converted; one
// 128-bit (fp32) or 64-bit (16-bit) store (and, for the epilogue, one load of
// the old values) when all four are inside C and C allows it.
template <Out TO>
__device__ __forceinline__ void store4(const Params& p, int m, int n, f32x4 v)
{
    const int64_t idx = (int64_t)m * p.ldc + n;
    const bool whole = p.c_vec && n + 3 < p.N;
    if (p.epi) {
        if (!whole) {
#pragma unroll 1
            for (int e = 0; e < 4; ++e)
                if (n + e < p.N) store_epi<TO>(p, m, n + e, v[e]);
            return;
        }
        // All four inside C: the epilogue on the four values (the operations
        // and their order of epi_value), then one vector store below.
        f32x4 old = {0.f, 0.f, 0.f, 0.f};
        if (p.beta != 0.f) {
            if constexpr (TO == Out::F32) {
                old = *(const f32x4*)((const float*)p.C + idx);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) old[e] = load_out<TO>(p.C, idx + e);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float t = p.alpha * v[e];
            if (p.beta != 0.f) t = __builtin_fmaf(p.beta, old[e], t);
            if (p.bias) t += p.bias[p.bias_rows ? m : n + e];
            if (p.act == kActRelu) t = t < 0.f ? 0.f : t;
            else if (p.act == kActGelu) t = 0.5f * t * (1.f + erf_as(t * 0.70710678118654752f));
            v[e] = t;
        }
    }
    if (whole) {
        if constexpr (TO == Out::F32) {
            *(f32x4*)((float*)p.C + idx) = v;
        } else {
            typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
            uint16_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                h[e] = TO == Out::F16 ? __builtin_bit_cast(uint16_t, (_Float16)v[e])
                                      : __builtin_bit_cast(uint16_t, (__bf16)v[e]);
            *(u32x2*)((uint16_t*)p.C + idx) = u32x2{h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16)};
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < p.N) store_out<TO>(p.C, idx + e, v[e]);
    }
}

// Tile epilogue through LDS, for the elementwise epilogue: the tile is
// handled in bands of RB rows; each lane parks its
// accumulators of the band at [row][col] in LDS (fp32), then every thread
// takes runs of 4 values along n and writes them with store4 -- row-major,
// coalesced vector stores instead of one store per accumulator, and one copy
// of the epilogue code.  get(v) returns accumulator v (a constant index once
// the loops are unrolled), pos(v, r, c) its tile-local row and column.  The
// LDS (LDS_BYTES from smem) is the kernel's operand ring; a barrier at entry
// waits until no wave still reads it or has loads into it in flight.
// ROLLED keeps the loop over bands rolled
// (fewer registers live at once: the persistent stream-K kernels, whose loop
// state stays live across the store, need that for 256x256 tiles).
template <Out TO, int BM, int BN, int NT, int NV, int LDS_BYTES, bool ROLLED = false, class Get, class Pos>
__device__ __forceinline__ void store_tile_via_lds(const Params& p, char* smem, int m0, int n0, int tid,
                                                   Get get, Pos pos)
{
    constexpr int FIT = LDS_BYTES / (BN * 4);
    constexpr int RB = FIT >= BM ? BM : FIT >= 128 ? 128 : FIT >= 64 ? 64 : FIT >= 32 ? 32 : FIT >= 16 ? 16 : 8;
    static_assert(FIT >= 8 && BM % RB == 0, "LDS too small for the staged epilogue");
    float* t = (float*)smem;
    // Every wave's loads into the ring (the asynchronous direct-to-LDS ones
    // included: the fence waits for this wave's vmcnt) and LDS reads of it are
    // complete before any wave writes the staging bands over it.
    __syncthreads();
    auto band = [&](int b0) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            int r, c;
            pos(v, r, c);
            if (r >= b0 && r < b0 + RB) t[(r - b0) * BN + c] = get(v);
        }
        __syncthreads();
#pragma unroll 1
        for (int q = tid; q < RB * BN / 4; q += NT) {
            const int r = q / (BN / 4), c = (q % (BN / 4)) * 4;
            const int m = m0 + b0 + r;
            if (m < p.M) store4<TO>(p, m, n0 + c, *(const f32x4*)(t + r * BN + c));
        }
        __syncthreads();
    };
    __syncthreads();
    if constexpr (ROLLED) {
#pragma unroll 1
        for (int b0 = 0; b0 < BM; b0 += RB) band(b0);
    } else {
#pragma unroll
        for (int b0 = 0; b0 < BM; b0 += RB) band(b0);
    }
}

// Linear tile index L -> (tile row, tile column) in groups of group_m tile rows.
__device__ __forceinline__ void raster(const Params& p, int L, int& tm, int& tn)
{
    const int width = p.group_m * p.tiles_n;
    const int first = (L / width) * p.group_m;
    const int gsz = min(p.tiles_m - first, p.group_m);
    const int r = L % width;
    tm = first + r % gsz;
    tn = r / gsz;
}

// Linear workgroup id -> (tile_m, tile_n): the 8 XCDs (workgroup w runs on
// XCD w mod 8) each own a contiguous range of the raster order.
__device__ __forceinline__ void tile_coords(const Params& p, int& tm, int& tn)
{
    const int G = p.tiles_m * p.tiles_n;
    const int w = blockIdx.x;
    const int per = G / 8, rem = G % 8;
    const int x = w % 8, idx = w / 8;
    const int L = x * per + (x < rem ? x : rem) + idx;
    raster(p, L, tm, tn);
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;

// Interleave NR LDS reads, NW LDS writes and NL global loads among NM MFMAs
// of one scheduling region: after each MFMA, the next share of each class.
template <int NM, int NR, int NW, int NL>
__device__ __forceinline__ void interleave()
{
    constexpr int PR = (NR + NM - 1) / NM, PW = (NW + NM - 1) / NM, PL = (NL + NM - 1) / NM;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (PR > 0 && i * PR < NR) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PR, 0);
        if (PW > 0 && i * PW < NW) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, PW, 0);
        if (PL > 0 && i * PL < NL) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, PL, 0);
    }
}

template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI, bool AK, bool BKM, bool SWZ,
          bool VEC = true>
struct GemmTile {
    static constexpr int NT = WM * WN * 64;
    static constexpr int ES = TI == In::F32 ? 4 : 2;
    static constexpr int CE = 16 / ES;
    static constexpr int CPR = BK / CE;
    static constexpr int RB = BK * ES;
    static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
    static constexpr int TM = WTM / MI, TN = WTN / MI;   // MFMA tiles per wave
    static constexpr int NQ = 64 / MI;                   // lane groups along k
    static constexpr int NG = CPR / NQ;                  // k-groups per BK
    static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int MF_PER = TI == In::F32 ? 4 : 1; // MFMAs per fragment pair
    static constexpr int NMF = TM * TN * MF_PER;         // MFMAs per k-group
    static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must be a multiple of the MFMA tile");
    static_assert(CPR % NQ == 0, "BK too small for this MFMA shape");
    static_assert(2 * STAGE <= 160 * 1024, "LDS budget");
    using Acc = typename std::conditional<MI == 32, f32x16, f32x4>::type;
    using LA = TileLoader<TI, BM, BK, NT, AK, SWZ, VEC>;
    using LB = TileLoader<TI, BN, BK, NT, BKM, SWZ, VEC>;
    static constexpr int NW = (AK ? LA::PER : LA::PER * CE) + (BKM ? LB::PER : LB::PER * CE);
    static constexpr int NL = LA::REGS + LB::REGS;

    LA la;
    LB lb;
    Acc acc[TM][TN];
    i32x4 fa[2][TM], fb[2][TN];
    int wm, wn, frow, fq, tid;

    __device__ __forceinline__ void read_frags(const char* sa, int g, int buf)
    {
        const char* sb = sa + A_BYTES;
        const int c = g * NQ + fq;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * MI + frow;
            fa[buf][i] = *(const i32x4*)(sa + row * RB + swz_chunk<CPR, SWZ>(row, c) * 16);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * WTN + j * MI + frow;
            fb[buf][j] = *(const i32x4*)(sb + row * RB + swz_chunk<CPR, SWZ>(row, c) * 16);
        }
    }

    __device__ __forceinline__ void mma(int buf)
    {
        if constexpr (TI == In::F32) {
            // The 4 k values of a fragment feed 4 MFMAs on one accumulator;
            // walk the accumulators innermost so consecutive MFMAs are independent.
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        mfma_f32_one<MI>(fa[buf][i][e], fb[buf][j][e], acc[i][j]);
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    mfma_step<TI, MI>(fa[buf][i], fb[buf][j], acc[i][j]);
        }
    }

    // One k-tile: MFMAs on LDS stage `cur` (whose group-0 fragments are already
    // in fa/fb[0]).  WRITE: the staged registers (tile t+1) go to the other
    // stage during group 0; LOAD: tile t+2 is fetched into the registers during
    // group 1 (group 0 when there is only one).  NEXT: after a barrier, the
    // group-0 fragments of the other stage are read for the next tile.
    template <bool WRITE, bool LOAD, bool NEXT>
    __device__ __forceinline__ void tile(char* smem, int cur, const Params& p, int m0, int n0,
                                         int k_load)
    {
        char* sa = smem + cur * STAGE;
        char* nxt = smem + (cur ^ 1) * STAGE;
        constexpr int LOAD_G = NG > 1 ? 1 : 0;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            // Fence: nothing moves between k-groups, so the reads issued here
            // for group g+1 are consumed only after this group's MFMAs.
            __builtin_amdgcn_sched_barrier(0);
            if (g + 1 < NG) read_frags(sa, g + 1, (g + 1) & 1);
            if (WRITE && g == 0) {
                la.store(nxt, tid);
                lb.store(nxt + A_BYTES, tid);
            }
            if (LOAD && g == LOAD_G) {
                la.load(p.A, p.a_bytes, p.lda, m0, k_load, tid);
                lb.load(p.B, p.b_bytes, p.ldb, n0, k_load, tid);
            }
            mma(g & 1);
            if (g + 1 < NG) {
                if (WRITE && g == 0 && LOAD && g == LOAD_G)
                    interleave<NMF, TM + TN, NW, NL>();
                else if (WRITE && g == 0)
                    interleave<NMF, TM + TN, NW, 0>();
                else if (LOAD && g == LOAD_G)
                    interleave<NMF, TM + TN, 0, NL>();
                else
                    interleave<NMF, TM + TN, 0, 0>();
            } else {
                if (WRITE && g == 0 && LOAD && g == LOAD_G)
                    interleave<NMF, 0, NW, NL>();
                else if (WRITE && g == 0)
                    interleave<NMF, 0, NW, 0>();
                else if (LOAD && g == LOAD_G)
                    interleave<NMF, 0, 0, NL>();
                else
                    interleave<NMF, 0, 0, 0>();
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (NEXT) {
            __syncthreads();
            read_frags(nxt, 0, 0);
        }
    }
};

// EPI: instantiation that runs the elementwise epilogue (only used for 16-bit
// outputs, whose plain epilogue and epilogue path do not share a kernel well:
// together they exhaust the registers; fp32 outputs take both in one kernel).
template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI, bool AK, bool BKM, bool SWZ, bool EPI,
          bool VEC>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_kernel(Params p)
{
    using T = GemmTile<TI, TO, BM, BN, BK, WM, WN, MI, AK, BKM, SWZ, VEC>;
    select_batch(p);
    __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

    T t;
    t.tid = threadIdx.x;
    const int lane = t.tid & 63;
    const int wave = t.tid >> 6;
    t.wm = wave / WN;
    t.wn = wave % WN;
    t.frow = lane % MI;
    t.fq = lane / MI;

    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    t.la.init(t.tid, p.lda);
    t.lb.init(t.tid, p.ldb);
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
            t.acc[i][j] = typename T::Acc{};

    const int nkt = (p.K + BK - 1) / BK;
    const bool ragged = (p.K % BK) != 0;

    if (nkt > 0) {
        // Prologue: tile 0 -> LDS stage 0, tile 1 -> registers, group-0 fragments.
        t.la.load(p.A, p.a_bytes, p.lda, m0, 0, t.tid);
        t.lb.load(p.B, p.b_bytes, p.ldb, n0, 0, t.tid);
        if (nkt == 1 && ragged) { t.la.mask(0, p.K, t.tid); t.lb.mask(0, p.K, t.tid); }
        t.la.store(smem, t.tid);
        t.lb.store(smem + T::A_BYTES, t.tid);
        if (nkt > 1) {
            t.la.load(p.A, p.a_bytes, p.lda, m0, BK, t.tid);
            t.lb.load(p.B, p.b_bytes, p.ldb, n0, BK, t.tid);
        }
        __syncthreads();
        t.read_frags(smem, 0, 0);

        // Steady state: every iteration writes tile kt+1 and loads tile kt+2.
        int kt = 0;
        for (; kt + 2 < nkt; ++kt)
            t.template tile<true, true, true>(smem, kt & 1, p, m0, n0, (kt + 2) * BK);
        // Tail: tile nkt-2 writes the (possibly ragged) last tile, then the last tile.
        if (kt + 1 < nkt) {
            if (ragged) { t.la.mask((kt + 1) * BK, p.K, t.tid); t.lb.mask((kt + 1) * BK, p.K, t.tid); }
            t.template tile<true, false, true>(smem, kt & 1, p, m0, n0, 0);
            ++kt;
        }
        t.template tile<false, false, false>(smem, kt & 1, p, m0, n0, 0);
    }

    // Epilogue: fp32 accumulators -> output type, predicated stores.
    constexpr int MI_ = MI;
    if (TO == Out::F32 ? p.epi : EPI) {
        constexpr int R = MI_ == 32 ? 16 : 4;
        store_tile_via_lds<TO, BM, BN, T::NT, T::TM * T::TN * R, 2 * T::STAGE>(
            p, smem, m0, n0, t.tid, [&](int v) { return t.acc[v / (T::TN * R)][(v / R) % T::TN][v % R]; },
            [&](int v, int& r, int& c) {
                const int i = v / (T::TN * R), j = (v / R) % T::TN, q = v % R;
                c = t.wn * T::WTN + j * MI_ + (lane % MI_);
                r = t.wm * T::WTM + i * MI_ + (MI_ == 32 ? (q / 4) * 8 + (lane / 32) * 4 + (q % 4) : (lane / 16) * 4 + q);
            });
        return;
    }
    if constexpr (TO != Out::F32 && EPI) return;
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int n = n0 + t.wn * T::WTN + j * MI_ + (lane % MI_);
            const int mb = m0 + t.wm * T::WTM + i * MI_;
            if constexpr (MI_ == 32) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = mb + (r / 4) * 8 + (lane / 32) * 4 + (r % 4);
                    if (m < p.M && n < p.N) store_out<TO>(p.C, (int64_t)m * p.ldc + n, t.acc[i][j][r]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = mb + (lane / 16) * 4 + r;
                    if (m < p.M && n < p.N) store_out<TO>(p.C, (int64_t)m * p.ldc + n, t.acc[i][j][r]);
                }
            }
        }
    }
}

// One tile configuration, instantiated for the four operand layouts.
using LaunchFn = hipError_t (*)(int layout, const Params& p, hipStream_t s);

struct KernelEntry {
    const char* name;
    int BM, BN, BK, WM, WN, MI;
    bool swz;
    LaunchFn launch;
    int stages;        // LDS ring depth
    bool dma;          // direct HBM -> LDS loads
    int sk_occ;        // stream-K: persistent workgroups per CU (0: one workgroup per tile)
    bool scalar;       // element-by-element loads: any leading dimension, element-aligned pointers
    bool c_trans;      // can store C transposed (Params::c_trans)
    int split_occ;     // split-k: workgroups per CU the k-ranges are counted for (0: not split-k)
};

// VEC = false: element-by-element operand loads, for operands that are not
// 16-byte aligned.
template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI, bool SWZ, bool VEC = true>
struct Inst {
    template <bool AK, bool BKM, bool EPI>
    static hipError_t go(const Params& p, hipStream_t s)
    {
        // hipLaunchKernel reports this launch's own status (a stale error left
        // by an earlier runtime call on the thread cannot be mistaken for it).
        Params copy = p;
        void* args[] = {&copy};
        return hipLaunchKernel((const void*)&gemm_kernel<TI, TO, BM, BN, BK, WM, WN, MI, AK, BKM, SWZ, EPI, VEC>,
                               dim3((unsigned)(p.tiles_m * p.tiles_n), (unsigned)p.batch), dim3(WM * WN * 64), args, 0, s);
    }
    template <bool AK, bool BKM>
    static hipError_t go(const Params& p, hipStream_t s)
    {
        if constexpr (TO != Out::F32)
            if (p.epi) return go<AK, BKM, true>(p, s);
        return go<AK, BKM, false>(p, s);
    }
    static hipError_t launch(int layout, const Params& p, hipStream_t s)
    {
        switch (layout) {
        case 0: return go<true, true>(p, s);
        case 1: return go<true, false>(p, s);
        case 2: return go<false, true>(p, s);
        default: return go<false, false>(p, s);
        }
    }
};

// Per-dtype registries, defined in the gemm_<dtype>.hip files.
const KernelEntry* entries_f32(int* n);
const KernelEntry* entries_f16_f32(int* n);
const KernelEntry* entries_bf16_bf16(int* n);
const KernelEntry* entries_f16_f16(int* n);
const KernelEntry* entries_bf16_f32(int* n);
// Widest last column (row) of C that the launch path gives to the strip
// kernel instead of a column (row) of tiles, and the least number of full
// tiles for which it does so (below that the extra launch costs more).
constexpr int kStripMax = 4;
constexpr int kStripMinTiles = 64;

// The strip kernel of each dtype (gemm_strip.hpp): layout as for a
// KernelEntry's launch; rows selects a strip of C's last rows.
hipError_t strip_f32(int layout, bool rows, const Params& p, hipStream_t s);
hipError_t strip_f16_f32(int layout, bool rows, const Params& p, hipStream_t s);
hipError_t strip_bf16_bf16(int layout, bool rows, const Params& p, hipStream_t s);
hipError_t strip_f16_f16(int layout, bool rows, const Params& p, hipStream_t s);
hipError_t strip_bf16_f32(int layout, bool rows, const Params& p, hipStream_t s);

}  // namespace mg
