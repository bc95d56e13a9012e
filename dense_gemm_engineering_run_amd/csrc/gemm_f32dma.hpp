// gemm_f32dma.hpp -- gfx950 fp32 GEMM with direct HBM -> LDS loads.
//
// Same operation and canonical form as gemm_kernel.hpp (C = A * B^T, C
// n-major; CuTe DSL Ampere SGEMM example, module docstring), for fp32 inputs on
// v_mfma_f32_32x32x2_f32.  Operands go from HBM straight into a ring of LDS
// stages with buffer_load_dwordx4 ... lds (as in gemm_dma.hpp), in their own
// layout: k-contiguous operands as [rows][BK], m/n-contiguous operands as
// [BK][rows].  No operand is transposed anywhere; instead each 128-bit LDS
// read feeds four MFMAs:
//
//  * k-contiguous operand: a lane reads 4 consecutive k of its row; MFMA e
//    (e = 0..3) takes element e.  Lane half h = lane/32 supplies k = 4h + e of
//    an 8-k step, the same relabelling for A and B, so each output element's
//    sum is unchanged up to rounding order.
//  * m-contiguous operand: for each e, a lane reads 4 consecutive m at
//    k = 4h + e; element v is row 4q + v of a 128-row block (q = lane mod 32),
//    i.e. the MFMA's 32 rows are 4 interleaved row sets v = 0..3.  The
//    epilogue undoes the interleave.  (The SGEMM example permutes its thread
//    layout along m and n for vectorised shared-memory reads in the same way.)
//
// Per 8-k step and per 128 rows (or columns) an operand needs 4 LDS reads of
// 128 bits in either layout; a 128x128 wave tile issues 64 MFMAs per step.
// When both A and B are m/n-contiguous, a lane's 16 accumulators hold 4x4
// blocks of C, written with 128-bit stores.
//
// The main loop over a range of k-tiles and the epilogue are separate pieces
// (F32Dma), so that the persistent stream-K kernel at the end of this file can
// run partial k-ranges of a tile.
#pragma once

#include "gemm_dma.hpp"
#include "gemm_streamk.hpp"

namespace mg {

// One fp32 operand's k-tile in the LDS ring.  VEC: each 1 KB group of the
// tile is one load of 16 bytes per lane (the operand and its leading
// dimension 16-byte aligned); else four loads of 4 bytes per lane, lane l of
// load e filling element l % 4 of 16-byte slot 16e + l / 4 -- the same LDS
// layout, for operands aligned only to their elements.
template <int ROWS, int BK, int NWAVES, bool KMAJ, bool VEC = true>
struct F32Operand {
    static constexpr int ES = 4, CE = 4;
    static constexpr int BYTES = ROWS * BK * ES;
    static constexpr int IPW = BYTES / 1024 / NWAVES;       // 1 KB groups per wave per tile
    static_assert(BYTES % (1024 * NWAVES) == 0, "tile must split into 1 KB loads per wave");
    static constexpr int SUB = VEC ? 1 : 4;                 // loads per group
    static constexpr int LOADS = IPW * SUB;                 // load instructions per wave per tile
    static constexpr int CPR = BK / CE, RB = BK * ES;       // k-contiguous layout
    static constexpr int RCH = ROWS / CE, RBM = ROWS * ES;  // m-contiguous layout (no swizzle:
                                                            // its reads are contiguous)
    int voff[LOADS];

    __device__ __forceinline__ void init(int wave, int lane, int64_t ld)
    {
#pragma unroll
        for (int j = 0; j < IPW; ++j)
#pragma unroll
            for (int e = 0; e < SUB; ++e) {
                const int slot = (wave * IPW + j) * 64 + (VEC ? lane : 16 * e + lane / 4);
                const int elem = VEC ? 0 : (lane % 4) * ES;
                if (KMAJ) {
                    const int row = slot / CPR, phys = slot % CPR;
                    voff[j * SUB + e] = (int)(row * ld * ES) + swz_chunk<CPR, true>(row, phys) * 16 + elem;
                } else {
                    const int k = slot / RCH, c = slot % RCH;
                    voff[j * SUB + e] = (int)(k * ld * ES) + c * 16 + elem;
                }
            }
    }

    __device__ __forceinline__ void issue(const char* base, uint64_t bytes, int64_t ld, int row0,
                                          int k0, char* lds_tile, int wave, int j0 = 0, int j1 = IPW)
    {
        const int64_t origin = KMAJ ? ((int64_t)row0 * ld + k0) * ES : ((int64_t)k0 * ld + row0) * ES;
        const uint64_t rem = (uint64_t)origin < bytes ? bytes - (uint64_t)origin : 0;
        const uint64_t addr = (uint64_t)(base + origin);
        i32x4 rs;
        rs[0] = (int)(uint32_t)addr;
        rs[1] = (int)((uint32_t)(addr >> 32) & 0xffffu);
        rs[2] = (int)(rem > 0xffffffffull ? 0xffffffffu : (uint32_t)rem);
        rs[3] = kBufferFlags;
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)lds_tile + (uint32_t)(wave * IPW * 1024);
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            if (j < j0 || j >= j1) continue;
            if constexpr (VEC) {
                asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                             :
                             : "s"(__builtin_amdgcn_readfirstlane(lds0 + j * 1024)), "v"(voff[j]), "s"(rs)
                             : "memory", "m0");
            } else {
#pragma unroll
                for (int e = 0; e < SUB; ++e)
                    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                                 :
                                 : "s"(__builtin_amdgcn_readfirstlane(lds0 + j * 1024 + e * 256)),
                                   "v"(voff[j * SUB + e]), "s"(rs)
                                 : "memory", "m0");
            }
        }
    }

    // k-contiguous: 4 consecutive k (4h .. 4h+3 of the 8-k step at kb) of row rbase + lane%32.
    __device__ __forceinline__ i32x4 frag_k(const char* t, int rbase, int kb, int lane) const
    {
        const int row = rbase + lane % 32;
        const int c = kb / CE + lane / 32;
        return *(const i32x4*)(t + row * RB + swz_chunk<CPR, true>(row, c) * 16);
    }

    // m-contiguous: rows cbase + RV*q .. RV*q + RV-1 (q = lane%32) at k = kb + 4h + e,
    // read with one 32-, 64- or 128-bit LDS load (RV = 1, 2, 4).
    template <int RV>
    __device__ __forceinline__ i32x4 frag_m(const char* t, int cbase, int kb, int e, int lane) const
    {
        const int k = kb + 4 * (lane / 32) + e;
        const char* q = t + k * RBM + (cbase + RV * (lane % 32)) * ES;
        i32x4 r = {0, 0, 0, 0};
        if constexpr (RV == 4) {
            r = *(const i32x4*)q;
        } else if constexpr (RV == 2) {
            typedef int i32x2 __attribute__((ext_vector_type(2)));
            const i32x2 v = *(const i32x2*)q;
            r[0] = v[0];
            r[1] = v[1];
        } else {
            r[0] = *(const int*)q;
        }
        return r;
    }

    template <int NT>
    __device__ __forceinline__ void zero_tail(char* t, int kvalid, int tid) const
    {
        if constexpr (KMAJ) {
            const int c0 = kvalid / CE;
#pragma unroll 1
            for (int idx = tid; idx < ROWS * CPR; idx += NT) {
                const int row = idx / CPR, c = idx % CPR;
                if (c < c0) continue;
                i32x4* q = (i32x4*)(t + row * RB + swz_chunk<CPR, true>(row, c) * 16);
                if (c * CE >= kvalid) *q = i32x4{0, 0, 0, 0};
                else *q = mask_k<In::F32>(*q, c * CE, kvalid);
            }
        }
    }
};

// Units of an operand within a wave tile (WT rows): k-contiguous -> WT/32 row
// blocks of 32 rows; m-contiguous -> blocks of 32*RV rows, each read as RV
// interleaved row variants (RV = 4 when WT is a multiple of 128, else 2 or 1).
template <bool KMAJ, int WT>
struct Units {
    static_assert(WT % 32 == 0, "wave tile must be a multiple of 32");
    static constexpr int N = WT / 32;
    static constexpr int RV = KMAJ ? 1 : (WT % 128 == 0 ? 4 : WT % 64 == 0 ? 2 : 1);
    static constexpr int BLK = 32 * RV;       // rows per block
    static constexpr int NBLK = WT / BLK;
    // row (relative to the wave tile) of MFMA row index r in unit u
    __device__ static __forceinline__ int row(int u, int r)
    {
        return KMAJ ? u * 32 + r : (u / RV) * BLK + RV * r + (u % RV);
    }
};

// The pieces of the kernel: a main loop over a range of k-tiles of one C tile,
// and the epilogue that stores a C tile.
template <Out TO, int BM, int BN, int BK, int WM, int WN, int STAGES, bool AK, bool BKM, bool VEC = true>
struct F32Dma {
    static constexpr int TILE_M = BM, TILE_N = BN, TILE_K = BK;
    static constexpr Out OUT = TO;
    static constexpr int NW = WM * WN, NT = NW * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    using UA = Units<AK, WTM>;
    using UB = Units<BKM, WTN>;
    static constexpr int NA = UA::N, NB = UB::N;
    static constexpr int NG = BK / 8;                  // 8-k steps per tile
    using OA = F32Operand<BM, BK, NW, AK, VEC>;
    using OB = F32Operand<BN, BK, NW, BKM, VEC>;
    static constexpr int STAGE = OA::BYTES + OB::BYTES;
    static constexpr int LPT = OA::LOADS + OB::LOADS;   // load instructions per wave per tile
    static constexpr int SMEM = STAGES * STAGE;
    static_assert(BK % 8 == 0, "BK must be a multiple of 8");
    static_assert(STAGES >= 2 && SMEM <= 160 * 1024, "LDS budget");
    static_assert(LPT * (STAGES - 2) < 64, "vmcnt range");
    typedef f32x16 Acc[NA][NB];

    __device__ static __forceinline__ void zero(Acc& acc)
    {
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};
    }

    // Accumulate k-tiles [kt0, kt1) of the C tile at (m0, n0) into acc.  The
    // LDS ring must be free on entry (no wave still reading it); on return
    // every load has landed.
    __device__ static __forceinline__ void mainloop(const Params& p, char* smem, OA& oa, OB& ob,
                                                    int m0, int n0, int kt0, int kt1, Acc& acc, int tid,
                                                    int lane, int wave)
    {
        const int wm = wave / WN, wn = wave % WN;
        const int nkt = (p.K + BK - 1) / BK;
        const int kvalid_last = p.K - (nkt - 1) * BK;
        // Operand fields as locals: read through `p` they would be reloaded
        // after every DMA asm statement (memory clobber) and the buffer
        // descriptors rebuilt per k-group.
        const char* const A = p.A;
        const char* const B = p.B;
        const uint64_t a_bytes = p.a_bytes, b_bytes = p.b_bytes;
        const int64_t lda = p.lda, ldb = p.ldb;
        const bool ragged = kvalid_last != BK;

        // Every k-tile issues the loads of the tile STAGES-1 ahead, also past the
        // end of the range: those get an empty extent (num_records 0), so they
        // write zeros into a stage that no later tile reads.  The steady state
        // then has no branch before each step's loads (a run-time test there
        // costs a branch and the compare feeding it between MFMA runs,
        // measured at 2 % of the loop time), and the number of loads in flight
        // is the same for every tile.
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s) {
            const bool live = kt0 + s < kt1;
            char* st = smem + s * STAGE;
            oa.issue(A, live ? a_bytes : 0, lda, m0, (kt0 + s) * BK, st, wave);
            ob.issue(B, live ? b_bytes : 0, ldb, n0, (kt0 + s) * BK, st + OA::BYTES, wave);
        }

        for (int t = kt0; t < kt1; ++t) {
            const int r = t - kt0;
            // Tile t has landed once the STAGES-2 later tiles' loads are all
            // that remain outstanding.
            wait_vmcnt<LPT * (STAGES - 2)>();
            char* st = smem + (r % STAGES) * STAGE;
            if (t == nkt - 1 && ragged && (AK || BKM)) {
                bare_barrier();
                oa.template zero_tail<NT>(st, kvalid_last, tid);
                ob.template zero_tail<NT>(st + OA::BYTES, kvalid_last, tid);
                __builtin_amdgcn_s_waitcnt(0xc07f);
            }
            bare_barrier();
            const bool more = t + STAGES - 1 < kt1;
            const uint64_t na = more ? a_bytes : 0, nb = more ? b_bytes : 0;
            char* nst = smem + ((r + STAGES - 1) % STAGES) * STAGE;
            const int nk0 = (t + STAGES - 1) * BK;
            const char* sa = st;
            const char* sb = st + OA::BYTES;

            // Fragments of one 8-k step: va[buf][e][u] is the A value of unit u for
            // k sub-index e; the next step's fragments are read during this step.
            int va[2][4][NA], vb[2][4][NB];
            auto read = [&](int g, int buf) {
                const int kb = g * 8;
                if constexpr (AK) {
#pragma unroll
                    for (int u = 0; u < NA; ++u) {
                        const i32x4 f = oa.frag_k(sa, wm * WTM + u * 32, kb, lane);
#pragma unroll
                        for (int e = 0; e < 4; ++e) va[buf][e][u] = f[e];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int cb = 0; cb < UA::NBLK; ++cb) {
                            const i32x4 f = oa.template frag_m<UA::RV>(sa, wm * WTM + cb * UA::BLK, kb, e, lane);
#pragma unroll
                            for (int v = 0; v < UA::RV; ++v) va[buf][e][cb * UA::RV + v] = f[v];
                        }
                }
                if constexpr (BKM) {
#pragma unroll
                    for (int u = 0; u < NB; ++u) {
                        const i32x4 f = ob.frag_k(sb, wn * WTN + u * 32, kb, lane);
#pragma unroll
                        for (int e = 0; e < 4; ++e) vb[buf][e][u] = f[e];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int cb = 0; cb < UB::NBLK; ++cb) {
                            const i32x4 f = ob.template frag_m<UB::RV>(sb, wn * WTN + cb * UB::BLK, kb, e, lane);
#pragma unroll
                            for (int v = 0; v < UB::RV; ++v) vb[buf][e][cb * UB::RV + v] = f[v];
                        }
                }
            };
            constexpr int RA = AK ? NA : 4 * UA::NBLK, RB_ = BKM ? NB : 4 * UB::NBLK;   // LDS reads per step
            read(0, 0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                __builtin_amdgcn_sched_barrier(0);
                oa.issue(A, na, lda, m0, nk0, nst, wave, g * OA::IPW / NG, (g + 1) * OA::IPW / NG);
                ob.issue(B, nb, ldb, n0, nk0, nst + OA::BYTES, wave, g * OB::IPW / NG, (g + 1) * OB::IPW / NG);
                if (g + 1 < NG) read(g + 1, (g + 1) & 1);
                const int b = g & 1;
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < NA; ++i)
#pragma unroll
                        for (int j = 0; j < NB; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(va[b][e][i]),
                                                                              __int_as_float(vb[b][e][j]), acc[i][j], 0, 0, 0);
                if (g + 1 < NG) interleave<4 * NA * NB, RA + RB_, 0, 0>();
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vmcnt<0>();   // the empty loads past the range have landed too
    }

    // Store the C tile at (m0, n0).  D row r of unit u maps to tile row
    // UA::row(u, r); likewise columns.
    // COHERENT: write with device-scope cache policy (partial tiles of the
    // stream-K kernel, read by a workgroup that may sit on another XCD).
    // With EPI and p.epi set the tile goes through the elementwise epilogue
    // via LDS, which must be free (smem = the kernel's LDS ring); ROLLED as
    // for store_tile_via_lds.
    template <bool COHERENT = false, bool EPI = true, bool ROLLED = false>
    __device__ static __forceinline__ void store(const Params& p, int m0, int n0, const Acc& acc, int lane,
                                                 int wave, char* smem = nullptr)
    {
        const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(p.C, (short)0, 0x7fffffff, kBufferFlags);
        const int wm = wave / WN, wn = wave % WN;
        const int rm0 = m0 + wm * WTM, cn0 = n0 + wn * WTN;
        if (!COHERENT && EPI && p.epi) {
            store_tile_via_lds<TO, BM, BN, NT, NA * NB * 16, SMEM, ROLLED>(
                p, smem, m0, n0, wave * 64 + lane, [&](int v) { return acc[v / (NB * 16)][(v / 16) % NB][v % 16]; },
                [&](int v, int& r, int& c) {
                    const int i = v / (NB * 16), j = (v / 16) % NB, q = v % 16;
                    r = wm * WTM + UA::row(i, (q / 4) * 8 + (lane / 32) * 4 + (q % 4));
                    c = wn * WTN + UB::row(j, lane % 32);
                });
            return;
        }
        if constexpr (!AK && !BKM && TO == Out::F32 && UA::RV == 4 && UB::RV == 4) {
            // Both interleaved: for register index i a lane holds rows 4r .. 4r+3 of
            // each 128-row block and columns 4c .. 4c+3 -> 128-bit row stores.
#pragma unroll
            for (int ca = 0; ca < NA / 4; ++ca)
#pragma unroll
                for (int cbk = 0; cbk < NB / 4; ++cbk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int r = (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
                        const int c = lane % 32;
                        const int n = cn0 + cbk * 128 + 4 * c;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int m = rm0 + ca * 128 + 4 * r + v;
                            f32x4 o = {acc[ca * 4 + v][cbk * 4 + 0][i], acc[ca * 4 + v][cbk * 4 + 1][i],
                                       acc[ca * 4 + v][cbk * 4 + 2][i], acc[ca * 4 + v][cbk * 4 + 3][i]};
                            if (COHERENT) {
                                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o), cr,
                                                                       (m * BN + n) * 4, 0, kDeviceCoherent);
                            } else if (m < p.M) {
                                float* dst = (float*)p.C + (int64_t)m * p.ldc + n;
                                // 128-bit stores only where C and ldc are 16-byte
                                // aligned (never in the element-by-element configs).
                                if (VEC && p.c_vec && n + 3 < p.N) {
                                    *(f32x4*)dst = o;
                                } else {
#pragma unroll
                                    for (int w = 0; w < 4; ++w)
                                        if (n + w < p.N) dst[w] = o[w];
                                }
                            }
                        }
                    }
        } else if constexpr (!BKM && UB::RV > 1 && TO == Out::F32 && !COHERENT && !ROLLED) {
            // B interleaved (columns RV * c + v of a block in units v = 0 ..
            // RV-1): for each row a lane holds RV consecutive columns, one
            // 64- or 128-bit store, whatever A's layout.  Not in the
            // persistent stream-K kernel's 256x256 tiles (ROLLED): inside its
            // tile loop this form put the accumulators on the stack (8-13 KB
            // per lane), so it keeps the element stores below.
            constexpr int RV = UB::RV;
            typedef float f32xr __attribute__((ext_vector_type(RV)));
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int cb = 0; cb < UB::NBLK; ++cb)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int m = rm0 + UA::row(i, (q / 4) * 8 + (lane / 32) * 4 + (q % 4));
                        const int n = cn0 + cb * UB::BLK + RV * (lane % 32);
                        f32xr o;
#pragma unroll
                        for (int v = 0; v < RV; ++v) o[v] = acc[i][cb * RV + v][q];
                        float* dst = (float*)p.C + (int64_t)m * p.ldc + n;
                        if (m < p.M) {
                            if (VEC && p.c_vec && n + RV - 1 < p.N) {
                                *(f32xr*)dst = o;
                            } else {
#pragma unroll
                                for (int v = 0; v < RV; ++v)
                                    if (n + v < p.N) dst[v] = o[v];
                            }
                        }
                    }
        } else if constexpr (COHERENT) {
            // Whole tile, row pitch BN: Units::row is linear in its row
            // argument, so each element's offset is a per-lane part plus a
            // compile-time constant.
            static_assert(BN % 4 == 0, "row pitch");
            const int voff = ((rm0 + UA::row(0, (lane / 32) * 4)) * BN + cn0 + UB::row(0, lane % 32)) * 4;
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int soff = (UA::row(i, (q / 4) * 8 + q % 4) * BN + UB::row(j, 0)) * 4;
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(acc[i][j][q]), cr, voff, soff,
                                                              kDeviceCoherent);
                    }
        } else {
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int r = (q / 4) * 8 + (lane / 32) * 4 + (q % 4);
                        const int m = rm0 + UA::row(i, r);
                        const int n = cn0 + UB::row(j, lane % 32);
                        if (m < p.M && n < p.N) store_out<TO>(p.C, (int64_t)m * p.ldc + n, acc[i][j][q]);
                    }
        }
    }

    static constexpr int PART_BYTES = BM * BN * 4;   // one partial tile, fp32 row-major
};

template <Out TO, int BM, int BN, int BK, int WM, int WN, int STAGES, bool AK, bool BKM, bool VEC>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_f32dma_kernel(Params p)
{
    using KT = F32Dma<TO, BM, BN, BK, WM, WN, STAGES, AK, BKM, VEC>;
    __shared__ __attribute__((aligned(1024))) char smem[KT::SMEM];

    select_batch(p);
    // wave index as a wave-uniform (scalar) value: the LDS addresses of the
    // direct loads (M0) then need no v_readfirstlane per load.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    typename KT::OA oa;
    typename KT::OB ob;
    oa.init(wave, lane, p.lda);
    ob.init(wave, lane, p.ldb);

    typename KT::Acc acc;
    KT::zero(acc);
    KT::mainloop(p, smem, oa, ob, m0, n0, 0, (p.K + BK - 1) / BK, acc, tid, lane, wave);
    KT::store(p, m0, n0, acc, lane, wave, smem);
}

// SK: the persistent stream-K kernel.  VEC = false: element-aligned operands
// (4-byte direct loads).
template <Out TO, int BM, int BN, int BK, int WM, int WN, int STAGES, bool SK = false, bool VEC = true>
struct F32DmaInst {
    template <bool AK, bool BKM>
    static hipError_t go(const Params& p, hipStream_t s)
    {
        Params copy = p;
        void* args[] = {&copy};
        if constexpr (SK)
            return hipLaunchKernel((const void*)&gemm_sk_kernel<F32Dma<TO, BM, BN, BK, WM, WN, STAGES, AK, BKM>>,
                                   dim3((unsigned)p.grid), dim3(WM * WN * 64), args, 0, s);
        return hipLaunchKernel((const void*)&gemm_f32dma_kernel<TO, BM, BN, BK, WM, WN, STAGES, AK, BKM, VEC>,
                               dim3((unsigned)(p.tiles_m * p.tiles_n), (unsigned)p.batch), dim3(WM * WN * 64), args, 0, s);
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

// Launcher of the fp32 split-k configs (gemm_split_kernel, gemm_split_reduce).
template <Out TO, int BM, int BN, int BK, int WM, int WN, int STAGES>
struct F32DmaSplitInst {
    static hipError_t launch(int layout, const Params& p, hipStream_t s)
    {
        switch (layout) {
        case 0: return launch_split<F32Dma<TO, BM, BN, BK, WM, WN, STAGES, true, true>>(p, s);
        case 1: return launch_split<F32Dma<TO, BM, BN, BK, WM, WN, STAGES, true, false>>(p, s);
        case 2: return launch_split<F32Dma<TO, BM, BN, BK, WM, WN, STAGES, false, true>>(p, s);
        default: return launch_split<F32Dma<TO, BM, BN, BK, WM, WN, STAGES, false, false>>(p, s);
        }
    }
};

}  // namespace mg
