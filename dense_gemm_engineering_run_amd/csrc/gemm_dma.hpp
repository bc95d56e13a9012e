// gemm_dma.hpp -- gfx950 GEMM for 16-bit inputs with direct HBM -> LDS loads.
//
// Same operation and canonical form as gemm_kernel.hpp (C = A * B^T with C
// n-major; CuTe DSL Ampere SGEMM example, module docstring).  This variant is
// built around two gfx950 instructions:
//
//  * buffer_load_dwordx4 ... lds: each lane's 16 bytes go straight from HBM
//    into LDS at (M0 + 16 * lane), with no VGPR staging and no LDS write
//    instruction.  Bounds checking of the buffer resource writes zeros for
//    out-of-range lanes.  The loads of one k-tile for both operands are issued
//    STAGES-1 tiles ahead into a ring of STAGES LDS buffers (or, for A, two
//    tiles ahead into 3 buffers while B uses 2; the multistage
//    shared-memory pipeline of the SGEMM example, mainloop comment), so several
//    hundred KB per CU are in flight and the one barrier per k-tile both
//    publishes tile t and frees the stage that tile t-1 used.
//  * ds_read_b64_tr_b16: a transposing LDS read.  Within each 16-lane group,
//    lane j receives element (j mod 4) of the 8-byte values addressed by lanes
//    4r + j/4, r = 0..3.  When lane s addresses row k0 + s/4, column
//    m0 + 4 (s mod 4) of an m-contiguous tile, lane j receives
//    A[k0 + r][m0 + j] for r = 0..3: four consecutive k of one row, the MFMA
//    operand order.  Operands whose contiguous index is m (or n) therefore
//    stay m-contiguous in LDS and are transposed on the read.
//
// LDS layouts (16-byte chunks XOR-swizzled for gfx950's 256-byte bank window):
//  k-contiguous operand: [ROWS][BK]; 16 lanes reading one logical chunk of 16
//    consecutive rows hit 16 distinct bank positions (as in gemm_kernel.hpp).
//  m-contiguous operand: [BK][ROWS]; a transposing read touches 4 rows x 64 B
//    (32x32x16 fragments) or 8 rows x 32 B (16x16x32) per 32 lanes, so row k's
//    chunks are XORed with a key that spreads those rows over the 16 chunk
//    positions (DmaOperand::mkey).
//
// K edge: rows k >= K of an m-contiguous operand lie outside its extent and
// read as zeros.  For a k-contiguous operand the elements k >= K of the last,
// partial k-tile hold whatever follows in memory (padding, possibly NaN), so
// after that tile lands they are overwritten with zeros in LDS, for both
// operands, before any wave reads it.
#pragma once

#include "gemm_kernel.hpp"

namespace mg {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Workgroup barrier without a memory fence: ordering of this workgroup's LDS
// traffic is ensured by explicit waits; the empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xf00);
}

// One operand's k-tile in the LDS ring, loaded with direct-to-LDS buffer loads.
// MI: the MFMA tile the fragments feed (it decides the m-contiguous swizzle).
template <int ROWS, int BK, int NWAVES, bool KMAJ, int MI_ = 32>
struct DmaOperand {
    static constexpr int ES = 2, CE = 8;
    static constexpr int BYTES = ROWS * BK * ES;
    static constexpr int IPW = BYTES / 1024 / NWAVES;        // 1 KB loads per wave per tile
    static_assert(BYTES % (1024 * NWAVES) == 0, "tile must split into 1 KB loads per wave");
    // k-contiguous layout
    static constexpr int CPR = BK / CE, RB = BK * ES;
    // m-contiguous layout
    static constexpr int RCH = ROWS * ES / 16, RBM = ROWS * ES;
    static constexpr int MRPW = RCH >= 16 ? 1 : 16 / RCH;   // rows per bank window
    static constexpr int MXR = (RCH >= 16 ? 16 : RCH) / 4;  // distinct 4-chunk offsets

    int voff[IPW];

    // Chunk XOR of row k of an m-contiguous tile.  A transposing read of a
    // 32x32x16 fragment touches, per 32 lanes, 4 rows x 4 chunks (rows k0 ..
    // k0+3): XOR with 4 (k mod 4) gives them 4 disjoint chunk groups.  A
    // 16x16x32 fragment touches 8 rows x 2 chunks (rows k0 .. k0+3 and
    // k0+8 .. k0+11): XOR with 2 ((k mod 4) + 4 ((k / 8) mod 2)) gives them
    // 8 disjoint chunk pairs; the 32x32 key would put rows k and k+8 on the
    // same banks (measured: SQ_LDS_BANK_CONFLICT at a quarter of the LDS
    // cycles per such operand).  Rows narrower than the bank window keep the
    // 32x32 key.
    __device__ static __forceinline__ int mkey(int k)
    {
        if constexpr (MI_ == 16 && RCH >= 16) return 2 * ((k & 3) | ((k >> 1) & 4));
        else return 4 * ((k / MRPW) % MXR);
    }

    __device__ __forceinline__ void init(int wave, int lane, int64_t ld)
    {
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int slot = (wave * IPW + j) * 64 + lane;    // 16-byte LDS slot
            if (KMAJ) {
                const int row = slot / CPR, phys = slot % CPR;
                const int c = swz_chunk<CPR, true>(row, phys);  // XOR is its own inverse
                voff[j] = (int)(row * ld * ES) + c * 16;
            } else {
                const int k = slot / RCH, phys = slot % RCH;
                const int c = phys ^ mkey(k);
                voff[j] = (int)(k * ld * ES) + c * 16;
            }
        }
    }

    // Issue this wave's loads of the tile at (row0, k0) into `lds_tile`.
    // The loads are written as inline assembly so that the compiler does not
    // track their LDS writes: it would otherwise wait for all of them (vmcnt(0))
    // before LDS reads it cannot prove independent, draining the ring.  The
    // kernel orders them itself with wait_vmcnt and a barrier.
    __device__ __forceinline__ void issue(const char* base, uint64_t bytes, int64_t ld, int row0,
                                          int k0, char* lds_tile, int wave, int j0 = 0, int j1 = IPW)
    {
        const int64_t origin = KMAJ ? ((int64_t)row0 * ld + k0) * ES : ((int64_t)k0 * ld + row0) * ES;
        const uint64_t rem = (uint64_t)origin < bytes ? bytes - (uint64_t)origin : 0;
        const uint64_t addr = (uint64_t)(base + origin);
        i32x4 rs;   // buffer resource: base, stride 0, num_records, raw 32-bit format
        rs[0] = (int)(uint32_t)addr;
        rs[1] = (int)((uint32_t)(addr >> 32) & 0xffffu);
        rs[2] = (int)(rem > 0xffffffffull ? 0xffffffffu : (uint32_t)rem);
        rs[3] = kBufferFlags;
        const uint32_t lds0 =
            (uint32_t)(uintptr_t)(lds_char*)lds_tile + (uint32_t)(wave * IPW * 1024);
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            if (j < j0 || j >= j1) continue;
            asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :
                         : "s"(__builtin_amdgcn_readfirstlane(lds0 + j * 1024)), "v"(voff[j]),
                           "s"(rs)
                         : "memory", "m0");
        }
    }

    // MFMA fragment: rows rbase .. rbase+MI-1 of the tile, k-group starting at kb.
    template <int MI>
    __device__ static __forceinline__ i32x4 frag(const char* t, int rbase, int kb, int lane)
    {
        if constexpr (KMAJ) {
            const int row = rbase + lane % MI;
            const int c = kb / CE + lane / MI;
            return *(const i32x4*)(t + row * RB + swz_chunk<CPR, true>(row, c) * 16);
        } else {
            const int g = lane / 16, s = lane % 16;
            int m, k;
            if constexpr (MI == 32) {
                m = rbase + 16 * (g % 2) + 4 * (s % 4);
                k = kb + 8 * (g / 2) + s / 4;
            } else {
                m = rbase + 4 * (s % 4);
                k = kb + 8 * g + s / 4;
            }
            const int k1 = k + 4;
            const int c = m / 8, w = (m % 8) * 2;
            const lds_char* p0 = (const lds_char*)(t + k * RBM + ((c ^ mkey(k)) * 16) + w);
            const lds_char* p1 = (const lds_char*)(t + k1 * RBM + ((c ^ mkey(k1)) * 16) + w);
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
            i32x4 r;
            r[0] = (int)(((uint32_t)(uint16_t)lo[0]) | ((uint32_t)(uint16_t)lo[1] << 16));
            r[1] = (int)(((uint32_t)(uint16_t)lo[2]) | ((uint32_t)(uint16_t)lo[3] << 16));
            r[2] = (int)(((uint32_t)(uint16_t)hi[0]) | ((uint32_t)(uint16_t)hi[1] << 16));
            r[3] = (int)(((uint32_t)(uint16_t)hi[2]) | ((uint32_t)(uint16_t)hi[3] << 16));
            return r;
        }
    }

    // Zero the elements k >= kvalid of every row of a k-contiguous tile (the
    // partial last k-tile), working with all NT threads of the workgroup.
    template <int NT>
    __device__ static __forceinline__ void zero_tail(char* t, int kvalid, int tid)
    {
        if constexpr (KMAJ) {
            const int c0 = kvalid / CE;
#pragma unroll 1
            for (int idx = tid; idx < ROWS * CPR; idx += NT) {
                const int row = idx / CPR, c = idx % CPR;
                if (c < c0) continue;
                i32x4* q = (i32x4*)(t + row * RB + swz_chunk<CPR, true>(row, c) * 16);
                if (c * CE >= kvalid) {
                    *q = i32x4{0, 0, 0, 0};
                } else {
                    i32x4 v = *q;
                    *q = mask_k<In::F16>(v, c * CE, kvalid);   // 16-bit element mask
                }
            }
        }
    }
};

// The pieces of the kernel: the main loop over a range of k-tiles of one C
// tile, and the ways to store the tile (so that the persistent stream-K
// kernel can run partial k-ranges with the same loop).
// STAGES: depth of the A ring; SBS: depth of the B ring (the same, or one
// less with two B stages: A, streamed from HBM, is then issued two k-tiles
// ahead and B, read from the caches, one; the 2 MB B panel of a tall-skinny
// problem stays in L2 while A needs every byte in flight that LDS can hold).
template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI, int STAGES, bool AK, bool BKM,
          int SBS = STAGES>
struct Dma16 {
    static_assert(TI != In::F32, "direct-to-LDS kernel is for 16-bit inputs");
    static constexpr int TILE_M = BM, TILE_N = BN, TILE_K = BK;
    static constexpr Out OUT = TO;
    static constexpr int NW = WM * WN, NT = NW * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / MI, TN = WTN / MI;
    static constexpr int KG = MI == 32 ? 16 : 32;      // k per MFMA
    static constexpr int NG = BK / KG;                 // k-groups per tile
    static constexpr int R = MI == 32 ? 16 : 4;        // accumulators per MFMA tile and lane
    using OA = DmaOperand<BM, BK, NW, AK, MI>;
    using OB = DmaOperand<BN, BK, NW, BKM, MI>;
    static constexpr int SA = STAGES, SB = SBS;        // ring depths
    static constexpr int DA = SA - 1, DB = SB - 1;     // k-tiles issued ahead
    static_assert(SA == SB || (SA == 3 && SB == 2), "A ring as deep as B's, or 3 A and 2 B stages");
    static constexpr int STAGE = OA::BYTES + OB::BYTES;
    static constexpr int LPT = OA::IPW + OB::IPW;      // loads per wave per tile
    static constexpr int SMEM = SA * OA::BYTES + SB * OB::BYTES;
    // Loads issued after tile t's B loads (each k-tile issues B first, then
    // A): those may still be in flight when tile t is waited for.
    static constexpr int WAIT = (DA == DB ? 0 : OA::IPW) + (DB - 1) * LPT;
    static_assert(BK % KG == 0, "BK must be a multiple of the MFMA k");
    static_assert(SB >= 2 && SMEM <= 160 * 1024, "LDS budget");
    static_assert(WAIT < 64, "vmcnt range");
    using AccT = typename std::conditional<MI == 32, f32x16, f32x4>::type;
    typedef AccT Acc[TM][TN];
    static constexpr int PART_BYTES = BM * BN * 4;     // one partial tile, fp32 row-major

    // LDS of k-tile i (counted from the first tile of a range) of each
    // operand: with equal rings, stage i mod SA holds A then B; otherwise the
    // A ring comes first and the B ring after it.
    __device__ static __forceinline__ char* a_stage(char* smem, int i)
    {
        if constexpr (SA == SB) return smem + (i % SA) * STAGE;
        else return smem + (i % SA) * OA::BYTES;
    }
    __device__ static __forceinline__ char* b_stage(char* smem, int i)
    {
        if constexpr (SA == SB) return smem + (i % SB) * STAGE + OA::BYTES;
        else return smem + SA * OA::BYTES + (i % SB) * OB::BYTES;
    }

    __device__ static __forceinline__ void zero(Acc& acc)
    {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = AccT{};
    }

    // Tile-local row and column of accumulator q of MFMA tile (i, j).
    __device__ static __forceinline__ int row(int wm, int i, int q, int lane)
    {
        return wm * WTM + i * MI + (MI == 32 ? (q / 4) * 8 + (lane / 32) * 4 + (q % 4) : (lane / 16) * 4 + q);
    }
    __device__ static __forceinline__ int col(int wn, int j, int lane) { return wn * WTN + j * MI + (lane % MI); }

    // Accumulate k-tiles [kt0, kt1) of the C tile at (m0, n0) into acc.  The
    // LDS ring must be free on entry (no wave still reading it); on return
    // every load has landed.  gemm_dma_kernel writes the same loop out for the
    // whole k-range (see there why); the two must stay in step.
    __device__ static __forceinline__ void mainloop(const Params& p, char* smem, OA& oa, OB& ob, int m0, int n0,
                                                    int kt0, int kt1, Acc& acc, int tid, int lane, int wave)
    {
        const int wm = wave / WN, wn = wave % WN;
        const int nkt = (p.K + BK - 1) / BK;
        const int kvalid_last = p.K - (nkt - 1) * BK;
        const bool ragged = kvalid_last != BK;
        // Operand fields as locals (the DMA asm statements clobber memory).
        const char* const A = p.A;
        const char* const B = p.B;
        const uint64_t a_bytes = p.a_bytes, b_bytes = p.b_bytes;
        const int64_t lda = p.lda, ldb = p.ldb;

        // Every k-tile issues the loads of the tiles DA (A) and DB (B) ahead,
        // also past the end of the range: those get an empty extent
        // (num_records 0) and write zeros into a stage that no later tile
        // reads.  No branch precedes each k-group's loads, and the number of
        // loads in flight is the same for every tile.
        if constexpr (DA == DB) {
#pragma unroll
            for (int s = 0; s < DA; ++s) {
                const bool live = kt0 + s < kt1;
                oa.issue(A, live ? a_bytes : 0, lda, m0, (kt0 + s) * BK, a_stage(smem, s), wave);
                ob.issue(B, live ? b_bytes : 0, ldb, n0, (kt0 + s) * BK, b_stage(smem, s), wave);
            }
        } else {
            // A one tile further ahead: A(0), then B(s), A(s + 1) as the loop does.
            oa.issue(A, kt0 < kt1 ? a_bytes : 0, lda, m0, kt0 * BK, a_stage(smem, 0), wave);
#pragma unroll
            for (int s = 0; s < DB; ++s) {
                ob.issue(B, kt0 + s < kt1 ? b_bytes : 0, ldb, n0, (kt0 + s) * BK, b_stage(smem, s), wave);
                oa.issue(A, kt0 + s + 1 < kt1 ? a_bytes : 0, lda, m0, (kt0 + s + 1) * BK, a_stage(smem, s + 1), wave);
            }
        }

        for (int t = kt0; t < kt1; ++t) {
            const int r = t - kt0;
            // Tile t has landed once the loads issued after its B loads are
            // all that remain outstanding.
            wait_vmcnt<WAIT>();
            char* sa = a_stage(smem, r);
            char* sb = b_stage(smem, r);
            if (t == nkt - 1 && ragged && (AK || BKM)) {
                bare_barrier();
                oa.template zero_tail<NT>(sa, kvalid_last, tid);
                ob.template zero_tail<NT>(sb, kvalid_last, tid);
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the zeros are written
            }
            // A bare barrier: this wave's loads of tile t are complete (the vmcnt
            // wait above), so after it every wave's part of tile t is in LDS.  A
            // fenced __syncthreads() would also wait for the later tiles still in
            // flight.
            bare_barrier();
            const uint64_t na = t + DA < kt1 ? a_bytes : 0, nb = t + DB < kt1 ? b_bytes : 0;
            char* nsa = a_stage(smem, r + DA);
            char* nsb = b_stage(smem, r + DB);
            const int nka = (t + DA) * BK, nkb = (t + DB) * BK;

            i32x4 fa[2][TM], fb[2][TN];
            auto read = [&](int g, int buf) {
#pragma unroll
                for (int i = 0; i < TM; ++i) fa[buf][i] = oa.template frag<MI>(sa, wm * WTM + i * MI, g * KG, lane);
#pragma unroll
                for (int j = 0; j < TN; ++j) fb[buf][j] = ob.template frag<MI>(sb, wn * WTN + j * MI, g * KG, lane);
            };
            read(0, 0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                __builtin_amdgcn_sched_barrier(0);
                // This k-group's share of the next loads (into the stages tile
                // t-1 used, which every wave has left at the barrier above),
                // spread over the first NI k-groups: spread, so the loads do
                // not leave in one burst after the barrier; within the first
                // half of the tile, so that with two stages the last share
                // still has half a tile to land (measured: 2-4 % faster than
                // spreading over all).  With unequal rings all of B goes
                // before any of A (the order WAIT counts on).
                constexpr int NI = NG < 2 ? NG : 2;
                if constexpr (DA == DB) {
                    if (g < NI) {
                        oa.issue(A, na, lda, m0, nka, nsa, wave, g * OA::IPW / NI, (g + 1) * OA::IPW / NI);
                        ob.issue(B, nb, ldb, n0, nkb, nsb, wave, g * OB::IPW / NI, (g + 1) * OB::IPW / NI);
                    }
                } else {
                    if (g == 0) ob.issue(B, nb, ldb, n0, nkb, nsb, wave);
                    if (g == NI - 1) oa.issue(A, na, lda, m0, nka, nsa, wave);
                }
                if (g + 1 < NG) read(g + 1, (g + 1) & 1);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) mfma_step<TI, MI>(fa[g & 1][i], fb[g & 1][j], acc[i][j]);
                if (g + 1 < NG) interleave<TM * TN, (AK ? 1 : 2) * TM + (BKM ? 1 : 2) * TN, 0, 0>();
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vmcnt<0>();   // the empty loads past the range have landed too
    }

    // The tile through LDS and the elementwise epilogue (the LDS ring must be
    // free); ROLLED as for store_tile_via_lds.
    template <bool ROLLED = false>
    __device__ static __forceinline__ void store_staged(const Params& p, char* smem, int m0, int n0, const Acc& acc,
                                                        int tid, int lane, int wave)
    {
        const int wm = wave / WN, wn = wave % WN;
        store_tile_via_lds<TO, BM, BN, NT, TM * TN * R, SMEM, ROLLED>(
            p, smem, m0, n0, tid, [&](int v) { return acc[v / (TN * R)][(v / R) % TN][v % R]; },
            [&](int v, int& r, int& c) {
                const int i = v / (TN * R), j = (v / R) % TN, q = v % R;
                c = col(wn, j, lane);
                r = row(wm, i, q, lane);
            });
    }

    // Direct predicated stores of the accumulators, converted to TO.
    __device__ static __forceinline__ void store_direct(const Params& p, int m0, int n0, const Acc& acc, int lane,
                                                        int wave)
    {
        const int wm = wave / WN, wn = wave % WN;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n0 + wn * WTN + j * MI + (lane % MI);
                const int mb = m0 + wm * WTM + i * MI;
                if constexpr (MI == 32) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = mb + (r / 4) * 8 + (lane / 32) * 4 + (r % 4);
                        if (m < p.M && n < p.N) store_out<TO>(p.C, (int64_t)m * p.ldc + n, acc[i][j][r]);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = mb + (lane / 16) * 4 + r;
                        if (m < p.M && n < p.N) store_out<TO>(p.C, (int64_t)m * p.ldc + n, acc[i][j][r]);
                    }
                }
            }
        }
    }

    // The plain store through LDS, each wave on its own.  In the accumulator
    // layout a store instruction writes 16 (or 32) consecutive columns of 4
    // rows: row pieces of 64 bytes for fp32 output, 32 for 16-bit.  Here each
    // wave writes its WTM x WTN block of C, converted to TO, into its share of
    // the (free) ring, row-major, and reads it back in 16-byte chunks, 16-32
    // lanes per row: row pieces of WTN * sizeof(TO) bytes, a quarter or less
    // of the store instructions.  Measured against the direct store: equal on
    // fp16 4096^3 with A and B k-contiguous, 1-2 % faster for m/n-contiguous
    // operands and 16-bit outputs (the store phase of a kernel with one tile
    // per CU, ~11 µs there, is mostly C's write-back, which neither form
    // hides).  Rows are padded so that the four (or two) row groups of an
    // MFMA tile's accumulators fall on disjoint banks.
    // Needs every wave's loads landed and its ring reads done (the caller's
    // barrier) and C allowing 16-byte stores (p.c_vec).
    static constexpr int OBY = TO == Out::F32 ? 4 : 2;                 // bytes per output element
    static constexpr int SPITCH = WTN * OBY + (MI == 16 ? 16 : 32);     // staged row pitch
    static constexpr int SHARE = SMEM / NW;                             // LDS bytes per wave
    static constexpr int SCPR = WTN * OBY / 16;                         // 16-byte chunks per row
    static_assert(SCPR <= 64 && 64 % SCPR == 0, "a read instruction covers whole rows");
    static constexpr int rows_per_pass()
    {
        for (int d = WTM; d >= MI; d -= MI)
            if (WTM % d == 0 && d * SPITCH <= SHARE) return d;
        return 0;
    }
    static constexpr int RPP = rows_per_pass();
    // Whether a share of the ring holds a pass of whole MFMA row blocks (else
    // the kernels store directly).
    static constexpr bool ROWS_OK = RPP >= MI && RPP % (64 / SCPR) == 0;

    __device__ static __forceinline__ void store_rows(const Params& p, char* smem, int m0, int n0, const Acc& acc,
                                                      int lane, int wave)
    {
        static_assert(ROWS_OK, "LDS share too small for the staged store");
        const int wm = wave / WN, wn = wave % WN;
        char* w = smem + wave * SHARE;
        constexpr int EPC = 16 / OBY;            // elements per chunk
        constexpr int RPI = 64 / SCPR;           // rows per read instruction
        const int mb = m0 + wm * WTM, nb = n0 + wn * WTN;
#pragma unroll
        for (int pass = 0; pass < WTM / RPP; ++pass) {
#pragma unroll
            for (int i = pass * RPP / MI; i < (pass + 1) * RPP / MI; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < R; ++q) {
                        const int r = row(0, i, q, lane) - pass * RPP, c = col(0, j, lane);
                        char* d = w + r * SPITCH + c * OBY;
                        const float v = acc[i][j][q];
                        if constexpr (TO == Out::F32) *(float*)d = v;
                        else if constexpr (TO == Out::F16) *(_Float16*)d = (_Float16)v;
                        else *(uint16_t*)d = __builtin_bit_cast(uint16_t, (__bf16)v);
                    }
#pragma unroll
            for (int r0 = 0; r0 < RPP; r0 += RPI) {
                const int r = r0 + lane / SCPR, ch = lane % SCPR;
                const i32x4 v = *(const i32x4*)(w + r * SPITCH + ch * 16);
                const int m = mb + pass * RPP + r, n = nb + ch * EPC;
                if (m >= p.M) continue;
                char* dst = p.C + ((int64_t)m * p.ldc + n) * OBY;
                if (n + EPC <= p.N) {
                    *(i32x4*)dst = v;
                } else {
#pragma unroll
                    for (int e = 0; e < EPC; ++e)
                        if (n + e < p.N) {
                            if constexpr (OBY == 4) ((int*)dst)[e] = v[e];
                            else ((uint16_t*)dst)[e] = (uint16_t)((uint32_t)v[e / 2] >> (16 * (e % 2)));
                        }
                }
            }
        }
    }

    // Direct stores of the accumulators with C transposed (element (m, n) at
    // n * ldc + m, Params::c_trans): a lane's 4 accumulators of a 16x16x32
    // tile are 4 consecutive m of one n, so they go out as one vector.
    __device__ static __forceinline__ void store_direct_t(const Params& p, int m0, int n0, const Acc& acc,
                                                          int lane, int wave)
    {
        static_assert(MI == 16, "transposed store of 16x16x32 tiles");
        const int wm = wave / WN, wn = wave % WN;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n0 + wn * WTN + j * MI + (lane % MI);
                const int m = m0 + wm * WTM + i * MI + (lane / 16) * 4;
                if (n >= p.N) continue;
                const int64_t idx = (int64_t)n * p.ldc + m;
                if (p.c_vec && m + 3 < p.M) {
                    if constexpr (TO == Out::F32) {
                        *(f32x4*)((float*)p.C + idx) = acc[i][j];
                    } else {
                        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
                        uint16_t h[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            h[e] = TO == Out::F16 ? __builtin_bit_cast(uint16_t, (_Float16)acc[i][j][e])
                                                  : __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][e]);
                        *(u32x2*)((uint16_t*)p.C + idx) = u32x2{(unsigned)h[0] | ((unsigned)h[1] << 16),
                                                                (unsigned)h[2] | ((unsigned)h[3] << 16)};
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (m + r < p.M) store_out<TO>(p.C, idx + r, acc[i][j][r]);
                }
            }
        }
    }

    // The fp32 partial tile, row-major with pitch BN, at p.C, with
    // device-scope stores (read back by a workgroup that may sit on another
    // XCD).  row() is linear in q apart from a per-lane part, so each element's
    // offset is a per-lane VGPR plus a compile-time constant.
    __device__ static __forceinline__ void store_partial(const Params& p, const Acc& acc, int lane, int wave)
    {
        const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(p.C, (short)0, 0x7fffffff, kBufferFlags);
        const int wm = wave / WN, wn = wave % WN;
        const int voff = (row(wm, 0, 0, lane) * BN + col(wn, 0, lane)) * 4;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < R; ++q) {
                    const int dr = i * MI + (MI == 32 ? (q / 4) * 8 + (q % 4) : q);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(acc[i][j][q]), cr, voff,
                                                          (dr * BN + j * MI) * 4, kDeviceCoherent);
                }
    }

    // The stream-K kernel's interface: COHERENT -> the partial tile at p.C;
    // else the tile at (m0, n0), through the epilogue when EPI and p.epi
    // (ROLLED as for store_tile_via_lds).
    template <bool COHERENT = false, bool EPI = true, bool ROLLED = false>
    __device__ static __forceinline__ void store(const Params& p, int m0, int n0, const Acc& acc, int lane,
                                                 int wave, char* smem = nullptr)
    {
        if constexpr (COHERENT) {
            store_partial(p, acc, lane, wave);
        } else {
            if constexpr (EPI)
                if (p.epi) {
                    store_staged<ROLLED>(p, smem, m0, n0, acc, wave * 64 + lane, lane, wave);
                    return;
                }
            store_direct(p, m0, n0, acc, lane, wave);
        }
    }
};

// EPI: as for gemm_kernel (a separate instantiation for 16-bit outputs that
// run the elementwise epilogue).
template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI, int STAGES, bool AK, bool BKM, bool EPI,
          int SBS = STAGES>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_dma_kernel(Params p)
{
    using KT = Dma16<TI, TO, BM, BN, BK, WM, WN, MI, STAGES, AK, BKM, SBS>;
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

    // The main loop of KT::mainloop for the whole k-range, written out here
    // (the two must stay in step): through the engine's function, even with
    // the range fixed at compile time, the compiler gives each fragment its
    // own LDS base register instead of folding the fragment offsets into the
    // ds_read offsets -- 12 more instructions per k-tile, 2 % slower.  The
    // stream-K kernel, which needs arbitrary k-ranges, uses KT::mainloop.
    constexpr int NG = KT::NG, KG = KT::KG, TM = KT::TM, TN = KT::TN;
    constexpr int DA = KT::DA, DB = KT::DB, WAIT = KT::WAIT;
    constexpr int NT = KT::NT, WTM = KT::WTM, WTN = KT::WTN;
    using OA = typename KT::OA;
    using OB = typename KT::OB;
    const int wm = wave / WN, wn = wave % WN;
    const int nkt = (p.K + BK - 1) / BK;
    const int kvalid_last = p.K - (nkt - 1) * BK;
    const bool ragged = kvalid_last != BK;
    if constexpr (DA == DB) {
#pragma unroll
        for (int s = 0; s < DA; ++s) {
            const bool live = s < nkt;
            oa.issue(p.A, live ? p.a_bytes : 0, p.lda, m0, s * BK, KT::a_stage(smem, s), wave);
            ob.issue(p.B, live ? p.b_bytes : 0, p.ldb, n0, s * BK, KT::b_stage(smem, s), wave);
        }
    } else {
        oa.issue(p.A, nkt > 0 ? p.a_bytes : 0, p.lda, m0, 0, KT::a_stage(smem, 0), wave);
#pragma unroll
        for (int s = 0; s < DB; ++s) {
            ob.issue(p.B, s < nkt ? p.b_bytes : 0, p.ldb, n0, s * BK, KT::b_stage(smem, s), wave);
            oa.issue(p.A, s + 1 < nkt ? p.a_bytes : 0, p.lda, m0, (s + 1) * BK, KT::a_stage(smem, s + 1), wave);
        }
    }
    for (int t = 0; t < nkt; ++t) {
        wait_vmcnt<WAIT>();
        char* sa = KT::a_stage(smem, t);
        char* sb = KT::b_stage(smem, t);
        if (t == nkt - 1 && ragged && (AK || BKM)) {
            bare_barrier();
            oa.template zero_tail<NT>(sa, kvalid_last, tid);
            ob.template zero_tail<NT>(sb, kvalid_last, tid);
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the zeros are written
        }
        bare_barrier();
        const uint64_t na = t + DA < nkt ? p.a_bytes : 0, nb = t + DB < nkt ? p.b_bytes : 0;
        char* nsa = KT::a_stage(smem, t + DA);
        char* nsb = KT::b_stage(smem, t + DB);
        const int nka = (t + DA) * BK, nkb = (t + DB) * BK;
        i32x4 fa[2][TM], fb[2][TN];
        auto read = [&](int g, int buf) {
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[buf][i] = oa.template frag<MI>(sa, wm * WTM + i * MI, g * KG, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[buf][j] = ob.template frag<MI>(sb, wn * WTN + j * MI, g * KG, lane);
        };
        read(0, 0);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            __builtin_amdgcn_sched_barrier(0);
            constexpr int NI = NG < 2 ? NG : 2;
            if constexpr (DA == DB) {
                if (g < NI) {
                    oa.issue(p.A, na, p.lda, m0, nka, nsa, wave, g * OA::IPW / NI, (g + 1) * OA::IPW / NI);
                    ob.issue(p.B, nb, p.ldb, n0, nkb, nsb, wave, g * OB::IPW / NI, (g + 1) * OB::IPW / NI);
                }
            } else {
                if (g == 0) ob.issue(p.B, nb, p.ldb, n0, nkb, nsb, wave);
                if (g == NI - 1) oa.issue(p.A, na, p.lda, m0, nka, nsa, wave);
            }
            if (g + 1 < NG) read(g + 1, (g + 1) & 1);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) mfma_step<TI, MI>(fa[g & 1][i], fb[g & 1][j], acc[i][j]);
            if (g + 1 < NG) interleave<TM * TN, (AK ? 1 : 2) * TM + (BKM ? 1 : 2) * TN, 0, 0>();
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();   // the empty loads past the last tile have landed too

    // Epilogue (as in gemm_kernel): fp32 accumulators -> output type, predicated stores.
    if (TO == Out::F32 ? p.epi : EPI) {
        KT::store_staged(p, smem, m0, n0, acc, tid, lane, wave);
        return;
    }
    if constexpr (TO != Out::F32 && EPI) return;
    if (KT::ROWS_OK && p.c_vec) {
        bare_barrier();   // every wave's loads have landed (vmcnt above) and its ring reads are done
        if constexpr (KT::ROWS_OK) KT::store_rows(p, smem, m0, n0, acc, lane, wave);
    } else {
        KT::store_direct(p, m0, n0, acc, lane, wave);
    }
}

// Ping-pong schedule of the 8-wave configs (two groups of four waves; waves
// w and w + 4 share a SIMD).  Under the schedule of
// gemm_dma_kernel the two waves of a SIMD take the MFMA pipe in turn, the
// older first, so after each k-tile's barrier one of them soon waits at the
// next barrier while the other runs the rest of its MFMAs alone between LDS
// waits (measured with per-wave cycle counters at 4096^3: ~2800 cycles per
// k-tile for 2048 cycles of MFMA work).  Here the groups trade roles in
// phases one k-tile of MFMAs long: while group 0 multiplies tile t out of
// registers, group 1 issues its loads and reads tile t's fragments; then
// group 1 multiplies tile t while group 0 issues its loads and reads tile
// t + 1.  A barrier closes each phase, so every SIMD always has one wave
// whose operands are all in registers (~2340 cycles per k-tile).
//
// Loads: group 1 issues every A load (3-stage ring; tile t + 2 in phase A
// of tile t), group 0 every B load (2-stage ring; tile t + 2 in phase B of
// tile t).  Each goes into the slot of a tile that both groups have read
// and waited for (lgkmcnt(0)) before the barrier that opens the phase.
// Tile t + 1 is published by the barrier that closes phase A of tile t:
// before it group 0 waits for all its loads (B of t + 1) and group 1 for
// all but the last tile's (A of t + 2 may still be in flight).
// The accumulation order of every C element is that of gemm_dma_kernel
// (k-groups in order, tiles in order), so the two give identical bits.
template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI, bool AK, bool BKM, bool EPI>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_pp_kernel(Params p)
{
    using KT = Dma16<TI, TO, BM, BN, BK, WM, WN, MI, 3, AK, BKM, 2>;
    static_assert(WM * WN == 8, "two groups of four waves");
    constexpr int NG = KT::NG, KG = KT::KG, TM = KT::TM, TN = KT::TN, NT = KT::NT;
    constexpr int WTM = KT::WTM, WTN = KT::WTN;
    using LA = DmaOperand<BM, BK, 4, AK, MI>;     // loaded by group 1
    using LB = DmaOperand<BN, BK, 4, BKM, MI>;    // loaded by group 0
    constexpr int IA = LA::IPW, IB = LB::IPW;
    static_assert(LA::BYTES == KT::OA::BYTES && LB::BYTES == KT::OB::BYTES, "same LDS tiles as Dma16");
    __shared__ __attribute__((aligned(1024))) char smem[KT::SMEM];

    select_batch(p);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, gw = wave & 3;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nkt = (p.K + BK - 1) / BK;
    const int kvalid_last = p.K - (nkt - 1) * BK;
    // A k-contiguous operand's partial last tile is zeroed past K (an
    // m-contiguous one reads zeros there: those rows lie past its extent).
    const bool zero_last = (AK || BKM) && kvalid_last != BK;

    // A wave loads one operand only: one set of per-lane offsets (the
    // operand's own layout) serves it, 8 registers fewer than two would take.
    static_assert(IA == IB, "one offset set for either operand");
    int voff[IA];
    if (grp) {
        LA o;
        o.init(gw, lane, p.lda);
#pragma unroll
        for (int j = 0; j < IA; ++j) voff[j] = o.voff[j];
    } else {
        LB o;
        o.init(gw, lane, p.ldb);
#pragma unroll
        for (int j = 0; j < IB; ++j) voff[j] = o.voff[j];
    }
    // Loads past the last tile get an empty extent (zeros into a free slot),
    // so every phase has the same loads in flight.
    auto issue_a = [&](int s) {
        LA o;
#pragma unroll
        for (int j = 0; j < IA; ++j) o.voff[j] = voff[j];
        o.issue(p.A, s < nkt ? p.a_bytes : 0, p.lda, m0, s * BK, KT::a_stage(smem, s), gw);
    };
    auto issue_b = [&](int s) {
        LB o;
#pragma unroll
        for (int j = 0; j < IB; ++j) o.voff[j] = voff[j];
        o.issue(p.B, s < nkt ? p.b_bytes : 0, p.ldb, n0, s * BK, KT::b_stage(smem, s), gw);
    };

    typename KT::Acc acc;
    KT::zero(acc);
    i32x4 fa[NG][TM], fb[NG][TN];
    auto read_all = [&](int s) {
        const char* sa = KT::a_stage(smem, s);
        const char* sb = KT::b_stage(smem, s);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[g][i] = LA::template frag<MI>(sa, wm * WTM + i * MI, g * KG, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[g][j] = LB::template frag<MI>(sb, wn * WTN + j * MI, g * KG, lane);
        }
    };
    auto mfma_all = [&]() {
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) mfma_step<TI, MI>(fa[g][i], fb[g][j], acc[i][j]);
    };
    // The partial last k-tile: zeros past K in both operands, by the whole
    // workgroup, between the barrier that publishes the tile and any read.
    auto zero_tail = [&](int s) {
        LA::template zero_tail<NT>(KT::a_stage(smem, s), kvalid_last, tid);
        LB::template zero_tail<NT>(KT::b_stage(smem, s), kvalid_last, tid);
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the zeros are written
        bare_barrier();
    };

    if (grp) {
        issue_a(0);
        issue_a(1);
        wait_vmcnt<IA>();
    } else {
        issue_b(0);
        issue_b(1);
        wait_vmcnt<IB>();
    }
    bare_barrier();
    if (nkt == 1 && zero_last) zero_tail(0);
    if (!grp) {
        read_all(0);
        __builtin_amdgcn_s_waitcnt(0xc07f);
    }
    // One loop per group, two barriers per k-tile in each (so they pair up);
    // straight-line bodies keep fragments and accumulators in fixed registers.
    if (!grp) {
        for (int t = 0; t < nkt; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            mfma_all();                       // phase A: tile t
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<0>();                  // B of tile t + 1
            bare_barrier();
            if (t + 2 == nkt && zero_last) zero_tail(t + 1);
            __builtin_amdgcn_sched_barrier(0);
            issue_b(t + 2);                   // phase B: into tile t's B slot
            if (t + 1 < nkt) read_all(t + 1);
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_sched_barrier(0);
            bare_barrier();
        }
    } else {
        for (int t = 0; t < nkt; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            issue_a(t + 2);                   // phase A: into tile t-1's A slot
            read_all(t);
            __builtin_amdgcn_s_waitcnt(0xc07f);
            wait_vmcnt<IA>();                 // A of tile t + 1
            __builtin_amdgcn_sched_barrier(0);
            bare_barrier();
            if (t + 2 == nkt && zero_last) zero_tail(t + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_all();                       // phase B: tile t
            __builtin_amdgcn_sched_barrier(0);
            bare_barrier();
        }
    }
    wait_vmcnt<0>();

    if (TO == Out::F32 ? p.epi : EPI) {
        KT::store_staged(p, smem, m0, n0, acc, tid, lane, wave);
        return;
    }
    if constexpr (TO != Out::F32 && EPI) return;
    if (p.c_trans) {
        KT::store_direct_t(p, m0, n0, acc, lane, wave);
    } else if (KT::ROWS_OK && p.c_vec) {
        bare_barrier();   // every wave's loads have landed (vmcnt above) and its ring reads are done
        if constexpr (KT::ROWS_OK) KT::store_rows(p, smem, m0, n0, acc, lane, wave);
    } else {
        KT::store_direct(p, m0, n0, acc, lane, wave);
    }
}

template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI, int STAGES, int SBS = STAGES>
struct DmaInst {
    template <bool AK, bool BKM, bool EPI>
    static hipError_t go(const Params& p, hipStream_t s)
    {
        Params copy = p;
        void* args[] = {&copy};
        return hipLaunchKernel((const void*)&gemm_dma_kernel<TI, TO, BM, BN, BK, WM, WN, MI, STAGES, AK, BKM, EPI, SBS>,
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

// Launcher of the ping-pong configs: A k with B k, A m with B k and A m with
// B n run gemm_pp_kernel (the last with both operands read by transposing
// loads: 254 VGPRs, no spills).  A k with B n reaches this launcher only with
// an epilogue (without one the operands are swapped and C stored
// transposed, which gives A m with B k) and runs the 3 + 2-stage
// gemm_dma_kernel.
template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI>
struct PpInst {
    template <bool AK, bool BKM, bool EPI>
    static hipError_t go(const Params& p, hipStream_t s)
    {
        Params copy = p;
        void* args[] = {&copy};
        return hipLaunchKernel((const void*)&gemm_pp_kernel<TI, TO, BM, BN, BK, WM, WN, MI, AK, BKM, EPI>,
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
        case 2: return go<false, true>(p, s);
        case 3: return go<false, false>(p, s);
        default: return DmaInst<TI, TO, BM, BN, BK, WM, WN, MI, 3, 2>::launch(layout, p, s);
        }
    }
};

}  // namespace mg
