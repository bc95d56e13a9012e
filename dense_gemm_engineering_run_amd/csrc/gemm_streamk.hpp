// gemm_streamk.hpp -- the persistent stream-K kernel, over either tile engine
// (F32Dma for fp32 inputs, Dma16 for 16-bit inputs).  An engine provides the
// LDS ring (SMEM, OA, OB), the accumulators (Acc, zero), mainloop over a range
// of k-tiles, store<COHERENT, EPI> and PART_BYTES; partial tiles are fp32
// whatever the output type, and the workgroup that completes a tile converts.
#pragma once

#include "gemm_dma.hpp"

namespace mg {

// Persistent stream-K form of the direct-to-LDS kernels, for grids that would leave
// part of the chip idle in their last wave (the persistent, load-balanced
// tile scheduling of the Gluon multi-CTA tutorial, "Persistent kernels" and
// its cluster launch control scheduler, reshaped for CDNA's plain grid).
//
// p.grid workgroups run (a multiple of 8; workgroup w runs on XCD w mod 8).
//  * Tiles [0, sk_first) are data-parallel: logical id g (XCD-major rank of
//    w) takes tiles g, g + grid, ...
//  * The k-iterations of the remaining tiles, tile after tile, are split into
//    sk_wgs contiguous ranges (sk_base or sk_base + 1 iterations each), one
//    per stream-K id; consecutive ids share an XCD and every XCD gets
//    sk_wgs / 8 of them.  A workgroup whose range covers a whole tile stores
//    it directly.  A tile split over several workgroups is finished by the
//    last one to arrive: every contributor writes its partial tile (fp32,
//    row-major) to its workspace slot, waits until the writes are
//    acknowledged, then increments the tile's counter atomically; the one
//    that sees the count reach the contributor count adds the partial tiles
//    in contributor order, stores C and resets the counter to zero.  Nobody
//    waits for anybody, and the order of the sum depends only on the
//    schedule, so results are deterministic.
//
// Coherence: the XCDs' L2 caches are not coherent with each other.  Partial
// tiles are written and read with device-scope cache policy (sc1, the
// encoding the compiler gives agent-scope atomic loads and stores), and the
// counter is an agent-scope atomic issued only after every partial write of
// the workgroup has completed (s_waitcnt vmcnt(0), then the barrier), so no
// whole-L2 write-back or invalidate is needed.
template <class KT>
__global__ void __launch_bounds__(KT::NT)
gemm_sk_kernel(Params p)
{
    constexpr int BM = KT::TILE_M, BN = KT::TILE_N, BK = KT::TILE_K;
    constexpr Out TO = KT::OUT;
    // Tiles above 128 x 128 hold 256 accumulators per lane: their staged
    // epilogue keeps its loop over row bands rolled.
    constexpr bool kBigTile = BM * BN > 128 * 128;
    __shared__ __attribute__((aligned(1024))) char smem[KT::SMEM];
    __shared__ int arrived;

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = p.grid;
    const int xcd = blockIdx.x % 8, rank = blockIdx.x / 8;
    const int g = xcd * (G / 8) + rank;
    const int nkt = (p.K + BK - 1) / BK;

    typename KT::OA oa;
    typename KT::OB ob;
    oa.init(wave, lane, p.lda);
    ob.init(wave, lane, p.ldb);
    typename KT::Acc acc;

    // Stream-K id: sk_wgs is a multiple of 8 (or below 8: XCDs 0 .. sk_wgs-1).
    const int per_xcd = p.sk_wgs >= 8 ? p.sk_wgs / 8 : 1;
    const bool streams = rank < per_xcd && xcd * per_xcd + rank < p.sk_wgs;
    const int k = xcd * per_xcd + rank;

    const __amdgpu_buffer_rsrc_t wsr = __builtin_amdgcn_make_buffer_rsrc(p.sk_part, (short)0, 0x7fffffff, kBufferFlags);
    const int base = p.sk_base, rem = p.sk_rem;
    auto start = [&](int w) { return w * base + min(w, rem); };
    auto owner = [&](int i) {
        const int cut = rem * (base + 1);
        return i < cut ? i / (base + 1) : rem + (i - cut) / base;
    };
    // Work units: this workgroup's data-parallel tiles, then its stream-K range.
    int L = g;
    int it = streams ? start(k) : 0;
    const int end = streams ? start(k + 1) : 0;
    while (true) {
        int tile, kt0, kt1, s = -1;
        if (L < p.sk_first) {
            tile = L;
            kt0 = 0;
            kt1 = nkt;
            L += G;
        } else if (it < end) {
            s = it / nkt;
            kt0 = it - s * nkt;
            kt1 = min(nkt, kt0 + (end - it));
            tile = p.sk_first + s;
            it += kt1 - kt0;
        } else {
            break;
        }
        int tm, tn;
        raster(p, tile, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        KT::zero(acc);
        KT::mainloop(p, smem, oa, ob, m0, n0, kt0, kt1, acc, tid, lane, wave);
        if (kt0 == 0 && kt1 == nkt) {
            KT::template store<false, true, kBigTile>(p, m0, n0, acc, lane, wave, smem);
        } else {
            const int ts = s * nkt;
            const int gf = owner(ts), gl = owner(ts + nkt - 1);
            // Slot of contributor w for this tile: 2w when the tile is w's first
            // range piece, 2w + 1 when it is its last (w started in an earlier tile).
            auto slot = [&](int w) { return (2 * w + (start(w) >= ts ? 0 : 1)) * KT::PART_BYTES; };
            {
                Params q = p;                 // the partial tile, row-major BM x BN
                q.C = (char*)p.sk_part + slot(k);
                q.ldc = BN;
                KT::template store<true>(q, 0, 0, acc, lane, wave);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0)
                arrived = __hip_atomic_fetch_add(p.sk_count + s, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (arrived == gl - gf) {
                // Last to arrive: C = partial(gf) + ... + partial(gl).  Thread
                // tid owns the 16-byte chunks tid + NT*u of the row-major
                // tile; U chunks per batch keep U loads in flight.  Eight, not
                // more: the 128x128 kernels run two workgroups per CU within
                // 256 registers, and the 256x256 ones keep their loop state
                // and the epilogue's loads of old values and bias live here.
                constexpr int CH = BM * BN / 4 / KT::NT, U = CH < 8 ? CH : 8;
                static_assert(CH % U == 0, "reduction batches");
                auto part = [&](int w, int c) {
                    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         wsr, slot(w) + tid * 16, c * KT::NT * 16, kDeviceCoherent));
                };
#pragma unroll 1
                for (int b = 0; b < CH; b += U) {
                    f32x4 sum[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) sum[u] = part(gf, b + u);
                    for (int w = gf + 1; w <= gl; ++w) {
                        f32x4 t[U];
#pragma unroll
                        for (int u = 0; u < U; ++u) t[u] = part(w, b + u);
#pragma unroll
                        for (int u = 0; u < U; ++u) sum[u] += t[u];
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int idx = tid + (b + u) * KT::NT;
                        const int m = m0 + idx / (BN / 4), n = n0 + (idx % (BN / 4)) * 4;
                        if (m < p.M) store4<TO>(p, m, n, sum[u]);   // the elementwise epilogue, if any
                    }
                }
                if (tid == 0) __hip_atomic_store(p.sk_count + s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        bare_barrier();                       // the LDS ring (and `arrived`) are reused next
    }
}

// Split-k form of the direct-to-LDS kernels (configs named `… split`), for
// problems with few tiles and a long K.  The k-tiles of every C tile are cut
// into p.split contiguous ranges, one workgroup per (tile, range): grid.x
// takes the tiles as the data-parallel kernels do, grid.y the ranges.  Each
// workgroup writes its fp32 partial tile (row-major BM x BN) to workspace
// slot tile * p.split + range; gemm_split_reduce, launched next on the same
// stream, adds the partials of every element in range order and stores C
// through the elementwise epilogue.  No workgroup waits for or reads another's
// partial, and the reduction is spread over the whole chip -- in the stream-K
// kernel the last contributor to arrive reads all of its tile's partials
// alone, which sets its tail (about 18 µs for eight 256 KB partials).
// Results are deterministic: the order of every sum is fixed by p.split.
template <class KT>
__global__ void __launch_bounds__(KT::NT)
gemm_split_kernel(Params p)
{
    constexpr int BM = KT::TILE_M, BN = KT::TILE_N, BK = KT::TILE_K;
    __shared__ __attribute__((aligned(1024))) char smem[KT::SMEM];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords(p, tm, tn);
    const int nkt = (p.K + BK - 1) / BK, r = blockIdx.y;
    const int kt0 = (int)((int64_t)r * nkt / p.split), kt1 = (int)((int64_t)(r + 1) * nkt / p.split);

    typename KT::OA oa;
    typename KT::OB ob;
    oa.init(wave, lane, p.lda);
    ob.init(wave, lane, p.ldb);
    typename KT::Acc acc;
    KT::zero(acc);
    KT::mainloop(p, smem, oa, ob, tm * BM, tn * BN, kt0, kt1, acc, tid, lane, wave);
    Params q = p;   // the partial tile, row-major BM x BN
    q.C = (char*)p.sk_part + ((int64_t)(tm * p.tiles_n + tn) * p.split + r) * KT::PART_BYTES;
    q.ldc = BN;
    KT::template store<true>(q, 0, 0, acc, lane, wave);
}

// Thread q adds the p.split partials of 16-byte chunk q of the partial
// tiles (tile q / (BM * BN / 4), chunks row-major within it) and stores the
// four elements through the epilogue.
template <Out TO, int BM, int BN>
__global__ void __launch_bounds__(256)
gemm_split_reduce(Params p)
{
    constexpr int CPT = BM * BN / 4;   // chunks per tile
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int t = (int)(q / CPT), c = (int)(q % CPT);
    if (t >= p.tiles_m * p.tiles_n) return;
    const int m = (t / p.tiles_n) * BM + c / (BN / 4), n = (t % p.tiles_n) * BN + (c % (BN / 4)) * 4;
    if (m >= p.M || n >= p.N) return;
    const f32x4* src = (const f32x4*)p.sk_part + (int64_t)t * p.split * CPT + c;
    f32x4 sum = src[0];
#pragma unroll 4
    for (int r = 1; r < p.split; ++r) sum += src[(int64_t)r * CPT];
    store4<TO>(p, m, n, sum);
}

template <class KT>
hipError_t launch_split(const Params& p, hipStream_t s)
{
    Params copy = p;
    void* args[] = {&copy};
    const unsigned tiles = (unsigned)(p.tiles_m * p.tiles_n);
    hipError_t e = hipLaunchKernel((const void*)&gemm_split_kernel<KT>, dim3(tiles, (unsigned)p.split),
                                   dim3(KT::NT), args, 0, s);
    if (e != hipSuccess) return e;
    const int64_t chunks = (int64_t)tiles * (KT::TILE_M * KT::TILE_N / 4);
    return hipLaunchKernel((const void*)&gemm_split_reduce<KT::OUT, KT::TILE_M, KT::TILE_N>,
                           dim3((unsigned)((chunks + 255) / 256)), dim3(256), args, 0, s);
}

// Launcher of the 16-bit split-k configs (A ring of SA stages, B ring of SB).
template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI, int SA, int SB>
struct Dma16SplitInst {
    static hipError_t launch(int layout, const Params& p, hipStream_t s)
    {
        switch (layout) {
        case 0: return launch_split<Dma16<TI, TO, BM, BN, BK, WM, WN, MI, SA, true, true, SB>>(p, s);
        case 1: return launch_split<Dma16<TI, TO, BM, BN, BK, WM, WN, MI, SA, true, false, SB>>(p, s);
        case 2: return launch_split<Dma16<TI, TO, BM, BN, BK, WM, WN, MI, SA, false, true, SB>>(p, s);
        default: return launch_split<Dma16<TI, TO, BM, BN, BK, WM, WN, MI, SA, false, false, SB>>(p, s);
        }
    }
};

// Launcher of the 16-bit stream-K configs (the fp32 ones launch through
// F32DmaInst<..., true>).
template <In TI, Out TO, int BM, int BN, int BK, int WM, int WN, int MI, int STAGES>
struct Dma16SkInst {
    template <bool AK, bool BKM>
    static hipError_t go(const Params& p, hipStream_t s)
    {
        Params copy = p;
        void* args[] = {&copy};
        return hipLaunchKernel((const void*)&gemm_sk_kernel<Dma16<TI, TO, BM, BN, BK, WM, WN, MI, STAGES, AK, BKM>>,
                               dim3((unsigned)p.grid), dim3(WM * WN * 64), args, 0, s);
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

}  // namespace mg
