// gemm_api.cpp -- host side of the C ABI declared in include/mi355_gemm.h.
//
// Argument checks (all before any HIP call), the C-m-major swap, tile config
// selection from the tuning table (stream-K configs only with a workspace,
// element-by-element configs for operands that are not 16-byte aligned), the
// stream-K schedule, the epilogue and batch parameters, and the launch.  The interface follows the
// pages' problem statement: device pointers, M/N/K, per-operand majors and
// leading dimensions, and a stream (CuTe DSL Ampere SGEMM example: docstring,
// SGemm.__call__ and run(); CK Tile practice GEMM README, "Kernel Launch").
#include "mi355_gemm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cctype>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "gemm_kernel.hpp"
#include "gemm_plan.hpp"

namespace {

struct DtypeInfo {
    const char* name;
    int in_bytes, out_bytes;
    const mg::KernelEntry* (*entries)(int*);
    hipError_t (*strip)(int, bool, const mg::Params&, hipStream_t);
};

const DtypeInfo kDtypes[GEMM_NUM_DTYPES] = {
    {"f32", 4, 4, mg::entries_f32, mg::strip_f32},
    {"f16_f32", 2, 4, mg::entries_f16_f32, mg::strip_f16_f32},
    {"bf16_bf16", 2, 2, mg::entries_bf16_bf16, mg::strip_bf16_bf16},
    {"f16_f16", 2, 2, mg::entries_f16_f16, mg::strip_f16_f16},
    {"bf16_f32", 2, 4, mg::entries_bf16_f32, mg::strip_bf16_f32},
};

const mg::KernelEntry* entries(int dtype, int* n)
{
    if (dtype < 0 || dtype >= GEMM_NUM_DTYPES) { *n = 0; return nullptr; }
    return kDtypes[dtype].entries(n);
}

int find_config(int dtype, const std::string& name)
{
    int n = 0;
    const mg::KernelEntry* e = entries(dtype, &n);
    for (int i = 0; i < n; ++i)
        if (name == e[i].name) return i;
    return -1;
}

// ---------------------------------------------------------------- arguments

struct Canon {
    int64_t M, N, K;
    char a, b;            // 'k'/'m' and 'k'/'n' after the swap
    const void* A;
    const void* B;
    int64_t lda, ldb, ldc;
    uint64_t a_bytes, b_bytes;
    int64_t batch, sa, sb, sc;   // batch count and strides in elements
    bool vec16;                  // 16-byte loads allowed (else scalar configs only)
    bool c_trans;                // C stored transposed (the swap below taken the other way)
};

// Largest span of one operand's rows, and of its batch entries, in bytes.
constexpr uint64_t kMaxSpanBytes = (uint64_t)1 << 48;

// Bytes spanned by `outer` rows of `ld` elements whose last row holds
// `inner` elements rounded up to 16 bytes.
uint64_t padded_extent(int64_t outer, int64_t inner, int64_t ld, int es)
{
    if (outer <= 0 || inner <= 0) return 0;
    uint64_t last = ((uint64_t)inner * es + 15) / 16 * 16;
    return (uint64_t)(outer - 1) * (uint64_t)ld * es + last;
}

uint64_t written_extent(int64_t outer, int64_t inner, int64_t ld, int es)
{
    if (outer <= 0 || inner <= 0) return 0;
    return ((uint64_t)(outer - 1) * (uint64_t)ld + (uint64_t)inner) * es;
}

bool overlap(const void* p, uint64_t pn, const void* q, uint64_t qn)
{
    if (!p || !q || pn == 0 || qn == 0) return false;
    uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + qn && b < a + pn;
}

// Argument checks.  *vec16 reports whether the operands allow 16-byte loads
// (pointers and leading dimensions and batch strides in 16-byte units); when
// they do not, only the element-by-element ("scalar") configs can run, and
// the pointers need only their element alignment.
int validate(int64_t M, int64_t N, int64_t K, char& a_major, char& b_major, char& c_major,
             int dtype, const void* A, const void* B, const void* C, int64_t lda, int64_t ldb,
             int64_t ldc, int64_t batch = 1, int64_t sa = 0, int64_t sb = 0, int64_t sc = 0,
             const void* ws = nullptr, size_t ws_bytes = 0, const gemm_epilogue_t* epi = nullptr,
             bool* vec16 = nullptr)
{
    const int64_t kMaxDim = (int64_t)1 << 30;
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_BAD_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMM_ERR_BAD_SHAPE;
    if (batch < 0 || batch > 65535) return GEMM_ERR_BAD_SHAPE;
    a_major = (char)std::tolower((unsigned char)a_major);
    b_major = (char)std::tolower((unsigned char)b_major);
    c_major = (char)std::tolower((unsigned char)c_major);
    if ((a_major != 'k' && a_major != 'm') || (b_major != 'k' && b_major != 'n') ||
        (c_major != 'n' && c_major != 'm'))
        return GEMM_ERR_BAD_MAJOR;
    if (dtype < 0 || dtype >= GEMM_NUM_DTYPES) return GEMM_ERR_BAD_DTYPE;
    const int es = kDtypes[dtype].in_bytes, eo = kDtypes[dtype].out_bytes;

    const int64_t a_inner = a_major == 'k' ? K : M, a_outer = a_major == 'k' ? M : K;
    const int64_t b_inner = b_major == 'k' ? K : N, b_outer = b_major == 'k' ? N : K;
    const int64_t c_inner = c_major == 'n' ? N : M, c_outer = c_major == 'n' ? M : N;
    if (lda < std::max<int64_t>(1, a_inner) || ldb < std::max<int64_t>(1, b_inner) ||
        ldc < std::max<int64_t>(1, c_inner))
        return GEMM_ERR_BAD_LD;
    if (sa < 0 || sb < 0 || sc < 0) return GEMM_ERR_BAD_LD;
    // Upper bounds: the rows of one entry (outer x ld) and the batch entries
    // (batch x stride) may each span at most 2^48 bytes, the GPU's virtual
    // address range; every byte offset and extent below then stays far inside
    // 64 bits.
    {
        const uint64_t nb = (uint64_t)std::max<int64_t>(1, batch);
        auto fits = [&](int64_t outer, int64_t ld, int64_t stride, int e) {
            const uint64_t lim = kMaxSpanBytes / (uint64_t)e;
            return (uint64_t)ld <= lim / (uint64_t)std::max<int64_t>(1, outer) && (uint64_t)stride <= lim / nb;
        };
        if (!fits(a_outer, lda, sa, es) || !fits(b_outer, ldb, sb, es) || !fits(c_outer, ldc, sc, eo))
            return GEMM_ERR_BAD_LD;
    }
    // C entries must not overlap one another.
    const uint64_t cn = written_extent(c_outer, c_inner, ldc, eo);
    if (batch > 1 && M > 0 && N > 0 && (uint64_t)sc * eo < cn) return GEMM_ERR_BAD_LD;

    const bool reads = M > 0 && N > 0 && K > 0 && batch > 0;
    const bool writes = M > 0 && N > 0 && batch > 0;
    if ((reads && (!A || !B)) || (writes && !C)) return GEMM_ERR_NULL_PTR;

    if (reads && (((uintptr_t)A | (uintptr_t)B) % es)) return GEMM_ERR_MISALIGNED;
    if (writes && ((uintptr_t)C % eo)) return GEMM_ERR_MISALIGNED;
    if (ws && ((uintptr_t)ws & 15)) return GEMM_ERR_MISALIGNED;
    const bool v16 = !(reads && (((uintptr_t)A | (uintptr_t)B) & 15)) && !(writes && ((uintptr_t)C & 15)) &&
                     (lda * es) % 16 == 0 && (ldb * es) % 16 == 0 && (ldc * eo) % 16 == 0 &&
                     (sa * es) % 16 == 0 && (sb * es) % 16 == 0 && (sc * eo) % 16 == 0;
    if (vec16) *vec16 = v16;
    const float* bias = epi ? epi->bias : nullptr;
    if (bias && ((uintptr_t)bias & 3)) return GEMM_ERR_MISALIGNED;

    if (writes) {
        // Whole ranges spanned by all batch entries (conservative); the
        // readable extents of the 16-byte path end on a 16-byte chunk.
        const uint64_t ca = v16 ? padded_extent(a_outer, a_inner, lda, es) : written_extent(a_outer, a_inner, lda, es);
        const uint64_t cb = v16 ? padded_extent(b_outer, b_inner, ldb, es) : written_extent(b_outer, b_inner, ldb, es);
        const uint64_t ct = cn + (uint64_t)(batch - 1) * sc * eo;
        const uint64_t at = ca + (uint64_t)(batch - 1) * sa * es;
        const uint64_t bt = cb + (uint64_t)(batch - 1) * sb * es;
        if (reads && (overlap(C, ct, A, at) || overlap(C, ct, B, bt))) return GEMM_ERR_ALIAS;
        if (ws && ws_bytes &&
            (overlap(ws, ws_bytes, C, ct) || (reads && (overlap(ws, ws_bytes, A, at) || overlap(ws, ws_bytes, B, bt)))))
            return GEMM_ERR_ALIAS;
        if (bias && overlap(bias, (uint64_t)N * 4, C, ct)) return GEMM_ERR_ALIAS;
    }
    return GEMM_OK;
}

// C m-major: C^T (N x M, n-major) = B * A^T.  Swap the operands and sizes.
// trans: the other way round (swap for C n-major, not for C m-major), for a
// kernel that then stores C transposed.
Canon canonicalise(int64_t M, int64_t N, int64_t K, char a, char b, char c, int dtype,
                   const void* A, const void* B, int64_t lda, int64_t ldb, int64_t ldc, bool vec16 = true,
                   bool trans = false)
{
    Canon x;
    x.c_trans = trans;
    if ((c == 'm') != trans) {
        x.M = N; x.N = M; x.K = K;
        x.A = B; x.lda = ldb; x.a = b == 'k' ? 'k' : 'm';
        x.B = A; x.ldb = lda; x.b = a == 'k' ? 'k' : 'n';
    } else {
        x.M = M; x.N = N; x.K = K;
        x.A = A; x.lda = lda; x.a = a;
        x.B = B; x.ldb = ldb; x.b = b;
    }
    x.ldc = ldc;
    x.batch = 1;
    x.sa = x.sb = x.sc = 0;
    const int es = kDtypes[dtype].in_bytes;
    auto ext = vec16 ? padded_extent : written_extent;
    x.a_bytes = x.a == 'k' ? ext(x.M, x.K, x.lda, es) : ext(x.K, x.M, x.lda, es);
    x.b_bytes = x.b == 'k' ? ext(x.N, x.K, x.ldb, es) : ext(x.K, x.N, x.ldb, es);
    x.vec16 = vec16;
    return x;
}

// ---------------------------------------------------------------- tuning table

struct TuneEntry {
    int dtype;
    char a, b, c;
    int64_t M, N, K;
    int config;
};

std::mutex g_table_mu;
std::vector<TuneEntry> g_table;
std::atomic<unsigned> g_table_gen{0};   // bumped whenever the table changes
std::once_flag g_env_once;

int dtype_from_name(const std::string& s)
{
    for (int d = 0; d < GEMM_NUM_DTYPES; ++d)
        if (s == kDtypes[d].name) return d;
    return -1;
}

int parse_table(const char* path, std::vector<TuneEntry>& out)
{
    std::ifstream f(path);
    if (!f) return GEMM_ERR_TUNING_FILE;
    std::string line;
    while (std::getline(f, line)) {
        size_t hash = line.find('#');
        if (hash != std::string::npos) line.resize(hash);
        std::istringstream ss(line);
        std::string dt, a, b, c;
        int64_t M, N, K;
        if (!(ss >> dt)) continue;  // blank line
        if (!(ss >> a >> b >> c >> M >> N >> K)) return GEMM_ERR_TUNING_FILE;
        std::string rest;
        std::getline(ss, rest);
        size_t s0 = rest.find_first_not_of(" \t");
        size_t s1 = rest.find_last_not_of(" \t\r");
        if (s0 == std::string::npos) return GEMM_ERR_TUNING_FILE;
        std::string cfg = rest.substr(s0, s1 - s0 + 1);
        int d = dtype_from_name(dt);
        if (d < 0 || a.size() != 1 || b.size() != 1 || c.size() != 1 || M < 0 || N < 0 || K < 0)
            return GEMM_ERR_TUNING_FILE;
        int id = find_config(d, cfg);
        if (id < 0) continue;       // a config this library does not contain
        out.push_back({d, (char)std::tolower(a[0]), (char)std::tolower(b[0]),
                       (char)std::tolower(c[0]), M, N, K, id});
    }
    return GEMM_OK;
}

void load_env_table()
{
    const char* p = std::getenv("MI355_GEMM_TUNING");
    if (!p || !*p) return;
    std::vector<TuneEntry> t;
    if (parse_table(p, t) == GEMM_OK) {
        std::lock_guard<std::mutex> g(g_table_mu);
        g_table.swap(t);
        ++g_table_gen;
    } else {
        std::fprintf(stderr, "mi355_gemm: cannot read tuning table %s; using built-in choices\n", p);
    }
}

// Built-in choice when the table has nothing for this dtype and layout.
int heuristic(int dtype, int64_t M, int64_t N, int64_t K, bool a_kmajor, bool b_kmajor, int64_t batch)
{
    auto pick = [&](const char* tile) {
        std::string name = std::string(kDtypes[dtype].name) + " " + tile;
        int id = find_config(dtype, name);
        return id < 0 ? 0 : id;
    };
    // Thresholds from a tuner sweep (M = N = 1024 .. 8192, K = 1024 and
    // 4096, every dtype, operands k-major or m/n-major, one MI355X): large
    // problems (at least a wave of 256x256 tiles) go to the direct-to-LDS
    // 256x256 kernels, mid-size ones to 128x128 direct-to-LDS tiles, small
    // ones to 64x64 tiles (register-staged for fp32, direct-to-LDS for
    // 16-bit inputs).  A strided batch counts all its entries' tiles
    // (64 x 512^3 fp16: the 256x256 tile runs at 507 TF/s, the register-staged
    // 64x64 one at 296).
    const double tiles256 = std::ceil(M / 256.0) * std::ceil(N / 256.0) * (double)std::max<int64_t>(batch, 1);
    const double tiles64 = std::ceil(M / 64.0) * std::ceil(N / 64.0) * (double)std::max<int64_t>(batch, 1);
    // Thin problems (C's shorter side at most 64 or 128 per entry): a wider
    // tile only multiplies zeros.  On 16384 .. 65536 x 64 .. 128, K 1024 ..
    // 8192, the 64-wide tiles ran 1.2-1.5x (16-bit) and about 3x (fp32) ahead
    // of the 128- and 256-wide ones the tile counts alone pick, and with 128
    // columns the 128x128 tile 8 % ahead of the 256x256 one.
    const int64_t short_side = std::min(M, N);
    if (short_side <= 64) {
        if (dtype == GEMM_DTYPE_F32)
            return pick(tiles64 > 128 ? "64x64x32 w2x2 mfma32 s4 dma" : "32x32x128 w2x2 mfma16 s2 swz");
        return pick(!a_kmajor && !b_kmajor ? "64x64x64 w2x2 mfma32 s4 dma" : "64x64x64 w2x2 mfma16 s4 dma");
    }
    // A short K (at most 256: a few k-tiles per tile) on up to 1024 tiles of
    // 64x64: the small-problem tiles below (16384 x 128 x 128: 15-17 % ahead
    // of the 128x128 tile for 16-bit inputs, 1.5x for fp32; at 4096^2 x 256,
    // 4096 such tiles, the 256x256 tile is ahead again).
    if (K <= 256 && tiles64 <= 1024) {
        if (dtype == GEMM_DTYPE_F32)
            return pick(tiles64 > 128 ? "64x64x32 w2x2 mfma32 s4 dma" : "32x32x128 w2x2 mfma16 s2 swz");
        return pick(!a_kmajor && !b_kmajor ? "64x64x64 w2x2 mfma32 s4 dma" : "64x64x64 w2x2 mfma16 s4 dma");
    }
    if (short_side <= 128 && tiles256 >= 64) {
        if (dtype == GEMM_DTYPE_F32) return pick("128x128x32 w2x2 mfma32 s2 dma");
        return pick(a_kmajor && b_kmajor ? "128x128x64 w2x2 mfma16 s4 dma" : "128x128x64 w2x2 mfma32 s4 dma");
    }
    if (dtype == GEMM_DTYPE_F32) {
        if (tiles256 >= 256) return pick("256x256x32 w2x2 mfma32 s2 dma");
        if (tiles256 >= 64) return pick("128x128x32 w2x2 mfma32 s2 dma");
        // Small: the 64x64 direct-to-LDS tile from 256 tiles of 64x64 up
        // (1024^2 .. 1536^2: 5-15 % ahead of the register-staged 64x64 tile);
        // below, the register-staged 32x32x128 tile (512^2, 768x512: about
        // twice as fast as either 64x64 tile, whose few workgroups leave CUs
        // idle).
        if (tiles64 > 128) return pick("64x64x32 w2x2 mfma32 s4 dma");
        return pick("32x32x128 w2x2 mfma16 s2 swz");
    }
    // Large problems with k-contiguous B (or k-contiguous A: the ping-pong
    // config then stores C transposed, with the operands the other way round)
    // and K >= 1024 take the ping-pong schedule (4-13 % ahead of the one-group schedules at 4096^3, 8192^2 x
    // 4096 and 2 x 4096^3 batched, every 16-bit dtype; level at K = 1024;
    // 2-3 % behind at K = 256 and 512, where the k-loop is a few tiles
    // long).  Otherwise the 256x256 tile on 16x16x32 MFMAs holds a higher
    // clock under the power limit than on 32x32x16 ones and wins on one wave
    // of tiles and for 16-bit outputs; with fp32 outputs on grids of several
    // waves (8192^2, 16384^2) the 32x32x16 form stays 3-7 % ahead.
    if (tiles256 >= 128) {
        // With both operands m/n-contiguous the ping-pong kernel reads both
        // with transposing loads: level with the one-group kernels on one
        // wave of tiles, 2-10 % ahead from 512 tiles (8192^2) up.
        if (K >= 1024 && (a_kmajor || b_kmajor || tiles256 >= 512)) return pick("256x256x64 w4x2 mfma16 s3x2 pp");
        return pick(kDtypes[dtype].out_bytes == 4 && tiles256 >= 512 ? "256x256x64 w4x2 mfma32 s2 dma"
                                                                      : "256x256x64 w4x2 mfma16 s2 dma");
    }
    // From half a wave of 256x256 tiles up (128; 2560 x 4096 .. 3328^2) the
    // branch above: those tiles ran 1.3-1.5x ahead of 128x128 ones, whose
    // four-stage ring fits one workgroup per CU and so takes 2-3 rounds.
    // Below that, with an operand k-contiguous, the 128x256 tile (one round;
    // 2304^2 .. 2816^2: 10-16 % ahead of 128x128).  Then the 128x128 tile,
    // on 16x16x32 MFMAs when both operands are k-contiguous (5-10 % faster
    // at 2048^2); with an m/n-contiguous operand the 32x32x16 form's
    // transposing LDS reads suit it better (up to 30 %).
    if (tiles256 > 64 && (a_kmajor || b_kmajor)) return pick("128x256x64 w2x2 mfma32 s3 dma");
    if (tiles256 >= 64)
        return pick(a_kmajor && b_kmajor ? "128x128x64 w2x2 mfma16 s4 dma" : "128x128x64 w2x2 mfma32 s4 dma");
    // Small: up to one wave of 64x64 tiles (256), the 64x64 direct-to-LDS
    // tile with a 4-stage ring, on 32x32x16 MFMAs only when neither operand is
    // k-contiguous (256^2 .. 1024^2, K 512 .. 4096: 5-8 us; 12-35 % ahead of
    // the 128x128 tile and up to 2.5x ahead of the register-staged 64x64 one
    // with m/n-contiguous operands); past that the 128x128 tile (1536^2:
    // 12.3-13.7 us against 14.0-17.2).
    if (tiles64 <= 256)
        return pick(!a_kmajor && !b_kmajor ? "64x64x64 w2x2 mfma32 s4 dma" : "64x64x64 w2x2 mfma16 s4 dma");
    return pick(a_kmajor && b_kmajor ? "128x128x64 w2x2 mfma16 s4 dma" : "128x128x64 w2x2 mfma32 s4 dma");
}

// Built-in choice among the element-by-element configs (operands that are
// not 16-byte aligned): fp32 problems of at least 64 tiles of 128x128 take
// the 4-byte direct-to-LDS loads, the rest the register-staged element loads.
int heuristic_scalar(int dtype, int64_t M, int64_t N)
{
    const bool big = std::ceil(M / 128.0) * std::ceil(N / 128.0) >= 64;
    if (dtype == GEMM_DTYPE_F32 && big) return find_config(dtype, "f32 128x128x32 w2x2 mfma32 s2 dma scalar");
    const std::string tile = big ? (dtype == GEMM_DTYPE_F32 ? "128x128x16 w2x2 mfma32" : "128x128x64 w2x2 mfma32")
                                 : (dtype == GEMM_DTYPE_F32 ? "64x64x16 w2x2 mfma16" : "64x64x64 w2x2 mfma16");
    return find_config(dtype, std::string(kDtypes[dtype].name) + " " + tile + " s2 swz scalar");
}

bool is_scalar(int dtype, int config)
{
    int n = 0;
    const mg::KernelEntry* all = entries(dtype, &n);
    return config >= 0 && config < n && all[config].scalar;
}

// The tuning table's choice for this problem, among the configs `usable`
// accepts (the first usable exact match, else the nearest usable entry within
// a factor 2 overall), else the built-in heuristic.  The table is tuned on
// single GEMMs, so a strided batch (batch > 1) goes to the heuristic.
// Where the last choice of this thread came from (for MI355_GEMM_LOG).
thread_local const char* t_source = "";

template <class Usable>
int select(int dtype, char a, char b, char c, int64_t M, int64_t N, int64_t K, int64_t batch, Usable usable)
{
    std::call_once(g_env_once, load_env_table);
    t_source = batch > 1 ? "heuristic, batched" : "heuristic";
    if (batch <= 1) {
        std::lock_guard<std::mutex> g(g_table_mu);
        const TuneEntry* best = nullptr;
        double best_d = 0;
        for (const TuneEntry& e : g_table) {
            if (e.dtype != dtype || e.a != a || e.b != b || e.c != c || !usable(e.config)) continue;
            if (e.M == M && e.N == N && e.K == K) {
                t_source = "table";
                return e.config;
            }
            double d = std::fabs(std::log2((double)std::max<int64_t>(M, 1) / std::max<int64_t>(e.M, 1))) +
                       std::fabs(std::log2((double)std::max<int64_t>(N, 1) / std::max<int64_t>(e.N, 1))) +
                       std::fabs(std::log2((double)std::max<int64_t>(K, 1) / std::max<int64_t>(e.K, 1)));
            if (!best || d < best_d) { best = &e; best_d = d; }
        }
        if (best && best_d <= 1.0) {   // within a factor 2 overall
            t_source = "table, nearest shape";
            return best->config;
        }
    }
    // The kernel only sees the canonical (C n-major) problem: for C m-major
    // the operands and sizes swap.
    return c == 'm' ? heuristic(dtype, N, M, K, b == 'k', a == 'k', batch)
                    : heuristic(dtype, M, N, K, a == 'k', b == 'k', batch);
}

int select(int dtype, char a, char b, char c, int64_t M, int64_t N, int64_t K)
{
    return select(dtype, a, b, c, M, N, K, 1, [](int) { return true; });
}

thread_local int t_last_config = -1;
thread_local int t_strip_m = 0, t_strip_n = 0;   // the last launch's strips (rows, columns of C)
thread_local bool t_c_trans = false;             // the last launch stored C transposed

// Stream-K schedule of a persistent config (mg::KernelEntry::sk_occ > 0).
// The grid is a fixed 256 CUs x sk_occ workgroups: nothing in the kernel
// waits for another workgroup, so correctness never depends on how many of
// them are resident at once.
constexpr int kSkCUs = 256;

struct SkPlan {
    int grid = 0, sk_first = 0, sk_tiles = 0, sk_wgs = 0, sk_base = 0, sk_rem = 0;
    uint64_t count_bytes = 0, bytes = 0;   // counters; whole workspace
    bool ok = true;                        // false: schedule does not fit 32-bit indexing
};

SkPlan sk_plan(const mg::KernelEntry& e, int64_t tiles, int64_t nkt)
{
    SkPlan s;
    s.grid = kSkCUs * e.sk_occ;
    s.sk_first = (int)tiles;
    if (nkt == 0 || tiles % s.grid == 0) return s;          // whole waves: data-parallel only
    // The tiles of the last, partial wave share their k-iterations.  Every
    // stream-K workgroup gets at least ceil(nkt / 8) of them, so a tile has at
    // most nine contributors (the last one adds up the others' partial
    // tiles).  Their count is a multiple of 8 (one share per XCD).
    const int64_t skt = tiles % s.grid;
    const int64_t iters = skt * nkt;
    if (iters >= ((int64_t)1 << 31) - nkt) { s.ok = false; return s; }
    const int64_t min_iters = (nkt + 7) / 8;
    int64_t wgs = std::min<int64_t>(s.grid, std::max<int64_t>(1, iters / min_iters));
    if (wgs >= 8) wgs -= wgs % 8;
    s.sk_first = (int)(tiles - skt);
    s.sk_tiles = (int)skt;
    s.sk_wgs = (int)wgs;
    s.sk_base = (int)(iters / wgs);
    s.sk_rem = (int)(iters % wgs);
    s.count_bytes = ((uint64_t)skt * 4 + 255) / 256 * 256;
    s.bytes = s.count_bytes + 2ull * wgs * e.BM * e.BN * 4;
    return s;
}

// k-ranges per tile of a split-k config (mg::KernelEntry::split_occ > 0):
// as many as fill 256 CUs with split_occ workgroups each, at most 32 and at
// least two k-tiles per range.
int split_count(const mg::KernelEntry& e, int64_t tiles, int64_t nkt)
{
    const int64_t slots = (int64_t)kSkCUs * e.split_occ;
    int64_t s = tiles > 0 ? slots / tiles : 1;
    s = std::min<int64_t>(s, std::min<int64_t>(32, nkt / 2));
    return (int)std::max<int64_t>(1, s);
}

// Workspace a config needs for the canonical problem x (0 when none).
uint64_t workspace_need(const mg::KernelEntry& e, int64_t M, int64_t N, int64_t K)
{
    if (e.sk_occ == 0 && e.split_occ == 0) return 0;
    const int64_t tiles = ((M + e.BM - 1) / e.BM) * ((N + e.BN - 1) / e.BN);
    const int64_t nkt = (K + e.BK - 1) / e.BK;
    if (e.split_occ > 0) return (uint64_t)tiles * split_count(e, tiles, nkt) * e.BM * e.BN * 4;
    return sk_plan(e, tiles, nkt).bytes;
}

// True when the epilogue does something (else the plain store runs).
bool epi_active(const gemm_epilogue_t* epi)
{
    return epi && (epi->alpha != 1.f || epi->beta != 0.f || epi->bias || epi->activation != GEMM_ACT_NONE);
}

// The config gemm_run* launches when none is forced: the table's choice,
// unless it is a stream-K config that cannot run here (batched call, or no
// workspace of the size it needs), then the heuristic.
int select_for_uncached(int dtype, char a, char b, char c, int64_t M, int64_t N, int64_t K, int64_t batch,
                        uint64_t ws_bytes, bool vec16)
{
    if (!vec16) {
        t_source = "heuristic, element-by-element loads";
        return c == 'm' ? heuristic_scalar(dtype, N, M) : heuristic_scalar(dtype, M, N);
    }
    int n = 0;
    const mg::KernelEntry* all = entries(dtype, &n);
    const bool swap = c == 'm';
    auto usable = [&](int config) {
        const mg::KernelEntry& e = all[config];
        return (e.sk_occ == 0 && e.split_occ == 0) ||
               (batch == 1 && workspace_need(e, swap ? N : M, swap ? M : N, K) <= ws_bytes);
    };
    return select(dtype, a, b, c, M, N, K, batch, usable);
}

// select_for_uncached with a one-entry memo per thread: repeated calls with
// the same problem (the common case in a loop) skip the table scan.
struct SelectMemo {
    bool valid = false;
    unsigned gen = 0;
    int dtype = 0;
    char a = 0, b = 0, c = 0;
    int64_t M = 0, N = 0, K = 0, batch = 0;
    uint64_t ws_bytes = 0;
    bool vec16 = false;
    int config = -1;
    const char* source = "";
};
thread_local SelectMemo t_memo;

int select_for(int dtype, char a, char b, char c, int64_t M, int64_t N, int64_t K, int64_t batch,
               uint64_t ws_bytes, bool vec16 = true)
{
    const unsigned gen = g_table_gen.load();
    SelectMemo& m = t_memo;
    if (m.valid && m.gen == gen && m.dtype == dtype && m.a == a && m.b == b && m.c == c && m.M == M &&
        m.N == N && m.K == K && m.batch == batch && m.ws_bytes == ws_bytes && m.vec16 == vec16) {
        t_source = m.source;
        return m.config;
    }
    const int config = select_for_uncached(dtype, a, b, c, M, N, K, batch, ws_bytes, vec16);
    m = SelectMemo{true, gen, dtype, a, b, c, M, N, K, batch, ws_bytes, vec16, config, t_source};
    return config;
}

int launch(const Canon& x, int dtype, void* C, int config, void* stream, void* ws = nullptr,
           uint64_t ws_bytes = 0, const gemm_epilogue_t* epi = nullptr, bool bias_rows = false)
{
    int n = 0;
    const mg::KernelEntry* all = entries(dtype, &n);
    if (config < 0 || config >= n) return GEMM_ERR_NO_CONFIG;
    const mg::KernelEntry& e = all[config];
    const int es = kDtypes[dtype].in_bytes;
    // Per-tile byte offsets are 32-bit: the rows a tile spans times the row
    // pitch, plus the tile's extent along the contiguous index.
    const int64_t a_span = ((x.a == 'k' ? e.BM : e.BK) * x.lda + std::max(e.BM, e.BK)) * es;
    const int64_t b_span = ((x.b == 'k' ? e.BN : e.BK) * x.ldb + std::max(e.BN, e.BK)) * es;
    if (a_span >= ((int64_t)1 << 31) || b_span >= ((int64_t)1 << 31)) return GEMM_ERR_BAD_SHAPE;
    // A last column (row) of C at most kStripMax wide past a multiple of the
    // tile goes to the strip kernel (gemm_strip.hpp); the tiled kernel runs
    // the full tiles.  Not for stream-K configs (their split tail already
    // shares such tiles out) nor for element-by-element ones.
    // Only where that saves a round of tiles: the workgroups of one round are
    // estimated from the config's LDS ring (256 CUs x how many rings fit in
    // 160 KB), and a strip that leaves the count of rounds unchanged would
    // only add its own time.
    int64_t strip_m = 0, strip_n = 0;
    if (e.sk_occ == 0 && e.split_occ == 0 && !e.scalar && x.K > 0) {
        const int64_t rm = x.M % e.BM, rn = x.N % e.BN;
        const int64_t sm = rm > 0 && rm <= mg::kStripMax && x.M > e.BM ? rm : 0;
        const int64_t sn = rn > 0 && rn <= mg::kStripMax && x.N > e.BN ? rn : 0;
        const int64_t ring = (int64_t)(e.dma ? e.stages : 2) * (e.BM + e.BN) * e.BK * es;
        const int64_t slots = 256 * std::max<int64_t>(1, std::min<int64_t>(8, (160 << 10) / ring));
        auto rounds = [&](int64_t dm, int64_t dn) {
            return ((x.M - dm + e.BM - 1) / e.BM * ((x.N - dn + e.BN - 1) / e.BN) * x.batch + slots - 1) / slots;
        };
        const int64_t r0 = rounds(0, 0), rn_only = rounds(0, sn), rm_only = rounds(sm, 0), both = rounds(sm, sn);
        if (rn_only < r0 && rn_only <= rm_only) strip_n = sn;
        else if (rm_only < r0) strip_m = sm;
        if (both < std::min(rn_only, rm_only)) { strip_m = sm; strip_n = sn; }
        if ((x.M - strip_m) / e.BM * ((x.N - strip_n) / e.BN) * x.batch < mg::kStripMinTiles) strip_m = strip_n = 0;
    }
    t_strip_m = (int)strip_m;
    t_strip_n = (int)strip_n;
    t_c_trans = x.c_trans;
    const int64_t tiles_m = (x.M - strip_m + e.BM - 1) / e.BM, tiles_n = (x.N - strip_n + e.BN - 1) / e.BN;
    if (tiles_m * tiles_n >= ((int64_t)1 << 31)) return GEMM_ERR_BAD_SHAPE;

    mg::Params p;
    p.A = (const char*)x.A;
    p.B = (const char*)x.B;
    p.C = (char*)C;
    p.M = (int)(x.M - strip_m); p.N = (int)(x.N - strip_n); p.K = (int)x.K;
    p.tiles_m = (int)tiles_m; p.tiles_n = (int)tiles_n;
    p.strip0 = 0;
    p.c_trans = x.c_trans;
    p.group_m = (int)std::min<int64_t>(8, tiles_m);
    p.lda = x.lda; p.ldb = x.ldb; p.ldc = x.ldc;
    p.a_bytes = x.K > 0 ? x.a_bytes : 0;
    p.b_bytes = x.K > 0 ? x.b_bytes : 0;
    p.batch = (int)x.batch;
    p.sA = x.sa * es;
    p.sB = x.sb * es;
    p.sC = x.sc * kDtypes[dtype].out_bytes;
    p.grid = 0;
    p.sk_first = p.sk_wgs = p.sk_base = p.sk_rem = 0;
    p.sk_part = nullptr;
    p.sk_count = nullptr;
    p.split = 1;
    p.epi = epi_active(epi);
    p.alpha = epi ? epi->alpha : 1.f;
    p.beta = epi ? epi->beta : 0.f;
    p.bias = epi ? epi->bias : nullptr;
    p.bias_rows = bias_rows;
    p.act = epi ? epi->activation : GEMM_ACT_NONE;
    p.c_vec = ((uintptr_t)C & 15) == 0 && (x.ldc * kDtypes[dtype].out_bytes) % 16 == 0;
    if (e.sk_occ > 0) {
        if (x.batch != 1) return GEMM_ERR_NO_CONFIG;
        const SkPlan sp = sk_plan(e, tiles_m * tiles_n, (x.K + e.BK - 1) / e.BK);
        if (!sp.ok) return GEMM_ERR_BAD_SHAPE;
        if (sp.bytes > 0 && (!ws || ws_bytes < sp.bytes)) return GEMM_ERR_WORKSPACE;
        p.grid = sp.grid;
        p.sk_first = sp.sk_first;
        p.sk_wgs = sp.sk_wgs;
        p.sk_base = sp.sk_base;
        p.sk_rem = sp.sk_rem;
        if (sp.bytes > 0) {
            p.sk_count = (int*)ws;
            p.sk_part = (float*)((char*)ws + sp.count_bytes);
        }
    }
    if (e.split_occ > 0) {
        if (x.batch != 1) return GEMM_ERR_NO_CONFIG;
        const uint64_t need = workspace_need(e, x.M, x.N, x.K);
        if (!ws || ws_bytes < need) return GEMM_ERR_WORKSPACE;
        p.split = split_count(e, tiles_m * tiles_n, (x.K + e.BK - 1) / e.BK);
        p.sk_part = (float*)ws;
    }
    const int layout = (x.a == 'k' ? 0 : 2) + (x.b == 'k' ? 0 : 1);
    hipError_t err = e.launch(layout, p, (hipStream_t)stream);
    if (err != hipSuccess) return GEMM_ERR_HIP;
    if (strip_n) {               // C's last columns, all rows
        mg::Params q = p;
        q.M = (int)x.M;
        q.N = (int)x.N;
        q.strip0 = (int)(x.N - strip_n);
        if (kDtypes[dtype].strip(layout, false, q, (hipStream_t)stream) != hipSuccess) return GEMM_ERR_HIP;
    }
    if (strip_m) {               // C's last rows, the columns the tiles cover
        mg::Params q = p;
        q.M = (int)x.M;
        q.strip0 = (int)(x.M - strip_m);
        if (kDtypes[dtype].strip(layout, true, q, (hipStream_t)stream) != hipSuccess) return GEMM_ERR_HIP;
    }
    t_last_config = config;
    return GEMM_OK;
}

// MI355_GEMM_LOG=1 (read once): one line on stderr per GEMM call that gets
// as far as choosing a config, naming the config, where the choice came from
// and the launch status.
bool log_enabled()
{
    static const bool on = [] {
        const char* v = std::getenv("MI355_GEMM_LOG");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

void log_call(const char* what, int dtype, int64_t M, int64_t N, int64_t K, char a, char b, char c, int64_t batch,
              int config, const char* source, int status)
{
    int n = 0;
    const mg::KernelEntry* all = entries(dtype, &n);
    char strips[96] = "";
    if (std::strcmp(what, "run") == 0) {   // strips in canonical rows / columns (C n-major)
        if (t_strip_m || t_strip_n)
            std::snprintf(strips, sizeof strips, " + strip kernel (%d rows, %d columns)", t_strip_m, t_strip_n);
        if (t_c_trans) std::strncat(strips, ", operands swapped, C stored transposed", sizeof strips - std::strlen(strips) - 1);
    }
    std::fprintf(stderr, "mi355_gemm: %s %s M=%lld N=%lld K=%lld a=%c b=%c c=%c batch=%lld -> %s%s [%s] %s\n", what,
                 kDtypes[dtype].name, (long long)M, (long long)N, (long long)K, a, b, c, (long long)batch,
                 config >= 0 && config < n ? all[config].name : "(none)", strips, source, gemm_status_str(status));
}

int run(int64_t M, int64_t N, int64_t K, char a, char b, char c, int dtype, const void* A,
        const void* B, void* C, int64_t lda, int64_t ldb, int64_t ldc, void* stream, int config,
        int64_t batch = 1, int64_t sa = 0, int64_t sb = 0, int64_t sc = 0, void* ws = nullptr,
        size_t ws_bytes = 0, const gemm_epilogue_t* epi = nullptr)
{
    t_last_config = -1;
    t_strip_m = t_strip_n = 0;
    t_c_trans = false;
    if (!ws) ws_bytes = 0;
    bool vec16 = true;
    int st = validate(M, N, K, a, b, c, dtype, A, B, C, lda, ldb, ldc, batch, sa, sb, sc, ws, ws_bytes, epi,
                      &vec16);
    if (st != GEMM_OK) return st;
    if (config >= 0) {
        int n = 0;
        entries(dtype, &n);
        if (config >= n) return GEMM_ERR_NO_CONFIG;
        if (!vec16 && !is_scalar(dtype, config)) return GEMM_ERR_MISALIGNED;   // needs 16-byte loads
    }
    if (epi && (epi->activation < GEMM_ACT_NONE || epi->activation > GEMM_ACT_GELU)) return GEMM_ERR_BAD_EPILOGUE;
    if (M == 0 || N == 0 || batch == 0) return GEMM_OK;
    Canon x = canonicalise(M, N, K, a, b, c, dtype, A, B, lda, ldb, ldc, vec16);
    x.batch = batch;
    x.sa = c == 'm' ? sb : sa;      // the C-m-major swap exchanges the operands
    x.sb = c == 'm' ? sa : sb;
    x.sc = sc;
    const char* source = "forced";
    if (config < 0) {
        config = select_for(dtype, a, b, c, M, N, K, batch, ws_bytes, vec16);
        source = t_source;
    }
    if (config < 0) return GEMM_ERR_NO_CONFIG;
    // A config that can store C transposed takes the other operand order when
    // that turns an n-contiguous B into a k-contiguous one (A k, B n becomes
    // A m, B k); not with an epilogue (its staged store runs along n).
    {
        int n = 0;
        const mg::KernelEntry* all = entries(dtype, &n);
        if (all[config].c_trans && !epi_active(epi) && x.a == 'k' && x.b == 'n') {
            const bool swap = c != 'm';
            x = canonicalise(M, N, K, a, b, c, dtype, A, B, lda, ldb, ldc, vec16, true);
            x.batch = batch;
            x.sa = swap ? sb : sa;
            x.sb = swap ? sa : sb;
            x.sc = sc;
        }
    }
    // bias follows the user's columns n: the canonical rows when C is m-major.
    st = launch(x, dtype, C, config, stream, ws, ws_bytes, epi, c == 'm');
    if (log_enabled()) log_call("run", dtype, M, N, K, a, b, c, batch, config, source, st);
    return st;
}

}  // namespace

namespace mg {

int plan_ws(int64_t M, int64_t N, int64_t K, char a, char b, char c, int dtype, const void* A,
            const void* B, const void* C, int64_t lda, int64_t ldb, int64_t ldc, size_t ws_bytes,
            int config_id, int* config, uint64_t* need, uint64_t* count_bytes)
{
    *config = -1;
    *need = *count_bytes = 0;
    bool vec16 = true;
    int st = validate(M, N, K, a, b, c, dtype, A, B, C, lda, ldb, ldc, 1, 0, 0, 0, nullptr, 0, nullptr, &vec16);
    if (st != GEMM_OK) return st;
    int n = 0;
    const KernelEntry* all = entries(dtype, &n);
    if (config_id >= 0) {
        if (config_id >= n) return GEMM_ERR_NO_CONFIG;
        if (!vec16 && !is_scalar(dtype, config_id)) return GEMM_ERR_MISALIGNED;
    }
    if (M == 0 || N == 0) return GEMM_OK;
    const int cfg = config_id >= 0 ? config_id : select_for(dtype, a, b, c, M, N, K, 1, ws_bytes, vec16);
    if (cfg < 0) return GEMM_ERR_NO_CONFIG;
    const bool swap = c == 'm';
    const KernelEntry& e = all[cfg];
    *config = cfg;
    if (e.sk_occ > 0) {
        const int64_t cm = swap ? N : M, cn = swap ? M : N;
        const SkPlan sp = sk_plan(e, ((cm + e.BM - 1) / e.BM) * ((cn + e.BN - 1) / e.BN), (K + e.BK - 1) / e.BK);
        if (!sp.ok) return GEMM_ERR_BAD_SHAPE;
        *need = sp.bytes;
        *count_bytes = sp.count_bytes;
    } else if (e.split_occ > 0) {
        *need = workspace_need(e, swap ? N : M, swap ? M : N, K);   // partial tiles only, no counters
    }
    return GEMM_OK;
}

}  // namespace mg

extern "C" {

int gemm_run(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major, int dtype,
             const void* A, const void* B, void* C, int64_t lda, int64_t ldb, int64_t ldc,
             void* stream)
{
    return run(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, stream, -1);
}

int gemm_run_batched(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                     int dtype, const void* A, const void* B, void* C, int64_t lda, int64_t ldb,
                     int64_t ldc, int64_t batch, int64_t stride_a, int64_t stride_b,
                     int64_t stride_c, void* stream)
{
    return run(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, stream, -1, batch,
               stride_a, stride_b, stride_c);
}

int gemm_run_ws(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major, int dtype,
                const void* A, const void* B, void* C, int64_t lda, int64_t ldb, int64_t ldc,
                void* workspace, size_t workspace_bytes, void* stream, int config_id)
{
    return run(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, stream,
               config_id < 0 ? -1 : config_id, 1, 0, 0, 0, workspace, workspace_bytes);
}

int gemm_run_ex(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major, int dtype,
                const void* A, const void* B, void* C, int64_t lda, int64_t ldb, int64_t ldc,
                const gemm_epilogue_t* epilogue, void* workspace, size_t workspace_bytes, void* stream,
                int config_id)
{
    return run(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, stream,
               config_id < 0 ? -1 : config_id, 1, 0, 0, 0, workspace, workspace_bytes, epilogue);
}

int gemm_workspace_size(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                        int dtype, int config_id, size_t* bytes)
{
    if (!bytes) return GEMM_ERR_NULL_PTR;
    *bytes = 0;
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_BAD_SHAPE;
    char a = (char)std::tolower((unsigned char)a_major);
    char b = (char)std::tolower((unsigned char)b_major);
    char c = (char)std::tolower((unsigned char)c_major);
    if ((a != 'k' && a != 'm') || (b != 'k' && b != 'n') || (c != 'n' && c != 'm'))
        return GEMM_ERR_BAD_MAJOR;
    if (dtype < 0 || dtype >= GEMM_NUM_DTYPES) return GEMM_ERR_BAD_DTYPE;
    int n = 0;
    const mg::KernelEntry* all = entries(dtype, &n);
    if (config_id >= n) return GEMM_ERR_NO_CONFIG;
    if (config_id < 0) config_id = select(dtype, a, b, c, M, N, K);
    const bool swap = c == 'm';
    *bytes = (size_t)workspace_need(all[config_id], swap ? N : M, swap ? M : N, K);
    return GEMM_OK;
}

int gemm_run_config(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                    int dtype, const void* A, const void* B, void* C, int64_t lda, int64_t ldb,
                    int64_t ldc, void* stream, int config_id)
{
    if (config_id < 0) {
        t_last_config = -1;
        return GEMM_ERR_NO_CONFIG;
    }
    return run(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, stream, config_id);
}

const char* gemm_status_str(int status)
{
    switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_BAD_SHAPE: return "bad shape: M, N, K or batch negative or too large";
    case GEMM_ERR_BAD_MAJOR: return "bad major: a in {k,m}, b in {k,n}, c in {n,m}";
    case GEMM_ERR_BAD_DTYPE: return "bad dtype";
    case GEMM_ERR_BAD_LD: return "bad leading dimension: smaller than the contiguous extent";
    case GEMM_ERR_NULL_PTR: return "null pointer for an operand that is accessed";
    case GEMM_ERR_MISALIGNED: return "misaligned: pointers and ld*element size must be 16-byte multiples";
    case GEMM_ERR_ALIAS: return "C overlaps A or B";
    case GEMM_ERR_NO_CONFIG: return "no such tile config for this dtype";
    case GEMM_ERR_HIP: return "HIP runtime error at launch";
    case GEMM_ERR_TUNING_FILE: return "tuning table missing or malformed";
    case GEMM_ERR_WORKSPACE: return "stream-K or split-k config without a workspace of the size it needs";
    case GEMM_ERR_BAD_EPILOGUE: return "unknown epilogue activation";
    case GEMM_ERR_SCRATCH_LIMIT:
        return "the config needs more workspace than the allocation-free entry point's fixed scratch (64 MiB)";
    default: return "unknown status";
    }
}

int gemm_num_configs(int dtype)
{
    int n = 0;
    entries(dtype, &n);
    return n;
}

int gemm_config_describe(int dtype, int config_id, char* buf, size_t len)
{
    if (dtype < 0 || dtype >= GEMM_NUM_DTYPES) return GEMM_ERR_BAD_DTYPE;
    int n = 0;
    const mg::KernelEntry* e = entries(dtype, &n);
    if (config_id < 0 || config_id >= n || !buf || len == 0) return GEMM_ERR_NO_CONFIG;
    std::snprintf(buf, len, "%s", e[config_id].name);
    return GEMM_OK;
}

int gemm_select_config(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                       int dtype)
{
    // Shape/major/dtype checks only: pointers and leading dims play no part in the choice.
    if (M < 0 || N < 0 || K < 0) return -GEMM_ERR_BAD_SHAPE;
    char a = (char)std::tolower((unsigned char)a_major);
    char b = (char)std::tolower((unsigned char)b_major);
    char c = (char)std::tolower((unsigned char)c_major);
    if ((a != 'k' && a != 'm') || (b != 'k' && b != 'n') || (c != 'n' && c != 'm'))
        return -GEMM_ERR_BAD_MAJOR;
    if (dtype < 0 || dtype >= GEMM_NUM_DTYPES) return -GEMM_ERR_BAD_DTYPE;
    const int config = select_for(dtype, a, b, c, M, N, K, 1, 0);
    if (log_enabled()) log_call("select", dtype, M, N, K, a, b, c, 1, config, t_source, GEMM_OK);
    return config;
}

int gemm_last_config(void) { return t_last_config; }

int gemm_load_tuning(const char* path)
{
    std::call_once(g_env_once, [] {});   // an explicit table wins over the environment
    std::vector<TuneEntry> t;
    if (path) {
        int st = parse_table(path, t);
        if (st != GEMM_OK) return st;
    }
    std::lock_guard<std::mutex> g(g_table_mu);
    g_table.swap(t);
    ++g_table_gen;
    return GEMM_OK;
}

int gemm_tuning_size(void)
{
    std::lock_guard<std::mutex> g(g_table_mu);
    return (int)g_table.size();
}

}  // extern "C"
