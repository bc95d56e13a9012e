// Host-logic driver for the sanitizer build: every C-ABI path that runs
// before a kernel launch (argument checks, config selection, the tuning
// table parser, workspace planning, the allocation-free entry point's checks,
// the probes' checks), built with AddressSanitizer and UndefinedBehavior-
// Sanitizer on the host code.  Launches nothing: every call either fails an
// argument check or has an empty problem.  Exit status 0 when every status is
// the one expected.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "mi355_gemm.h"
#include "mi355_gemm_probe.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static const uintptr_t P = (uintptr_t)1 << 20;   // fake, aligned device addresses (never dereferenced)
static const void* ptr(uintptr_t a) { return (const void*)a; }

static void write_file(const char* path, const char* text)
{
    FILE* f = std::fopen(path, "w");
    if (!f) { ++failures; return; }
    std::fputs(text, f);
    std::fclose(f);
}

int main(int argc, char** argv)
{
    const char* table = argc > 1 ? argv[1] : nullptr;
    const char* tmpdir = argc > 2 ? argv[2] : "/tmp";

    for (int s = -5; s < 20; ++s) EXPECT(gemm_status_str(s) != nullptr);

    // config registries
    char buf[256];
    for (int d = -1; d <= GEMM_NUM_DTYPES; ++d) {
        const int n = gemm_num_configs(d);
        EXPECT((d >= 0 && d < GEMM_NUM_DTYPES) ? n > 0 : n == 0);
        for (int c = -1; c <= n; ++c) {
            const int st = gemm_config_describe(d, c, buf, sizeof buf);
            if (d < 0 || d >= GEMM_NUM_DTYPES) EXPECT(st == GEMM_ERR_BAD_DTYPE);
            else if (c < 0 || c >= n) EXPECT(st == GEMM_ERR_NO_CONFIG);
            else EXPECT(st == GEMM_OK && std::strlen(buf) > 0);
        }
        if (n > 0) {
            char one[1];
            EXPECT(gemm_config_describe(d, 0, one, 1) == GEMM_OK && one[0] == 0);   // truncated
            EXPECT(gemm_config_describe(d, 0, buf, 0) == GEMM_ERR_NO_CONFIG);
            EXPECT(gemm_config_describe(d, 0, nullptr, 8) == GEMM_ERR_NO_CONFIG);
        }
    }

    // argument checks (all before any HIP call)
    auto run = [](int64_t M, int64_t N, int64_t K, char a, char b, char c, int dt, uintptr_t A, uintptr_t B,
                  uintptr_t C, int64_t lda, int64_t ldb, int64_t ldc) {
        return gemm_run(M, N, K, a, b, c, dt, ptr(A), ptr(B), (void*)C, lda, ldb, ldc, nullptr);
    };
    EXPECT(run(-1, 8, 8, 'k', 'k', 'n', 0, P, 2 * P, 3 * P, 8, 8, 8) == GEMM_ERR_BAD_SHAPE);
    EXPECT(run((int64_t)1 << 40, 8, 8, 'k', 'k', 'n', 0, P, 2 * P, 3 * P, 8, 8, 8) == GEMM_ERR_BAD_SHAPE);
    EXPECT(run(8, 8, 8, 'x', 'k', 'n', 0, P, 2 * P, 3 * P, 8, 8, 8) == GEMM_ERR_BAD_MAJOR);
    EXPECT(run(8, 8, 8, 'k', 'k', 'n', 9, P, 2 * P, 3 * P, 8, 8, 8) == GEMM_ERR_BAD_DTYPE);
    EXPECT(run(8, 8, 8, 'k', 'k', 'n', 0, P, 2 * P, 3 * P, 7, 8, 8) == GEMM_ERR_BAD_LD);
    EXPECT(run(8, 8, 8, 'k', 'k', 'n', 0, 0, 2 * P, 3 * P, 8, 8, 8) == GEMM_ERR_NULL_PTR);
    EXPECT(run(8, 8, 8, 'k', 'k', 'n', 0, P + 2, 2 * P, 3 * P, 8, 8, 8) == GEMM_ERR_MISALIGNED);
    EXPECT(run(8, 8, 8, 'k', 'k', 'n', 0, P, 2 * P, P + 16, 8, 8, 8) == GEMM_ERR_ALIAS);
    EXPECT(run(0, 8, 8, 'k', 'k', 'n', 0, P, 2 * P, 3 * P, 8, 8, 8) == GEMM_OK);   // empty: no launch
    EXPECT(gemm_run_config(8, 8, 8, 'k', 'k', 'n', 0, ptr(P), ptr(2 * P), (void*)(3 * P), 8, 8, 8, nullptr,
                           100000) == GEMM_ERR_NO_CONFIG);
    gemm_epilogue_t bad = {1.f, 0.f, nullptr, 7};
    EXPECT(gemm_run_ex(8, 8, 8, 'k', 'k', 'n', 0, ptr(P), ptr(2 * P), (void*)(3 * P), 8, 8, 8, &bad, nullptr, 0,
                       nullptr, -1) == GEMM_ERR_BAD_EPILOGUE);
    EXPECT(gemm_run_batched(8, 8, 8, 'k', 'k', 'n', 0, ptr(P), ptr(2 * P), (void*)(3 * P), 8, 8, 8, 70000, 0, 0,
                            64, nullptr) == GEMM_ERR_BAD_SHAPE);
    EXPECT(gemm_run_batched(8, 8, 8, 'k', 'k', 'n', 0, ptr(P), ptr(2 * P), (void*)(3 * P), 8, 8, 8, 4, 0, 0, 32,
                            nullptr) == GEMM_ERR_BAD_LD);   // C entries overlap

    // selection and workspace planning over a grid of shapes, every dtype and layout
    const int64_t sizes[] = {0, 1, 17, 255, 256, 1000, 4095, 8192, 65536};
    const char ams[] = {'k', 'm'}, bms[] = {'k', 'n'}, cms[] = {'n', 'm'};
    for (int d = 0; d < GEMM_NUM_DTYPES; ++d)
        for (int64_t M : sizes)
            for (int64_t N : sizes)
                for (int64_t K : {(int64_t)0, (int64_t)64, (int64_t)1028, (int64_t)4096})
                    for (char a : ams)
                        for (char b : bms)
                            for (char c : cms) {
                                const int cfg = gemm_select_config(M, N, K, a, b, c, d);
                                EXPECT(cfg >= 0 && cfg < gemm_num_configs(d));
                                size_t ws = 0;
                                EXPECT(gemm_workspace_size(M, N, K, a, b, c, d, -1, &ws) == GEMM_OK);
                                for (int id = 0; id < gemm_num_configs(d); id += 3)
                                    EXPECT(gemm_workspace_size(M, N, K, a, b, c, d, id, &ws) == GEMM_OK);
                            }
    EXPECT(gemm_workspace_size(8, 8, 8, 'k', 'k', 'n', 0, -1, nullptr) == GEMM_ERR_NULL_PTR);
    EXPECT(gemm_select_config(8, 8, 8, 'q', 'k', 'n', 0) == -GEMM_ERR_BAD_MAJOR);

    // the tuning table parser
    const std::string good = std::string(tmpdir) + "/san_good.txt", badf = std::string(tmpdir) + "/san_bad.txt";
    write_file(good.c_str(), "# comment\n\nf32 k k n 100 100 100 f32 64x64x16 w2x2 mfma16 s2 swz  # trailing\n"
                             "f32 k k n 1 2 3 no such config\n");
    write_file(badf.c_str(), "f32 k k n 100 100\n");
    EXPECT(gemm_load_tuning(good.c_str()) == GEMM_OK && gemm_tuning_size() == 1);
    EXPECT(gemm_load_tuning(badf.c_str()) == GEMM_ERR_TUNING_FILE && gemm_tuning_size() == 1);
    EXPECT(gemm_load_tuning("/nonexistent/table") == GEMM_ERR_TUNING_FILE);
    if (table) EXPECT(gemm_load_tuning(table) == GEMM_OK && gemm_tuning_size() > 10);
    for (int64_t M : sizes)
        EXPECT(gemm_select_config(M, 4096, 4096, 'k', 'k', 'n', 1) >= 0);
    EXPECT(gemm_load_tuning(nullptr) == GEMM_OK && gemm_tuning_size() == 0);
    EXPECT(gemm_last_config() == -1);

    // the allocation-free entry point's checks
    EXPECT(gemm_run_noalloc(-1, 8, 8, 'k', 'k', 'n', 0, ptr(P), ptr(2 * P), (void*)(3 * P), 8, 8, 8, nullptr, -1) ==
           GEMM_ERR_BAD_SHAPE);
    EXPECT(gemm_run_noalloc(0, 8, 8, 'k', 'k', 'n', 0, ptr(P), ptr(2 * P), (void*)(3 * P), 8, 8, 8, nullptr, -1) ==
           GEMM_OK);
    int sk = -1;
    for (int id = 0; id < gemm_num_configs(0); ++id) {
        gemm_config_describe(0, id, buf, sizeof buf);
        if (std::strcmp(buf, "f32 256x256x32 w2x2 mfma32 s2 dma sk") == 0) sk = id;
    }
    EXPECT(sk >= 0);
    const uintptr_t big = (uintptr_t)1 << 34;
    EXPECT(gemm_run_noalloc(6144, 5888, 8192, 'k', 'k', 'n', 0, ptr(big), ptr(2 * big), (void*)(3 * big), 8192, 8192,
                            5888, nullptr, sk) == GEMM_ERR_SCRATCH_LIMIT);

    // probes' checks
    EXPECT(gemm_probe_mfma(9, 1, ptr(P), 1, 1, (float*)(2 * P), nullptr) == GEMM_ERR_BAD_SHAPE);
    EXPECT(gemm_probe_hbm_read(ptr(P), 255, 8192, 128, (float*)(2 * P), nullptr) == GEMM_ERR_BAD_SHAPE);

    std::fprintf(stderr, "host driver: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
