/*
 * mi355_gemm.h -- C ABI of the MI355X (gfx950) dense GEMM library.
 *
 * Operation (CuTe DSL Ampere SGEMM example, module docstring and the
 * einsum('mk,nk->mn') reference check in run(); CK Tile practice GEMM README,
 * "Host Matrix Creation"):
 *
 *     C[m][n] = sum over k < K of A[m][k] * B[n][k]
 *
 * with A logically M x K, B logically N x K and C logically M x N.  C is
 * overwritten and never read (the SGEMM example's epilogue is the identity
 * and the initial contents of C are discarded).  Products are formed exactly
 * and accumulated in fp32 on the MFMA units; the summation order is the
 * library's own.
 *
 * Storage.  Each matrix has one contiguous ("major") index, as in the SGEMM
 * example's --a_major / --b_major / --c_major flags and its
 * create_and_permute_tensor():
 *     a_major 'k': A[m][k] at A + m*lda + k     'm': at A + m + k*lda
 *     b_major 'k': B[n][k] at B + n*ldb + k     'n': at B + n + k*ldb
 *     c_major 'n': C[m][n] at C + m*ldc + n     'm': at C + m + n*ldc
 * Major characters are case-insensitive.  Leading dimensions and sizes are in
 * ELEMENTS.  All pointers are device pointers (HBM), owned by the caller; the
 * library keeps no pointer after a call returns and allocates nothing (the
 * one device array it owns, for gemm_run_noalloc, is described there).
 *
 * Alignment (SGEMM example, "Constraints" in its docstring: the contiguous
 * dimension must be at least 16-byte aligned for its vectorised copies, and
 * the example falls back to scalar copies otherwise).  Pointers must be
 * aligned to their element size.  When A, B and C are 16-byte aligned and
 * every ld * sizeof(element) (and every batch stride) is a multiple of 16,
 * all tile configs can run and each operand must be readable (C: writable)
 * over its padded extent: for A k-major, (M-1)*lda elements plus K rounded up
 * to a 16-byte multiple; likewise for the other majors.  Otherwise only the
 * element-by-element ("scalar") configs run, with any ld >= the contiguous
 * extent, and the exact extent ((M-1)*lda + K elements for A k-major) is
 * read.  The ld padding may hold anything, NaN included: it never reaches C.
 * C's padding is never written.
 *
 * Asynchrony.  gemm_run only enqueues work on `stream` (a hipStream_t; NULL is
 * the default stream) and returns.  The caller synchronises.  Launch errors
 * are reported as GEMM_ERR_HIP; faults inside a kernel surface at the
 * caller's synchronisation.
 *
 * Errors.  Every function returns a status and never throws.  All argument
 * checks run before any HIP call, so they can be exercised without a GPU, in
 * this order: shape (GEMM_ERR_BAD_SHAPE), majors (BAD_MAJOR), dtype
 * (BAD_DTYPE), leading dimensions and batch strides (BAD_LD), pointers
 * (NULL_PTR), alignment (MISALIGNED), overlap (ALIAS), then the config
 * (NO_CONFIG), the epilogue (BAD_EPILOGUE) and the workspace (WORKSPACE).
 * The first failing check decides the status.
 *
 * Degenerate sizes.  M == 0 or N == 0: nothing is launched, GEMM_OK.
 * K == 0: C is filled with zeros (the empty sum); A and B are not read.
 *
 * Logging.  With the environment variable MI355_GEMM_LOG set (to anything but
 * 0) when the library first checks it, every GEMM call that chooses a config
 * prints one line on stderr: the problem, the config (and, when the last
 * rows or columns of C went to the strip kernel, how many; and whether the
 * operands were swapped and C stored transposed), where the choice
 * came from (forced, table, table nearest shape, heuristic) and the launch
 * status; gemm_select_config prints its choice too.
 *
 * Thin edges.  When C's last 1-4 columns (or rows, of C as computed: C
 * n-major, or its transpose for C m-major) lie past a multiple of the
 * chosen tile and leaving them to a small strip kernel saves a round of
 * tiles, the call launches the tiled kernel on the full tiles and the strip
 * kernel after it, on the same stream (not for stream-K, split-k or
 * element-by-element configs).
 *
 * Transposed store.  Configs whose names end in " pp" store C transposed when
 * that gives them a k-contiguous B: for A k-major and B n-major (C n-major),
 * or A m-major and B k-major (C m-major), without an epilogue, they compute
 * C^T = B A^T and write it transposed, which is C in the caller's layout.
 *
 * Threads.  All functions are reentrant.  The only global state is the tuning
 * table, guarded by a mutex, a per-thread record of the last config, and the
 * device scratch array of gemm_run_noalloc (whose calls on one GPU must not
 * overlap).
 */
#ifndef MI355_GEMM_H
#define MI355_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input type -> output type; accumulation is always fp32. */
typedef enum {
    GEMM_DTYPE_F32 = 0,        /* A, B fp32 -> C fp32                         */
    GEMM_DTYPE_F16_F32 = 1,    /* A, B fp16 -> C fp32                         */
    GEMM_DTYPE_BF16_BF16 = 2,  /* A, B bf16 -> C bf16 (round to nearest even) */
    GEMM_DTYPE_F16_F16 = 3,    /* A, B fp16 -> C fp16 (round to nearest even) */
    GEMM_DTYPE_BF16_F32 = 4,   /* A, B bf16 -> C fp32                         */
    GEMM_NUM_DTYPES = 5
} gemm_dtype_t;

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_NULL_PTR = 1,     /* A or B NULL while M*N*K > 0, or C NULL while M*N > 0   */
    GEMM_ERR_BAD_SHAPE = 2,    /* M, N, K or batch negative, or too large for the tile indexing */
    GEMM_ERR_BAD_MAJOR = 3,    /* major character not in {k,m} / {k,n} / {n,m}          */
    GEMM_ERR_BAD_DTYPE = 4,    /* dtype not a gemm_dtype_t                               */
    GEMM_ERR_BAD_LD = 5,       /* ld below the contiguous extent (or 1); bad batch stride;
                                  an operand's rows (outer extent x ld) or its batch
                                  entries (batch x stride) spanning over 2^48 bytes      */
    GEMM_ERR_MISALIGNED = 6,   /* pointer not element-aligned (workspace: 16 bytes), or a
                                  forced config that needs 16-byte alignment the operands lack */
    GEMM_ERR_ALIAS = 7,        /* C's extent overlaps A's or B's                         */
    GEMM_ERR_NO_CONFIG = 8,    /* config id out of range for this dtype                  */
    GEMM_ERR_HIP = 9,          /* the HIP runtime reported an error at launch            */
    GEMM_ERR_TUNING_FILE = 10, /* tuning table missing or malformed                      */
    GEMM_ERR_BAD_EPILOGUE = 11, /* unknown epilogue activation                              */
    GEMM_ERR_WORKSPACE = 12,   /* stream-K / split-k config without a large enough workspace */
    GEMM_ERR_SCRATCH_LIMIT = 13 /* gemm_run_noalloc: the forced config needs more workspace
                                   than the library's fixed scratch holds               */
} gemm_status_t;

/* Activations of the elementwise epilogue. */
typedef enum {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1,         /* x < 0 ? 0 : x (NaN stays NaN)          */
    GEMM_ACT_GELU = 2          /* x/2 * (1 + erf(x / sqrt(2)))            */
} gemm_activation_t;

/*
 * Elementwise epilogue applied to every output element before the store, in
 * fp32, as the SGEMM example's epilogue_op is applied to the accumulator
 * fragment right before it is copied out (identity by default), and as CK
 * Tile composes a kernel from a problem, a pipeline policy and an Epilogue:
 *
 *     C[m][n] = act(alpha * sum_k A[m][k] B[n][k] + beta * C_old[m][n] + bias[n])
 *
 * C_old is C's value before the call, in C's type, read only when beta != 0
 * (beta == 0 ignores whatever C holds, NaN included).  bias is a device
 * array of N fp32 values (one per column n of C, whatever c_major), 4-byte
 * aligned, or NULL.  The result is rounded to C's type (RNE) as without an
 * epilogue.  alpha = 1, beta = 0, bias = NULL, act = GEMM_ACT_NONE is the
 * plain product.
 */
typedef struct {
    float alpha;
    float beta;
    const float* bias;
    int activation;            /* gemm_activation_t */
} gemm_epilogue_t;

/*
 * C = A * B^T (storage B is N x K) as described above, with the tile config
 * chosen from the tuning table (exact key match, else the nearest tuned shape
 * of the same dtype and layout, else a built-in heuristic).
 */
int gemm_run(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
             int dtype, const void* A, const void* B, void* C,
             int64_t lda, int64_t ldb, int64_t ldc, void* stream);

/*
 * Strided batched form: for l < batch, C_l = A_l * B_l^T with
 * A_l = A + l*stride_a, B_l = B + l*stride_b, C_l = C + l*stride_c (strides in
 * elements).  This is the "L" mode of the CuTe DSL Ampere SGEMM example, whose
 * run() documents an (M, N, K, L) problem size.  Strides must be >= 0
 * (strides that are not 16-byte multiples select the element-by-element
 * configs, as unaligned pointers do); stride_a or stride_b may be 0 (the same
 * operand for every entry); C entries must not overlap (stride_c covers one
 * C, else GEMM_ERR_BAD_LD); batch <= 65535 (else GEMM_ERR_BAD_SHAPE); batch
 * == 0 launches nothing.  Aliasing is checked over the whole range each
 * operand spans.  One launch covers every entry, so the tile config is chosen
 * by the built-in heuristic from the tile count of all entries together (the
 * tuning table holds single GEMMs and is not consulted).  gemm_run is the
 * batch == 1 case.
 */
int gemm_run_batched(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                     int dtype, const void* A, const void* B, void* C,
                     int64_t lda, int64_t ldb, int64_t ldc,
                     int64_t batch, int64_t stride_a, int64_t stride_b, int64_t stride_c,
                     void* stream);

/*
 * gemm_run with a caller-owned device workspace, which lets the stream-K
 * configs run (persistent workgroups that split the k-iterations of the last
 * waves of tiles between them, for grids that would leave CUs idle; after the
 * Gluon multi-CTA tutorial, "Persistent kernels"), and the split-k configs
 * (names ending in " split": every tile's k-tiles cut into ranges, one
 * workgroup per tile and range writing a partial tile, then a second kernel
 * on the same stream adding the partials in range order, for problems with
 * few tiles and a long K).  config_id < 0 chooses as gemm_run does, except
 * that a stream-K or split-k config named by the tuning table is used when
 * workspace_bytes covers gemm_workspace_size() for it; config_id >= 0 forces
 * that config (GEMM_ERR_WORKSPACE if it needs a workspace and the workspace
 * is NULL or smaller than it needs).
 *
 * The workspace must be 16-byte aligned (else GEMM_ERR_MISALIGNED), must not
 * overlap A, B or C (GEMM_ERR_ALIAS), and must be zero-filled before its
 * first use: it holds per-tile arrival counters that every completed call
 * leaves at zero again, and partial tiles that need no initialisation.  Two
 * calls that may run at the same time (e.g. on different streams) need
 * different workspaces.  NULL / 0 is allowed: then this is gemm_run_config
 * (or gemm_run for config_id < 0).  Results are deterministic for a given
 * config and shape.  No batched form: stream-K and split-k configs take
 * batch == 1.
 */
int gemm_run_ws(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                int dtype, const void* A, const void* B, void* C,
                int64_t lda, int64_t ldb, int64_t ldc,
                void* workspace, size_t workspace_bytes, void* stream, int config_id);

/*
 * gemm_run_ws with an elementwise epilogue (NULL: none).  Errors besides
 * gemm_run_ws's: bias not 4-byte aligned -> GEMM_ERR_MISALIGNED; bias
 * overlapping C -> GEMM_ERR_ALIAS; unknown activation -> GEMM_ERR_BAD_EPILOGUE.
 * Every config runs the epilogue; in a stream-K config it is applied once per
 * element, by the workgroup that completes the tile, in a split-k config by
 * the reduction kernel.
 */
int gemm_run_ex(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                int dtype, const void* A, const void* B, void* C,
                int64_t lda, int64_t ldb, int64_t ldc, const gemm_epilogue_t* epilogue,
                void* workspace, size_t workspace_bytes, void* stream, int config_id);

/*
 * For callers that cannot allocate device memory or call hipMalloc (code
 * under HIP graph capture, tight serving loops, harnesses that forbid it):
 * gemm_run_ws with the workspace taken from a fixed array that the library
 * owns in device memory, GEMM_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it
 * runs on, held from the first call on that GPU until the process ends.
 * Nothing is allocated per call; the caller passes A, B, C and the stream as
 * for gemm_run_ws.  config_id < 0 chooses as gemm_run_ws does with a
 * workspace of that size (a stream-K or split-k config only when it fits); a forced
 * config that needs more returns GEMM_ERR_SCRATCH_LIMIT.  When the config is
 * a stream-K one, a small kernel on `stream` first zeroes the arrival
 * counters, then the GEMM runs.  The array is the GPU's (the stream's
 * device; the current device for a NULL stream): every call on one GPU
 * shares it and it keeps the last call's partial tiles, so calls that may
 * overlap on one GPU (different streams, or host threads) race and must not
 * be issued.  The first call on a GPU looks up the array's device address
 * (GEMM_ERR_HIP if that fails).  Results equal gemm_run_ws's for the same
 * config bit for bit.
 */
#define GEMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gemm_run_noalloc(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                     int dtype, const void* A, const void* B, void* C,
                     int64_t lda, int64_t ldb, int64_t ldc, void* stream, int config_id);

/*
 * Bytes of workspace that gemm_run_ws needs for this problem with config
 * config_id (< 0: the config the tuning table or the heuristic names for it),
 * written to *bytes; 0 when the config needs none (neither stream-K nor
 * split-k, or a stream-K config whose grid is whole waves).  Host only: no HIP call.  Returns GEMM_OK,
 * GEMM_ERR_NULL_PTR (bytes NULL), GEMM_ERR_BAD_SHAPE, GEMM_ERR_BAD_MAJOR,
 * GEMM_ERR_BAD_DTYPE or GEMM_ERR_NO_CONFIG.
 */
int gemm_workspace_size(int64_t M, int64_t N, int64_t K, char a_major, char b_major,
                        char c_major, int dtype, int config_id, size_t* bytes);

/*
 * Same as gemm_run but with an explicit tile config (0 <= config_id <
 * gemm_num_configs(dtype)).  Used by the offline tuner and by the tests that
 * cover every config; GEMM_ERR_NO_CONFIG when the id is out of range,
 * GEMM_ERR_WORKSPACE for a stream-K or split-k config that needs a workspace
 * (use gemm_run_ws).
 */
int gemm_run_config(int64_t M, int64_t N, int64_t K, char a_major, char b_major, char c_major,
                    int dtype, const void* A, const void* B, void* C,
                    int64_t lda, int64_t ldb, int64_t ldc, void* stream, int config_id);

/* Static description of a status code; never NULL. */
const char* gemm_status_str(int status);

/* Number of tile configs built for `dtype` (0 for an unknown dtype). */
int gemm_num_configs(int dtype);

/*
 * Writes a NUL-terminated description of config `config_id` of `dtype` into
 * buf (at most len bytes, truncated): its name, e.g.
 * "f16 256x256x64 w2x2 mfma32 s2 swz".  Returns GEMM_OK, GEMM_ERR_BAD_DTYPE or
 * GEMM_ERR_NO_CONFIG (also when buf is NULL or len is 0).
 */
int gemm_config_describe(int dtype, int config_id, char* buf, size_t len);

/*
 * The config id gemm_run would launch for these arguments (after the
 * C-m-major swap and the table lookup; never a stream-K config, since
 * gemm_run has no workspace), or a negative gemm_status_t negated
 * when the arguments are invalid.  Host only: no HIP call.
 */
int gemm_select_config(int64_t M, int64_t N, int64_t K, char a_major, char b_major,
                       char c_major, int dtype);

/*
 * Config id launched by the calling thread's last successful gemm_run /
 * gemm_run_config (-1 if none, or if that call launched no GEMM kernel).
 * Lets a tuner verify that the kernel it timed is the candidate it asked for.
 */
int gemm_last_config(void);

/*
 * Replace the tuning table with the one in `path` (text; one entry per line:
 * "dtype a_major b_major c_major M N K config_name", '#' starts a comment).
 * path NULL clears the table.  Entries naming unknown configs are skipped.
 * Returns GEMM_OK or GEMM_ERR_TUNING_FILE (the old table is then kept).  The
 * table is also read once, at the first call, from $MI355_GEMM_TUNING if set.
 */
int gemm_load_tuning(const char* path);

/* Number of entries in the current tuning table. */
int gemm_tuning_size(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355_GEMM_H */
