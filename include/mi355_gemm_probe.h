/*
 * mi355_gemm_probe.h -- measurement probes of the MI355X GEMM library.
 *
 * Not part of the GEMM path.  These two kernels measure the ceilings that
 * the GEMM kernels are compared with, so that a benchmark can report them on
 * the machine it runs on (the CuTe DSL benchmark/autotune notebook's
 * benchmark() notes that results depend on the clocks the part runs at; the
 * MFMA rate of this part depends on the data, through its power limit).
 * Status codes are gemm_status_t.  Both only enqueue work on `stream`.
 */
#ifndef MI355_GEMM_PROBE_H
#define MI355_GEMM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_PROBE_F16_16x16x32 = 0,   /* v_mfma_f32_16x16x32_f16  */
    GEMM_PROBE_F16_32x32x16 = 1,   /* v_mfma_f32_32x32x16_f16  */
    GEMM_PROBE_BF16_16x16x32 = 2   /* v_mfma_f32_16x16x32_bf16 */
} gemm_probe_shape_t;

/* Floating-point operations of one MFMA of `shape` (0 for an unknown shape). */
double gemm_probe_mfma_flops(int shape);

/*
 * MFMA-only throughput: `grid` workgroups of 4 waves; each wave runs `iters`
 * iterations of 64 MFMAs of `shape` on 8 independent accumulators, its
 * operands held in registers (no memory traffic in the loop).  operands:
 * device array of 16 x 64 16-byte values (A sets 0..7, then B sets 0..7, one
 * value per lane: 8 fp16 or bf16 elements), 16-byte aligned.
 * rotate != 0: every MFMA of an iteration takes a different (A, B) pair, so
 * the operand bits change from one MFMA to the next; 0: all take set 0.
 * sink: grid * 256 floats (one per thread, written at the end).  Flops =
 * grid * 4 * iters * 64 * gemm_probe_mfma_flops(shape).  Errors: BAD_SHAPE
 * (shape, iters < 0, grid outside 1 .. 2^20), NULL_PTR, MISALIGNED, HIP.
 */
int gemm_probe_mfma(int shape, int rotate, const void* operands, int64_t iters, int grid, float* sink,
                    void* stream);

/*
 * HBM -> LDS read rate for a row-major operand read the way the GEMM main
 * loop reads a k-contiguous tile: rows of row_bytes bytes (row i at
 * A + i * row_bytes); each workgroup (8 waves) owns 32768 / seg_bytes
 * consecutive rows and walks them seg_bytes of each row per step, through a
 * 3-stage ring of 32 KB with direct-to-LDS 16-byte loads, one barrier per
 * step.  seg_bytes in {128, 256, 512, 1024}; rows a multiple of
 * 32768 / seg_bytes; row_bytes a multiple of seg_bytes, with
 * row_bytes * 32768 / seg_bytes < 2^31.  A: rows * row_bytes readable bytes,
 * 16-byte aligned.  sink: (rows * seg_bytes / 32768) * 512 floats.  Bytes
 * read = rows * row_bytes.  Errors: BAD_SHAPE, BAD_LD, NULL_PTR,
 * MISALIGNED, HIP.
 */
int gemm_probe_hbm_read(const void* A, int64_t rows, int64_t row_bytes, int seg_bytes, float* sink,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MI355_GEMM_PROBE_H */
