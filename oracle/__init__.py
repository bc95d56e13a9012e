"""CPU reference oracle for the dense GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, links or calls it, and the two share no code.

``gemm_ref`` wraps ``oracle_gemm.c``: the plain fp64 triple loop
C[m][n] = sum_k A[m][k] * B[n][k] of the CuTe DSL Ampere SGEMM example (module
docstring; reference check in ``run()``) and the CK Tile practice GEMM README
("Host Matrix Creation", "Result Verification").  The comparison helpers in
``compare`` implement the acceptance test on top of it.
"""
import ctypes
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

IN_TYPES = {"f32": 0, "f16": 1, "bf16": 2}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, c, vp, dp = ctypes.c_int64, ctypes.c_char, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_gemm.argtypes = [i64, i64, i64, c, c, ctypes.c_int, vp, i64, vp, i64,
                                i64, i64, dp, ctypes.c_int]
    lib.oracle_gemm.restype = ctypes.c_int
    for name in ("oracle_round_f32_n", "oracle_round_bf16_n", "oracle_round_f16_n",
                 "oracle_decode_f16_n", "oracle_decode_bf16_n"):
        getattr(lib, name).argtypes = [vp, vp, i64]
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a.size else ctypes.c_void_p(0)


def gemm_ref(M, N, K, a_major, b_major, in_type, A, lda, B, ldb, rows=None, threads=None):
    """Rows ``rows`` (a (begin, end) pair, default all) of C = A * B^T in fp64.

    ``A`` and ``B`` are flat numpy storage arrays: float32 for ``in_type='f32'``,
    uint16 bit patterns for ``'f16'``/``'bf16'``.  Majors and leading dimensions
    follow the SGEMM example's convention ('k'/'m' for A, 'k'/'n' for B).
    Returns a dense (end-begin) x N float64 array.  ``threads`` defaults to
    every CPU this process may run on.
    """
    lib = _load()
    r0, r1 = (0, M) if rows is None else rows
    want = np.float32 if in_type == "f32" else np.uint16
    A = np.ascontiguousarray(A, dtype=want)
    B = np.ascontiguousarray(B, dtype=want)
    out = np.zeros((max(r1 - r0, 0), N), dtype=np.float64)
    if threads is None:
        threads = len(os.sched_getaffinity(0)) or 1
    rc = lib.oracle_gemm(M, N, K, a_major.encode(), b_major.encode(), IN_TYPES[in_type],
                         _ptr(A), lda, _ptr(B), ldb, r0, r1, _ptr(out), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_gemm failed with {rc}")
    return out


def round_to(x, out_type):
    """Round fp64 values to the output type (round to nearest even).

    Returns float32 for 'f32', uint16 bit patterns for 'f16' and 'bf16'."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    if out_type == "f32":
        y = np.empty(x.shape, dtype=np.float32)
        lib.oracle_round_f32_n(_ptr(x), _ptr(y), x.size)
    elif out_type == "bf16":
        y = np.empty(x.shape, dtype=np.uint16)
        lib.oracle_round_bf16_n(_ptr(x), _ptr(y), x.size)
    elif out_type == "f16":
        y = np.empty(x.shape, dtype=np.uint16)
        lib.oracle_round_f16_n(_ptr(x), _ptr(y), x.size)
    else:
        raise ValueError(out_type)
    return y


def decode(bits, in_type):
    """fp64 values of fp16 / bf16 bit patterns (uint16 array)."""
    lib = _load()
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    y = np.empty(bits.shape, dtype=np.float64)
    fn = {"f16": lib.oracle_decode_f16_n, "bf16": lib.oracle_decode_bf16_n}[in_type]
    fn(_ptr(bits), _ptr(y), bits.size)
    return y


ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2


def epilogue_ref(acc, alpha=1.0, beta=0.0, c_old=None, bias=None, activation=ACT_NONE):
    """The elementwise epilogue, in fp64, on an M x N array of exact sums:

        act(alpha * acc + beta * c_old + bias[n])

    The SGEMM example applies its ``epilogue_op`` (identity by default) to the
    accumulator fragment right before copying it out; CK Tile composes a kernel
    from a problem, a pipeline policy and an Epilogue stage.  The engine's
    epilogue offers a scale, a scaled read of the old C, a per-column bias and
    an activation: relu(x) = 0 if x < 0 else x (NaN stays NaN), gelu(x) =
    x/2 * (1 + erf(x / sqrt 2)) with the library erf.  ``c_old`` (fp64, M x N)
    is used only when beta != 0.  The caller rounds the result to the output
    type.
    """
    y = alpha * np.asarray(acc, dtype=np.float64)
    if beta != 0.0:
        y = y + beta * np.asarray(c_old, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if activation == ACT_RELU:
        y = np.where(y < 0.0, 0.0, y)
    elif activation == ACT_GELU:
        erf = np.vectorize(math.erf, otypes=[np.float64])
        y = 0.5 * y * (1.0 + erf(y / math.sqrt(2.0)))
    elif activation != ACT_NONE:
        raise ValueError(activation)
    return y
