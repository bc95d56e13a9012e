"""Seeded synthetic GEMM inputs, shared by the tests, the benchmark and the smoke check.

This module holds no GEMM arithmetic: it only draws logical matrices, casts
them to the input type and lays them out in storage.  Both the HIP path and
the oracle consume what it produces.

Logical shapes follow the CuTe DSL Ampere SGEMM example (module docstring) and
the CK Tile practice GEMM README ("Host Matrix Creation"): A is M x K, B is
N x K, C is M x N.  The value distributions are the ones the workloads name:

  'int5'  integers drawn uniformly from {-5, ..., 5} (both pages fill A and B
          with small uniform integers; the inclusive upper bound is a reading)
  'u11'   uniform(-1, 1) in fp32
  'n01'   normal(0, 1) drawn in fp32
  'n002'  normal(0, 0.02) drawn in fp32

One numpy PCG64 generator seeded with ``seed`` (default 1024, the SGEMM
example's seed) draws A first, then B, each in logical row-major order, so the
same logical inputs feed every storage layout.
"""
import numpy as np

DTYPES = {
    # gemm dtype code: (name, input type, output type)
    0: ("f32", "f32", "f32"),
    1: ("f16_f32", "f16", "f32"),
    2: ("bf16_bf16", "bf16", "bf16"),
    3: ("f16_f16", "f16", "f16"),
    4: ("bf16_f32", "bf16", "f32"),
}
DTYPE_CODE = {v[0]: k for k, v in DTYPES.items()}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def draw(rng, rows, cols, kind):
    if kind == "int5":
        return rng.integers(-5, 6, size=(rows, cols)).astype(np.float32)
    if kind == "u11":
        return rng.uniform(-1.0, 1.0, size=(rows, cols)).astype(np.float32)
    if kind == "n01":
        return rng.standard_normal(size=(rows, cols), dtype=np.float32)
    if kind == "n002":
        return (rng.standard_normal(size=(rows, cols), dtype=np.float32) * np.float32(0.02))
    if kind == "ones":
        return np.ones((rows, cols), dtype=np.float32)
    raise ValueError(kind)


def draw_ab(M, N, K, kind, seed=1024):
    rng = np.random.Generator(np.random.PCG64(seed))
    a = draw(rng, M, K, kind)
    b = draw(rng, N, K, kind)
    return a, b


def _f32_to_bf16_bits(x):
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def cast(x, in_type):
    """Logical fp32 matrix -> storage element type: float32, or uint16 bit
    patterns for fp16 / bf16 (round to nearest even)."""
    if in_type == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if in_type == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    if in_type == "bf16":
        return _f32_to_bf16_bits(x)
    raise ValueError(in_type)


def min_ld(contig_extent, elem_bytes):
    """Smallest leading dimension >= the contiguous extent whose byte size is a
    multiple of 16 (the pages require 16-byte aligned contiguous dimensions)."""
    per = 16 // elem_bytes
    return max(per, -(-contig_extent // per) * per)


def store(x, first_contig, ld, fill=0):
    """Lay out logical 2-D ``x`` (rows x cols) in flat storage.

    first_contig=False: row-major, element (i, j) at i*ld + j (ld >= cols).
    first_contig=True:  column-major, element (i, j) at i + j*ld (ld >= rows).
    The padding of every row/column holds ``fill``.
    """
    rows, cols = x.shape
    if first_contig:
        outer, inner, src = cols, rows, x.T
    else:
        outer, inner, src = rows, cols, x
    assert ld >= inner
    buf = np.empty((outer, ld), dtype=x.dtype)
    if ld > inner:
        buf[:, inner:] = fill
    buf[:, :inner] = src
    return buf.reshape(-1)


def load(buf, rows, cols, first_contig, ld):
    """Inverse of ``store``: logical rows x cols view of flat storage."""
    outer = cols if first_contig else rows
    inner = rows if first_contig else cols
    m = np.asarray(buf)[: outer * ld].reshape(outer, ld)[:, :inner]
    return m.T if first_contig else m


def problem(M, N, K, a_major, b_major, c_major, dtype, kind, seed=1024,
            lda=None, ldb=None, ldc=None, pad_fill=None):
    """A complete seeded problem: flat storage for A and B, and the layout of C.

    ``dtype`` is a gemm dtype code or name.  Returns a dict with the storage
    arrays, leading dimensions and types.  ``pad_fill`` (default 0) is written
    into the leading-dimension padding of A and B.
    """
    code = DTYPE_CODE[dtype] if isinstance(dtype, str) else int(dtype)
    _, tin, tout = DTYPES[code]
    a_log, b_log = draw_ab(M, N, K, kind, seed)
    a_t, b_t = cast(a_log, tin), cast(b_log, tin)
    eb, ebo = ELEM_BYTES[tin], ELEM_BYTES[tout]
    a_first = a_major == "m"
    b_first = b_major == "n"
    c_first = c_major == "m"
    lda = lda or min_ld(M if a_first else K, eb)
    ldb = ldb or min_ld(N if b_first else K, eb)
    ldc = ldc or min_ld(M if c_first else N, ebo)
    fill = 0 if pad_fill is None else pad_fill
    if tin != "f32" and pad_fill is not None:
        fill = cast(np.array([[pad_fill]], dtype=np.float32), tin)[0, 0]
    A = store(a_t, a_first, lda, fill)
    B = store(b_t, b_first, ldb, fill)
    return dict(M=M, N=N, K=K, a_major=a_major, b_major=b_major, c_major=c_major,
                dtype=code, in_type=tin, out_type=tout, A=A, B=B, lda=lda, ldb=ldb,
                ldc=ldc, c_first=c_first)
