"""ctypes binding of libmi355_gemm.so -- argument marshalling only.

Every function here forwards to the C ABI of the same name (see
include/mi355_gemm.h); all GEMM work runs in the library's HIP kernels.  There
is no fallback: importing this module fails loudly when the library has not
been built.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmi355_gemm.so")
DEFAULT_TABLE = os.path.join(HERE, "tuning", "table.txt")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python dense_gemm_engineering_run_amd/build.py, or __graft_entry__.build())")

# PyTorch (used for device memory and streams) ships its own HIP runtime with
# the same SONAME as /opt/rocm's.  Loading torch first makes the library bind
# to that one copy; loading the library first would leave two HIP runtimes in
# the process and kernel launches on torch's memory would fail.
try:
    import torch  # noqa: F401
except ImportError:
    pass

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                p = line.split()[-1]
                if "libamdhip64.so" in os.path.basename(p):
                    paths.add(os.path.realpath(p))
    except OSError:
        pass
    return sorted(paths)


if len(_hip_runtimes()) > 1:
    raise ImportError(f"two HIP runtimes are loaded ({_hip_runtimes()}); import torch before any "
                      "other HIP library, or load this package first")

_i64, _int, _chr, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_char, ctypes.c_void_p
class Epilogue(ctypes.Structure):
    """gemm_epilogue_t: C = act(alpha * A.B^T + beta * C_old + bias)."""
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("bias", ctypes.c_void_p), ("activation", ctypes.c_int)]


_RUN_ARGS = [_i64, _i64, _i64, _chr, _chr, _chr, _int, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.gemm_run.argtypes = _RUN_ARGS
_lib.gemm_run.restype = _int
_lib.gemm_run_batched.argtypes = _RUN_ARGS[:-1] + [_i64, _i64, _i64, _i64, _vp]
_lib.gemm_run_batched.restype = _int
_lib.gemm_run_ws.argtypes = _RUN_ARGS[:-1] + [_vp, ctypes.c_size_t, _vp, _int]
_lib.gemm_run_ws.restype = _int
_lib.gemm_run_noalloc.argtypes = _RUN_ARGS + [_int]
_lib.gemm_run_noalloc.restype = _int
_lib.gemm_run_ex.argtypes = _RUN_ARGS[:-1] + [ctypes.POINTER(Epilogue), _vp, ctypes.c_size_t, _vp,
                                              _int]
_lib.gemm_run_ex.restype = _int
_lib.gemm_workspace_size.argtypes = [_i64, _i64, _i64, _chr, _chr, _chr, _int, _int,
                                     ctypes.POINTER(ctypes.c_size_t)]
_lib.gemm_workspace_size.restype = _int
_lib.gemm_run_config.argtypes = _RUN_ARGS + [_int]
_lib.gemm_run_config.restype = _int
_lib.gemm_status_str.argtypes = [_int]
_lib.gemm_status_str.restype = ctypes.c_char_p
_lib.gemm_num_configs.argtypes = [_int]
_lib.gemm_num_configs.restype = _int
_lib.gemm_config_describe.argtypes = [_int, _int, ctypes.c_char_p, ctypes.c_size_t]
_lib.gemm_config_describe.restype = _int
_lib.gemm_select_config.argtypes = [_i64, _i64, _i64, _chr, _chr, _chr, _int]
_lib.gemm_select_config.restype = _int
_lib.gemm_last_config.argtypes = []
_lib.gemm_last_config.restype = _int
_lib.gemm_load_tuning.argtypes = [ctypes.c_char_p]
_lib.gemm_load_tuning.restype = _int
_lib.gemm_tuning_size.argtypes = []
_lib.gemm_tuning_size.restype = _int
_lib.gemm_probe_mfma_flops.argtypes = [_int]
_lib.gemm_probe_mfma_flops.restype = ctypes.c_double
_lib.gemm_probe_mfma.argtypes = [_int, _int, _vp, _i64, _int, _vp, _vp]
_lib.gemm_probe_mfma.restype = _int
_lib.gemm_probe_hbm_read.argtypes = [_vp, _i64, _i64, _int, _vp, _vp]
_lib.gemm_probe_hbm_read.restype = _int

# gemm_dtype_t
DTYPE_F32, DTYPE_F16_F32, DTYPE_BF16_BF16, DTYPE_F16_F16, DTYPE_BF16_F32 = range(5)
DTYPE_NAMES = ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"]

# gemm_status_t (values as in include/mi355_gemm.h)
GEMM_OK = 0
GEMM_ERR_NULL_PTR = 1
GEMM_ERR_BAD_SHAPE = 2
GEMM_ERR_BAD_MAJOR = 3
GEMM_ERR_BAD_DTYPE = 4
GEMM_ERR_BAD_LD = 5
GEMM_ERR_MISALIGNED = 6
GEMM_ERR_ALIAS = 7
GEMM_ERR_NO_CONFIG = 8
GEMM_ERR_HIP = 9
GEMM_ERR_TUNING_FILE = 10
GEMM_ERR_BAD_EPILOGUE = 11
GEMM_ERR_WORKSPACE = 12
GEMM_ERR_SCRATCH_LIMIT = 13

# bytes of the device scratch array behind gemm_run_noalloc
GEMM_NOALLOC_SCRATCH_BYTES = 64 << 20

# gemm_activation_t
GEMM_ACT_NONE, GEMM_ACT_RELU, GEMM_ACT_GELU = range(3)



class GemmError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"gemm status {status}: {gemm_status_str(status)}")


def _c(ch):
    return ch.encode() if isinstance(ch, str) else bytes([ch])


def gemm_run(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, stream=0):
    """C ABI gemm_run; A, B, C and stream are integer addresses. Returns the status."""
    return _lib.gemm_run(M, N, K, _c(a_major), _c(b_major), _c(c_major), dtype, A, B, C,
                         lda, ldb, ldc, stream)


def gemm_run_batched(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, batch,
                     stride_a, stride_b, stride_c, stream=0):
    """C ABI gemm_run_batched (strides in elements). Returns the status."""
    return _lib.gemm_run_batched(M, N, K, _c(a_major), _c(b_major), _c(c_major), dtype, A, B, C,
                                 lda, ldb, ldc, batch, stride_a, stride_b, stride_c, stream)


def gemm_run_noalloc(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, stream=0,
                     config_id=-1):
    """C ABI gemm_run_noalloc (the library's own device scratch as workspace). Returns the status."""
    return _lib.gemm_run_noalloc(M, N, K, _c(a_major), _c(b_major), _c(c_major), dtype, A, B, C,
                                 lda, ldb, ldc, stream, config_id)


def gemm_run_ws(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, workspace,
                workspace_bytes, stream=0, config_id=-1):
    """C ABI gemm_run_ws. Returns the status."""
    return _lib.gemm_run_ws(M, N, K, _c(a_major), _c(b_major), _c(c_major), dtype, A, B, C,
                            lda, ldb, ldc, workspace, workspace_bytes, stream, config_id)


def gemm_run_ex(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, epilogue=None,
                workspace=0, workspace_bytes=0, stream=0, config_id=-1):
    """C ABI gemm_run_ex; `epilogue` is an Epilogue or None. Returns the status."""
    epi = ctypes.byref(epilogue) if epilogue is not None else None
    return _lib.gemm_run_ex(M, N, K, _c(a_major), _c(b_major), _c(c_major), dtype, A, B, C,
                            lda, ldb, ldc, epi, workspace, workspace_bytes, stream, config_id)


def gemm_workspace_size(M, N, K, a_major, b_major, c_major, dtype, config_id=-1):
    """Workspace bytes for gemm_run_ws; raises GemmError on invalid arguments."""
    n = ctypes.c_size_t(0)
    st = _lib.gemm_workspace_size(M, N, K, _c(a_major), _c(b_major), _c(c_major), dtype,
                                  config_id, ctypes.byref(n))
    if st != GEMM_OK:
        raise GemmError(st)
    return n.value


def gemm_run_config(M, N, K, a_major, b_major, c_major, dtype, A, B, C, lda, ldb, ldc, stream,
                    config_id):
    return _lib.gemm_run_config(M, N, K, _c(a_major), _c(b_major), _c(c_major), dtype, A, B, C,
                                lda, ldb, ldc, stream, config_id)


def gemm_status_str(status):
    return _lib.gemm_status_str(status).decode()


def gemm_num_configs(dtype):
    return _lib.gemm_num_configs(dtype)


def gemm_config_describe(dtype, config_id):
    buf = ctypes.create_string_buffer(128)
    st = _lib.gemm_config_describe(dtype, config_id, buf, len(buf))
    if st != GEMM_OK:
        raise GemmError(st)
    return buf.value.decode()


def gemm_select_config(M, N, K, a_major, b_major, c_major, dtype):
    return _lib.gemm_select_config(M, N, K, _c(a_major), _c(b_major), _c(c_major), dtype)


def gemm_last_config():
    return _lib.gemm_last_config()


def gemm_load_tuning(path):
    return _lib.gemm_load_tuning(None if path is None else os.fsencode(path))


def gemm_tuning_size():
    return _lib.gemm_tuning_size()


# ---------------------------------------------------------------- torch convenience

def _major(t, first, second):
    """Major character of a 2-D tensor view: `first` if dim 0 is contiguous."""
    s0, s1 = t.stride()
    if s1 == 1 and (s0 >= max(1, t.shape[1]) or t.shape[0] <= 1):
        return second, s0 if t.shape[0] > 1 else max(1, t.shape[1])
    if s0 == 1 and (s1 >= max(1, t.shape[0]) or t.shape[1] <= 1):
        return first, s1 if t.shape[1] > 1 else max(1, t.shape[0])
    raise ValueError(f"tensor with strides {t.stride()} has no contiguous dimension")


def dtype_code(in_dtype, out_dtype):
    import torch
    table = {(torch.float32, torch.float32): DTYPE_F32,
             (torch.float16, torch.float32): DTYPE_F16_F32,
             (torch.bfloat16, torch.bfloat16): DTYPE_BF16_BF16,
             (torch.float16, torch.float16): DTYPE_F16_F16,
             (torch.bfloat16, torch.float32): DTYPE_BF16_F32}
    try:
        return table[(in_dtype, out_dtype)]
    except KeyError:
        raise ValueError(f"unsupported dtype pair {in_dtype} -> {out_dtype}") from None


def gemm(a, b, c, stream=None, config=None):
    """C = A * B^T for torch device tensors: a is (M, K), b is (N, K), c is (M, N),
    each a 2-D view with one contiguous dimension.  Majors and leading dims are
    read from the strides; the stream defaults to torch's current stream."""
    import torch
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or tuple(c.shape) != (M, N):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}, c {tuple(c.shape)}")
    am, lda = _major(a, "m", "k")
    bm, ldb = _major(b, "n", "k")
    cm, ldc = _major(c, "m", "n")
    code = dtype_code(a.dtype, c.dtype)
    if b.dtype != a.dtype:
        raise ValueError("a and b must have the same dtype")
    if stream is None:
        stream = torch.cuda.current_stream(c.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    args = (M, N, K, am, bm, cm, code, a.data_ptr(), b.data_ptr(), c.data_ptr(), lda, ldb, ldc,
            stream)
    st = gemm_run(*args) if config is None else gemm_run_config(*args, config)
    if st != GEMM_OK:
        raise GemmError(st)
    return c


if not os.environ.get("MI355_GEMM_TUNING") and os.path.exists(DEFAULT_TABLE):
    gemm_load_tuning(DEFAULT_TABLE)


# ---------------------------------------------------------------- measurement probes
# (include/mi355_gemm_probe.h; not part of the GEMM path)

PROBE_F16_16x16x32, PROBE_F16_32x32x16, PROBE_BF16_16x16x32 = range(3)


def gemm_probe_mfma_flops(shape):
    return _lib.gemm_probe_mfma_flops(shape)


def gemm_probe_mfma(shape, rotate, operands, iters, grid, sink, stream=0):
    """C ABI gemm_probe_mfma (device addresses). Returns the status."""
    return _lib.gemm_probe_mfma(shape, int(bool(rotate)), operands, iters, grid, sink, stream)


def gemm_probe_hbm_read(A, rows, row_bytes, seg_bytes, sink, stream=0):
    """C ABI gemm_probe_hbm_read (device addresses). Returns the status."""
    return _lib.gemm_probe_hbm_read(A, rows, row_bytes, seg_bytes, sink, stream)
