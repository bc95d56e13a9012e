"""The C-ABI library without a GPU: it loads, exports every function the header
declares, and rejects bad arguments before touching the HIP runtime.  Config
selection and the tuning table are host logic and are covered here too."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import dense_gemm_engineering_run_amd as g
from dense_gemm_engineering_run_amd import _binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355_gemm.h")

NULL = 0
P = 1 << 20          # a fake, 16-byte aligned device address (never dereferenced)


def declared_functions():
    """Every function declared in include/*.h."""
    import glob
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(gemm_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "gemm_run" in names and "gemm_probe_mfma" in names and len(names) >= 9
    lib = ctypes.CDLL(b.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


# Status values of the boundary: success 0, then the argument errors in the
# order null pointer, shape, major, dtype, leading dimension, alignment,
# aliasing, config, launch; the library's own additions follow.
STATUS_VALUES = {
    "GEMM_OK": 0, "GEMM_ERR_NULL_PTR": 1, "GEMM_ERR_BAD_SHAPE": 2, "GEMM_ERR_BAD_MAJOR": 3,
    "GEMM_ERR_BAD_DTYPE": 4, "GEMM_ERR_BAD_LD": 5, "GEMM_ERR_MISALIGNED": 6, "GEMM_ERR_ALIAS": 7,
    "GEMM_ERR_NO_CONFIG": 8, "GEMM_ERR_HIP": 9, "GEMM_ERR_TUNING_FILE": 10,
    "GEMM_ERR_BAD_EPILOGUE": 11, "GEMM_ERR_WORKSPACE": 12, "GEMM_ERR_SCRATCH_LIMIT": 13,
}


def header_enum(name):
    """{enumerator: value} of the typedef enum `name` in the header."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef enum \{([^}]*)\}\s*" + name + ";", text).group(1)
    return {k: int(v) for k, v in re.findall(r"(\w+)\s*=\s*(\d+)", body)}


def test_status_values_pinned_in_header_and_binding():
    assert header_enum("gemm_status_t") == STATUS_VALUES
    for k, v in STATUS_VALUES.items():
        assert getattr(b, k) == v, k
    assert header_enum("gemm_dtype_t") == {"GEMM_DTYPE_F32": 0, "GEMM_DTYPE_F16_F32": 1,
                                           "GEMM_DTYPE_BF16_BF16": 2, "GEMM_DTYPE_F16_F16": 3,
                                           "GEMM_DTYPE_BF16_F32": 4, "GEMM_NUM_DTYPES": 5}
    assert header_enum("gemm_activation_t") == {"GEMM_ACT_NONE": 0, "GEMM_ACT_RELU": 1, "GEMM_ACT_GELU": 2}
    assert (b.GEMM_ACT_NONE, b.GEMM_ACT_RELU, b.GEMM_ACT_GELU) == (0, 1, 2)


def test_status_strings():
    for st in range(len(STATUS_VALUES)):
        s = g.gemm_status_str(st)
        assert s and s != "unknown status"
    assert g.gemm_status_str(99) == "unknown status"


def run(M=64, N=64, K=64, a="k", bm="k", c="n", dtype=0, A=P, B=2 * P, C=3 * P, lda=None,
        ldb=None, ldc=None):
    lda = lda if lda is not None else (K if a in "kK" else M)
    ldb = ldb if ldb is not None else (K if bm in "kK" else N)
    ldc = ldc if ldc is not None else (N if c in "nN" else M)
    return g.gemm_run(M, N, K, a, bm, c, dtype, A, B, C, lda, ldb, ldc, 0)


def test_validation_errors_without_gpu():
    assert run(M=-1) == b.GEMM_ERR_BAD_SHAPE
    assert run(K=-5) == b.GEMM_ERR_BAD_SHAPE
    assert run(M=1 << 31) == b.GEMM_ERR_BAD_SHAPE
    assert run(a="n") == b.GEMM_ERR_BAD_MAJOR
    assert run(bm="m") == b.GEMM_ERR_BAD_MAJOR
    assert run(c="k") == b.GEMM_ERR_BAD_MAJOR
    assert run(dtype=5) == b.GEMM_ERR_BAD_DTYPE
    assert run(dtype=-1) == b.GEMM_ERR_BAD_DTYPE
    assert run(lda=63) == b.GEMM_ERR_BAD_LD
    assert run(a="m", lda=32) == b.GEMM_ERR_BAD_LD
    assert run(ldc=0, N=0) == b.GEMM_ERR_BAD_LD           # ld must be >= 1
    # At most 2^48 bytes spanned by an operand's rows: one row of fp32 allows
    # ld up to 2^46 elements, 64 rows up to 2^40; beyond that (and near 2^63,
    # where the byte offsets would wrap) the call is refused before any offset
    # is formed.  At 2^46 validation passes and the launch then refuses the
    # tile's 32-bit row offsets.
    assert run(M=1, lda=1 << 46) == b.GEMM_ERR_BAD_SHAPE
    assert run(M=1, lda=(1 << 46) + 1) == b.GEMM_ERR_BAD_LD
    assert run(lda=(1 << 40) + 1) == b.GEMM_ERR_BAD_LD
    assert run(ldb=(1 << 62) + 64) == b.GEMM_ERR_BAD_LD
    assert run(ldc=(1 << 63) - 1) == b.GEMM_ERR_BAD_LD
    assert run(a="m", lda=(1 << 61)) == b.GEMM_ERR_BAD_LD
    assert run(A=NULL) == b.GEMM_ERR_NULL_PTR
    assert run(B=NULL) == b.GEMM_ERR_NULL_PTR
    assert run(C=NULL) == b.GEMM_ERR_NULL_PTR
    assert run(A=P + 2) == b.GEMM_ERR_MISALIGNED               # fp32 needs 4-byte alignment
    assert run(C=3 * P + 1, dtype=2) == b.GEMM_ERR_MISALIGNED   # bf16 C needs 2
    assert run(B=2 * P + 1, dtype=1) == b.GEMM_ERR_MISALIGNED
    assert run(C=P + 64 * 16) == b.GEMM_ERR_ALIAS          # C starts inside A
    assert run(C=P - 64 * 64 * 4 + 16) == b.GEMM_ERR_ALIAS  # C ends inside A
    assert run(lda=63, a="x") == b.GEMM_ERR_BAD_MAJOR       # checks run in header order
    assert g.gemm_last_config() == -1


def test_unaligned_operands_take_the_scalar_configs_without_gpu():
    """Operands that are not 16-byte aligned pass validation (the launch then
    fails only for lack of a GPU here) and run on the element-by-element
    configs; a forced 16-byte config is refused."""
    scalar = [i for i in range(g.gemm_num_configs(0)) if g.gemm_config_describe(0, i).endswith("scalar")]
    assert len(scalar) == 4          # fp32: two with 4-byte direct loads, two register-staged
    for kw in (dict(K=30, lda=30, ldb=32), dict(A=P + 4), dict(C=3 * P + 8), dict(ldc=65),
               dict(K=60, dtype=1, lda=60, ldb=64), dict(A=P + 2, dtype=2)):
        assert run(**kw) == b.GEMM_ERR_HIP, kw
    assert run_batched(sa=2) == b.GEMM_ERR_HIP                  # 8-byte batch stride
    args = (64, 64, 30, "k", "k", "n", 0, P, 2 * P, 3 * P, 30, 30, 64, 0)
    assert g.gemm_run_config(*args, 0) == b.GEMM_ERR_MISALIGNED
    assert g.gemm_run_config(*args, scalar[0]) == b.GEMM_ERR_HIP
    # aligned operands may use a scalar config too
    assert g.gemm_run_config(64, 64, 64, "k", "k", "n", 0, P, 2 * P, 3 * P, 64, 64, 64, 0,
                             scalar[1]) == b.GEMM_ERR_HIP
    for d in range(5):
        assert sum(g.gemm_config_describe(d, i).endswith("scalar")
                   for i in range(g.gemm_num_configs(d))) == (4 if d == 0 else 2)
    # the large unaligned fp32 problems take the direct-to-LDS element loads
    assert g.gemm_config_describe(0, g.gemm_select_config(4095, 2049, 1028, "k", "k", "n", 0)) != ""


def test_degenerate_sizes_without_gpu():
    # M == 0 or N == 0: no launch, OK; pointers may be NULL.
    assert run(M=0, A=NULL, B=NULL, C=NULL) == b.GEMM_OK
    assert run(N=0, A=NULL, B=NULL, C=NULL, ldc=4) == b.GEMM_OK
    # K == 0 needs no A/B (but does need C): the NULL checks reflect that.
    assert run(K=0, A=NULL, B=NULL, C=NULL, lda=1, ldb=1) == b.GEMM_ERR_NULL_PTR
    assert g.gemm_last_config() == -1


def run_batched(batch=2, sa=64 * 64, sb=64 * 64, sc=64 * 64, M=64, N=64, K=64, A=P, B=2 * P,
                C=3 * P):
    return g.gemm_run_batched(M, N, K, "k", "k", "n", 0, A, B, C, K, K, N, batch, sa, sb, sc, 0)


def test_batched_validation_without_gpu():
    assert run_batched(batch=-1) == b.GEMM_ERR_BAD_SHAPE
    assert run_batched(batch=65536) == b.GEMM_ERR_BAD_SHAPE
    assert run_batched(sa=-64) == b.GEMM_ERR_BAD_LD
    assert run_batched(sc=64 * 64 - 4) == b.GEMM_ERR_BAD_LD     # C entries would overlap
    assert run_batched(sc=0) == b.GEMM_ERR_BAD_LD               # ... also when identical
    # batch x stride at most 2^48 bytes: two fp32 entries allow strides up to 2^45.
    assert run_batched(sa=1 << 45, sb=1 << 45, C=1 << 49) == b.GEMM_ERR_HIP
    assert run_batched(sa=(1 << 45) + 4) == b.GEMM_ERR_BAD_LD
    assert run_batched(sb=1 << 62) == b.GEMM_ERR_BAD_LD
    assert run_batched(sc=(1 << 63) - 1) == b.GEMM_ERR_BAD_LD

    # A's entries reach into C's range: entry 2 of A starts at 3P.
    assert run_batched(batch=3, sa=(1 << 20) // 4) == b.GEMM_ERR_ALIAS
    # batch 0 launches nothing and needs no pointers; strides may then be anything >= 0.
    assert run_batched(batch=0, A=NULL, B=NULL, C=NULL, sc=0) == b.GEMM_OK
    # Broadcast operands (stride 0) and an empty M pass validation without a launch.
    assert run_batched(M=0, sa=0, sb=0, sc=0) == b.GEMM_OK
    assert g.gemm_last_config() == -1


def sk_config(name):
    for i in range(g.gemm_num_configs(0)):
        if g.gemm_config_describe(0, i) == name:
            return i
    raise KeyError(name)


def test_stream_k_workspace_size_and_errors_without_gpu():
    sk = sk_config("f32 256x256x32 w2x2 mfma32 s2 dma sk")
    # 4095 x 2049: 16 x 9 = 144 tiles of 256 x 256 (< 256 workgroups, so all are
    # stream-K), 33 k-tiles each: 4752 iterations over 256 workgroups; counters
    # (144 ints -> 768 bytes) plus two 256 KB partial tiles per workgroup.
    need = g.gemm_workspace_size(4095, 2049, 1028, "k", "k", "n", 0, sk)
    assert need == 768 + 2 * 256 * 256 * 256 * 4
    # The C-m-major swap exchanges M and N: same tile count.
    assert g.gemm_workspace_size(2049, 4095, 1028, "k", "k", "m", 0, sk) == need
    # Whole waves (1024 tiles = 4 x 256) and K = 0 need no workspace.
    assert g.gemm_workspace_size(8192, 8192, 8192, "m", "n", "n", 0, sk) == 0
    assert g.gemm_workspace_size(4095, 2049, 0, "k", "k", "n", 0, sk) == 0
    # 257 tiles: one data-parallel wave, then the last tile's 8 k-iterations
    # shared by 8 workgroups (at least an eighth of a tile each).
    n257 = g.gemm_workspace_size(257 * 256, 256, 256, "k", "k", "n", 0, sk)
    assert n257 == 256 + 2 * 8 * 256 * 256 * 4
    # Not a stream-K config: no workspace.
    assert g.gemm_workspace_size(4095, 2049, 1028, "k", "k", "n", 0, 0) == 0
    with pytest.raises(g.GemmError):
        g.gemm_workspace_size(-1, 2, 3, "k", "k", "n", 0)
    with pytest.raises(g.GemmError):
        g.gemm_workspace_size(1, 2, 3, "k", "k", "n", 0, 999)

    def run_ws(ws, nbytes, config=sk, C=3 * P):
        return g.gemm_run_ws(4095, 2049, 1028, "k", "k", "n", 0, P, P + (1 << 24), C, 1028, 1028,
                             2052, ws, nbytes, 0, config)

    A_end = P + (1 << 24) + 2049 * 1028 * 4
    C = 1 << 32
    assert run_ws(0, 0, C=C) == b.GEMM_ERR_WORKSPACE
    assert run_ws(1 << 34, need - 16, C=C) == b.GEMM_ERR_WORKSPACE
    assert run_ws((1 << 34) + 8, need, C=C) == b.GEMM_ERR_MISALIGNED
    assert run_ws(A_end - 64, need, C=C) == b.GEMM_ERR_ALIAS          # overlaps B
    assert run_ws(C + 4096, need, C=C) == b.GEMM_ERR_ALIAS            # overlaps C
    assert g.gemm_run_config(4095, 2049, 1028, "k", "k", "n", 0, P, P + (1 << 24), C, 1028, 1028,
                             2052, 0, sk) == b.GEMM_ERR_WORKSPACE
    # Stream-K configs take no batch.
    assert g.gemm_last_config() == -1


def test_split_k_workspace_size_and_errors_without_gpu():
    """Split-k configs: k-ranges per tile S = floor(256 * workgroups per CU /
    tiles), at most 32 and at most half the k-tiles (at least 1), and a
    workspace of tiles * S partial fp32 tiles; without one, or with a batch,
    a forced split-k config is refused before any HIP call."""
    def cfg(dtype, name):
        return next(i for i in range(g.gemm_num_configs(dtype)) if g.gemm_config_describe(dtype, i) == name)
    big = cfg(2, "bf16_bf16 256x256x64 w4x2 mfma16 s3x2 dma split")
    small = cfg(2, "bf16_bf16 128x128x64 w2x2 mfma32 s2x2 dma split")
    f32 = cfg(0, "f32 128x128x32 w2x2 mfma32 s2 dma split")
    ws = lambda c, M, N, K, dtype=2, cm="n": g.gemm_workspace_size(M, N, K, "k", "k", cm, dtype, c)
    # 8192 x 256: 32 tiles of 256x256 -> S = 8; 128 tiles of 128x128 at two per CU -> S = 4
    assert ws(big, 8192, 256, 4096) == 32 * 8 * 256 * 256 * 4
    assert ws(small, 8192, 256, 4096) == 128 * 4 * 128 * 128 * 4
    # 600 x 520: 9 tiles -> 28 ranges; 25 tiles -> 20 (K = 4100: 65 k-tiles)
    assert ws(big, 600, 520, 4100) == 9 * 28 * 256 * 256 * 4
    assert ws(small, 600, 520, 4100) == 25 * 20 * 128 * 128 * 4
    # one tile: capped at 32 ranges; a short K: at most half its k-tiles
    assert ws(big, 256, 256, 8192) == 32 * 256 * 256 * 4
    assert ws(big, 256, 256, 320) == 2 * 256 * 256 * 4          # 5 k-tiles -> 2 ranges
    assert ws(big, 256, 256, 64) == 256 * 256 * 4               # one k-tile, one range
    # many tiles: one range each (still a partial tile per tile)
    assert ws(big, 8192, 8192, 1024) == 1024 * 256 * 256 * 4
    # fp32 (32-deep k-tiles) and the C-m-major swap
    assert ws(f32, 1024, 1024, 4096, dtype=0) == 64 * 8 * 128 * 128 * 4
    assert ws(f32, 1024, 2048, 4096, dtype=0, cm="m") == ws(f32, 2048, 1024, 4096, dtype=0)

    # K = 4104 (65 k-tiles as for 4100; rows of 8208 bytes, 16-byte multiples)
    def run(config, ws_ptr, nbytes):
        return g.gemm_run_ws(600, 520, 4104, "k", "k", "n", 2, P, P + (1 << 26), 1 << 32, 4104, 4104,
                             520, ws_ptr, nbytes, 0, config)
    need = ws(small, 600, 520, 4104)
    assert need == ws(small, 600, 520, 4100)
    assert run(small, 0, 0) == b.GEMM_ERR_WORKSPACE
    assert run(small, 1 << 34, need - 16) == b.GEMM_ERR_WORKSPACE
    assert run(small, (1 << 34) + 8, need) == b.GEMM_ERR_MISALIGNED
    assert g.gemm_run_config(600, 520, 4104, "k", "k", "n", 2, P, P + (1 << 26), 1 << 32, 4104, 4104,
                             520, 0, small) == b.GEMM_ERR_WORKSPACE
    assert g.gemm_last_config() == -1
    # The allocation-free entry point refuses a split that outgrows its scratch.
    st = g.gemm_run_noalloc(8192, 8192, 8192, "k", "k", "n", 2, 1 << 34, 1 << 35, 1 << 36, 8192, 8192,
                            8192, 0, big)
    assert ws(big, 8192, 8192, 8192) > b.GEMM_NOALLOC_SCRATCH_BYTES
    assert st == b.GEMM_ERR_SCRATCH_LIMIT, g.gemm_status_str(st)


def test_select_config_never_returns_stream_k(tmp_path):
    sk_name = "f32 256x256x32 w2x2 mfma32 s2 dma sk"
    t = tmp_path / "t.txt"
    t.write_text(f"f32 k k n 4095 2049 1028 {sk_name}\n")
    try:
        assert g.gemm_load_tuning(str(t)) == 0
        chosen = g.gemm_select_config(4095, 2049, 1028, "k", "k", "n", 0)
        assert chosen >= 0 and not g.gemm_config_describe(0, chosen).endswith(" sk")
        # With a workspace the table's stream-K choice is the one sized.
        assert g.gemm_workspace_size(4095, 2049, 1028, "k", "k", "n", 0) > 0
    finally:
        g.gemm_load_tuning(os.path.join(ROOT, "dense_gemm_engineering_run_amd", "tuning", "table.txt"))


def test_epilogue_errors_without_gpu():
    def run_ex(epi, C=3 * P):
        return g.gemm_run_ex(64, 64, 64, "k", "k", "n", 0, P, 2 * P, C, 64, 64, 64, epi)
    assert run_ex(g.Epilogue(1.0, 0.0, P + 2, 0)) == b.GEMM_ERR_MISALIGNED   # bias not 4-byte aligned
    assert run_ex(g.Epilogue(1.0, 0.0, 3 * P + 64, 0)) == b.GEMM_ERR_ALIAS   # bias inside C
    assert run_ex(g.Epilogue(1.0, 0.0, 0, 7)) == b.GEMM_ERR_BAD_EPILOGUE
    assert run_ex(g.Epilogue(1.0, 0.0, 0, -1)) == b.GEMM_ERR_BAD_EPILOGUE
    # Forced stream-K configs of either tile size accept an active epilogue
    # (and then need their workspace).
    def sk_id(name):
        return next(i for i in range(g.gemm_num_configs(0)) if g.gemm_config_describe(0, i) == name)
    relu = g.Epilogue(1.0, 0.0, 0, g.GEMM_ACT_RELU)
    big, small = sk_id("f32 256x256x32 w2x2 mfma32 s2 dma sk"), sk_id("f32 128x128x32 w2x2 mfma32 s2 dma sk")
    def run_sk(config, epi):
        return g.gemm_run_ex(4095, 2049, 1028, "k", "k", "n", 0, P, P + (1 << 24), 1 << 32, 1028, 1028,
                             2052, epi, 0, 0, 0, config)
    assert run_sk(big, relu) == b.GEMM_ERR_WORKSPACE
    assert run_sk(big, g.Epilogue(1.0, 0.0, 0, g.GEMM_ACT_NONE)) == b.GEMM_ERR_WORKSPACE   # identity
    assert run_sk(small, relu) == b.GEMM_ERR_WORKSPACE
    # argument errors come first, in status order
    assert g.gemm_run_ex(-1, 64, 64, "k", "k", "n", 0, P, 2 * P, 3 * P, 64, 64, 64,
                         g.Epilogue(1.0, 0.0, 0, 7)) == b.GEMM_ERR_BAD_SHAPE
    # an empty problem still rejects a bad activation, launches nothing otherwise
    assert g.gemm_run_ex(0, 64, 64, "k", "k", "n", 0, 0, 0, 0, 64, 64, 64,
                         g.Epilogue(1.0, 0.0, 0, 7)) == b.GEMM_ERR_BAD_EPILOGUE
    assert g.gemm_run_ex(0, 64, 64, "k", "k", "n", 0, 0, 0, 0, 64, 64, 64,
                         g.Epilogue(2.0, 1.0, 0, 1)) == b.GEMM_OK
    assert g.gemm_last_config() == -1


def test_majors_case_insensitive():
    assert run(a="X") == b.GEMM_ERR_BAD_MAJOR
    assert run(M=0, a="K", bm="N", c="M", ldc=4) == b.GEMM_OK


def test_config_registry():
    for d in range(5):
        n = g.gemm_num_configs(d)
        assert n >= 3
        names = [g.gemm_config_describe(d, i) for i in range(n)]
        assert len(set(names)) == n
        assert all(nm.startswith(b.DTYPE_NAMES[d] + " ") for nm in names)
        with pytest.raises(b.GemmError):
            g.gemm_config_describe(d, n)
    assert g.gemm_num_configs(7) == 0
    buf = ctypes.create_string_buffer(8)
    assert b._lib.gemm_config_describe(0, 0, buf, 8) == b.GEMM_OK and len(buf.value) == 7
    assert g.gemm_run_config(64, 64, 64, "k", "k", "n", 0, P, 2 * P, 3 * P, 64, 64, 64, 0,
                             999) == b.GEMM_ERR_NO_CONFIG
    assert g.gemm_run_config(64, 64, 64, "k", "k", "n", 0, P, 2 * P, 3 * P, 64, 64, 64, 0,
                             -1) == b.GEMM_ERR_NO_CONFIG


def test_select_config_is_host_logic():
    for d in range(5):
        for shape in [(1, 1, 1), (1024, 512, 256), (8192, 8192, 8192), (65536, 256, 4096)]:
            for c in "nm":
                cfg = g.gemm_select_config(*shape, "k", "k", c, d)
                assert 0 <= cfg < g.gemm_num_configs(d)
    assert g.gemm_select_config(-1, 1, 1, "k", "k", "n", 0) == -b.GEMM_ERR_BAD_SHAPE
    assert g.gemm_select_config(1, 1, 1, "q", "k", "n", 0) == -b.GEMM_ERR_BAD_MAJOR
    assert g.gemm_select_config(1, 1, 1, "k", "k", "n", 9) == -b.GEMM_ERR_BAD_DTYPE


def test_heuristic_for_large_untuned_16bit_shapes():
    """Shapes far from every tuned key take the heuristic: with K >= 1024 and
    a k-contiguous operand the ping-pong 256x256 config (for A k, B n it
    stores C transposed with the operands swapped), and with neither
    operand k-contiguous from 512 such tiles up; otherwise the 256x256 tile
    on 16x16x32 MFMAs, except for fp32 outputs on grids of 512 or more of
    its tiles, which keep the 32x32x16 form."""
    def chosen(M, N, K, d, a="k", b="k"):
        return g.gemm_config_describe(d, g.gemm_select_config(M, N, K, a, b, "n", d))
    assert chosen(16384, 16384, 1024, 3) == "f16_f16 256x256x64 w4x2 mfma16 s3x2 pp"
    assert chosen(3008, 12000, 3008, 2) == "bf16_bf16 256x256x64 w4x2 mfma16 s3x2 pp"
    assert chosen(16384, 16384, 1024, 1) == "f16_f32 256x256x64 w4x2 mfma16 s3x2 pp"
    assert chosen(16384, 16384, 1024, 1, a="m") == "f16_f32 256x256x64 w4x2 mfma16 s3x2 pp"
    assert chosen(16384, 16384, 1024, 3, b="n") == "f16_f16 256x256x64 w4x2 mfma16 s3x2 pp"
    assert chosen(16384, 16384, 512, 3) == "f16_f16 256x256x64 w4x2 mfma16 s2 dma"
    assert chosen(16384, 16384, 1024, 3, a="m", b="n") == "f16_f16 256x256x64 w4x2 mfma16 s3x2 pp"
    assert chosen(3008, 12000, 3008, 2, a="m", b="n") == "bf16_bf16 256x256x64 w4x2 mfma16 s3x2 pp"
    assert chosen(16384, 16384, 1024, 1, a="m", b="n") == "f16_f32 256x256x64 w4x2 mfma16 s3x2 pp"
    assert chosen(16384, 16384, 512, 1, a="m", b="n") == "f16_f32 256x256x64 w4x2 mfma32 s2 dma"
    assert chosen(16384, 16384, 512, 4) == "bf16_f32 256x256x64 w4x2 mfma32 s2 dma"
    # mid-size (65 to 127 tiles of 256x256): the 128x256 tile with a
    # k-contiguous operand, else the 128x128 tile on 32x32x16 MFMAs
    assert chosen(2560, 2560, 16384, 1) == "f16_f32 128x256x64 w2x2 mfma32 s3 dma"
    sel = g.gemm_select_config(2560, 2560, 16384, "m", "n", "n", 1)
    assert g.gemm_config_describe(1, sel) == "f16_f32 128x128x64 w2x2 mfma32 s4 dma"


def test_tuning_table_lookup(tmp_path):
    saved = g.gemm_tuning_size()
    name0 = g.gemm_config_describe(0, 0)
    name2 = g.gemm_config_describe(0, 2)
    t = tmp_path / "t.txt"
    t.write_text(f"# comment\n\nf32 k k n 1000 1000 1000 {name2}\n"
                 f"f32 m n n 8192 8192 8192 {name0}   # trailing comment\n"
                 f"f32 k k n 5 5 5 f32 no such config\n")
    try:
        assert g.gemm_load_tuning(str(t)) == b.GEMM_OK
        assert g.gemm_tuning_size() == 2            # the unknown config is skipped
        assert g.gemm_select_config(1000, 1000, 1000, "k", "k", "n", 0) == 2   # exact
        assert g.gemm_select_config(1100, 900, 1000, "k", "k", "n", 0) == 2    # nearest
        assert g.gemm_select_config(8192, 8192, 8192, "m", "n", "n", 0) == 0
        bad = tmp_path / "bad.txt"
        bad.write_text("f32 k k n 10 10\n")
        assert g.gemm_load_tuning(str(bad)) == b.GEMM_ERR_TUNING_FILE
        assert g.gemm_tuning_size() == 2                                        # kept
        assert g.gemm_load_tuning(str(tmp_path / "missing.txt")) == b.GEMM_ERR_TUNING_FILE
        assert g.gemm_load_tuning(None) == b.GEMM_OK and g.gemm_tuning_size() == 0
    finally:
        if os.path.exists(b.DEFAULT_TABLE):
            g.gemm_load_tuning(b.DEFAULT_TABLE)
        else:
            g.gemm_load_tuning(None)
    assert g.gemm_tuning_size() == saved


def test_committed_tuning_table_is_whole():
    """Every line of the shipped table names a config the library has (the
    loader skips unknown names, so a renamed config would otherwise drop its
    keys silently), its keys are exactly those of keys.txt, and a key with two
    lines is a stream-K or split-k winner followed by its no-workspace
    fallback."""
    tdir = os.path.join(ROOT, "dense_gemm_engineering_run_amd", "tuning")
    rows = [l.split("#")[0].split() for l in open(os.path.join(tdir, "table.txt"))]
    rows = [r for r in rows if r]
    keys = [l.split("#")[0].split() for l in open(os.path.join(tdir, "keys.txt"))]
    keys = {" ".join(k) for k in keys if len(k) == 7}
    saved = g.gemm_tuning_size()
    try:
        assert g.gemm_load_tuning(os.path.join(tdir, "table.txt")) == b.GEMM_OK
        assert g.gemm_tuning_size() == len(rows)
    finally:
        g.gemm_load_tuning(b.DEFAULT_TABLE)
    assert g.gemm_tuning_size() == saved
    by_key = {}
    for r in rows:
        by_key.setdefault(" ".join(r[:7]), []).append(" ".join(r[7:]))
    assert set(by_key) == keys
    for k, cfgs in by_key.items():
        assert len(cfgs) in (1, 2), k
        ws = [c.endswith(" sk") or c.endswith(" split") for c in cfgs]
        if len(cfgs) == 2:
            assert ws == [True, False], (k, cfgs)


def test_torch_helper_derives_majors_from_strides():
    torch = pytest.importorskip("torch")
    a = torch.empty(64, 40)                      # (M, K) row-major -> 'k', lda 40
    assert b._major(a, "m", "k") == ("k", 40)
    at = torch.empty(40, 72)[:, :64].t()         # (M, K) view of column storage, ld 72
    assert b._major(at, "m", "k") == ("m", 72)
    with pytest.raises(ValueError):
        b._major(torch.empty(8, 8)[::2, ::2], "m", "k")
    assert b.dtype_code(torch.float16, torch.float32) == b.DTYPE_F16_F32
    with pytest.raises(ValueError):
        b.dtype_code(torch.float64, torch.float64)


def test_import_fails_loudly_without_the_library(tmp_path):
    """A copy of the package without libmi355_gemm.so must refuse to import
    (no CPU or eager fallback exists to take over)."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(ROOT, "dense_gemm_engineering_run_amd")
    dst = tmp_path / "dense_gemm_engineering_run_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    assert not any(p.suffix == ".so" for p in dst.iterdir())
    r = subprocess.run([sys.executable, "-c", "import dense_gemm_engineering_run_amd"], cwd=tmp_path,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)}, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libmi355_gemm.so is missing" in r.stderr, r.stderr[-2000:]


def test_build_scripts_need_no_built_library():
    """__graft_entry__.build() must work on a fresh checkout, where the
    libraries do not exist yet: the build scripts load by path and import
    neither package (both packages load their library on import)."""
    import subprocess
    code = (
        "import sys, builtins\n"
        "real = builtins.__import__\n"
        "def guard(name, *a, **k):\n"
        "    if name.split('.')[0] in ('dense_gemm_engineering_run_amd', 'oracle'):\n"
        "        raise ImportError('package imported: ' + name)\n"
        "    return real(name, *a, **k)\n"
        "builtins.__import__ = guard\n"
        "import __graft_entry__ as e\n"
        "import os\n"
        "for p in ('dense_gemm_engineering_run_amd/build.py', 'oracle/build.py'):\n"
        "    m = e._load_script(os.path.join(e.ROOT, p), 'x')\n"
        "    assert callable(m.build), p\n"
        "print('ok')\n")
    import sys
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-2000:]


def test_noalloc_entry_point_host_checks():
    """gemm_run_noalloc validates like gemm_run_ws before any HIP call; a
    forced config that needs more workspace than the fixed scratch is refused
    with its own status; an empty problem is a no-op."""
    text = open(HEADER).read()
    m = re.search(r"#define GEMM_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == b.GEMM_NOALLOC_SCRATCH_BYTES == 64 << 20

    def na(M=64, N=64, K=64, A=P, B=2 * P, C=3 * P, cfg=-1, **kw):
        return g.gemm_run_noalloc(M, N, K, "k", "k", "n", kw.get("dtype", 0), A, B, C,
                                  kw.get("lda", K), kw.get("ldb", K), kw.get("ldc", N), 0, cfg)
    assert na(M=-1) == b.GEMM_ERR_BAD_SHAPE
    assert na(A=NULL) == b.GEMM_ERR_NULL_PTR
    assert na(lda=3) == b.GEMM_ERR_BAD_LD
    assert na(C=P + 16) == b.GEMM_ERR_ALIAS
    assert na(cfg=10 ** 6) == b.GEMM_ERR_NO_CONFIG
    assert na(M=0) == b.GEMM_OK and g.gemm_last_config() == -1
    # the 256x256 fp32 stream-K tile on 24 x 23 tiles with a long K splits 40
    # tiles over 256 workgroups: 128 MiB of partial tiles
    sk = next(i for i in range(g.gemm_num_configs(0))
              if g.gemm_config_describe(0, i) == "f32 256x256x32 w2x2 mfma32 s2 dma sk")
    M, N, K = 6144, 5888, 8192
    need = g.gemm_workspace_size(M, N, K, "k", "k", "n", 0, sk)
    assert need > b.GEMM_NOALLOC_SCRATCH_BYTES
    big = 1 << 34
    st = g.gemm_run_noalloc(M, N, K, "k", "k", "n", 0, big, 2 * big, 3 * big, K, K, N, 0, sk)
    assert st == b.GEMM_ERR_SCRATCH_LIMIT, g.gemm_status_str(st)
    assert "scratch" in g.gemm_status_str(st)


def test_probe_entry_points_host_checks():
    """The measurement probes validate their arguments before any HIP call."""
    assert b.gemm_probe_mfma_flops(b.PROBE_F16_16x16x32) == 16 * 16 * 32 * 2
    assert b.gemm_probe_mfma_flops(b.PROBE_F16_32x32x16) == 32 * 32 * 16 * 2
    assert b.gemm_probe_mfma_flops(b.PROBE_BF16_16x16x32) == 16 * 16 * 32 * 2
    assert b.gemm_probe_mfma_flops(3) == 0
    assert b.gemm_probe_mfma(7, 1, P, 10, 256, 2 * P) == b.GEMM_ERR_BAD_SHAPE
    assert b.gemm_probe_mfma(0, 1, P, -1, 256, 2 * P) == b.GEMM_ERR_BAD_SHAPE
    assert b.gemm_probe_mfma(0, 1, P, 10, 0, 2 * P) == b.GEMM_ERR_BAD_SHAPE
    assert b.gemm_probe_mfma(0, 1, NULL, 10, 256, 2 * P) == b.GEMM_ERR_NULL_PTR
    assert b.gemm_probe_mfma(0, 1, P + 4, 10, 256, 2 * P) == b.GEMM_ERR_MISALIGNED
    assert b.gemm_probe_hbm_read(P, 256, 8192, 96, 2 * P) == b.GEMM_ERR_BAD_SHAPE
    assert b.gemm_probe_hbm_read(P, 255, 8192, 128, 2 * P) == b.GEMM_ERR_BAD_SHAPE
    assert b.gemm_probe_hbm_read(P, 256, 8000, 128, 2 * P) == b.GEMM_ERR_BAD_LD
    assert b.gemm_probe_hbm_read(NULL, 256, 8192, 128, 2 * P) == b.GEMM_ERR_NULL_PTR
    assert b.gemm_probe_hbm_read(P + 8, 256, 8192, 128, 2 * P) == b.GEMM_ERR_MISALIGNED


def test_log_env_prints_the_choice():
    """MI355_GEMM_LOG=1: the config choice is printed with its source; a call
    that fails validation prints nothing."""
    code = (
        "import dense_gemm_engineering_run_amd as g\n"
        "g.gemm_load_tuning(None)\n"
        f"assert g.gemm_run(-1, 8, 8, 'k', 'k', 'n', 0, {P}, {2 * P}, {3 * P}, 8, 8, 8, 0) != 0\n"
        "print(g.gemm_select_config(4096, 4096, 4096, 'K', 'k', 'n', 1))\n")
    env = dict(os.environ, MI355_GEMM_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("mi355_gemm:")]
    assert len(lines) == 1, r.stderr
    cfg = int(r.stdout.strip())
    assert f"-> {g.gemm_config_describe(1, cfg)} [heuristic] ok" in lines[0], lines[0]
    assert "select f16_f32 M=4096 N=4096 K=4096 a=k b=k c=n" in lines[0], lines[0]
    env["MI355_GEMM_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=120)
    assert r.returncode == 0 and "mi355_gemm:" not in r.stderr


def test_heuristic_picks_without_table():
    """With no tuning table the built-in heuristic chooses by C's shorter
    side first (thin problems take tiles no wider than it) and, for 16-bit
    inputs, a K of at most 256 (64x64 tiles), then by tile counts: the register-staged 32x32 fp32 tile and the 64x64 direct tiles
    for small problems, 128x128 in between, 256x256 (the ping-pong config
    for 16-bit inputs with a k-contiguous operand and K >= 1024) for large."""
    cases = [
        (65536, 64, 1024, "k", "k", "n", 0, "f32 64x64x32 w2x2 mfma32 s4 dma"),
        (4096, 64, 1024, "k", "k", "n", 0, "f32 32x32x128 w2x2 mfma16 s2 swz"),
        (512, 512, 512, "k", "k", "n", 0, "f32 32x32x128 w2x2 mfma16 s2 swz"),
        (1024, 1024, 1024, "m", "n", "n", 0, "f32 64x64x32 w2x2 mfma32 s4 dma"),
        (2048, 2048, 1024, "k", "n", "n", 0, "f32 128x128x32 w2x2 mfma32 s2 dma"),
        (32768, 128, 1024, "m", "n", "n", 0, "f32 128x128x32 w2x2 mfma32 s2 dma"),
        (8192, 8192, 8192, "m", "n", "n", 0, "f32 256x256x32 w2x2 mfma32 s2 dma"),
        (65536, 64, 4096, "k", "k", "n", 1, "f16_f32 64x64x64 w2x2 mfma16 s4 dma"),
        (64, 65536, 4096, "m", "n", "m", 1, "f16_f32 64x64x64 w2x2 mfma32 s4 dma"),
        (65536, 128, 4096, "k", "k", "n", 2, "bf16_bf16 128x128x64 w2x2 mfma16 s4 dma"),
        (16384, 128, 128, "k", "k", "n", 1, "f16_f32 64x64x64 w2x2 mfma16 s4 dma"),
        (16384, 128, 128, "k", "k", "n", 0, "f32 64x64x32 w2x2 mfma32 s4 dma"),
        (4096, 4096, 256, "k", "k", "n", 0, "f32 256x256x32 w2x2 mfma32 s2 dma"),
        (32768, 512, 512, "k", "k", "n", 1, "f16_f32 256x256x64 w4x2 mfma16 s2 dma"),
        (1024, 1024, 1024, "k", "n", "n", 3, "f16_f16 64x64x64 w2x2 mfma16 s4 dma"),
        (1024, 1024, 4096, "m", "n", "n", 4, "bf16_f32 64x64x64 w2x2 mfma32 s4 dma"),
        (2048, 2048, 2048, "m", "k", "n", 1, "f16_f32 128x128x64 w2x2 mfma32 s4 dma"),
        (2304, 2304, 2048, "k", "k", "n", 1, "f16_f32 128x256x64 w2x2 mfma32 s3 dma"),
        (3072, 3072, 1024, "k", "k", "n", 1, "f16_f32 256x256x64 w4x2 mfma16 s3x2 pp"),
        (3072, 3072, 2048, "m", "n", "n", 1, "f16_f32 256x256x64 w4x2 mfma16 s2 dma"),
        (4096, 4096, 4096, "k", "k", "n", 1, "f16_f32 256x256x64 w4x2 mfma16 s3x2 pp"),
        (8192, 8192, 512, "m", "n", "n", 1, "f16_f32 256x256x64 w4x2 mfma32 s2 dma"),
        (8192, 8192, 4096, "m", "n", "n", 1, "f16_f32 256x256x64 w4x2 mfma16 s3x2 pp"),
        (4096, 4096, 4096, "m", "n", "n", 2, "bf16_bf16 256x256x64 w4x2 mfma16 s2 dma"),
    ]
    code = "import dense_gemm_engineering_run_amd as g\ng.gemm_load_tuning(None)\n"
    for M, N, K, a, bm, c, d, _ in cases:
        code += f"print(g.gemm_config_describe({d}, g.gemm_select_config({M}, {N}, {K}, '{a}', '{bm}', '{c}', {d})))\n"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    got = r.stdout.strip().splitlines()
    assert got == [want for *_, want in cases], list(zip(got, [c[:7] for c in cases]))
