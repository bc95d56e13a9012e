"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Workloads (seeded, synthetic; see gemm_inputs):
  1. fp32 1024x512x256, A k-major, B k-major, C n-major, integers in [-5,5]   -> bit-exact
  2. fp32 8192^3, A m-major, B n-major, C n-major, uniform(-1,1)             -> normwise <= 1e-5
  3. fp16 4096^3 -> fp32, all 8 layouts, normal(0,1)                         -> normwise <= 1e-5
  4. fp32 4095x2049x1028 ragged, A k, B k, C n (ldc 2052), uniform(-1,1)     -> normwise <= 1e-5
  5. bf16 65536x256x4096 -> bf16, A k, B k, C n, normal(0,0.02)              -> normwise <= 8e-3
Integer-valued inputs at each shape must match bit for bit.  Every workload
is compared with the oracle over the whole of C, every element; C starts
filled with a NaN sentinel, so a tile that is never written fails the check.
"""
import itertools
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
import gemm_inputs as gi  # noqa: E402
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS8 = [(a, b, c) for a in "km" for b in "kn" for c in "nm"]


def log(msg):
    print(msg, flush=True)


def full_check(prob, exact, config=None, ref=None, dev=None):
    """Run `prob` and compare all of C with the oracle (computed here unless
    `ref` is given); C's ld padding must keep the sentinel."""
    c, flat, st = gu.run(prob, config=config, dev=dev)
    assert st == 0, st
    if ref is None:
        ref = gu.reference(prob)
    assert gu.no_sentinel(c, prob), "C holds unwritten elements"
    ok, info = gu.check(c, ref, prob, exact)
    assert ok, info
    assert gu.padding_intact(flat, prob)
    return info


# ---------------------------------------------------------------- the five workloads

def test_w1_fp32_1024x512x256_integer_exact():
    log("w1 fp32 1024x512x256 kkn int5")
    prob = gi.problem(1024, 512, 256, "k", "k", "n", "f32", "int5")
    full_check(prob, exact=True)


@pytest.mark.parametrize("kind,exact", [("u11", False), ("int5", True)])
def test_w2_fp32_8192_cube(kind, exact):
    log(f"w2 fp32 8192^3 mnn {kind}")
    prob = gi.problem(8192, 8192, 8192, "m", "n", "n", "f32", kind)
    info = full_check(prob, exact)
    log(f"  {info}")


@pytest.mark.parametrize("kind,exact", [("n01", False), ("int5", True)])
def test_w3_fp16_4096_cube_all_layouts(kind, exact):
    M = N = K = 4096
    a_log, b_log = gi.draw_ab(M, N, K, kind)
    a16, b16 = gi.cast(a_log, "f16"), gi.cast(b_log, "f16")
    ref = None
    for am, bm, cm in LAYOUTS8:
        log(f"w3 fp16 4096^3 {am}{bm}{cm} {kind}")
        prob = dict(M=M, N=N, K=K, a_major=am, b_major=bm, c_major=cm, dtype=1, in_type="f16",
                    out_type="f32", lda=4096, ldb=4096, ldc=4096, c_first=(cm == "m"),
                    A=gi.store(a16, am == "m", 4096), B=gi.store(b16, bm == "n", 4096))
        if ref is None:  # same logical inputs for every layout: compute the oracle once
            ref = gu.reference(prob)
        info = full_check(prob, exact, ref=ref)
        log(f"  {info}")


@pytest.mark.parametrize("kind,exact", [("u11", False), ("int5", True)])
def test_w4_fp32_ragged(kind, exact):
    log(f"w4 fp32 4095x2049x1028 kkn {kind}")
    prob = gi.problem(4095, 2049, 1028, "k", "k", "n", "f32", kind, ldc=2052)
    info = full_check(prob, exact)
    log(f"  {info}")


@pytest.mark.parametrize("kind,exact", [("n002", False), ("int5", True)])
def test_w5_bf16_tall_skinny(kind, exact):
    log(f"w5 bf16 65536x256x4096 kkn {kind}")
    prob = gi.problem(65536, 256, 4096, "k", "k", "n", "bf16_bf16", kind)
    info = full_check(prob, exact)
    log(f"  {info}")


# One GPU's share of the two largest problems split over eight GPUs with no
# reduction (the fp32 cube over a 4 x 2 grid of GPUs, the tall-skinny GEMM
# along M): tile counts of a half and an eighth of the chip's CUs, where the
# tuned configs differ from those of the whole problems.
@pytest.mark.parametrize("kind,exact", [("u11", False), ("int5", True)])
def test_shard_fp32_2048x4096x8192(kind, exact):
    log(f"shard fp32 2048x4096x8192 mnn {kind}")
    prob = gi.problem(2048, 4096, 8192, "m", "n", "n", "f32", kind)
    info = full_check(prob, exact)
    log(f"  {info}")


@pytest.mark.parametrize("kind,exact", [("n002", False), ("int5", True)])
def test_shard_bf16_8192x256x4096(kind, exact):
    log(f"shard bf16 8192x256x4096 kkn {kind}")
    prob = gi.problem(8192, 256, 4096, "k", "k", "n", "bf16_bf16", kind)
    info = full_check(prob, exact)
    log(f"  {info}")


# ---------------------------------------------------------------- edges and configs

EDGE = [1, 2, 3, 15, 16, 17, 31, 33, 63, 65, 127, 129, 255, 257]


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"])
def test_edge_sizes_integer_exact(dtype):
    rng = np.random.Generator(np.random.PCG64(sum(map(ord, dtype))))
    triples = [(int(rng.choice(EDGE)), int(rng.choice(EDGE)), int(rng.choice(EDGE)))
               for _ in range(6)] + [(1, 1, 1), (257, 255, 1), (3, 129, 257)]
    for (M, N, K), (am, bm, cm) in itertools.product(triples, LAYOUTS8):
        prob = gi.problem(M, N, K, am, bm, cm, dtype, "int5", seed=M * 7 + N * 3 + K)
        c, flat, st = gu.run(prob)
        assert st == 0
        ok, info = gu.check(c, gu.reference(prob), prob, exact=True)
        assert ok, (dtype, M, N, K, am, bm, cm, info)
        assert gu.padding_intact(flat, prob), (dtype, M, N, K, am, bm, cm)
    log(f"{dtype}: {len(triples) * 8} edge cases exact")


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"])
def test_every_config_every_layout(dtype):
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    for cfg in range(g.gemm_num_configs(code)):
        name = g.gemm_config_describe(code, cfg)
        for (M, N, K), (am, bm, cm) in itertools.product([(300, 200, 136), (97, 65, 37)], LAYOUTS8):
            prob = gi.problem(M, N, K, am, bm, cm, dtype, "int5", seed=cfg, pad_fill=float("nan"))
            c, flat, st = gu.run(prob, config=cfg)
            assert st == 0
            assert g.gemm_last_config() == cfg
            ok, info = gu.check(c, gu.reference(prob), prob, exact=True)
            assert ok, (name, M, N, K, am, bm, cm, info)
            assert gu.padding_intact(flat, prob)
        log(f"{name}: 8 layouts exact")


def _config_shape(name):
    """(BK, stages) from a config description such as
    'f16_f32 256x256x64 w4x2 mfma32 s2 dma'."""
    import re
    m = re.search(r"\d+x\d+x(\d+) w\dx\d mfma\d+ s(\d+)", name)
    assert m, name
    return int(m.group(1)), int(m.group(2))


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"])
def test_every_config_pipeline_depths(dtype):
    """K giving 1, 2, STAGES-1, STAGES and STAGES+1 k-tiles, each with a
    partial last tile, for every config: the load ring's prologue and tail
    (including loads issued past the last k-tile, which must read nothing
    and disturb nothing) at every depth the config can reach."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    count = 0
    for cfg in range(g.gemm_num_configs(code)):
        name = g.gemm_config_describe(code, cfg)
        bk, stages = _config_shape(name)
        tiles = sorted({1, 2, max(stages - 1, 1), stages, stages + 1})
        ks = sorted({max(1, (t - 1) * bk + (bk // 2 + 1)) for t in tiles} | {1, bk})
        for K in ks:
            for am, bm, cm in [(a, b, "n") for a in "km" for b in "kn"]:
                prob = gi.problem(130, 70, K, am, bm, cm, dtype, "int5", seed=cfg * 131 + K,
                                  pad_fill=float("nan"))
                c, flat, st = gu.run(prob, config=cfg)
                assert st == 0, (name, K, am, bm)
                ok, info = gu.check(c, gu.reference(prob), prob, exact=True)
                assert ok, (name, K, am, bm, info)
                assert gu.padding_intact(flat, prob), (name, K, am, bm)
                count += 1
    log(f"{dtype}: {count} pipeline-depth cases exact")


STRIP_TILE = {"f32": "f32 128x128x32 w2x2 mfma32 s2 dma", "f16_f32": "f16_f32 128x128x64 w2x2 mfma16 s4 dma",
              "bf16_bf16": "bf16_bf16 128x128x64 w2x2 mfma16 s4 dma", "f16_f16": "f16_f16 128x128x64 w2x2 mfma16 s4 dma",
              "bf16_f32": "bf16_f32 128x128x64 w2x2 mfma16 s4 dma"}
# Shapes whose last tile row and column (128x128 tiles) hold 1-4 rows and
# columns of C, and where leaving them to the strip kernel saves a round of
# tiles: 561 -> 512 tiles for the fp32 config (two rings per CU), 289 -> 256
# for the 16-bit ones (one ring per CU).
STRIP_SHAPES = {"f32": [(2049, 4099), (4098, 2050)], "16": [(2049, 2051), (2050, 2052)]}


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"])
def test_thin_edge_strips(dtype):
    """C's last rows and columns, when 1-4 wide past a multiple of the tile,
    go to the strip kernel and the rest to the tiled kernel: both strips and
    their corner, one K chunk of the strip kernel and two (the second
    partial), all 8 layouts, NaN in the ld padding; all of C against the
    oracle, bit-exact on integer inputs; then 4095x2049x1028 (a column strip
    only) on real-valued data within the tolerance."""
    code = gi.DTYPE_CODE[dtype]
    cfg = _config_id(code, STRIP_TILE[dtype])
    k2 = 2200 if dtype == "f32" else 4200
    shapes = STRIP_SHAPES["f32" if dtype == "f32" else "16"]
    for (M, N), K in zip(shapes, (200, k2)):
        for am, bm, cm in LAYOUTS8:
            log(f"strips {dtype} {M}x{N}x{K} {am}{bm}{cm}")
            prob = gi.problem(M, N, K, am, bm, cm, dtype, "int5", seed=M + K, pad_fill=float("nan"))
            full_check(prob, exact=True, config=cfg)
    kind = {"f32": "u11", "bf16_bf16": "n002", "bf16_f32": "n002"}.get(dtype, "n01")
    ldc = 2052 if gi.DTYPES[code][2] == "f32" else 2056       # 16-byte rows of C
    prob = gi.problem(4095, 2049, 1028, "k", "k", "n", dtype, kind, seed=4, ldc=ldc)
    full_check(prob, exact=False, config=cfg)


def test_thin_edge_strips_with_epilogue_and_batch():
    """The strip kernel runs the same epilogue (alpha, beta, bias, relu; bias
    along rows for C m-major) and serves every entry of a strided batch; the
    call log names the strips."""
    import subprocess
    import dense_gemm_engineering_run_amd as g
    for dtype in ("f32", "bf16_bf16"):
        cfg = _config_id(gi.DTYPE_CODE[dtype], STRIP_TILE[dtype])
        M, N = STRIP_SHAPES["f32" if dtype == "f32" else "16"][0]
        for layout in [("k", "k", "n"), ("m", "n", "m")]:
            epi_case(M, N, 136, layout, dtype, "int5", 2.0, -0.5, g.GEMM_ACT_RELU, config=cfg)
    batched_case(1026, 1027, 72, ("m", "n", "m"), "f32", "int5", 2)       # 64x64 tiles: 578 -> 512
    batched_case(1026, 1027, 72, ("k", "k", "n"), "f16_f32", "int5", 4)   # 128x128 tiles: 324 -> 256
    code = (
        "import sys, torch; sys.path.insert(0, '.');"
        "import dense_gemm_engineering_run_amd as g;"
        "a = torch.zeros(4095 * 1028, device='cuda'); b = torch.zeros(2049 * 1028, device='cuda');"
        "c = torch.zeros(4095 * 2052, device='cuda');"
        f"cfg = [g.gemm_config_describe(0, i) for i in range(g.gemm_num_configs(0))].index('{STRIP_TILE['f32']}');"
        "st = g.gemm_run_config(4095, 2049, 1028, 'k', 'k', 'n', 0, a.data_ptr(), b.data_ptr(), c.data_ptr(),"
        " 1028, 1028, 2052, torch.cuda.current_stream().cuda_stream, cfg);"
        "torch.cuda.synchronize(); assert st == 0, st")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, MI355_GEMM_LOG="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    assert "strip kernel (0 rows, 1 columns)" in r.stderr, r.stderr[-2000:]
    log("strips with epilogue and batch: exact; log names the strip")


def test_ping_pong_transposed_store():
    """A k with B n (C n-major) and A m with B k (C m-major): the ping-pong
    config swaps the operands and stores C transposed (the other two layouts
    are controls).  All of C against the oracle, bit-exact on integer inputs,
    NaN in the ld padding; thin edges (4097 x 4098: both strips, stored
    transposed too) and ragged K; a strided batch, which the heuristic gives
    the ping-pong config; an epilogue (the plain order); the call log."""
    import subprocess
    import dense_gemm_engineering_run_amd as g
    for dtype in ("f16_f32", "bf16_bf16", "f16_f16"):
        code = gi.DTYPE_CODE[dtype]
        cfg = _config_id(code, dtype + " 256x256x64 w4x2 mfma16 s3x2 pp")
        for layout in (("k", "n", "n"), ("m", "k", "m"), ("k", "n", "m"), ("m", "k", "n")):
            for M, N, K in ((4097, 4098, 72), (1000, 700, 300)):
                log(f"transposed store {dtype} {M}x{N}x{K} {''.join(layout)}")
                prob = gi.problem(M, N, K, *layout, dtype, "int5", seed=M + K, pad_fill=float("nan"))
                full_check(prob, exact=True, config=cfg)
    used = batched_case(1024, 1024, 1024, ("k", "n", "n"), "f16_f32", "int5", 12)
    assert g.gemm_config_describe(1, used).endswith(" pp"), g.gemm_config_describe(1, used)
    cfg = _config_id(1, "f16_f32 256x256x64 w4x2 mfma16 s3x2 pp")
    epi_case(1000, 700, 300, ("k", "n", "n"), "f16_f32", "int5", 2.0, -0.5, g.GEMM_ACT_RELU, config=cfg)
    code = (
        "import sys, torch; sys.path.insert(0, '.');"
        "import dense_gemm_engineering_run_amd as g;"
        "a = torch.zeros(1024 * 1024, dtype=torch.float16, device='cuda');"
        "b = torch.zeros(1024 * 1024, dtype=torch.float16, device='cuda');"
        "c = torch.zeros(1024 * 1024, device='cuda');"
        "cfg = [g.gemm_config_describe(1, i) for i in range(g.gemm_num_configs(1))].index("
        "'f16_f32 256x256x64 w4x2 mfma16 s3x2 pp');"
        "st = g.gemm_run_config(1024, 1024, 1024, 'k', 'n', 'n', 1, a.data_ptr(), b.data_ptr(), c.data_ptr(),"
        " 1024, 1024, 1024, torch.cuda.current_stream().cuda_stream, cfg);"
        "torch.cuda.synchronize(); assert st == 0, st")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, MI355_GEMM_LOG="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    assert "operands swapped, C stored transposed" in r.stderr, r.stderr[-2000:]
    log("transposed store: exact on every layout; batch and epilogue exact; log names it")


def test_every_config_nonintegers_multi_tile():
    import dense_gemm_engineering_run_amd as g
    for dtype, kind in [("f32", "u11"), ("f16_f32", "n01"), ("bf16_bf16", "n002")]:
        code = gi.DTYPE_CODE[dtype]
        prob = gi.problem(515, 777, 333, "m", "k", "n", dtype, kind, seed=3)
        ref = gu.reference(prob)
        for cfg in range(g.gemm_num_configs(code)):
            c, _, st = gu.run(prob, config=cfg)
            assert st == 0
            ok, info = gu.check(c, ref, prob, exact=False)
            assert ok, (g.gemm_config_describe(code, cfg), info)


def _config_id(code, name):
    import dense_gemm_engineering_run_amd as g
    return next(i for i in range(g.gemm_num_configs(code)) if g.gemm_config_describe(code, i) == name)


def test_ping_pong_matches_single_group_schedule():
    """The ping-pong config accumulates every C element in the order of the
    3 + 2-stage kernel of the same tile, so the two give identical bits: fp16
    4096^3 on N(0,1) in all 8 layouts (A m with B n reads both operands with
    transposing loads), each also checked against the oracle over the whole of
    C; then ragged bf16 -> bf16 and fp16 -> fp32 shapes (a partial last
    k-tile, 2-tile and 3-tile k ranges, partial edge tiles)."""
    M = N = K = 4096
    a_log, b_log = gi.draw_ab(M, N, K, "n01", seed=77)
    a16, b16 = gi.cast(a_log, "f16"), gi.cast(b_log, "f16")
    pp = _config_id(1, "f16_f32 256x256x64 w4x2 mfma16 s3x2 pp")
    one = _config_id(1, "f16_f32 256x256x64 w4x2 mfma16 s3x2 dma")
    ref = None
    for am, bm, cm in LAYOUTS8:
        log(f"ping-pong fp16 4096^3 {am}{bm}{cm}")
        prob = dict(M=M, N=N, K=K, a_major=am, b_major=bm, c_major=cm, dtype=1, in_type="f16",
                    out_type="f32", lda=4096, ldb=4096, ldc=4096, c_first=(cm == "m"),
                    A=gi.store(a16, am == "m", 4096), B=gi.store(b16, bm == "n", 4096))
        if ref is None:
            ref = gu.reference(prob)
        full_check(prob, exact=False, config=pp, ref=ref)
        c_pp, _, st = gu.run(prob, config=pp)
        assert st == 0
        c_one, _, st = gu.run(prob, config=one)
        assert st == 0
        assert np.array_equal(c_pp.view(np.uint32), c_one.view(np.uint32)), (am, bm, cm)
    for dtype, kind, code in (("bf16_bf16", "n002", 2), ("f16_f32", "n01", 1)):
        pfx = dtype + " 256x256x64 w4x2 mfma16 s3x2 "
        pp, one = _config_id(code, pfx + "pp"), _config_id(code, pfx + "dma")
        for (m, n, k), (am, bm) in itertools.product([(1000, 1100, 1000), (520, 770, 100), (300, 260, 150)],
                                                     [("k", "k"), ("m", "k"), ("m", "n")]):
            log(f"ping-pong {dtype} {m}x{n}x{k} {am}{bm}n")
            prob = gi.problem(m, n, k, am, bm, "n", dtype, kind, seed=m + k)
            full_check(prob, exact=False, config=pp)
            c_pp, _, _ = gu.run(prob, config=pp)
            c_one, _, _ = gu.run(prob, config=one)
            assert np.array_equal(c_pp.view(np.uint8), c_one.view(np.uint8)), (dtype, m, n, k, am, bm)


# ---------------------------------------------------------------- canaries and edge semantics

@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16"])
def test_nan_in_ld_padding_does_not_reach_c(dtype):
    for am, bm, cm in LAYOUTS8:
        prob = gi.problem(130, 67, 77, am, bm, cm, dtype, "int5", seed=9,
                          lda=(136 if am == "m" else 88), ldb=(72 if bm == "n" else 88),
                          ldc=(136 if cm == "m" else 72), pad_fill=float("nan"))
        c, flat, st = gu.run(prob)
        assert st == 0
        ok, info = gu.check(c, gu.reference(prob), prob, exact=True)
        assert ok, (am, bm, cm, info)
        assert gu.padding_intact(flat, prob)


def test_deterministic_bitwise():
    prob = gi.problem(1000, 700, 900, "m", "k", "n", "f32", "u11", seed=4)
    c1, _, st1 = gu.run(prob)
    c2, _, st2 = gu.run(prob)
    assert st1 == 0 and st2 == 0
    ok, info = gu.check(c1, gu.reference(prob), prob, exact=False)
    assert ok, info
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


def test_nondefault_stream():
    import torch
    s = torch.cuda.Stream()
    prob = gi.problem(500, 300, 200, "k", "n", "m", "f16_f32", "int5", seed=2)
    with torch.cuda.stream(s):
        c, _, st = gu.run(prob, stream=s)
    assert st == 0
    ok, info = gu.check(c, gu.reference(prob), prob, exact=True)
    assert ok, info


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16", "f16_f16"])
def test_k_zero_gives_zeros_and_empty_is_noop(dtype):
    prob = gi.problem(70, 50, 0, "k", "k", "n", dtype, "int5")
    c, flat, st = gu.run(prob)
    assert st == 0
    assert np.all(gu.compare.as_f64(c, prob["out_type"]) == 0)
    assert gu.padding_intact(flat, prob)
    for M, N in [(0, 50), (70, 0)]:
        prob = gi.problem(M, N, 16, "k", "k", "n", dtype, "int5")
        _, flat, st = gu.run(prob)
        assert st == 0
        got = flat.view(np.uint32 if prob["out_type"] == "f32" else np.uint16)
        assert np.all(got == gu.SENTINEL[prob["out_type"]])      # C untouched


def test_large_integer_sums_stay_exact():
    # K * 25 < 2^24: every fp32 partial sum is an exact integer.
    prob = gi.problem(64, 96, 20000, "k", "n", "n", "f32", "int5", seed=12)
    full_check(prob, exact=True)


def test_graph_capture_and_replay():
    """gemm_run enqueued under HIP graph capture: every replay (with eager work
    and synchronisation between replays) reproduces the eager result."""
    import torch

    import dense_gemm_engineering_run_amd as g
    prob = gi.problem(300, 260, 200, "m", "k", "n", "f16_f32", "int5", seed=21)
    ref_c, _, st = gu.run(prob)
    assert st == 0
    a, b = gu.to_device(prob["A"]), gu.to_device(prob["B"])
    c = gu.c_buffer(prob)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    args = (prob["M"], prob["N"], prob["K"], "m", "k", "n", prob["dtype"], a.data_ptr(),
            b.data_ptr(), c.data_ptr(), prob["lda"], prob["ldb"], prob["ldc"], s.cuda_stream)
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            assert g.gemm_run(*args) == 0
    torch.cuda.synchronize()
    for rep in range(4):
        c.fill_(0)                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got, _ = gu.host_c(c, prob)
        assert np.array_equal(got.view(np.uint32), ref_c.view(np.uint32)), rep


# ---------------------------------------------------------------- second workload: fp16 K sweep

@pytest.mark.parametrize("K,kind,exact", [(512, "n01", False), (16384, "n01", False), (2048, "int5", True)])
def test_fp16_out_sweep_8192(K, kind, exact):
    """M = N = 8192, fp16 in and out, A k-major, B n-major (B stored K x N
    row-major), C n-major; all of C against the oracle rounded to fp16."""
    log(f"sweep f16_f16 8192x8192x{K} knn {kind}")
    prob = gi.problem(8192, 8192, K, "k", "n", "n", "f16_f16", kind)
    info = full_check(prob, exact)
    log(f"  {info}")


# ---------------------------------------------------------------- strided batched ("L") mode

_GAP_BITS16 = np.uint16(0x7FFF)      # NaN in both fp16 and bf16


def _pack(arrs, shared):
    """Concatenate per-entry storage with a NaN gap between entries; stride 0
    when every entry is the same array.  Returns (flat array, stride)."""
    n = arrs[0].size
    per = 16 // arrs[0].itemsize
    if shared:
        return arrs[0], 0
    stride = -(-n // per) * per + 2 * per
    fill = np.float32(np.nan) if arrs[0].dtype == np.float32 else _GAP_BITS16
    buf = np.full(stride * (len(arrs) - 1) + n, fill, dtype=arrs[0].dtype)
    for i, a in enumerate(arrs):
        buf[i * stride: i * stride + n] = a
    return buf, stride


def batched_case(M, N, K, layout, dtype, kind, batch, share="", seed=11):
    """Run one strided-batched call and compare every entry with the oracle.
    share: "a" and/or "b" give that operand stride 0 (one matrix for all).
    Every entry is compared in full."""
    import torch
    import dense_gemm_engineering_run_amd as g
    a_m, b_m, c_m = layout
    probs = [gi.problem(M, N, K, a_m, b_m, c_m, dtype, kind, seed=seed + l) for l in range(batch)]
    for key in ("A", "B"):
        if key.lower() in share:
            for p in probs:
                p[key] = probs[0][key]
    A, sa = _pack([p["A"] for p in probs], "a" in share)
    B, sb = _pack([p["B"] for p in probs], "b" in share)
    p0 = probs[0]
    outer = N if p0["c_first"] else M
    per_out = 16 // gi.ELEM_BYTES[p0["out_type"]]
    sc = outer * p0["ldc"] + 2 * per_out
    c = gu.c_buffer(dict(p0, ldc=1, M=sc * (batch - 1) + outer * p0["ldc"], N=1, c_first=False))
    s = torch.cuda.current_stream()
    a_dev, b_dev = gu.to_device(A), gu.to_device(B)
    st = g.gemm_run_batched(M, N, K, a_m, b_m, c_m, p0["dtype"], a_dev.data_ptr(),
                            b_dev.data_ptr(), c.data_ptr(), p0["lda"], p0["ldb"], p0["ldc"],
                            batch, sa, sb, sc, s.cuda_stream)
    assert st == 0, g.gemm_status_str(st)
    cfg = g.gemm_last_config()
    s.synchronize()
    flat = c.cpu().numpy()
    if p0["out_type"] != "f32":
        flat = flat.view(np.uint16)
    sentinel = gu.SENTINEL[p0["out_type"]]
    for l, p in enumerate(probs):
        part = flat[l * sc: l * sc + outer * p["ldc"]]
        got = np.ascontiguousarray(gi.load(part, M, N, p["c_first"], p["ldc"]))
        assert gu.no_sentinel(got, p), l
        ok, info = gu.check(got, gu.reference(p), p, kind == "int5")
        assert ok, (l, info)
        assert gu.padding_intact(part, p), l
        gap = flat[l * sc + outer * p["ldc"]: (l + 1) * sc] if l + 1 < batch else flat[:0]
        assert np.all(gap.view(np.uint32 if p["out_type"] == "f32" else np.uint16) == sentinel), l
    return cfg


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"])
def test_batched_every_layout(dtype):
    """Three entries of a ragged 200x136x72 problem, integer inputs: bit-exact
    per entry, NaN between entries never read, C gaps never written."""
    for layout in LAYOUTS8:
        log(f"batched {dtype} {''.join(layout)} 200x136x72 x3")
        batched_case(200, 136, 72, layout, dtype, "int5", 3)


@pytest.mark.parametrize("share", ["a", "b", "ab"])
def test_batched_broadcast_operand(share):
    log(f"batched broadcast {share}")
    batched_case(96, 160, 40, ("k", "n", "n"), "f32", "int5", 4, share=share)
    batched_case(96, 160, 40, ("m", "k", "m"), "f16_f32", "u11", 3, share=share)


@pytest.mark.parametrize("dtype,layout", [("f32", "mnn"), ("f32", "kkn"), ("f16_f32", "kkn"),
                                          ("f16_f32", "mnm"), ("bf16_bf16", "kkn")])
def test_batched_direct_to_lds_kernels(dtype, layout):
    """Shapes large enough for the direct-to-LDS kernels; every entry in full."""
    import dense_gemm_engineering_run_amd as g
    log(f"batched large {dtype} {layout}")
    cfg = batched_case(4096, 4096, 104, tuple(layout), dtype, "int5", 2)
    name = g.gemm_config_describe(gi.DTYPE_CODE[dtype], cfg)
    log(f"  config {name}")
    assert name.endswith(("dma", "pp")), name


def test_batched_selection_counts_every_entry():
    """A strided batch is one launch over all its entries' tiles: 64 x 512^3
    and 16 x 1024^3 (whose batch-1 table entry names a 64x64 tile) both go to
    a 256x256 direct-to-LDS kernel (one wave of its tiles) -- the one-group
    16x16x32 schedule at K = 512, the ping-pong one at K = 1024 -- and stay
    exact (every entry in full)."""
    import dense_gemm_engineering_run_amd as g
    for M, batch, want in ((512, 64, "s2 dma"), (1024, 16, "s3x2 pp")):
        cfg = batched_case(M, M, M, ("k", "k", "n"), "f16_f32", "int5", batch)
        assert g.gemm_config_describe(1, cfg) == "f16_f32 256x256x64 w4x2 mfma16 " + want, g.gemm_config_describe(1, cfg)
    log("batched selection: 256x256 tile for 64 x 512^3 and 16 x 1024^3")


def test_batched_k_zero_and_empty():
    import torch
    import dense_gemm_engineering_run_amd as g
    c = torch.full((3 * 64 * 32,), 7.0, device="cuda")
    st = g.gemm_run_batched(64, 32, 0, "k", "k", "n", 0, 0, 0, c.data_ptr(), 4, 4, 32, 3, 0, 0,
                            64 * 32, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0
    st = g.gemm_run_batched(64, 32, 8, "k", "k", "n", 0, 0, 0, 0, 8, 8, 32, 0, 0, 0, 0, 0)
    assert st == 0


# ---------------------------------------------------------------- stream-K (persistent) fp32 configs

SK_DTYPES = ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"]


def _sk_configs(dtype="f32"):
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    return [i for i in range(g.gemm_num_configs(code)) if g.gemm_config_describe(code, i).endswith(" sk")]


def sk_case(M, N, K, layout, config, kind, ldc=None, seed=5, dtype="f32", ref=None):
    """Run a stream-K config through gemm_run_ws twice (fresh C each time) and
    compare all of C with the oracle (`ref` if given); the second run also
    checks that the first left the workspace's arrival counters at zero."""
    import torch
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    prob = gi.problem(M, N, K, *layout, dtype, kind, seed=seed, ldc=ldc)
    need = g.gemm_workspace_size(M, N, K, *layout, code, config)
    ws = torch.zeros(max(need, 16) // 4, dtype=torch.int32, device="cuda")
    a, b = gu.to_device(prob["A"]), gu.to_device(prob["B"])
    outs = []
    for _ in range(2):
        c = gu.c_buffer(prob)
        s = torch.cuda.current_stream()
        st = g.gemm_run_ws(M, N, K, *layout, code, a.data_ptr(), b.data_ptr(), c.data_ptr(),
                           prob["lda"], prob["ldb"], prob["ldc"], ws.data_ptr() if need else 0,
                           need, s.cuda_stream, config)
        assert st == 0, g.gemm_status_str(st)
        assert g.gemm_last_config() == config
        s.synchronize()
        outs.append(gu.host_c(c, prob))
    (c0, f0), (c1, f1) = outs
    assert np.array_equal(f0.view(np.uint8), f1.view(np.uint8)), "not deterministic"
    assert gu.padding_intact(f0, prob)
    assert gu.no_sentinel(c0, prob), "C holds unwritten elements"
    if ref is None:
        ref = gu.reference(prob)
    ok, info = gu.check(c0, ref, prob, kind == "int5")
    assert ok, info
    return need, info


@pytest.mark.parametrize("dtype", SK_DTYPES)
def test_stream_k_every_config_every_layout(dtype):
    """Shapes with fewer tiles than persistent workgroups (every tile split
    over 2-3 workgroups), ragged in M, N and K; full oracle comparison."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    for cfg in _sk_configs(dtype):
        for layout in [("k", "k", "n"), ("k", "n", "n"), ("m", "k", "n"), ("m", "n", "n"), ("m", "n", "m")]:
            log(f"stream-K {g.gemm_config_describe(code, cfg)} {''.join(layout)} 600x520x200")
            need, _ = sk_case(600, 520, 200, layout, cfg, "int5", dtype=dtype)
            assert need > 0


@pytest.mark.parametrize("kind,exact", [("int5", True), ("u11", False)])
def test_stream_k_ragged_workload(kind, exact):
    """4095x2049x1028, A k, B k, C n with ldc 2052: 144 tiles of 256x256 over
    256 workgroups; all of C."""
    import dense_gemm_engineering_run_amd as g
    ref = gu.reference(gi.problem(4095, 2049, 1028, "k", "k", "n", "f32", kind, seed=5, ldc=2052))
    for cfg in _sk_configs():
        log(f"stream-K ragged {g.gemm_config_describe(0, cfg)} {kind}")
        sk_case(4095, 2049, 1028, ("k", "k", "n"), cfg, kind, ldc=2052, ref=ref)


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16"])
def test_stream_k_thin_edge_tiles(dtype):
    """A last tile row and column that are almost entirely outside C (4097 x
    2049: one row and one column past a multiple of 128 and of 256), whose
    tiles fall partly in the data-parallel part and partly in the split
    stream-K share.  Every stream-K config, C n-major and m-major (the thin
    edge then lies along the other canonical index), all of C against the
    oracle, bit-exact on integer inputs."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    for cfg in _sk_configs(dtype):
        name = g.gemm_config_describe(code, cfg)
        for M, N, K, layout in [(4097, 2049, 200, ("k", "k", "n")), (2049, 4097, 136, ("m", "k", "m"))]:
            log(f"stream-K thin edges {name} {M}x{N}x{K} {''.join(layout)}")
            need, _ = sk_case(M, N, K, layout, cfg, "int5", dtype=dtype)
            assert need > 0


@pytest.mark.parametrize("dtype", SK_DTYPES)
def test_stream_k_data_parallel_waves_plus_split_tail(dtype):
    """More than two waves of tiles, not whole waves: data-parallel tiles
    first, then the stream-K share (the tiles of the partial wave).  256x256
    tiles: 24 x 23 = 552 over 256 workgroups; 128x128 tiles: 34 x 34 = 1156
    over 512."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    for cfg in _sk_configs(dtype):
        name = g.gemm_config_describe(code, cfg)
        M, N = (6144, 5888) if " 256x256x" in name else (4352, 4352)
        log(f"stream-K dp+sk {name} {M}x{N}x96")
        sk_case(M, N, 96, ("k", "n", "n"), cfg, "int5", dtype=dtype)


@pytest.mark.parametrize("dtype,kind", [("f16_f32", "n01"), ("bf16_bf16", "n002"), ("f16_f16", "int5")])
def test_stream_k_16bit_ragged(dtype, kind):
    """The ragged shape in 16-bit inputs, K not a multiple of the 64-wide
    k-tile (a zero-filled partial last k-tile inside split ranges)."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    ref = gu.reference(gi.problem(4095, 2049, 1028, "k", "k", "n", dtype, kind, seed=5, ldc=2056))
    for cfg in _sk_configs(dtype):
        log(f"stream-K ragged {g.gemm_config_describe(code, cfg)} {kind}")
        sk_case(4095, 2049, 1028, ("k", "k", "n"), cfg, kind, ldc=2056, dtype=dtype, ref=ref)


def test_stream_k_whole_waves_and_k_zero_need_no_workspace():
    import dense_gemm_engineering_run_amd as g
    cfg = _sk_configs()[0]
    assert g.gemm_config_describe(0, cfg).startswith("f32 256x256")
    need, _ = sk_case(4096, 4096, 64, ("k", "k", "n"), cfg, "int5")
    assert need == 0
    need, _ = sk_case(700, 300, 0, ("k", "k", "n"), cfg, "int5")
    assert need == 0


# ---------------------------------------------------------------- split-k configs

def _split_configs(dtype="f32"):
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    return [i for i in range(g.gemm_num_configs(code)) if g.gemm_config_describe(code, i).endswith(" split")]


SPLIT_LAYOUTS = [("k", "k", "n"), ("k", "n", "n"), ("m", "k", "n"), ("m", "n", "n"), ("m", "n", "m")]


@pytest.mark.parametrize("dtype", SK_DTYPES)
def test_split_k_every_config_every_layout(dtype):
    """Few tiles and a long, ragged K: 600 x 520 x 4100 is 9 tiles of 256x256
    (28 k-ranges each) or 25 of 128x128 (20 each), the last k-tile partial,
    M and N ragged; five layouts, C m-major among them.  All of C against the
    oracle, bit-exact on integer inputs, twice (deterministic)."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    ref = gu.reference(gi.problem(600, 520, 4100, "k", "k", "n", dtype, "int5", seed=5))
    cfgs = _split_configs(dtype)
    assert len(cfgs) == 2
    for cfg in cfgs:
        for layout in SPLIT_LAYOUTS:
            log(f"split-k {g.gemm_config_describe(code, cfg)} {''.join(layout)} 600x520x4100")
            need, _ = sk_case(600, 520, 4100, layout, cfg, "int5", dtype=dtype, ref=ref)
            assert need > 0


@pytest.mark.parametrize("dtype,kind", [("f32", "u11"), ("bf16_bf16", "n002"), ("f16_f32", "n01")])
def test_split_k_float_inputs_and_short_k(dtype, kind):
    """Real-valued inputs on the bf16 shard shape 8192 x 256 x 4096 (32 tiles
    of 256x256 cut into 8 k-ranges; 128 of 128x128 into 4), within the
    normwise tolerance; and K too short to split (one k-range: partial tiles
    written and added back unchanged)."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    ref = gu.reference(gi.problem(8192, 256, 4096, "k", "k", "n", dtype, kind, seed=5))
    for cfg in _split_configs(dtype):
        name = g.gemm_config_describe(code, cfg)
        log(f"split-k {name} 8192x256x4096 {kind}")
        need, info = sk_case(8192, 256, 4096, ("k", "k", "n"), cfg, kind, dtype=dtype, ref=ref)
        log(f"  {info}")
        assert need == 8192 * 256 * 4 * (8 if " 256x256x" in name else 4)
        log(f"split-k {name} 300x200x40 int5")
        sk_case(300, 200, 40, ("k", "n", "n"), cfg, "int5", dtype=dtype)


def test_split_k_epilogue_and_no_alloc_entry_point():
    """The epilogue applied by the reduction kernel (bias, ReLU, beta != 0,
    against the oracle on exact sums), and the allocation-free entry point
    running a split-k config bit-identical to gemm_run_ws."""
    import torch
    import dense_gemm_engineering_run_amd as g
    for dtype in ["f32", "bf16_bf16"]:
        for cfg in _split_configs(dtype):
            log(f"split-k epilogue {g.gemm_config_describe(gi.DTYPE_CODE[dtype], cfg)}")
            assert epi_case(600, 520, 1100, ("k", "n", "n"), dtype, "int5", 2.0, -0.5, g.GEMM_ACT_RELU,
                            config=cfg) == cfg
            # C m-major: the swapped problem, the bias indexed by its rows
            assert epi_case(520, 600, 1100, ("m", "k", "m"), dtype, "int5", 1.0, 1.0, g.GEMM_ACT_RELU,
                            config=cfg) == cfg
    cfg = _split_configs("bf16_bf16")[0]
    prob = gi.problem(1000, 300, 4100, "k", "k", "n", "bf16_bf16", "int5", seed=3)
    need = g.gemm_workspace_size(1000, 300, 4100, "k", "k", "n", prob["dtype"], cfg)
    assert 0 < need <= g.GEMM_NOALLOC_SCRATCH_BYTES
    a, b = gu.to_device(prob["A"]), gu.to_device(prob["B"])
    ws = torch.zeros(need // 4, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    outs = []
    for noalloc in (False, True):
        c = gu.c_buffer(prob)
        args = (1000, 300, 4100, "k", "k", "n", prob["dtype"], a.data_ptr(), b.data_ptr(), c.data_ptr(),
                prob["lda"], prob["ldb"], prob["ldc"])
        if noalloc:
            st = g.gemm_run_noalloc(*args, s.cuda_stream, cfg)
        else:
            st = g.gemm_run_ws(*args, ws.data_ptr(), need, s.cuda_stream, cfg)
        assert st == 0, g.gemm_status_str(st)
        s.synchronize()
        outs.append(gu.host_c(c, prob)[1])
    assert np.array_equal(outs[0].view(np.uint8), outs[1].view(np.uint8))


# ---------------------------------------------------------------- elementwise epilogue

def _c_storage(c_log_bits, prob):
    """Flat C storage (outer x ldc) holding logical M x N bits, padding = sentinel."""
    tout = prob["out_type"]
    bits = np.uint32 if tout == "f32" else np.uint16
    outer = prob["N"] if prob["c_first"] else prob["M"]
    flat = np.full(outer * prob["ldc"], gu.SENTINEL[tout], dtype=bits)
    view = flat.reshape(outer, prob["ldc"])
    view[:, :c_log_bits.shape[1] if not prob["c_first"] else c_log_bits.shape[0]] = \
        (c_log_bits.T if prob["c_first"] else c_log_bits).view(bits)
    return flat


def epi_case(M, N, K, layout, dtype, kind, alpha, beta, act, with_bias=True, config=None, seed=9,
             nan_c=False, expect=0):
    """One gemm_run_ex call with an epilogue against oracle.epilogue_ref on the
    oracle's exact sums.  C starts with integers in [-5, 5] (NaN with nan_c),
    the bias holds halves in [-4, 4]."""
    import torch
    import dense_gemm_engineering_run_amd as g
    import oracle
    prob = gi.problem(M, N, K, *layout, dtype, kind, seed=seed)
    tout = prob["out_type"]
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    c_old = rng.integers(-5, 6, size=(M, N)).astype(np.float32)
    if nan_c:
        c_old[:] = np.nan
    c_bits = gi.cast(c_old, tout)
    flat = _c_storage(np.ascontiguousarray(c_bits), prob)
    c = gu.to_device(flat.view(np.float32) if tout == "f32" else flat)
    bias = (rng.integers(-8, 9, size=N) / 2).astype(np.float32)
    bias_dev = torch.from_numpy(bias).cuda()
    need = g.gemm_workspace_size(M, N, K, *layout, prob["dtype"], -1 if config is None else config)
    ws = torch.zeros(max(need, 16) // 4, dtype=torch.int32, device="cuda")
    a, b = gu.to_device(prob["A"]), gu.to_device(prob["B"])
    s = torch.cuda.current_stream()
    epi = g.Epilogue(alpha, beta, bias_dev.data_ptr() if with_bias else 0, act)
    st = g.gemm_run_ex(M, N, K, *layout, prob["dtype"], a.data_ptr(), b.data_ptr(), c.data_ptr(),
                       prob["lda"], prob["ldb"], prob["ldc"], epi, ws.data_ptr() if need else 0,
                       need, s.cuda_stream, -1 if config is None else config)
    if expect:
        assert st == expect, g.gemm_status_str(st)
        return None
    assert st == 0, g.gemm_status_str(st)
    s.synchronize()
    got, out_flat = gu.host_c(c, prob)
    old64 = c_old.astype(np.float64) if tout == "f32" else oracle.decode(c_bits, tout)
    want = oracle.epilogue_ref(gu.reference(prob), alpha, beta, old64,
                               bias if with_bias else None, act)
    ok, info = gu.check(got, want, prob, kind == "int5")
    assert ok, (layout, dtype, config, info)
    assert gu.padding_intact(out_flat, prob)
    return g.gemm_last_config()


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"])
def test_epilogue_every_config_exact(dtype):
    """alpha = 2, beta = -0.5, per-column bias, relu on integer inputs: every
    intermediate is exact in fp32, so the result must match bit for bit.
    C n-major and m-major (the bias then runs along the canonical rows)."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    for cfg in range(g.gemm_num_configs(code)):
        name = g.gemm_config_describe(code, cfg)
        for layout in [("k", "k", "n"), ("m", "n", "m")]:
            epi_case(300, 200, 136, layout, dtype, "int5", 2.0, -0.5, g.GEMM_ACT_RELU, config=cfg)
        log(f"{name}: epilogue exact")


def test_epilogue_stream_k_ragged():
    """The ragged fp32 workload with an epilogue: the 128x128 stream-K config
    runs 512 whole tiles through the staged epilogue and 32 split tiles
    through the reduction's; with no forced config the table's choice (the
    128x128 tile with the strip kernel for the last column) is taken; both
    bit-exact on integer inputs."""
    import dense_gemm_engineering_run_amd as g
    sk = next(i for i in range(g.gemm_num_configs(0))
              if g.gemm_config_describe(0, i) == "f32 128x128x32 w2x2 mfma32 s2 dma sk")
    table = g.gemm_select_config(4095, 2049, 1028, "k", "k", "n", 0)
    for config, want in ((sk, sk), (None, table)):
        used = epi_case(4095, 2049, 1028, ("k", "k", "n"), "f32", "int5", 2.0, -0.5, g.GEMM_ACT_RELU,
                        config=config, seed=21)
        assert used == want, g.gemm_config_describe(0, used)
    log("ragged 4095x2049x1028 with epilogue, stream-K and the table's choice: exact")


@pytest.mark.parametrize("dtype", ["f32", "bf16_bf16", "f16_f32"])
def test_epilogue_stream_k_256_whole_and_split_tiles(dtype):
    """The 256x256 stream-K configs with an epilogue: 17 x 16 = 272 tiles on
    a grid of 256 workgroups, so 256 whole tiles go through the staged
    epilogue and 16 split tiles (three contributors each) through the
    reduction's; bit-exact on integer inputs, C n-major and m-major."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    names = [n for n in (g.gemm_config_describe(code, i) for i in range(g.gemm_num_configs(code)))
             if n.endswith(" sk") and " 256x256x" in n]
    assert names
    for name in names:
        cfg = next(i for i in range(g.gemm_num_configs(code)) if g.gemm_config_describe(code, i) == name)
        k = 72 if dtype == "f32" else 136          # three k-tiles, the last one partial
        for layout, (M, N) in [(("k", "k", "n"), (4352, 4096)), (("m", "n", "m"), (4096, 4352))]:
            used = epi_case(M, N, k, layout, dtype, "int5", 2.0, -0.5, g.GEMM_ACT_RELU, config=cfg, seed=23)
            assert used == cfg
        log(f"{name}: 256 whole + 16 split tiles with epilogue exact")


def test_epilogue_random_shapes_configs_exact():
    """80 seeded random epilogue cases: M, N in [1, 600], K in [0, 600], any
    layout, dtype and config (stream-K ones with a workspace), alpha and beta
    from powers of two and zero, with or without a bias, relu or none.  Every
    intermediate is exact in fp32 (|sum| <= 600 * 25), so the result must
    match the oracle's epilogue bit for bit."""
    import dense_gemm_engineering_run_amd as g
    rng = np.random.Generator(np.random.PCG64(4242))
    for case in range(80):
        dtype = ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"][rng.integers(5)]
        code = gi.DTYPE_CODE[dtype]
        M, N = (int(x) for x in rng.integers(1, 601, size=2))
        K = int(rng.integers(0, 601))
        layout = LAYOUTS8[rng.integers(8)]
        cfg = int(rng.integers(g.gemm_num_configs(code)))
        alpha = float(rng.choice([1.0, 2.0, -0.5, 0.25]))
        beta = float(rng.choice([0.0, 1.0, -0.5, 2.0]))
        act = int(rng.choice([g.GEMM_ACT_NONE, g.GEMM_ACT_RELU]))
        with_bias = bool(rng.random() < 0.7)
        log(f"case {case}: {dtype} {M}x{N}x{K} {''.join(layout)} {g.gemm_config_describe(code, cfg)} "
            f"alpha={alpha} beta={beta} act={act} bias={with_bias}")
        used = epi_case(M, N, K, layout, dtype, "int5", alpha, beta, act, with_bias=with_bias, config=cfg,
                        seed=100 + case)
        assert used == cfg or (M == 0 or N == 0)
    log("80 random epilogue cases exact")


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16"])
def test_epilogue_gelu_and_scale(dtype):
    import dense_gemm_engineering_run_amd as g
    kind = {"f32": "u11", "f16_f32": "n01", "bf16_bf16": "n002"}[dtype]
    for layout in LAYOUTS8:
        epi_case(257, 190, 96, layout, dtype, kind, 0.75, 0.25, g.GEMM_ACT_GELU)
    log(f"{dtype}: gelu epilogue, 8 layouts")


def test_epilogue_beta_zero_ignores_c_and_k_zero():
    import dense_gemm_engineering_run_amd as g
    epi_case(200, 120, 64, ("k", "k", "n"), "f32", "int5", 1.0, 0.0, g.GEMM_ACT_NONE, nan_c=True)
    epi_case(200, 120, 64, ("k", "n", "m"), "bf16_bf16", "int5", -1.0, 0.0, g.GEMM_ACT_RELU,
             nan_c=True)
    # K = 0: C = act(beta * C_old + bias)
    epi_case(130, 70, 0, ("k", "k", "n"), "f32", "int5", 3.0, 2.0, g.GEMM_ACT_NONE)


def test_epilogue_large_direct_kernels():
    """Shapes that take the direct-to-LDS kernels by default (several bands of
    the staged epilogue per tile, and 16-bit outputs)."""
    import dense_gemm_engineering_run_amd as g
    for dtype, layout in [("f32", "mnn"), ("f32", "kkn"), ("f16_f16", "knn"), ("bf16_bf16", "kkm")]:
        cfg = epi_case(4096, 4096, 64, tuple(layout), dtype, "int5", 2.0, 1.0, g.GEMM_ACT_RELU)
        name = g.gemm_config_describe(gi.DTYPE_CODE[dtype], cfg)
        log(f"  {dtype} {layout}: {name}")
        assert name.endswith(("dma", "pp")), name


# ---------------------------------------------------------------- operands not 16-byte aligned

def _upload_at(arr, off):
    """Device copy of flat storage `arr` starting `off` elements into a fresh
    buffer (so the pointer is only element-aligned); returns (tensor, ptr)."""
    t = gu.to_device(np.concatenate([np.zeros(off, arr.dtype), arr, np.zeros(8, arr.dtype)]))
    return t, t.data_ptr() + off * arr.itemsize


def unaligned_case(M, N, K, layout, dtype, kind, pads=(1, 3, 1), offs=(1, 2, 1), config=None, seed=21):
    """Leading dimensions extent + pads and pointers offs elements past a
    16-byte boundary; compared with the oracle, C's padding must keep the
    sentinel."""
    import torch
    import dense_gemm_engineering_run_amd as g
    a_m, b_m, c_m = layout
    code = gi.DTYPE_CODE[dtype]
    lda = (K if a_m == "k" else M) + pads[0]
    ldb = (K if b_m == "k" else N) + pads[1]
    ldc = (N if c_m == "n" else M) + pads[2]
    prob = gi.problem(M, N, K, a_m, b_m, c_m, dtype, kind, seed=seed, lda=lda, ldb=ldb, ldc=ldc,
                      pad_fill=float("nan"))
    ta, pa = _upload_at(prob["A"], offs[0])
    tb, pb = _upload_at(prob["B"], offs[1])
    c0 = gu.c_buffer(prob).cpu().numpy()
    tc, pc = _upload_at(c0, offs[2])
    s = torch.cuda.current_stream()
    args = (M, N, K, a_m, b_m, c_m, code, pa, pb, pc, lda, ldb, ldc, s.cuda_stream)
    st = g.gemm_run(*args) if config is None else g.gemm_run_config(*args, config)
    assert st == 0, g.gemm_status_str(st)
    used = g.gemm_config_describe(code, g.gemm_last_config())
    s.synchronize()
    flat = tc.cpu().numpy()[offs[2]:offs[2] + c0.size]
    got, flat = gu.host_c(torch.from_numpy(flat.view(np.int16) if flat.dtype == np.uint16 else flat), prob)
    ok, info = gu.check(got, gu.reference(prob), prob, kind == "int5")
    assert ok, (layout, dtype, used, info)
    assert gu.padding_intact(flat, prob)
    return used


@pytest.mark.parametrize("dtype", ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"])
def test_unaligned_operands_every_layout(dtype):
    """Odd leading dimensions and pointers one or two elements past a 16-byte
    boundary (NaN in the ld padding): the element-by-element configs, chosen
    automatically, bit-exact on integer inputs; both scalar configs forced."""
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    scalar = [i for i in range(g.gemm_num_configs(code)) if g.gemm_config_describe(code, i).endswith("scalar")]
    for layout in LAYOUTS8:
        used = unaligned_case(200, 136, 72, layout, dtype, "int5")
        assert used.endswith("scalar"), used
        for cfg in scalar:
            unaligned_case(97, 65, 37, layout, dtype, "int5", pads=(3, 1, 5), offs=(3, 1, 2), config=cfg)
            # several tiles and k-tiles, a partial last k-tile
            unaligned_case(300, 260, 100, layout, dtype, "int5", pads=(1, 5, 3), offs=(1, 3, 3), config=cfg,
                           seed=23)
    log(f"{dtype}: unaligned operands, 8 layouts")


def test_unaligned_large_and_noninteger():
    used = unaligned_case(2049, 1537, 515, ("k", "k", "n"), "f32", "u11")
    assert used.startswith("f32 128x128")
    unaligned_case(1031, 777, 300, ("m", "n", "m"), "bf16_bf16", "n002", pads=(5, 7, 9), offs=(7, 5, 3))


def test_unaligned_aligned_pointers_odd_ld_only():
    used = unaligned_case(300, 200, 136, ("k", "k", "n"), "f32", "int5", pads=(1, 1, 1), offs=(0, 0, 0))
    assert used.endswith("scalar")


def test_graph_capture_stream_k_and_epilogue():
    """gemm_run_ex on a stream-K config (workspace counters reset by the
    kernel itself, no memset), on a plain config with an epilogue, on the
    stream-K config with the epilogue, and on a split-k config (two kernels
    per call) with and without it, each captured once: every replay, with
    eager work between replays, equals the oracle bit for bit."""
    import torch

    import dense_gemm_engineering_run_amd as g
    import oracle
    sk = [i for i in range(g.gemm_num_configs(0)) if g.gemm_config_describe(0, i).endswith(" sk")][2]
    prob = gi.problem(600, 520, 200, "k", "k", "n", "f32", "int5", seed=33)
    ref = gu.reference(prob)
    a, b = gu.to_device(prob["A"]), gu.to_device(prob["B"])
    bias = torch.arange(520, dtype=torch.float32, device="cuda") - 260.0
    want_epi = oracle.epilogue_ref(ref, 2.0, 0.0, None, bias.cpu().numpy(), oracle.ACT_RELU)
    relu = g.Epilogue(2.0, 0.0, bias.data_ptr(), g.GEMM_ACT_RELU)
    split = [i for i in range(g.gemm_num_configs(0)) if g.gemm_config_describe(0, i).endswith(" split")][1]
    cases = [(sk, None, ref), (-1, relu, want_epi), (sk, relu, want_epi), (split, None, ref),
             (split, relu, want_epi)]
    for cfg, epi, want in cases:
        need = g.gemm_workspace_size(600, 520, 200, "k", "k", "n", 0, cfg)
        assert (need > 0) == (cfg >= 0)
        ws = torch.zeros(max(need, 16) // 4, dtype=torch.int32, device="cuda")
        c = gu.c_buffer(prob)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                assert g.gemm_run_ex(600, 520, 200, "k", "k", "n", 0, a.data_ptr(), b.data_ptr(),
                                     c.data_ptr(), prob["lda"], prob["ldb"], prob["ldc"], epi,
                                     ws.data_ptr(), need, s.cuda_stream, cfg) == 0
        torch.cuda.synchronize()
        for rep in range(4):
            c.fill_(-1.0)                    # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got, _ = gu.host_c(c, prob)
            ok, info = gu.check(got, want, prob, True)
            assert ok, (cfg, rep, info)
        if cfg == sk:
            assert int(torch.count_nonzero(ws[:256 // 4])) == 0     # counters back at zero


# ---------------------------------------------------------------- large sizes

def _exact_case(M, N, K, layout, dtype, A_log, B_log, batch=1):
    """Upload logical A (M x K) and B (N x K) in the given majors, run, and
    compare with the exact integer product (values keep every fp32 partial
    sum exact)."""
    import torch
    import dense_gemm_engineering_run_amd as g
    a_m, b_m, c_m = layout
    code = gi.DTYPE_CODE[dtype]
    _, tin, tout = gi.DTYPES[code]
    lda = gi.min_ld(M if a_m == "m" else K, gi.ELEM_BYTES[tin])
    ldb = gi.min_ld(N if b_m == "n" else K, gi.ELEM_BYTES[tin])
    ldc = gi.min_ld(M if c_m == "m" else N, gi.ELEM_BYTES[tout])
    A = gi.store(gi.cast(A_log, tin), a_m == "m", lda)
    B = gi.store(gi.cast(B_log, tin), b_m == "n", ldb)
    outer = N if c_m == "m" else M
    a, b = gu.to_device(A), gu.to_device(B)
    c = torch.zeros(outer * ldc * batch, dtype=torch.float32 if tout == "f32" else torch.int16, device="cuda")
    s = torch.cuda.current_stream()
    st = g.gemm_run_batched(M, N, K, a_m, b_m, c_m, code, a.data_ptr(), b.data_ptr(), c.data_ptr(),
                            lda, ldb, ldc, batch, 0, 0, outer * ldc, s.cuda_stream)
    assert st == 0, g.gemm_status_str(st)
    s.synchronize()
    want = A_log.astype(np.float64) @ B_log.astype(np.float64).T
    flat = c.cpu().numpy()
    if tout != "f32":
        flat = flat.view(np.uint16)
    for l in (0, batch // 2, batch - 1):
        got = gi.load(flat[l * outer * ldc:(l + 1) * outer * ldc], M, N, c_m == "m", ldc)
        ok, info = gu.compare.check(np.ascontiguousarray(got), want, tout, True)
        assert ok, (l, info)


def test_long_k_exact():
    """K = 2^22 (a 16 MiB row per operand row): values in {-1, 0, 1} keep
    every fp32 partial sum an exact integer."""
    rng = np.random.Generator(np.random.PCG64(5))
    K = 1 << 22
    A = rng.integers(-1, 2, size=(48, K)).astype(np.float32)
    B = rng.integers(-1, 2, size=(40, K)).astype(np.float32)
    log(f"long K {K}")
    _exact_case(48, 40, K, ("k", "k", "n"), "f32", A, B)
    _exact_case(48, 40, K, ("m", "n", "m"), "bf16_f32", A, B)


def test_tall_m_exact():
    """M = 2^20 rows (4096 tiles of 256 along M)."""
    rng = np.random.Generator(np.random.PCG64(6))
    M = 1 << 20
    A = rng.integers(-5, 6, size=(M, 64)).astype(np.float32)
    B = rng.integers(-5, 6, size=(48, 64)).astype(np.float32)
    log(f"tall M {M}")
    _exact_case(M, 48, 64, ("k", "k", "n"), "f16_f32", A, B)
    _exact_case(M, 48, 64, ("m", "k", "n"), "f32", A, B)


def test_max_batch_exact():
    """The largest batch (65535 entries on grid.y) of a broadcast 16x24x8 problem."""
    rng = np.random.Generator(np.random.PCG64(7))
    A = rng.integers(-5, 6, size=(16, 8)).astype(np.float32)
    B = rng.integers(-5, 6, size=(24, 8)).astype(np.float32)
    log("batch 65535")
    _exact_case(16, 24, 8, ("k", "k", "n"), "f32", A, B, batch=65535)


# (M, N, K, layout, dtype, which operand is the 2^20-row one).  Each long
# operand takes 4.5 GiB and C over 4 GiB, so tile origins, the 32-bit
# extents of the buffer loads and the C offsets all pass the 2^32-byte mark;
# the short side is 4 past a multiple of 256 or 8 past one (ragged tiles).
OVER_4GIB = [
    (1 << 20, 1028, 2304, ("k", "k", "n"), "f16_f32", "A"),
    (1032, 1 << 20, 2304, ("m", "n", "m"), "bf16_f32", "B"),
    (1 << 20, 1028, 1152, ("k", "k", "n"), "f32", "A"),
]


@pytest.mark.parametrize("M,N,K,layout,dtype,big", OVER_4GIB)
def test_operands_and_c_over_4gib_exact(M, N, K, layout, dtype, big):
    """The long operand's rows repeat a seeded 997-row integer pattern
    (so an offset that wrapped at 2^32 would read another row phase, or
    another k, than the one it should); every element of C is compared
    with the fp64 product of the pattern, which is exact for these values."""
    import torch
    import dense_gemm_engineering_run_amd as g
    a_m, b_m, c_m = layout
    code = gi.DTYPE_CODE[dtype]
    _, tin, tout = gi.DTYPES[code]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[tin]
    P = 997
    rng = np.random.Generator(np.random.PCG64(11))
    long_rows = M if big == "A" else N
    short_rows = N if big == "A" else M
    pat = rng.integers(-2, 3, size=(P, K)).astype(np.float32)
    short = rng.integers(-2, 3, size=(short_rows, K)).astype(np.float32)
    # C restricted to the pattern: (short x P) products, then spread by row phase.
    small = (short.astype(np.float64) @ pat.astype(np.float64).T).astype(np.float32)
    log(f"over 4 GiB {dtype} {M}x{N}x{K} {a_m}{b_m}{c_m} long {big}")

    phase = torch.arange(long_rows, device="cuda") % P
    pat_d = torch.from_numpy(pat).cuda().to(tdt)
    # The long operand, k-contiguous (rows x K) or not (K x rows).
    long_kmaj = (a_m if big == "A" else b_m) == "k"
    long_d = pat_d[phase] if long_kmaj else pat_d.t()[:, phase].contiguous()
    del pat_d
    short_kmaj = (b_m if big == "A" else a_m) == "k"
    short_d = torch.from_numpy(short).cuda().to(tdt)
    short_d = short_d if short_kmaj else short_d.t().contiguous()
    a_d, b_d = (long_d, short_d) if big == "A" else (short_d, long_d)
    assert long_d.numel() * long_d.element_size() > (1 << 32)
    lda = a_d.shape[1]
    ldb = b_d.shape[1]
    ldc = N if c_m == "n" else M
    outer = M if c_m == "n" else N
    assert outer * ldc * 4 > (1 << 32)
    c = torch.full((outer, ldc), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    st = g.gemm_run(M, N, K, a_m, b_m, c_m, code, a_d.data_ptr(), b_d.data_ptr(), c.data_ptr(),
                    lda, ldb, ldc, s.cuda_stream)
    assert st == 0, g.gemm_status_str(st)
    s.synchronize()
    log(f"  config {g.gemm_config_describe(code, g.gemm_last_config())}")
    del a_d, b_d, long_d, short_d
    # small[s, p] = C at (short row s, long row with phase p).
    small_d = torch.from_numpy(small).cuda()
    if big == "A":
        want = small_d.t()[phase]            # (M x N): row i is small[:, i % P]
        got = c if c_m == "n" else c.t()
    else:
        want = small_d[:, phase]             # (M x N): column j is small[:, j % P]
        got = c if c_m == "n" else c.t()
    bad = int((got != want).sum())
    assert bad == 0, f"{bad} of {M * N} elements differ"


# ---------------------------------------------------------------- seeded random sweep

def test_random_shapes_configs_layouts_exact():
    """120 seeded random cases: M, N, K in [1, 400], any layout and dtype,
    extra leading-dimension padding (16-byte multiples or odd), a random
    config among those the operands allow (stream-K ones with a workspace);
    integer inputs, bit-exact against the oracle, C padding untouched."""
    import torch
    import dense_gemm_engineering_run_amd as g
    rng = np.random.Generator(np.random.PCG64(2024))
    for case in range(120):
        dtype = ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"][rng.integers(5)]
        code = gi.DTYPE_CODE[dtype]
        M, N, K = (int(x) for x in rng.integers(1, 401, size=3))
        a_m, b_m, c_m = LAYOUTS8[rng.integers(8)]
        _, tin, tout = gi.DTYPES[code]
        aligned = rng.random() < 0.7
        def ld(inner, es):
            base = gi.min_ld(inner, es) if aligned else inner
            return base + (int(rng.integers(0, 3)) * (16 // es) if aligned else int(rng.integers(0, 4)))
        lda = ld(M if a_m == "m" else K, gi.ELEM_BYTES[tin])
        ldb = ld(N if b_m == "n" else K, gi.ELEM_BYTES[tin])
        ldc = ld(M if c_m == "m" else N, gi.ELEM_BYTES[tout])
        vec = all((x * e) % 16 == 0 for x, e in ((lda, gi.ELEM_BYTES[tin]), (ldb, gi.ELEM_BYTES[tin]),
                                                   (ldc, gi.ELEM_BYTES[tout])))
        names = [g.gemm_config_describe(code, i) for i in range(g.gemm_num_configs(code))]
        allowed = [i for i, nm in enumerate(names) if vec or nm.endswith("scalar")]
        cfg = int(rng.choice(allowed))
        prob = gi.problem(M, N, K, a_m, b_m, c_m, dtype, "int5", seed=case, lda=lda, ldb=ldb, ldc=ldc,
                          pad_fill=float("nan"))
        need = g.gemm_workspace_size(M, N, K, a_m, b_m, c_m, code, cfg)
        ws = torch.zeros(max(need, 16) // 4, dtype=torch.int32, device="cuda")
        a, b = gu.to_device(prob["A"]), gu.to_device(prob["B"])
        c = gu.c_buffer(prob)
        s = torch.cuda.current_stream()
        st = g.gemm_run_ws(M, N, K, a_m, b_m, c_m, code, a.data_ptr(), b.data_ptr(), c.data_ptr(),
                           lda, ldb, ldc, ws.data_ptr() if need else 0, need, s.cuda_stream, cfg)
        what = (case, dtype, M, N, K, a_m + b_m + c_m, lda, ldb, ldc, names[cfg])
        assert st == 0, (what, g.gemm_status_str(st))
        s.synchronize()
        got, flat = gu.host_c(c, prob)
        ok, info = gu.check(got, gu.reference(prob), prob, True)
        assert ok, (what, info)
        assert gu.padding_intact(flat, prob), what
    log("120 random cases exact")


# ---------------------------------------------------------------- Python helper and threads

def test_torch_helper_all_layouts():
    """gemm(a, b, c) on torch views: majors and leading dimensions come from
    the strides (transposed views give the m/n-major storage); integer inputs,
    exact against the fp64 product."""
    import torch
    import dense_gemm_engineering_run_amd as g
    rng = np.random.Generator(np.random.PCG64(8))
    M, N, K = 150, 90, 70
    A = rng.integers(-5, 6, size=(M, K)).astype(np.float32)
    B = rng.integers(-5, 6, size=(N, K)).astype(np.float32)
    want = A.astype(np.float64) @ B.astype(np.float64).T
    for tin, tout in [(torch.float32, torch.float32), (torch.float16, torch.float32),
                      (torch.bfloat16, torch.bfloat16)]:
        for at, bt, ct in itertools.product([False, True], repeat=3):
            a = torch.from_numpy(A).to(tin)
            b = torch.from_numpy(B).to(tin)
            a = (a.t().contiguous().cuda().t() if at else a.cuda())
            b = (b.t().contiguous().cuda().t() if bt else b.cuda())
            c = torch.zeros((N, M) if ct else (M, N), dtype=tout, device="cuda")
            c = c.t() if ct else c
            g.gemm(a, b, c)
            torch.cuda.synchronize()
            got = c.float().cpu().numpy().astype(np.float64)
            want_t = torch.from_numpy(want).to(tout).double().numpy()   # exact sums, rounded to C's type
            assert np.array_equal(got, want_t), (tin, at, bt, ct)


def test_concurrent_host_threads():
    """Four host threads, each on its own stream, enqueue different problems
    through the C ABI at the same time (ctypes releases the GIL): every result
    is exact."""
    import threading
    import torch
    import dense_gemm_engineering_run_amd as g
    shapes = [(256, 192, 96, "f32"), (300, 200, 136, "f16_f32"), (130, 260, 72, "bf16_bf16"),
              (512, 512, 64, "f16_f16")]
    probs = [gi.problem(M, N, K, "k", "n", "n", dt, "int5", seed=40 + i) for i, (M, N, K, dt) in enumerate(shapes)]
    devs = [(gu.to_device(p["A"]), gu.to_device(p["B"]), gu.c_buffer(p)) for p in probs]
    streams = [torch.cuda.Stream() for _ in probs]
    errors = []

    def work(i):
        p, (a, b, c), s = probs[i], devs[i], streams[i]
        for _ in range(25):
            st = g.gemm_run(p["M"], p["N"], p["K"], "k", "n", "n", p["dtype"], a.data_ptr(), b.data_ptr(),
                            c.data_ptr(), p["lda"], p["ldb"], p["ldc"], s.cuda_stream)
            if st != 0:
                errors.append((i, st))
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(probs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for p, (a, b, c) in zip(probs, devs):
        got, flat = gu.host_c(c, p)
        ok, info = gu.check(got, gu.reference(p), p, True)
        assert ok, info
