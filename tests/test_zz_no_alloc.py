"""gemm_run_noalloc (the library's own device scratch as the stream-K
workspace) against gemm_run_ws with a caller-owned workspace and the same
config: bit for bit, on two calls in a row, the second with a smaller input;
both also against the oracle (integer inputs, exact)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
import gemm_inputs as gi  # noqa: E402
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def _run_both(M, N, K, layout, dtype, config, seed, ldc=None):
    """C from gemm_run_noalloc and from gemm_run_ws (same config), and the
    config each launched."""
    import torch
    import dense_gemm_engineering_run_amd as g
    code = gi.DTYPE_CODE[dtype]
    prob = gi.problem(M, N, K, *layout, dtype, "int5", seed=seed, ldc=ldc)
    a, b = gu.to_device(prob["A"]), gu.to_device(prob["B"])
    s = torch.cuda.current_stream()
    args = (M, N, K, *layout, code, a.data_ptr(), b.data_ptr())
    c_na = gu.c_buffer(prob)
    st = g.gemm_run_noalloc(*args, c_na.data_ptr(), prob["lda"], prob["ldb"], prob["ldc"], s.cuda_stream, config)
    assert st == 0, g.gemm_status_str(st)
    used = g.gemm_last_config()
    need = g.gemm_workspace_size(M, N, K, *layout, code, used)
    ws = torch.zeros(max(need, 16) // 4, dtype=torch.int32, device="cuda")
    c_ws = gu.c_buffer(prob)
    st = g.gemm_run_ws(*args, c_ws.data_ptr(), prob["lda"], prob["ldb"], prob["ldc"],
                       ws.data_ptr() if need else 0, need, s.cuda_stream, used)
    assert st == 0, g.gemm_status_str(st)
    assert g.gemm_last_config() == used
    s.synchronize()
    got_na, flat_na = gu.host_c(c_na, prob)
    got_ws, _ = gu.host_c(c_ws, prob)
    return prob, got_na, flat_na, got_ws, g.gemm_config_describe(code, used), need


def _check(prob, got_na, flat_na, got_ws):
    bits = np.uint32 if prob["out_type"] == "f32" else np.uint16
    assert np.array_equal(got_na.view(bits), got_ws.view(bits))
    assert gu.no_sentinel(got_na, prob)
    ok, info = gu.check(got_na, gu.reference(prob), prob, True)
    assert ok, info
    assert gu.padding_intact(flat_na, prob)


def test_noalloc_matches_workspace_entry_point_two_calls():
    import dense_gemm_engineering_run_amd as g
    # 1: the ragged fp32 problem on the 128x128 stream-K config (its split
    # tail's partial tiles and counters in the scratch array).
    sk = next(i for i in range(g.gemm_num_configs(0))
              if g.gemm_config_describe(0, i) == "f32 128x128x32 w2x2 mfma32 s2 dma sk")
    log("noalloc 1: f32 4095x2049x1028 kkn, f32 128x128x32 w2x2 mfma32 s2 dma sk")
    prob, na, flat, ws, name, need = _run_both(4095, 2049, 1028, ("k", "k", "n"), "f32", sk, seed=3, ldc=2052)
    log(f"  {name}, workspace {need} bytes")
    assert name.endswith(" sk") and 0 < need <= g.GEMM_NOALLOC_SCRATCH_BYTES
    _check(prob, na, flat, ws)
    # 2: a smaller problem right after, on a 16-bit stream-K config whose
    # split tiles use fewer partial slots and counters than call 1 left.
    code = gi.DTYPE_CODE["f16_f32"]
    sk16 = [i for i in range(g.gemm_num_configs(code)) if g.gemm_config_describe(code, i).endswith(" sk")]
    for cfg in sk16:
        log(f"noalloc 2: f16_f32 600x520x200 mnm, {g.gemm_config_describe(code, cfg)}")
        prob, na, flat, ws, name, need = _run_both(600, 520, 200, ("m", "n", "m"), "f16_f32", cfg, seed=4)
        assert need > 0
        _check(prob, na, flat, ws)
    # 3: smaller again, fp32, a config without a workspace (no counters to clear).
    log("noalloc 3: f32 300x200x136 kkn, default config")
    prob, na, flat, ws, name, need = _run_both(300, 200, 136, ("k", "k", "n"), "f32", -1, seed=5)
    log(f"  {name}, workspace {need} bytes")
    _check(prob, na, flat, ws)
