"""bench.py's host-side contract without a GPU: more than one GPU is refused
with a message, every workload is well formed, and the traffic table lookup
only answers for the current kernel sources."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_workloads_are_well_formed():
    import gemm_inputs as gi
    assert bench.HEADLINE in bench.WORKLOADS
    for name, (M, N, K, a, b, c, dtype, kind, ldc, desc) in bench.WORKLOADS.items():
        assert a in "km" and b in "kn" and c in "nm", name
        assert dtype in gi.DTYPE_CODE and desc, name
        assert min(M, N, K) > 0, name
    assert set(bench.OPTIONS) <= set(bench.WORKLOADS)
    assert set(bench.NEXT_ROWS) == set(bench.OPTIONS)


def test_traffic_lookup_needs_current_sources(tmp_path, monkeypatch):
    src = bench.kernel_source_hash()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "hbm_traffic.md").write_text(
        "| workload | src hash | fetch | write | total |\n|---|---|---|---|---|\n"
        f"| fp32_8192 | {src} | 1 | 2 | 3 |\n| fp16_4096_kkn | 0000000000000000 | 1 | 2 | 3 |\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: src)
    assert bench.read_traffic("fp32_8192") == 3.0
    assert bench.read_traffic("fp16_4096_kkn") is None
    assert bench.read_traffic("bf16_skinny") is None


def test_host_facts_and_stats():
    h = bench.host_info()
    assert h["nproc"] == len(os.sched_getaffinity(0)) and h["cpu_count"] >= 1
    assert 1 <= bench.oracle_threads() <= h["nproc"]
    c = bench.clocks()
    assert set(c) == {"sclk_mhz", "mclk_mhz"} and len(c["sclk_mhz"]) == len(c["mclk_mhz"])
    st = bench._stats([3.0, 1.0, 2.0, 10.0])
    assert st["median_ms"] == 2.5 and st["mean_ms"] == 4.0 and st["n"] == 4
    assert bench._stats([5.0, 1.0, 2.0])["median_ms"] == 2.0
    assert bench._mfma_cycles("f16 16x16x32") == 16 and bench._mfma_cycles("f16 32x32x16") == 32


def test_cli_mnk_and_sweep_in_default_run():
    assert bench.parse_mnk("1,2,3") == (1, 2, 3)
    import argparse
    import pytest
    with pytest.raises(argparse.ArgumentTypeError):
        bench.parse_mnk("1,2")
    # the default run ("--others all") covers every workload, the sweep included
    assert bench.SWEEP and all(w in bench.WORKLOADS for w in bench.SWEEP)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True,
                       text=True, timeout=120)
    for flag in ("--mnk", "--a_major", "--b_major", "--c_major", "--dtype", "--iterations",
                 "--warmup_iterations", "--skip_ref_check", "--use_cold_l2", "--probe"):
        assert flag in r.stdout, flag
