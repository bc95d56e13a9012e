"""The offline tuner's GPU path end to end: every candidate of a small shape is
launched, verified bit for bit against the default config on integer inputs,
timed, and the written table makes gemm_run pick the winner."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import gemm_inputs as gi  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,layout", [("f32", "mnn"), ("f16_f32", "kkm"), ("bf16_bf16", "knn")])
def test_tuner_gpu_end_to_end(tmp_path, dtype, layout):
    import dense_gemm_engineering_run_amd as g
    from dense_gemm_engineering_run_amd import _binding as b
    from dense_gemm_engineering_run_amd import tune as T
    code = gi.DTYPE_CODE[dtype]
    key = (code, layout[0], layout[1], layout[2], 520, 300, 136)

    def inputs(k):
        p = gi.problem(k[4], k[5], k[6], k[1], k[2], k[3], k[0], "int5")
        return p["A"], p["B"], p["lda"], p["ldb"], p["ldc"]

    meas = T.GpuMeasure(inputs, warmup=2, iters=5, timing_inputs=inputs)
    table = tmp_path / "table.txt"
    best = T.tune([key], meas, T.config_names, str(tmp_path / "log.jsonl"), str(table),
                  verbose=False)
    recs = [l for l in open(tmp_path / "log.jsonl")]
    assert len(recs) == g.gemm_num_configs(code)
    import json
    assert all(json.loads(r)["pass"] for r in recs), [json.loads(r) for r in recs if not json.loads(r)["pass"]]
    winner = best[T.key_str(key)]["config"]
    try:
        assert g.gemm_load_tuning(str(table)) == 0
        assert g.gemm_select_config(520, 300, 136, layout[0], layout[1], layout[2], code) == winner
    finally:
        g.gemm_load_tuning(b.DEFAULT_TABLE if os.path.exists(b.DEFAULT_TABLE) else None)
