"""The offline tuner's search, resume and table logic against a scripted fake
backend (no GPU): the fastest passing candidate wins, failing / mislaunched /
crashing candidates are dropped, a rerun resumes from the log, and the table
it writes is one the library loads."""
import json

import dense_gemm_engineering_run_amd as g
from dense_gemm_engineering_run_amd import tune as T


def names(dtype):
    return [g.gemm_config_describe(dtype, i) for i in range(g.gemm_num_configs(dtype))]


def scripted(script, calls):
    def measure(key, cid):
        calls.append((key, cid))
        r = script[cid]
        if r == "raise":
            raise RuntimeError("launch failed")
        t, ok, launched = r
        return dict(launched=launched, error=None, median_us=t, mean_us=t, **{"pass": ok})
    return measure


def test_fastest_passing_candidate_wins_and_failures_are_dropped(tmp_path):
    key = (0, "k", "k", "n", 1000, 1000, 1000)
    n = g.gemm_num_configs(0)
    script = {i: (100.0 + i, True, i) for i in range(n)}
    script[1] = (5.0, True, 1)        # the winner
    script[2] = (3.0, False, 2)       # faster but wrong result
    script[3] = "raise"               # crashes
    script[4] = (1.0, True, 0)        # reports a different config than requested
    calls = []
    log = tmp_path / "log.jsonl"
    table = tmp_path / "table.txt"
    best = T.tune([key], scripted(script, calls), names, str(log), str(table), verbose=False)
    assert best[T.key_str(key)]["config"] == 1
    recs = [json.loads(l) for l in open(log)]
    assert len(recs) == n
    by = {r["config"]: r for r in recs}
    assert not by[2]["pass"] and not by[3]["pass"] and not by[4]["pass"]
    assert "instead of" in by[4]["error"]
    # resume: nothing is measured again
    calls.clear()
    with open(log, "a") as f:
        f.write('{"torn": ')      # an interrupted write
    best2 = T.tune([key], scripted(script, calls), names, str(log), str(table), verbose=False)
    assert calls == [] and best2[T.key_str(key)]["config"] == 1
    # the library reads the table and selects the tuned config
    saved = g.gemm_tuning_size()
    try:
        assert g.gemm_load_tuning(str(table)) == 0
        assert g.gemm_select_config(1000, 1000, 1000, "k", "k", "n", 0) == 1
    finally:
        from dense_gemm_engineering_run_amd import _binding as b
        import os
        g.gemm_load_tuning(b.DEFAULT_TABLE if os.path.exists(b.DEFAULT_TABLE) else None)
    assert g.gemm_tuning_size() == saved


def test_no_passing_candidate_leaves_key_untuned(tmp_path):
    key = (1, "m", "n", "m", 64, 64, 64)
    n = g.gemm_num_configs(1)
    script = {i: (1.0, False, i) for i in range(n)}
    best = T.tune([key], scripted(script, []), names, None, str(tmp_path / "t.txt"),
                  verbose=False)
    assert best == {}
    assert [l for l in open(tmp_path / "t.txt") if not l.startswith("#")] == []


def test_stream_k_winner_gets_a_fallback_line(tmp_path):
    """A stream-K config needs a workspace that gemm_run does not have: the
    table then also names the best config without one, and selection without
    a workspace takes that line."""
    key = (0, "k", "k", "n", 4095, 2049, 1028)
    all_names = names(0)
    sk = [i for i, nm in enumerate(all_names) if nm.endswith(" sk")]
    plain = [i for i, nm in enumerate(all_names) if not nm.endswith(" sk")]
    script = {i: (200.0 + i, True, i) for i in range(len(all_names))}
    script[sk[0]] = (150.0, True, sk[0])        # the overall winner
    script[plain[3]] = (160.0, True, plain[3])  # the best without a workspace
    table = tmp_path / "table.txt"
    T.tune([key], scripted(script, []), names, None, str(table), verbose=False)
    lines = [l.split("#")[0].split() for l in open(table) if not l.startswith("#")]
    assert [" ".join(l[7:]) for l in lines] == [all_names[sk[0]], all_names[plain[3]]]
    try:
        assert g.gemm_load_tuning(str(table)) == 0
        assert g.gemm_tuning_size() == 2
        assert g.gemm_select_config(4095, 2049, 1028, "k", "k", "n", 0) == plain[3]
        # with a workspace the stream-K line is the one sized
        assert g.gemm_workspace_size(4095, 2049, 1028, "k", "k", "n", 0) == \
            g.gemm_workspace_size(4095, 2049, 1028, "k", "k", "n", 0, sk[0]) > 0
    finally:
        from dense_gemm_engineering_run_amd import _binding as b
        import os
        g.gemm_load_tuning(b.DEFAULT_TABLE if os.path.exists(b.DEFAULT_TABLE) else None)


def test_reference_rows_exact_check_catches_planted_mistakes():
    """The tuner's check of its reference output: the exact product, laid out
    as C, passes for every dtype and C layout; a changed element, a C written
    row-shifted and column-shifted each fail at the right place."""
    import numpy as np

    import gemm_inputs as gi
    from dense_gemm_engineering_run_amd import tune as T
    for dtype, lay in [("f32", "mnn"), ("f16_f32", "kkm"), ("bf16_bf16", "knn"), ("f16_f16", "mkm"),
                       ("bf16_f32", "knm")]:
        code = gi.DTYPE_CODE[dtype]
        M, N, K = 70, 45, 300
        p = gi.problem(M, N, K, lay[0], lay[1], lay[2], dtype, "int5", seed=3)
        a_log, b_log = gi.draw_ab(M, N, K, "int5", seed=3)
        exact = a_log.astype(np.float64) @ b_log.astype(np.float64).T
        tout = gi.DTYPES[code][2]
        cbits = T._round_bits(exact, tout)
        flat = gi.store(cbits, lay[2] == "m", p["ldc"], fill=0)
        key = (code, lay[0], lay[1], lay[2], M, N, K)
        rows = T.sample_rows(M, n=20)
        assert T.reference_rows_exact(key, p["A"], p["B"], p["lda"], p["ldb"], p["ldc"], flat, rows) == (True, None)
        bad = flat.copy()
        r, col = rows[5], 7
        idx = (col * p["ldc"] + r) if lay[2] == "m" else (r * p["ldc"] + col)
        bad[idx] ^= 1
        assert T.reference_rows_exact(key, p["A"], p["B"], p["lda"], p["ldb"], p["ldc"], bad, rows) == (False, (r, col))
        row_shift = gi.store(np.roll(cbits, 1, axis=0), lay[2] == "m", p["ldc"], fill=0)
        assert not T.reference_rows_exact(key, p["A"], p["B"], p["lda"], p["ldb"], p["ldc"], row_shift, rows)[0]
        shifted = gi.store(np.roll(cbits, 1, axis=1), lay[2] == "m", p["ldc"], fill=0)
        assert not T.reference_rows_exact(key, p["A"], p["B"], p["lda"], p["ldb"], p["ldc"], shifted, rows)[0]
    # row sample: first and last 16 rows, the rest seeded, sorted and unique
    s = T.sample_rows(1000)
    assert s == sorted(set(s)) and s[:16] == list(range(16)) and s[-16:] == list(range(984, 1000))
