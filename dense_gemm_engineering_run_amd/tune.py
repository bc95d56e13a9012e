"""Offline tile-config autotuner.

For every tuning key (dtype, a_major, b_major, c_major, M, N, K) it runs each
tile config the library was built with, checks it, times it, and writes the
fastest passing config per key into a tuning table that gemm_run reads.  The
search space, the per-key cache and the warm-up / iteration counts follow the
CuTe DSL benchmark/autotune notebook (autotune_jit's params_dict and
update_on_change, tune(), benchmark()); the candidates are this library's
compiled tile configs rather than JIT parameters.

Each candidate is
  1. launched through gemm_run_config (gemm_run_ws with a workspace for stream-K and split-k configs) and must report that the config it ran
     is the one requested (gemm_last_config) -- the notebook's tune() example
     compiles a fixed copy width whatever candidate it is given, which is the
     mistake this check rules out;
  2. checked on integer-valued inputs, whose exact result is unique: its
     output must equal, bit for bit, the output of the library's default
     config for the same key.  That reference output is itself checked first,
     on 64 sampled rows (the first, the last and seeded ones, all columns),
     against the exact product computed in fp64 on the host and rounded to
     C's type; a key whose reference fails is not tuned;
  3. timed: `warmup` untimed runs, then `iters` runs each bracketed by HIP
     events on the launch stream; the median is the score.
Every result is appended to a JSONL log as it is measured; a rerun skips the
(key, config) pairs already in the log, so an interrupted tuning resumes.  The
table is written atomically (temporary file, then rename).
"""
import json
import os
import statistics
import sys
import time

DTYPE_NAMES = ["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"]


# Kernels whose eager median is below GRAPH_BELOW_US are ranked by their time
# per launch in a captured graph (GRAPH_LAUNCHES launches, median of
# GRAPH_REPLAYS replays).
GRAPH_BELOW_US = 30.0
GRAPH_LAUNCHES = 20
GRAPH_REPLAYS = 5

def key_str(key):
    dt, a, b, c, M, N, K = key
    return f"{DTYPE_NAMES[dt]} {a} {b} {c} {M} {N} {K}"


def load_log(path):
    done = {}
    if path and os.path.exists(path):
        with open(path) as f:
            for line in f:
                line = line.strip()
                if not line:
                    continue
                try:
                    r = json.loads(line)
                except ValueError:
                    continue   # a torn last line from an interrupted run
                done[(r["key"], r["config_name"])] = r
    return done


def needs_workspace(name):
    """Stream-K and split-k configs (names ending in ' sk' or ' split') run
    only with a workspace."""
    return name.endswith(" sk") or name.endswith(" split")


def best_per_key(records, plain=False):
    """Fastest passing record per key (plain: among configs that need no workspace)."""
    best = {}
    for r in records:
        if not r.get("pass") or r.get("median_us") is None:
            continue
        if plain and needs_workspace(r["config_name"]):
            continue
        k = r["key"]
        if k not in best or r["median_us"] < best[k]["median_us"]:
            best[k] = r
    return best


def write_table(path, best, header="", fallback=None):
    """One line per key with its best config; when that config needs a
    workspace, a second line with the best config that does not (the library
    takes the first line it can use: gemm_run has no workspace)."""
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        f.write("# dtype a_major b_major c_major M N K config  (written by tune.py)\n")
        if header:
            f.write(f"# {header}\n")
        for k in sorted(best):
            r = best[k]
            f.write(f"{k} {r['config_name']}   # {r['median_us']:.2f} us\n")
            alt = (fallback or {}).get(k)
            if needs_workspace(r["config_name"]) and alt is not None:
                f.write(f"{k} {alt['config_name']}   # {alt['median_us']:.2f} us, no workspace\n")
    os.replace(tmp, path)


def tune(keys, measure, config_names, log_path=None, table_path=None, verbose=True,
         header=""):
    """Core search, independent of the GPU.

    keys:          list of (dtype, a, b, c, M, N, K)
    measure:       measure(key, config_id) -> dict(launched=int, pass=bool,
                   median_us=float|None, mean_us=float|None, err=float|None, error=str|None)
    config_names:  config_names(dtype) -> list of names (index = config id)
    Returns {key_str: best record}.
    """
    done = load_log(log_path)
    records = list(done.values())
    logf = open(log_path, "a") if log_path else None
    try:
        for key in keys:
            ks = key_str(key)
            names = config_names(key[0])
            for cid, name in enumerate(names):
                if (ks, name) in done:
                    if verbose:
                        print(f"[tune] {ks} | {name}: cached", flush=True)
                    continue
                t0 = time.time()
                try:
                    m = measure(key, cid)
                except Exception as e:   # a failing candidate is dropped, tuning goes on
                    m = dict(launched=None, error=f"{type(e).__name__}: {e}")
                ok = (m.get("error") is None and m.get("launched") == cid and bool(m.get("pass")))
                if m.get("error") is None and m.get("launched") != cid:
                    m["error"] = f"launched config {m.get('launched')} instead of {cid}"
                rec = dict(key=ks, config=cid, config_name=name, **m)
                rec["pass"] = ok
                rec["seconds"] = round(time.time() - t0, 3)
                records.append(rec)
                if logf:
                    logf.write(json.dumps(rec) + "\n")
                    logf.flush()
                if verbose:
                    t = rec.get("median_us")
                    print(f"[tune] {ks} | {name}: {'%.2f us' % t if t else '-'} "
                          f"{'ok' if ok else 'REJECTED ' + str(rec.get('error'))}", flush=True)
    finally:
        if logf:
            logf.close()
    best = best_per_key(records)
    if table_path:
        write_table(table_path, best, header, fallback=best_per_key(records, plain=True))
    if verbose:
        for k in sorted(best):
            print(f"[tune] best {k}: {best[k]['config_name']} {best[k]['median_us']:.2f} us",
                  flush=True)
    return best


# ---------------------------------------------------------------- exact check of the reference

def _logical(flat, dt_in, major_first, ld, rows, cols):
    """fp64 logical rows x cols matrix from flat storage (float32, or fp16 /
    bf16 bit patterns as uint16); major_first: the row index is contiguous."""
    import numpy as np
    flat = np.asarray(flat)
    if dt_in == "f32":
        v = flat.astype(np.float64)
    elif dt_in == "f16":
        v = flat.view(np.float16).astype(np.float64)
    else:
        v = (flat.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if major_first:
        return v[: cols * ld].reshape(cols, ld)[:, :rows].T
    return v[: rows * ld].reshape(rows, ld)[:, :cols]


def _round_bits(x, dt_out):
    """Bits of fp64 values (exact integers below 2^24) rounded to the output
    type, to nearest even: uint32 for fp32, uint16 for fp16 / bf16."""
    import numpy as np
    if dt_out == "f32":
        return x.astype(np.float32).view(np.uint32)
    if dt_out == "f16":
        return x.astype(np.float16).view(np.uint16)
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)       # exact: |x| < 2^24
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def sample_rows(M, n=64, seed=0):
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(seed))
    picks = set(range(min(16, M))) | set(range(max(0, M - 16), M))
    picks |= set(int(r) for r in rng.integers(0, M, size=max(0, n - len(picks))))
    return sorted(picks)


def reference_rows_exact(key, A, B, lda, ldb, ldc, C, rows):
    """True when rows `rows` of C (flat storage: float32, or uint16 bits for
    16-bit outputs) equal the exact product of the integer-valued inputs,
    rounded to C's type; else False and the first (row, column) that differs."""
    import numpy as np
    dt, a, b, c, M, N, K = key
    din = {"f32": "f32", "f16_f32": "f16", "bf16_bf16": "bf16", "f16_f16": "f16", "bf16_f32": "bf16"}[DTYPE_NAMES[dt]]
    dout = {"f32": "f32", "f16_f32": "f32", "bf16_bf16": "bf16", "f16_f16": "f16", "bf16_f32": "f32"}[DTYPE_NAMES[dt]]
    Al = _logical(A, din, a == "m", lda, M, K)
    Bl = _logical(B, din, b == "n", ldb, N, K)
    want = _round_bits(Al[rows] @ Bl.T, dout)
    flat = np.asarray(C)
    bits = flat.view(np.uint32) if dout == "f32" else flat.view(np.uint16)
    got = bits[: N * ldc].reshape(N, ldc)[:, :M].T[rows] if c == "m" else bits[: M * ldc].reshape(M, ldc)[rows, :N]
    diff = np.argwhere(got != want)
    if diff.size:
        i, j = (int(v) for v in diff[0])
        return False, (rows[i], j)
    return True, None


# ---------------------------------------------------------------- GPU measurement

class GpuMeasure:
    """Checks and times candidates on the GPU through the C ABI.

    `inputs(key)` returns (A, B, lda, ldb, ldc) as flat numpy storage; the
    inputs should be integer-valued so that every correct config produces the
    same bits as the reference config (gemm_select_config's choice).
    `timing_inputs(key)`, if given, returns the data to time on (the MFMA
    units draw more power on realistic values than on small integers, and
    the clock follows)."""

    def __init__(self, inputs, warmup=10, iters=100, timing_inputs=None):
        import torch  # noqa: F401  (device memory and streams)
        self.inputs = inputs
        self.timing_inputs = timing_inputs
        self.warmup, self.iters = warmup, iters
        self._cache_key, self._dev, self._ref, self._tdev = None, None, None, None

    def _args(self, key, C):
        dt, a, b, c, M, N, K = key
        A, B, _, lda, ldb, ldc = self._dev
        import torch
        return (M, N, K, a, b, c, dt, A.data_ptr(), B.data_ptr(), C.data_ptr(), lda, ldb, ldc,
                torch.cuda.current_stream().cuda_stream)

    def _prepare(self, key):
        import numpy as np
        import torch

        import dense_gemm_engineering_run_amd as g
        if self._cache_key == key:
            return
        self._dev = self._ref = self._tdev = None
        torch.cuda.empty_cache()
        dt, a, b, c, M, N, K = key
        A, B, lda, ldb, ldc = self.inputs(key)

        def dev(x):
            x = np.ascontiguousarray(x)
            return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
        out_f32 = DTYPE_NAMES[dt] in ("f32", "f16_f32", "bf16_f32")
        outer = N if c == "m" else M
        C = torch.zeros(max(outer * ldc, 1), dtype=torch.float32 if out_f32 else torch.int16,
                        device="cuda")
        self._dev = (dev(A), dev(B), C, lda, ldb, ldc)
        ref = torch.zeros_like(C)
        st = g.gemm_run(*self._args(key, ref))
        if st != 0:
            raise RuntimeError(f"reference config failed: {g.gemm_status_str(st)}")
        torch.cuda.synchronize()
        ok, where = reference_rows_exact(key, A, B, lda, ldb, ldc, (ref.view(torch.int32) if out_f32 else ref).cpu().numpy(),
                                         sample_rows(M))
        if not ok:
            raise RuntimeError(f"reference config differs from the exact product at (row, column) {where}")
        self._ref = ref
        if self.timing_inputs is not None:
            TA, TB, tlda, tldb, _ = self.timing_inputs(key)
            assert (tlda, tldb) == (lda, ldb)
            self._tdev = (dev(TA), dev(TB))
        self._cache_key = key

    def __call__(self, key, cid):
        import torch

        import dense_gemm_engineering_run_amd as g
        dt, a, b, c, M, N, K = key
        self._prepare(key)
        C = self._dev[2]
        C.zero_()
        args = self._args(key, C) + (cid,)
        s = torch.cuda.current_stream()
        # Stream-K and split-k configs run through gemm_run_ws with a zero-filled workspace.
        need = g.gemm_workspace_size(M, N, K, a, b, c, dt, cid)
        ws = torch.zeros(max(need, 16) // 4, dtype=torch.int32, device="cuda") if need else None

        def launch(args):
            if ws is None:
                return g.gemm_run_config(*args)
            return g.gemm_run_ws(*args[:-2], ws.data_ptr(), need, args[-2], args[-1])
        st = launch(args)
        if st != 0:
            return dict(launched=None, error=g.gemm_status_str(st))
        launched = g.gemm_last_config()
        s.synchronize()
        res = dict(launched=launched, error=None)
        res["pass"] = bool(torch.equal(C.view(torch.int32) if C.dtype == torch.float32 else C,
                                       self._ref.view(torch.int32) if C.dtype == torch.float32
                                       else self._ref))
        if self._tdev is not None:
            args = (M, N, K, a, b, c, dt, self._tdev[0].data_ptr(), self._tdev[1].data_ptr(),
                    C.data_ptr(), self._dev[3], self._dev[4], self._dev[5], s.cuda_stream, cid)
        for _ in range(self.warmup):
            launch(args)
        # keep the GPU busy for at least 50 ms before timing (clock ramp-up)
        s.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.05:
            for _ in range(8):
                launch(args)
            s.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(self.iters)]
        for e0, e1 in ev:
            e0.record(s)
            launch(args)
            e1.record(s)
        s.synchronize()
        t = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
        res["median_us"] = statistics.median(t)
        res["mean_us"] = statistics.fmean(t)
        if res["median_us"] < GRAPH_BELOW_US:
            # A short kernel's eager time is mostly the host's launch latency,
            # the same whatever the config: rank by the time per launch inside
            # a captured graph of GRAPH_LAUNCHES launches instead (what a
            # caller that captures graphs sees); the eager median stays logged.
            res["eager_median_us"] = res["median_us"]
            res["median_us"] = self._graph_time(launch, args)
        res["tflops"] = 2.0 * M * N * K / (res["median_us"] * 1e-6) / 1e12
        return res

    def _graph_time(self, launch, args):
        import torch
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        gargs = args[:-2] + (gs.cuda_stream, args[-1])
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(graph, stream=gs):
                for _ in range(GRAPH_LAUNCHES):
                    launch(gargs)
        torch.cuda.synchronize()
        rs = torch.cuda.current_stream()           # replay() launches on the current stream
        times = []
        for _ in range(GRAPH_REPLAYS + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(rs)
            graph.replay()
            e1.record(rs)
            rs.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / GRAPH_LAUNCHES)
        return statistics.median(times[1:])       # the first replay warms up


def config_names(dtype):
    import dense_gemm_engineering_run_amd as g
    return [g.gemm_config_describe(dtype, i) for i in range(g.gemm_num_configs(dtype))]


def main(argv=None):
    import argparse
    ap = argparse.ArgumentParser(description="Tune tile configs per GEMM shape.")
    ap.add_argument("--keys", required=True,
                    help="file with one key per line: dtype a_major b_major c_major M N K")
    ap.add_argument("--log", required=True, help="JSONL log (appended; resumes)")
    ap.add_argument("--table", required=True, help="tuning table to write")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--iters", type=int, default=100)
    args = ap.parse_args(argv)

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import gemm_inputs as gi

    keys = []
    with open(args.keys) as f:
        for line in f:
            line = line.split("#")[0].split()
            if len(line) == 7:
                keys.append((DTYPE_NAMES.index(line[0]), line[1], line[2], line[3],
                             int(line[4]), int(line[5]), int(line[6])))

    def inputs(key):
        dt, a, b, c, M, N, K = key
        p = gi.problem(M, N, K, a, b, c, dt, "int5")
        return p["A"], p["B"], p["lda"], p["ldb"], p["ldc"]

    def timing_inputs(key):
        dt, a, b, c, M, N, K = key
        kind = {"f32": "u11", "bf16_bf16": "n002", "bf16_f32": "n002"}.get(DTYPE_NAMES[dt], "n01")
        p = gi.problem(M, N, K, a, b, c, dt, kind)
        return p["A"], p["B"], p["lda"], p["ldb"], p["ldc"]

    meas = GpuMeasure(inputs, warmup=args.warmup, iters=args.iters, timing_inputs=timing_inputs)
    tune(keys, meas, config_names, args.log, args.table)


if __name__ == "__main__":
    main()
