"""Benchmark of the MI355X GEMM library.

One step = one GEMM C = A * B^T through the C ABI on inputs already resident
in HBM.  The headline workload is the fp32 SGEMM M=N=K=8192 with A m-major,
B n-major and C n-major (the size and layouts the CuTe DSL Ampere SGEMM
example is run with in its docstring); the value is 2*M*N*K / t in TFLOP/s,
timed with HIP events on the stream the kernels are launched on, after
warm-up runs (the example's benchmark and the CuTe DSL benchmark notebook
time runs the same way): the mean over a window of back-to-back launches,
and the median of a second pass with an event after every launch.

The JSON line also carries:
  roofline      achieved TFLOP/s of the GEMM kernel against the MI355X dense
                MFMA peak for its input type, plus the HBM traffic measured
                with rocprofv3 counters (profiles/hbm_traffic.md) when that
                measurement matches the current kernel sources;
  cpu_baseline  the CPU oracle timed on a bounded row sample of the same
                problem on this host's CPUs, with the GPU rows compared to it;
  host, clocks  the host's CPUs and the GPU's shader and memory clocks read
                before and after the run (and sampled during the timed runs);
  workloads     the other measured GEMM workloads (fp16 4096^3 in all eight
                layouts, fp32 1024x512x256, fp32 4095x2049x1028 ragged, bf16
                65536x256x4096 tall-skinny with its HBM GB/s, the fp16 -> fp16
                K sweep at 8192^2), and the rows built on the plain GEMM:
                stream-K, the fused epilogue, the strided-batched mode,
                operands that are not 16-byte aligned; and one GPU's share of
                the fp32 cube and of the tall-skinny GEMM split over eight GPUs.

Other modes:
  --mnk M,N,K [--a_major --b_major --c_major --dtype ...]
                one problem of the caller's choice, checked against the
                oracle unless --skip_ref_check (the SGEMM example's command
                line: --mnk, the three majors, --iterations,
                --warmup_iterations, --skip_ref_check, --use_cold_l2);
  --use_cold_l2 rotate through enough copies of each problem's buffers
                (at least 512 MB) that the caches cannot hold them;
  --probe mfma|hbm|all
                the ceilings the kernels are measured against: 16-bit MFMA-only
                throughput on register operands (per shape, operands changing
                every MFMA or one fixed pair), and HBM -> LDS read rates per
                segment size (include/mi355_gemm_probe.h).
"""
import argparse
import glob
import hashlib
import json
import math
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (2MNK/t) + % of MFMA peak, fp32 8192³ and fp16 4096³"
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}   # MI355X dense MFMA
HBM_PEAK_GBS = 8000.0
COLD_BYTES = 512 << 20          # rotated working set of --use_cold_l2 (> the 256 MB MALL)

WORKLOADS = {
    # name: (M, N, K, a, b, c, dtype, kind, ldc or None, description)
    "fp32_8192": (8192, 8192, 8192, "m", "n", "n", "f32", "u11", None,
                  "fp32 SGEMM 8192x8192x8192, A m-major, B n-major, C n-major, uniform(-1,1)"),
    "fp32_1024x512x256": (1024, 512, 256, "k", "k", "n", "f32", "int5", None,
                          "fp32 GEMM 1024x512x256, A k-major, B k-major, C n-major, integers in [-5,5]"),
    "fp32_ragged": (4095, 2049, 1028, "k", "k", "n", "f32", "u11", 2052,
                    "fp32 ragged GEMM 4095x2049x1028, A k, B k, C n (ldc 2052), uniform(-1,1)"),
    "bf16_skinny": (65536, 256, 4096, "k", "k", "n", "bf16_bf16", "n002", None,
                    "bf16 GEMM 65536x256x4096 -> bf16, A k, B k, C n, normal(0,0.02)"),
}
for _a in "km":
    for _b in "kn":
        for _c in "nm":
            WORKLOADS[f"fp16_4096_{_a}{_b}{_c}"] = (
                4096, 4096, 4096, _a, _b, _c, "f16_f32", "n01", None,
                f"fp16 GEMM 4096^3 -> fp32, A {_a}, B {_b}, C {_c}, normal(0,1)")

# The fp16 -> fp16 sweep M = N = 8192, K = 512 .. 16384 with B stored K x N
# row-major (= N x K n-major here), the persistent-matmul benchmark of the
# Triton Gluon multi-CTA tutorial.
for _k in (512, 1024, 2048, 4096, 8192, 16384):
    WORKLOADS[f"fp16_sweep_k{_k}"] = (
        8192, 8192, _k, "k", "n", "n", "f16_f16", "n01", None,
        f"fp16 GEMM 8192x8192x{_k} -> fp16, A k, B n, C n, normal(0,1)")

# The rows built on top of the plain GEMM, each timed on a workload of its
# own: stream-K (persistent) scheduling on the ragged fp32 problem, the fused
# elementwise epilogue on the headline problem and on stream-K, the
# strided-batched mode, and the element-by-element path for operands that are
# not 16-byte aligned.
WORKLOADS["fp32_ragged_streamk"] = WORKLOADS["fp32_ragged"][:9] + (
    "fp32 ragged GEMM 4095x2049x1028 on the stream-K config f32 128x128x32 sk (workspace)",)
WORKLOADS["fp32_8192_epilogue"] = WORKLOADS["fp32_8192"][:9] + (
    "fp32 SGEMM 8192^3 (A m, B n, C n) with epilogue relu(A.B^T + bias[n])",)
WORKLOADS["fp32_ragged_streamk_epilogue"] = WORKLOADS["fp32_ragged"][:9] + (
    "fp32 ragged GEMM 4095x2049x1028 on the stream-K config f32 128x128x32 sk with epilogue relu(A.B^T + bias[n])",)
WORKLOADS["fp16_batched_64x512"] = (512, 512, 512, "k", "k", "n", "f16_f32", "n01", None,
                                    "fp16 strided-batched GEMM, 64 x (512x512x512) -> fp32, A k, B k, C n")
WORKLOADS["fp32_ragged_unaligned"] = WORKLOADS["fp32_ragged"][:8] + (2049,
    "fp32 ragged GEMM 4095x2049x1028 with lda = ldb = 1029, ldc = 2049 (not 16-byte multiples)",)
# One GPU's share when the two largest problems are split over eight GPUs
# without a reduction: the fp32 cube with C over a 4 x 2 grid of GPUs (rows
# M/4, columns N/2, each GPU holding its own slices of A and B), the
# tall-skinny GEMM split along M.
WORKLOADS["fp32_8192_shard8"] = (2048, 4096, 8192, "m", "n", "n", "f32", "u11", None,
    "fp32 SGEMM 2048x4096x8192 (one GPU's share of 8192^3 over a 4 x 2 GPU grid), A m, B n, C n, uniform(-1,1)")
WORKLOADS["bf16_skinny_shard8"] = (8192, 256, 4096, "k", "k", "n", "bf16_bf16", "n002", None,
    "bf16 GEMM 8192x256x4096 -> bf16 (one GPU's share of 65536x256x4096 split along M over 8 GPUs), A k, B k, C n, normal(0,0.02)")
OPTIONS = {
    "fp32_ragged_streamk": {"config": "f32 128x128x32 w2x2 mfma32 s2 dma sk"},
    "fp32_8192_epilogue": {"epilogue": "bias_relu"},
    "fp32_ragged_streamk_epilogue": {"config": "f32 128x128x32 w2x2 mfma32 s2 dma sk", "epilogue": "bias_relu"},
    "fp16_batched_64x512": {"batch": 64},
    "fp32_ragged_unaligned": {"lda": 1029, "ldb": 1029},
}
NEXT_ROWS = list(OPTIONS)
SWEEP = [w for w in WORKLOADS if w.startswith("fp16_sweep")]
SHARD = [w for w in WORKLOADS if w.endswith("_shard8")]

HEADLINE = "fp32_8192"

# Sources the GEMM kernels and their launch parameters are built from (the
# probes and the allocation-free entry point's wrapper do not change them).
_NOT_KERNEL_SOURCES = {"gemm_probe.hip", "gemm_noalloc.hip", "gemm_plan.hpp"}


def kernel_source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "dense_gemm_engineering_run_amd", "csrc", "*"))):
        if os.path.basename(p) in _NOT_KERNEL_SOURCES:
            continue
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per launch from profiles/hbm_traffic.md, if it was measured on
    the current kernel sources: a table row '| workload | src hash | fetch | write | total |'."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    src = kernel_source_hash()
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 5 and cells[0] == workload and cells[1] == src:
            try:
                return float(cells[4])
            except ValueError:
                return None
    return None


# ---------------------------------------------------------------- host and clocks

def _dpm_current(path):
    """MHz of the level marked '*' in an amdgpu pp_dpm_* file, or None."""
    try:
        for line in open(path):
            if "*" in line:
                m = re.search(r"(\d+)\s*Mhz", line, re.I)
                if m:
                    return int(m.group(1))
    except OSError:
        pass
    return None


def clocks():
    """Current shader and memory clock (MHz) of every GPU whose amdgpu sysfs
    entries this process can read (file reads only, no GPU call)."""
    out = {"sclk_mhz": [], "mclk_mhz": []}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        s = _dpm_current(os.path.join(dev, "pp_dpm_sclk"))
        m = _dpm_current(os.path.join(dev, "pp_dpm_mclk"))
        if s is not None or m is not None:
            out["sclk_mhz"].append(s)
            out["mclk_mhz"].append(m)
    return out


class ClockSampler:
    """Samples the shader clock from sysfs every 5 ms on a host thread while
    the timed runs execute; reports the range seen."""

    def __init__(self):
        self.samples = []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            s = [v for v in clocks()["sclk_mhz"] if v is not None]
            if s:
                self.samples.append(max(s))
            self._stop.wait(0.005)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def summary(self):
        if not self.samples:
            return None
        return {"min": min(self.samples), "max": max(self.samples), "n": len(self.samples)}


def cgroup_cpu_quota():
    """CPUs granted by the cgroup v2 (cpu.max) or v1 (cfs quota) limit, or None."""
    try:
        q, p = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            return int(q) / int(p)
    except (OSError, ValueError):
        pass
    try:
        q = int(open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us").read())
        p = int(open("/sys/fs/cgroup/cpu/cpu.cfs_period_us").read())
        if q > 0:
            return q / p
    except (OSError, ValueError):
        pass
    return None


def host_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    quota = cgroup_cpu_quota()
    return {"nproc": affinity, "cpu_count": os.cpu_count(), "cgroup_cpus": quota, "cpu_model": model}


def oracle_threads():
    """Threads for the CPU oracle: every CPU this process may run on (its
    affinity mask), capped by the cgroup's CPU quota when one is set (threads
    beyond the quota only share the same CPU time)."""
    n = len(os.sched_getaffinity(0))
    q = cgroup_cpu_quota()
    if q is not None:
        n = max(1, min(n, int(math.floor(q + 1e-9))))
    return n


# ---------------------------------------------------------------- problems

def _stats(ms_list):
    xs = sorted(ms_list)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"mean_ms": sum(xs) / n, "median_ms": med, "min_ms": xs[0], "max_ms": xs[-1], "n": n}


class Problem:
    """A seeded problem on the device.  spec = WORKLOADS tuple; opt = OPTIONS
    entry.  With cold_l2, ceil(COLD_BYTES / working set) copies of A, B, C
    (and the workspace) are made and launches rotate through them."""

    def __init__(self, name, spec=None, opt=None, seed=1024, cold_l2=False):
        import numpy as np
        import torch

        import dense_gemm_engineering_run_amd as g
        import gemm_inputs as gi
        M, N, K, a, b, c, dtype, kind, ldc, desc = spec or WORKLOADS[name]
        opt = OPTIONS.get(name, {}) if opt is None else opt
        self.name, self.desc = name, desc
        self.p = gi.problem(M, N, K, a, b, c, dtype, kind, seed=seed, ldc=ldc,
                            lda=opt.get("lda"), ldb=opt.get("ldb"))
        p = self.p
        self.batch = opt.get("batch", 1)

        def dev(x):
            x = np.ascontiguousarray(x)
            if self.batch > 1:                  # the same operand in every batch entry
                x = np.tile(x, self.batch)
            return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
        a0, b0 = dev(p["A"]), dev(p["B"])
        outer = N if p["c_first"] else M
        ct = torch.float32 if p["out_type"] == "f32" else torch.int16
        self.sc = outer * p["ldc"]
        c0 = torch.zeros(self.sc * self.batch, dtype=ct, device="cuda")
        self.stream = torch.cuda.current_stream()
        self.config = -1
        if "config" in opt:
            names = [g.gemm_config_describe(p["dtype"], i) for i in range(g.gemm_num_configs(p["dtype"]))]
            self.config = names.index(opt["config"])
        self.ws_bytes = g.gemm_workspace_size(M, N, K, a, b, c, p["dtype"], self.config)
        ws0 = torch.zeros(max(self.ws_bytes, 16) // 4, dtype=torch.int32, device="cuda")
        eb = gi.ELEM_BYTES[p["in_type"]]
        eo = gi.ELEM_BYTES[p["out_type"]]
        work = a0.numel() * a0.element_size() + b0.numel() * b0.element_size() + c0.numel() * c0.element_size()
        self.n_sets = max(1, math.ceil(COLD_BYTES / work)) if cold_l2 else 1
        self.sets = [(a0, b0, c0, ws0)]
        for _ in range(self.n_sets - 1):
            self.sets.append((a0.clone(), b0.clone(), torch.zeros_like(c0), torch.zeros_like(ws0)))
        self.working_set_bytes = work
        self.epi = None
        if opt.get("epilogue") == "bias_relu":
            self.bias = torch.linspace(-1, 1, N, device="cuda")
            self.epi = g.Epilogue(1.0, 0.0, self.bias.data_ptr(), g.GEMM_ACT_RELU)
        self.flops = 2.0 * M * N * K * self.batch
        self.bytes = float(M * K * eb + N * K * eb + M * N * eo) * self.batch
        self._next = 0

    @property
    def c(self):
        return self.sets[0][2]

    def launch(self, stream=None, set_index=None):
        import dense_gemm_engineering_run_amd as g
        i = self._next if set_index is None else set_index
        self._next = (i + 1) % self.n_sets
        a, b, c, ws = self.sets[i]
        p = self.p
        s = self.stream.cuda_stream if stream is None else stream
        args = (p["M"], p["N"], p["K"], p["a_major"], p["b_major"], p["c_major"], p["dtype"], a.data_ptr(),
                b.data_ptr(), c.data_ptr(), p["lda"], p["ldb"], p["ldc"])
        if self.batch > 1:
            st = g.gemm_run_batched(*args, self.batch, len(p["A"]), len(p["B"]), self.sc, s)
        elif self.epi is not None or self.config >= 0 or self.ws_bytes:
            st = g.gemm_run_ex(*args, self.epi, ws.data_ptr(), self.ws_bytes, s, self.config)
        else:
            st = g.gemm_run(*args, s)
        if st != 0:
            raise RuntimeError(g.gemm_status_str(st))

    def warm(self, warmup, min_warm_s=0.0):
        """`warmup` untimed launches, then (min_warm_s) more until the GPU has
        been busy that long (clocks ramp up over tens of ms after idle)."""
        import torch
        for _ in range(warmup):
            self.launch()
        torch.cuda.synchronize()
        if min_warm_s > 0:
            t0 = time.perf_counter()
            n = 1
            while time.perf_counter() - t0 < min_warm_s:
                for _ in range(n):
                    self.launch()
                torch.cuda.synchronize()
                n *= 2

    def time(self, iters):
        """Two passes of `iters` back-to-back launches on the launch stream:
        the first bracketed by one pair of events (mean_ms: the window over
        iters), the second with an event after every launch (the per-launch
        median, min and max; for kernels of a few microseconds the events
        between launches add their own time)."""
        import torch
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(iters):
            self.launch()
        e1.record(self.stream)
        torch.cuda.synchronize()
        window = e0.elapsed_time(e1) / iters
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        ev[0].record(self.stream)
        for i in range(iters):
            self.launch()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        st = _stats([ev[i].elapsed_time(ev[i + 1]) for i in range(iters)])
        st["mean_ms"] = window
        return st

    def time_sustained(self, min_s=0.1, per_launch_ms=None):
        """Mean ms per launch over at least min_s of back-to-back launches."""
        import torch
        n = max(10, math.ceil(min_s * 1e3 / max(per_launch_ms or 1.0, 1e-3)))
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(n):
            self.launch()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, n

    def time_graph(self, steps, min_warm_s=0.3):
        """Mean ms per launch when `steps` launches are captured once into a HIP
        graph and the graph is replayed (no per-launch host overhead)."""
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            self.launch(s.cuda_stream)              # eager warm-up on the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=s):
                for _ in range(steps):
                    self.launch(s.cuda_stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min_warm_s:
            graph.replay()
            torch.cuda.synchronize()
        rs = torch.cuda.current_stream()          # replay() launches on the current stream
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(rs)
        graph.replay()
        e1.record(rs)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def ref_check(self, max_flops=2e11):
        """The first run's C against the oracle: all of C when 2*M*N*K is at
        most max_flops, else the first rows that fit in that budget."""
        import numpy as np

        import gemm_inputs as gi
        import oracle
        from oracle import compare
        import torch
        p = self.p
        M, N, K = p["M"], p["N"], p["K"]
        torch.cuda.synchronize()
        self.launch(set_index=0)
        torch.cuda.synchronize()
        rows = M if 2.0 * M * N * K <= max_flops else max(1, int(max_flops / (2.0 * N * max(K, 1))))
        ref = oracle.gemm_ref(M, N, K, p["a_major"], p["b_major"], p["in_type"], p["A"], p["lda"], p["B"],
                              p["ldb"], rows=(0, rows), threads=oracle_threads())
        flat = self.c.cpu().numpy()
        if p["out_type"] != "f32":
            flat = flat.view(np.uint16)
        got = np.ascontiguousarray(gi.load(flat, M, N, p["c_first"], p["ldc"])[:rows])
        ok, info = compare.check(got, ref, p["out_type"], exact=(p.get("kind") == "int5"))
        return {"rows": rows, "of": M, "pass": bool(ok),
                **{k: v for k, v in info.items() if k in ("normwise_err", "mismatches", "nonfinite")}}

    def summary(self, st):
        import dense_gemm_engineering_run_amd as g
        tin = self.p["in_type"]
        ms = st["mean_ms"]
        tflops = self.flops / (ms * 1e-3) / 1e12
        return {
            "workload": self.desc,
            "config": g.gemm_config_describe(self.p["dtype"], g.gemm_last_config()),
            "ms": round(ms, 5),
            "median_ms": round(st["median_ms"], 5),
            "tflops": round(tflops, 2),
            "median_tflops": round(self.flops / (st["median_ms"] * 1e-3) / 1e12, 2),
            "pct_mfma_peak": round(100.0 * tflops / PEAK_TFLOPS[tin], 2),
            "hbm_gbs_algorithmic": round(self.bytes / (ms * 1e-3) / 1e9, 1),
            "iterations": st["n"],
            "buffer_sets": self.n_sets,
        }


def cpu_baseline(prob, target_s):
    """Time the oracle on the first R rows of the problem, R sized so the run
    takes about target_s seconds, and compare the GPU's rows with it."""
    import numpy as np

    import gemm_inputs as gi
    import oracle
    from oracle import compare
    p = prob.p
    threads = oracle_threads()
    M, N, K = p["M"], p["N"], p["K"]

    def run(rows):
        t = time.perf_counter()
        ref = oracle.gemm_ref(M, N, K, p["a_major"], p["b_major"], p["in_type"], p["A"], p["lda"],
                              p["B"], p["ldb"], rows=(0, rows), threads=threads)
        return ref, time.perf_counter() - t

    # Size the sample: a probe run, then rescale once more if the first sized
    # run is still well short of the target (the repack of B is a fixed cost).
    rows = min(M, 2 * threads)
    ref, t = run(rows)
    for _ in range(2):
        if t >= 0.6 * target_s or rows >= M:
            break
        rows = int(min(M, max(threads, rows * target_s / max(t, 1e-3))))
        rows = max(min(threads, M), rows // threads * threads)
        ref, t = run(rows)
    flat = prob.c.cpu().numpy()
    if p["out_type"] != "f32":
        flat = flat.view(np.uint16)
    got = np.ascontiguousarray(gi.load(flat, M, N, p["c_first"], p["ldc"])[:rows])
    ok, info = compare.check(got, ref, p["out_type"], exact=False)
    h = host_info()
    return {
        "value": round(2.0 * rows * N * K / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of C for the {prob.desc} problem (all {N} columns, "
                  f"full K={K}), fp64 sums on {threads} threads, {t:.1f} s",
        "seconds": round(t, 2),
        "nproc": h["nproc"],
        "cgroup_cpus": h["cgroup_cpus"],
        "cpu_model": h["cpu_model"],
        "sample_normwise_err": info.get("normwise_err"),
        "sample_pass": bool(ok),
    }


# ---------------------------------------------------------------- probes

def run_probes(which, min_s=0.15):
    """MFMA-only and HBM-read ceilings (include/mi355_gemm_probe.h)."""
    import numpy as np
    import torch

    import dense_gemm_engineering_run_amd as g
    import gemm_inputs as gi
    out = {"probe": which, "clocks_before": clocks()}
    s = torch.cuda.current_stream()
    if which in ("mfma", "all"):
        rng = np.random.Generator(np.random.PCG64(1024))
        shapes = [(g.PROBE_F16_16x16x32, "f16 16x16x32", "f16", "n01"),
                  (g.PROBE_F16_32x32x16, "f16 32x32x16", "f16", "n01"),
                  (g.PROBE_BF16_16x16x32, "bf16 16x16x32", "bf16", "n01")]
        grid = 1024                     # 4 workgroups of 4 waves per CU
        sink = torch.zeros(grid * 256, dtype=torch.float32, device="cuda")
        res = []
        for shape, label, tin, kind in shapes:
            vals = gi.cast(gi.draw(rng, 16 * 64, 8, kind), tin)
            ops = torch.from_numpy(np.ascontiguousarray(vals).view(np.int32).reshape(-1)).cuda()
            for rot in (1, 0):
                def go(iters):
                    st = g.gemm_probe_mfma(shape, rot, ops.data_ptr(), iters, grid, sink.data_ptr(), s.cuda_stream)
                    assert st == 0, g.gemm_status_str(st)
                go(200)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                go(2000)
                e1.record(s)
                torch.cuda.synchronize()
                iters = max(1000, int(2000 * min_s * 1e3 / max(e0.elapsed_time(e1), 1e-3)))
                go(iters)                  # warm at the measured length
                torch.cuda.synchronize()
                with ClockSampler() as cs:
                    e0.record(s)
                    go(iters)
                    e1.record(s)
                    torch.cuda.synchronize()
                ms = e0.elapsed_time(e1)
                flops = grid * 4.0 * iters * 64 * g.gemm_probe_mfma_flops(shape)
                tf = flops / (ms * 1e-3) / 1e12
                peak = PEAK_TFLOPS[tin]
                res.append({"mfma": label, "operands": "N(0,1), changing every MFMA" if rot else "one fixed pair", "ms": round(ms, 3), "tflops": round(tf, 1),
                            "pct_spec_peak": round(100 * tf / peak, 1),
                            "clock_mhz_implied": round(tf * 1e12 / (256 * 4 * g.gemm_probe_mfma_flops(shape) /
                                                                    _mfma_cycles(label)) / 1e6),
                            "sclk_sampled": cs.summary()})
                print(f"probe mfma {label} rotate={rot}: {tf:.1f} TF/s ({100 * tf / peak:.1f} % of spec)",
                      file=sys.stderr, flush=True)
        out["mfma"] = res
    if which in ("hbm", "all"):
        rows, row_bytes = 65536, 8192
        buf = torch.randn(rows * row_bytes // 2, dtype=torch.float16, device="cuda")
        sink = torch.zeros(rows * 1024 // 32768 * 512, dtype=torch.float32, device="cuda")
        res = []
        for seg in (128, 256, 512, 1024):
            def go():
                st = g.gemm_probe_hbm_read(buf.data_ptr(), rows, row_bytes, seg, sink.data_ptr(), s.cuda_stream)
                assert st == 0, g.gemm_status_str(st)
            for _ in range(5):
                go()
            torch.cuda.synchronize()
            ts = []
            for _ in range(30):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                go()
                e1.record(s)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            med = sorted(ts)[len(ts) // 2]
            tbs = rows * row_bytes / (med * 1e-3) / 1e12
            res.append({"segment_bytes": seg, "rows_per_workgroup": 32768 // seg, "median_us": round(med * 1e3, 1),
                        "tb_s": round(tbs, 2), "pct_hbm_peak": round(100 * tbs * 1e3 / HBM_PEAK_GBS, 1)})
            print(f"probe hbm seg {seg}: {tbs:.2f} TB/s", file=sys.stderr, flush=True)
        out["hbm"] = {"matrix": f"{rows} rows x {row_bytes} B (512 MiB), 3-stage 32 KB LDS ring, 8 waves",
                      "results": res}
    out["clocks_after"] = clocks()
    return out


def _mfma_cycles(label):
    """Issue cycles per MFMA on one SIMD at the spec rate: 1024 fp16 / bf16
    flops per SIMD per clock (2516.6 TFLOP/s = 256 CUs x 4 SIMDs x 1024 x 2.4 GHz)."""
    m = re.match(r"(\w+) (\d+)x(\d+)x(\d+)", label)
    a, b, c = int(m.group(2)), int(m.group(3)), int(m.group(4))
    return 2.0 * a * b * c / 1024


# ---------------------------------------------------------------- main

def parse_mnk(s):
    m = [int(x) for x in s.split(",")]
    if len(m) != 3 or min(m) < 0:
        raise argparse.ArgumentTypeError("--mnk takes M,N,K")
    return tuple(m)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed launches of the headline workload")
    ap.add_argument("--warmup", type=int, default=10, help="untimed launches before timing")
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--others", default="all",
                    help="comma list of extra workloads to time, 'all' (every other workload: the five "
                         "workloads' others, the fp16 K sweep, the stream-K / epilogue / batched / "
                         "unaligned rows and the eight-GPU shard shapes), 'sweep' (the fp16 K sweep), "
                         "'next' (those four rows), 'shard' (the shard shapes) or 'none'")
    ap.add_argument("--iterations", "--other-steps", dest="iterations", type=int, default=100,
                    help="timed launches of each other workload (and of --mnk)")
    ap.add_argument("--warmup_iterations", type=int, default=10)
    ap.add_argument("--sustained-ms", type=float, default=100.0,
                    help="also time at least this long of back-to-back launches for workloads under 5 ms")
    ap.add_argument("--use_cold_l2", action="store_true",
                    help=f"rotate {COLD_BYTES >> 20} MB or more of buffer copies so caches cannot hold them")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU oracle sample (0 disables it)")
    ap.add_argument("--mnk", type=parse_mnk, help="time one problem M,N,K instead of the named workloads")
    ap.add_argument("--a_major", default="k", choices=["k", "m"])
    ap.add_argument("--b_major", default="k", choices=["k", "n"])
    ap.add_argument("--c_major", default="n", choices=["n", "m"])
    ap.add_argument("--dtype", default="f32", choices=["f32", "f16_f32", "bf16_bf16", "f16_f16", "bf16_f32"])
    ap.add_argument("--integer_inputs", action="store_true", help="integers in [-5, 5] (exact check)")
    ap.add_argument("--skip_ref_check", action="store_true")
    ap.add_argument("--seed", type=int, default=1024)
    ap.add_argument("--probe", choices=["mfma", "hbm", "all"], help="measure the MFMA / HBM-read ceilings")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the engine runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the GEMM would shard along M or N with a broadcast of B, which is not built).",
              file=sys.stderr)
        sys.exit(2)

    clocks_before = clocks()
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_each_way": n * 4}), flush=True)
        return

    if args.probe:
        print(json.dumps(run_probes(args.probe)), flush=True)
        return

    if args.mnk:
        M, N, K = args.mnk
        kind = "int5" if args.integer_inputs else {"f32": "u11", "f16_f32": "n01", "f16_f16": "n01",
                                                    "bf16_bf16": "n002", "bf16_f32": "n002"}[args.dtype]
        desc = (f"{args.dtype} GEMM {M}x{N}x{K}, A {args.a_major}, B {args.b_major}, C {args.c_major}, "
                f"{ {'int5': 'integers in [-5,5]', 'u11': 'uniform(-1,1)', 'n01': 'normal(0,1)', 'n002': 'normal(0,0.02)'}[kind] }")
        spec = (M, N, K, args.a_major, args.b_major, args.c_major, args.dtype, kind, None, desc)
        pr = Problem("custom", spec=spec, opt={}, seed=args.seed, cold_l2=args.use_cold_l2)
        pr.p["kind"] = kind
        check = None if args.skip_ref_check else pr.ref_check()
        pr.warm(args.warmup_iterations, 0.3)
        with ClockSampler() as cs:
            st = pr.time(args.iterations)
        s = pr.summary(st)
        tin = pr.p["in_type"]
        rec = {"metric": "GEMM TFLOP/s (2MNK/t)", "value": s["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
               "steps": args.iterations, "warmup": args.warmup_iterations, "ms_per_step": s["ms"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": tin,
               "data": "synthetic", "config": {"workload": desc, "kernel_config": s["config"],
                                               "cold_l2_buffer_sets": pr.n_sets},
               "median_ms": s["median_ms"], "pct_mfma_peak": s["pct_mfma_peak"],
               "hbm_gbs_algorithmic": s["hbm_gbs_algorithmic"], "ref_check": check,
               "clocks": {"before": clocks_before, "during_sclk": cs.summary(), "after": clocks()}}
        print(json.dumps(rec), flush=True)
        return

    print(f"bench: preparing {args.workload}", file=sys.stderr, flush=True)
    head = Problem(args.workload, cold_l2=args.use_cold_l2)
    head.warm(args.warmup)
    with ClockSampler() as cs:
        st = head.time(args.steps)
    ms = st["mean_ms"]
    s = head.summary(st)
    print(f"bench: {args.workload} {s['ms']} ms (median {s['median_ms']}) {s['tflops']} TFLOP/s",
          file=sys.stderr, flush=True)
    tin = head.p["in_type"]
    achieved = head.flops / (ms * 1e-3) / 1e12
    traffic = read_traffic(args.workload)

    record = {
        "metric": METRIC,
        "value": round(achieved, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": tin,
        "data": "synthetic",
        "config": {"workload": head.desc, "M": head.p["M"], "N": head.p["N"], "K": head.p["K"],
                   "a_major": head.p["a_major"], "b_major": head.p["b_major"],
                   "c_major": head.p["c_major"], "kernel_config": s["config"],
                   "cold_l2_buffer_sets": head.n_sets},
        "median_ms": s["median_ms"],
        "pct_mfma_peak": s["pct_mfma_peak"],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_TFLOPS[tin],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[tin], 4),
                     "traffic": traffic},
        "host": host_info(),
    }

    if args.cpu_seconds > 0:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        record["cpu_baseline"] = cpu_baseline(head, args.cpu_seconds)

    default_others = [w for w in WORKLOADS if w != args.workload]
    if args.others == "none":
        others = []
    elif args.others == "all":
        others = default_others
    elif args.others == "sweep":
        others = SWEEP
    elif args.others == "next":
        others = NEXT_ROWS
    elif args.others == "shard":
        others = SHARD
    else:
        others = [w for w in args.others.split(",") if w]
    if others:
        record["workloads"] = {}
        del head
        torch.cuda.empty_cache()
        for w in others:
            print(f"bench: {w}", file=sys.stderr, flush=True)
            pr = Problem(w, cold_l2=args.use_cold_l2)
            pr.warm(args.warmup_iterations, 0.3)
            st = pr.time(args.iterations)
            rec = pr.summary(st)
            if args.sustained_ms > 0 and st["mean_ms"] < 5.0:
                sms, n = pr.time_sustained(args.sustained_ms * 1e-3, st["mean_ms"])
                rec["sustained_ms"] = round(sms, 5)
                rec["sustained_launches"] = n
                rec["sustained_tflops"] = round(pr.flops / (sms * 1e-3) / 1e12, 2)
            if st["mean_ms"] < 0.05:
                # launch-bound: also time back-to-back launches replayed from a HIP graph
                gms = pr.time_graph(max(args.iterations, 100))
                rec["graph_ms"] = round(gms, 5)
                rec["graph_tflops"] = round(pr.flops / (gms * 1e-3) / 1e12, 2)
            record["workloads"][w] = rec
            del pr
            torch.cuda.empty_cache()

    record["clocks"] = {"before": clocks_before, "during_headline_sclk": cs.summary(), "after": clocks()}
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
