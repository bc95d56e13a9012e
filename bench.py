"""Benchmark of the MI355X GEMM library.

One step = one GEMM C = A * B^T through the C ABI on inputs already resident
in HBM.  The headline workload is the fp32 SGEMM M=N=K=8192 with A m-major,
B n-major and C n-major (the size and layouts the CuTe DSL Ampere SGEMM
example is run with in its docstring); the value is 2*M*N*K / t in TFLOP/s,
timed with HIP events on the stream the kernels are launched on.

The JSON line also carries:
  roofline      achieved TFLOP/s of the GEMM kernel against the MI355X dense
                MFMA peak for its input type, plus the HBM traffic measured
                with rocprofv3 counters (profiles/hbm_traffic.md) when that
                measurement matches the current kernel sources;
  cpu_baseline  the CPU oracle timed on a bounded row sample of the same
                problem on this host's cores, with the GPU rows compared to it;
  workloads     the other measured GEMM workloads (fp16 4096^3 in all eight
                layouts, fp32 1024x512x256, fp32 4095x2049x1028 ragged, bf16
                65536x256x4096 tall-skinny with its HBM GB/s), and the rows
                built on the plain GEMM: stream-K, the fused epilogue, the
                strided-batched mode, operands that are not 16-byte aligned.
"""
import argparse
import hashlib
import glob
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (2MNK/t) + % of MFMA peak, fp32 8192³ and fp16 4096³"
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}   # MI355X dense MFMA
HBM_PEAK_GBS = 8000.0

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
# strided-batched mode, and
# the element-by-element path for operands that are not 16-byte aligned.
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
OPTIONS = {
    "fp32_ragged_streamk": {"config": "f32 128x128x32 w2x2 mfma32 s2 dma sk"},
    "fp32_8192_epilogue": {"epilogue": "bias_relu"},
    "fp32_ragged_streamk_epilogue": {"config": "f32 128x128x32 w2x2 mfma32 s2 dma sk", "epilogue": "bias_relu"},
    "fp16_batched_64x512": {"batch": 64},
    "fp32_ragged_unaligned": {"lda": 1029, "ldb": 1029},
}
NEXT_ROWS = list(OPTIONS)

HEADLINE = "fp32_8192"


def kernel_source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "dense_gemm_engineering_run_amd", "csrc", "*"))):
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


def sclk_mhz():
    """Current shader clock from sysfs (the entry marked '*'), if readable."""
    for p in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            for line in open(p):
                if "*" in line:
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    if m:
                        return int(m.group(1))
        except OSError:
            pass
    return None


class Problem:
    def __init__(self, name, seed=1024):
        import numpy as np
        import torch

        import dense_gemm_engineering_run_amd as g
        import gemm_inputs as gi
        M, N, K, a, b, c, dtype, kind, ldc, desc = WORKLOADS[name]
        opt = OPTIONS.get(name, {})
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
        self.a, self.b = dev(p["A"]), dev(p["B"])
        outer = N if p["c_first"] else M
        ct = torch.float32 if p["out_type"] == "f32" else torch.int16
        self.sc = outer * p["ldc"]
        self.c = torch.zeros(self.sc * self.batch, dtype=ct, device="cuda")
        self.stream = torch.cuda.current_stream()
        self.args = (M, N, K, a, b, c, p["dtype"], self.a.data_ptr(), self.b.data_ptr(),
                     self.c.data_ptr(), p["lda"], p["ldb"], p["ldc"], self.stream.cuda_stream)
        self.config = -1
        if "config" in opt:
            names = [g.gemm_config_describe(p["dtype"], i) for i in range(g.gemm_num_configs(p["dtype"]))]
            self.config = names.index(opt["config"])
        self.ws_bytes = g.gemm_workspace_size(M, N, K, a, b, c, p["dtype"], self.config)
        self.ws = torch.zeros(max(self.ws_bytes, 16) // 4, dtype=torch.int32, device="cuda")
        self.epi = None
        if opt.get("epilogue") == "bias_relu":
            self.bias = torch.linspace(-1, 1, N, device="cuda")
            self.epi = g.Epilogue(1.0, 0.0, self.bias.data_ptr(), g.GEMM_ACT_RELU)
        eb = gi.ELEM_BYTES[p["in_type"]]
        eo = gi.ELEM_BYTES[p["out_type"]]
        self.flops = 2.0 * M * N * K * self.batch
        self.bytes = float(M * K * eb + N * K * eb + M * N * eo) * self.batch

    def launch(self, stream=None):
        import dense_gemm_engineering_run_amd as g
        args = self.args if stream is None else self.args[:-1] + (stream,)
        if self.batch > 1:
            st = g.gemm_run_batched(*args[:-1], self.batch, len(self.p["A"]), len(self.p["B"]),
                                    self.sc, args[-1])
        elif self.epi is not None or self.config >= 0 or self.ws_bytes:
            st = g.gemm_run_ex(*args[:-1], self.epi, self.ws.data_ptr(), self.ws_bytes, args[-1],
                               self.config)
        else:
            st = g.gemm_run(*args)
        if st != 0:
            raise RuntimeError(g.gemm_status_str(st))

    def time(self, steps, warmup, min_warm_s=0.0):
        """Mean ms per launch over `steps` launches, after `warmup` untimed
        launches and, with min_warm_s, enough further launches to keep the GPU
        busy that long first (clocks ramp up over tens of ms after idle)."""
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
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for _ in range(steps):
            self.launch()
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps      # ms per launch

    def time_graph(self, steps, min_warm_s=0.3):
        """Mean ms per launch when `steps` launches are captured once into a HIP
        graph and the graph is replayed (no per-launch host overhead)."""
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            self.launch()                           # eager warm-up on the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=s):
                for _ in range(steps):
                    self.launch(s.cuda_stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min_warm_s:
            graph.replay()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def summary(self, ms):
        import dense_gemm_engineering_run_amd as g
        tin = self.p["in_type"]
        tflops = self.flops / (ms * 1e-3) / 1e12
        return {
            "workload": self.desc,
            "config": g.gemm_config_describe(self.p["dtype"], g.gemm_last_config()),
            "ms": round(ms, 5),
            "tflops": round(tflops, 2),
            "pct_mfma_peak": round(100.0 * tflops / PEAK_TFLOPS[tin], 2),
            "hbm_gbs_algorithmic": round(self.bytes / (ms * 1e-3) / 1e9, 1),
        }


def cpu_baseline(prob, target_s):
    """Time the oracle on the first R rows of the problem, R sized so the run
    takes about target_s seconds, and compare the GPU's rows with it."""
    import numpy as np

    import oracle
    from oracle import compare
    p = prob.p
    threads = min(16, len(os.sched_getaffinity(0)))
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
    import gemm_inputs as gi
    got = np.ascontiguousarray(gi.load(flat, M, N, p["c_first"], p["ldc"])[:rows])
    ok, info = compare.check(got, ref, p["out_type"], exact=False)
    return {
        "value": round(2.0 * rows * N * K / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of C for the {prob.desc} problem (all {N} columns, "
                  f"full K={K}), fp64 triple loop on {threads} threads, {t:.1f} s",
        "seconds": round(t, 2),
        "sample_normwise_err": info.get("normwise_err"),
        "sample_pass": bool(ok),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--others", default="all",
                    help="comma list of extra workloads to time, 'all' (the five workloads' "
                         "others and the stream-K / epilogue / batched / unaligned rows), "
                         "'sweep' (the fp16 K sweep), 'next' (those four rows) or 'none'")
    ap.add_argument("--other-steps", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU oracle sample (0 disables it)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the engine runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the GEMM would shard along M or N with a broadcast of B, which is not built).",
              file=sys.stderr)
        sys.exit(2)

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

    print(f"bench: preparing {args.workload}", file=sys.stderr, flush=True)
    head = Problem(args.workload)
    ms = head.time(args.steps, args.warmup)
    s = head.summary(ms)
    print(f"bench: {args.workload} {s['ms']} ms {s['tflops']} TFLOP/s", file=sys.stderr, flush=True)
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
                   "c_major": head.p["c_major"], "kernel_config": s["config"]},
        "pct_mfma_peak": s["pct_mfma_peak"],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_TFLOPS[tin],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[tin], 4),
                     "traffic": traffic},
        "sclk_mhz": sclk_mhz(),
    }

    if args.cpu_seconds > 0:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        record["cpu_baseline"] = cpu_baseline(head, args.cpu_seconds)

    default_others = [w for w in WORKLOADS if w != args.workload and not w.startswith("fp16_sweep")]
    if args.others == "none":
        others = []
    elif args.others == "all":
        others = default_others
    elif args.others == "sweep":
        others = [w for w in WORKLOADS if w.startswith("fp16_sweep")]
    elif args.others == "next":
        others = NEXT_ROWS
    else:
        others = [w for w in args.others.split(",") if w]
    if others:
        record["workloads"] = {}
        del head
        torch.cuda.empty_cache()
        for w in others:
            print(f"bench: {w}", file=sys.stderr, flush=True)
            pr = Problem(w)
            ms = pr.time(args.other_steps, args.warmup, 0.3)
            rec = pr.summary(ms)
            if ms < 0.05:
                # launch-bound: also time back-to-back launches replayed from a HIP graph
                gms = pr.time_graph(max(args.other_steps, 100))
                rec["graph_ms"] = round(gms, 5)
                rec["graph_tflops"] = round(pr.flops / (gms * 1e-3) / 1e12, 2)
            record["workloads"][w] = rec
            del pr
            torch.cuda.empty_cache()

    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
