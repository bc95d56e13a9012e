"""Build libmi355_gemm.so (the HIP GEMM library) in-tree for gfx950.

Every source under csrc/ is compiled with hipcc for --offload-arch=gfx950 into
_build/, in parallel, and linked into ``libmi355_gemm.so`` beside this file.
Packed-fp32 instructions are disabled for all device code.  The build fails if
a kernel spills more than SPILL_LIMIT bytes per lane to scratch memory (the
compiler's resource-usage remarks are checked): accumulators spilled around a
GEMM main loop cost several times its runtime.  The limit admits the few
values (up to 9) that the plain 16-bit-output epilogues of the 256x256 tiles
park in scratch at the loop exit, which cost nothing measurable.
"""
import glob
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmi355_gemm.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SPILL_LIMIT = 40        # bytes of scratch per lane
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wno-inline-asm",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _spills(remarks):
    """(function, scratch bytes per lane) for every kernel whose ScratchSize in
    hipcc's kernel-resource-usage remarks exceeds SPILL_LIMIT."""
    bad, fn = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            fn = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > SPILL_LIMIT:
            bad.append((fn, int(m.group(1))))
    return bad


def _includes(path, seen):
    """Local headers that `path` includes, transitively (quoted #includes
    found in csrc/ or include/)."""
    for name in re.findall(r'^\s*#\s*include\s+"([^"]+)"', open(path).read(), flags=re.M):
        for d in (CSRC, os.path.join(ROOT, "include")):
            h = os.path.join(d, name)
            if os.path.exists(h) and h not in seen:
                seen.add(h)
                _includes(h, seen)
    return seen


def _fresh(src, obj):
    """True when obj is newer than src and than every local header it includes."""
    if not os.path.exists(obj):
        return False
    t = os.path.getmtime(obj)
    return all(os.path.getmtime(d) < t for d in [src, *_includes(src, set())])


def _compile(src, verbose, incremental=False):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and _fresh(src, obj):
        return obj
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    bad = _spills(out)
    if bad:
        raise RuntimeError(f"register spills in {src}: " + ", ".join(f"{f} ({b} B/lane)" for f, b in bad))
    if verbose:
        print("\n".join(l for l in out.splitlines() if "remark" not in l))
    return obj


def build(verbose=False, jobs=None, incremental=False):
    """Compile every source (incremental: only those whose object is older
    than the source or a header) and link the library."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, incremental), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv)
