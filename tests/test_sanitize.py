"""The host-side logic and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

* The library's sources are compiled for the host only (hipcc
  --cuda-host-only: argument checks, config selection, the tuning-table
  parser, workspace planning, the entry points' checks; no device code) with
  both sanitizers on host code, and linked with tests/sanitize/host_driver.cpp,
  which drives every C-ABI path that ends before a kernel launch.
* oracle/oracle_gemm.c is compiled with gcc and both sanitizers and linked
  with tests/sanitize/oracle_driver.c, which runs every oracle entry point and
  checks its results against a direct double loop.
Any sanitizer report stops the program with a non-zero status."""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_gemm_engineering_run_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-g", "-O1", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
          os.path.join(ROOT, "oracle", "oracle_gemm.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=SAN_ENV)
    assert "oracle driver: 0 failure(s)" in r.stderr, r.stderr[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_library_logic_under_sanitizers(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", "-std=c++17", "-g", "-O1",
             "-Wno-inline-asm", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, *san, "-c", src, "-o", obj])
        return obj
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    # Host-only objects still name their files' device-code blobs; the driver
    # never loads device code (every call stops before a launch), so
    # zero-filled arrays stand in for the blobs the objects reference.
    nm = _run(["nm", "-u", *objs]).stdout.split()
    blobs = sorted({w for w in nm if w.startswith("__hip_fatbin_")})
    stub = tmp_path / "blobs.c"
    stub.write_text("".join(f"const char {b}[16] = {{0}};\n" for b in blobs))
    _run(["gcc", "-c", str(stub), "-o", str(tmp_path / "blobs.o")])
    objs.append(str(tmp_path / "blobs.o"))
    exe = str(tmp_path / "host_san")
    _run([HIPCC, "--offload-arch=gfx950", *san, *objs, "-o", exe])
    table = os.path.join(ROOT, "dense_gemm_engineering_run_amd", "tuning", "table.txt")
    r = _run([exe, table, str(tmp_path)], env=SAN_ENV)
    assert "host driver: 0 failure(s)" in r.stderr, r.stderr[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
