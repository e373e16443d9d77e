"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU oracle and
of the C ABI's host code (CPU only; no device is touched).

  * oracle/moe_oracle.c with tests/sanitize/oracle_driver.c (gcc): every
    oracle function on small seeded layers and the edge cases;
  * the library's sources with tests/sanitize/abi_host_driver.cpp (hipcc,
    the sanitizers on the host pass only): argument checks, capacity, row
    bounds and workspace sizing over valid, invalid and extreme parameters.
Each driver must exit 0 with no sanitizer report.
"""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_mixture_experts_gemm_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="moe_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r.stdout


def test_oracle_under_asan_ubsan(tmp):
    exe = os.path.join(tmp, "oracle_driver")
    run(["gcc", "-g", "-O1", "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wall", "-Wno-unknown-pragmas", "-o", exe,
         os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    assert "oracle driver ok" in run([exe], env=ENV)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_abi_host_code_under_asan_ubsan(tmp):
    host_san = []
    for f in ("address", "undefined"):
        host_san += ["-Xarch_host", "-fsanitize=" + f]
    host_san += ["-Xarch_host", "-fno-omit-frame-pointer"]
    srcs = [os.path.join(CSRC, f) for f in
            ("route.hip", "dispatch.hip", "expert_gemm.hip", "combine.hip", "backward.hip", "moe_api.cpp")]
    srcs.append(os.path.join(SAN, "abi_host_driver.cpp"))

    def comp(src):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        run(["hipcc", "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", *host_san, "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(comp, srcs))
    exe = os.path.join(tmp, "abi_driver")
    run(["hipcc", "--offload-arch=gfx950", *host_san, "-o", exe, *objs])
    out = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1"))
    assert "abi host driver ok" in out
