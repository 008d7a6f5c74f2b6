"""Memory and undefined-behaviour checks on the CPU: the oracle (C) and the host side of the HIP
library (argument checks, shape planning, workspace layout) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through every entry point, malformed inputs included.

  * oracle/sanitize_driver.c: every oracle function on small seeded inputs (trees, chains,
    malformed trees, empty contexts, out-of-range tokens, exact ties, recurrent commits at
    accepted_len -1, 0, K-1, K and with a bad node id, every bf16 pattern through W12), built
    with gcc -fsanitize=address,undefined in one unit with the oracle source.
  * tree_verification_skinny_amd/csrc/host_sanitize_driver.c: workspace sizes over batches, draft
    sizes and page budgets, and every refusal path of the C ABI (no GPU is touched), against a
    libspecverify whose host code is built with the sanitizers (hipcc, each -fsanitize after
    -Xarch_host, so the device code is built as usual).
A sanitizer report aborts the driver (-fno-sanitize-recover=all), failing the test.
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.slow

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _have(tool):
    return shutil.which(tool) is not None or os.path.exists(tool)


def test_oracle_under_asan_ubsan(tmp_path):
    if not _have("gcc"):
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_san")
    src = os.path.join(ROOT, "oracle", "sanitize_driver.c")
    r = subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-fopenmp", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"), src, "-o", exe,
                        "-lm"], capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("gcc without the sanitizer runtimes")
    assert r.returncode == 0, r.stderr
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all cases clean" in run.stdout


def test_library_host_code_under_asan_ubsan(tmp_path):
    from tree_verification_skinny_amd import build as b
    clang = "/opt/rocm/llvm/bin/clang"
    if not (_have(b.HIPCC) and _have(clang)):
        pytest.skip("no hipcc / clang")
    san = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]

    def comp(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([b.HIPCC, *b.FLAGS, *san, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, b.sources()))
    lib = str(tmp_path / "libspecverify.so")
    subprocess.run([b.HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", lib, *objs], check=True)
    exe = str(tmp_path / "host_san")
    drv = os.path.join(ROOT, "tree_verification_skinny_amd", "csrc", "host_sanitize_driver.c")
    r = subprocess.run([clang, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                        drv, "-L", str(tmp_path), "-lspecverify", f"-Wl,-rpath,{tmp_path}", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all cases clean" in run.stdout
