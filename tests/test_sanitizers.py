"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer runs.

* The CPU oracle (oracle/oracle.c) built with gcc -fsanitize=address,undefined
  and driven through every entry point on small seeded problems
  (tests/sanitize/oracle_driver.c).
* The C ABI's argument validation and workspace sizing: the HIP library's
  sources built with the sanitizers on their host code only, linked into a
  host program (tests/sanitize/abi_driver.cpp) that calls every entry point
  with arguments it must reject before any launch, and sizes the largest
  shapes the checks accept.  No GPU is touched.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_attention_token_dsa_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-pthread", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "oracle"), "-o", exe,
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "oracle sanitizer driver ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm toolchain not found")
def test_abi_validation_under_asan_ubsan(tmp_path):
    from sparse_attention_token_dsa_amd import build
    objs = []
    cmds = []
    for src in build.SOURCES:
        o = str(tmp_path / src.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
                     "-fno-honor-nans", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                     "-Xarch_host", "-fno-omit-frame-pointer",
                     "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", o])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(_run, cmds))
    drv = str(tmp_path / "abi_driver.o")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(SAN, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX, "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "abi sanitizer driver ok" in r.stdout
