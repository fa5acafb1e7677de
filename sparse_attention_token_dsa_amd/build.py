"""Build the gfx950 HIP library ``libsaindexer.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libsaindexer.so")
SOURCES = ["abi.hip", "scan.hip", "scan8.hip", "topk.hip", "pool.hip", "prefill.hip",
           "lisa.hip", "tidy.hip"]

# Packed fp32 ops are switched off for device code: hipcc -O3 would otherwise
# form v_pk_* fp32 instructions on its own.  -fno-honor-nans: inputs are
# finite by contract, so max(x, 0) needs no NaN quieting.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# The prefill kernel's and the FP8 scan's epilogues read every MFMA result with
# VALU: results in VGPRs save one accumulator-to-VGPR move per element.  (The
# bf16 scan kernels keep the default: there it would cost occupancy.)
FILE_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "scan8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              # the key scans' 64-step loops unroll completely (waits stay
              # exact), including the one that pools the keys as well
              "scan.hip": ["-mllvm", "-pragma-unroll-threshold=200000"]}
_NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d): %s\n%s" % (res.returncode, " ".join(cmd), msgs))
    return msgs


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link one shared library; returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    with tempfile.TemporaryDirectory(prefix="sa_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(s, []), "-I", INCLUDE, "-c",
                 os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
            msgs = list(ex.map(_run, cmds))
        tmp = LIB + ".tmp%d" % os.getpid()
        msgs.append(_run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]))
    if verbose and any(m.strip() for m in msgs):
        print("\n".join(m for m in msgs if m.strip()))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
