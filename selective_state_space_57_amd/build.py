"""Build libssm57.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree next to this file."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("ssm_scan.hip", "ssm_conv_scan.hip", "ssm_complex_scan.hip",
                                                  "ssm_scan_bwd.hip", "ssm_ssd.hip")]
INC = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssm57.so")
# the issue-rate probe that bench.py runs beside the scan (not part of the scan library's ABI)
PROBE_SRC = os.path.join(HERE, "csrc", "issue_probe.hip")
PROBE_LIB = os.path.join(HERE, "libssm57_probe.so")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-Wall",
    # packed FP32 (v_pk_*_f32) stays off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every translation unit (in parallel), link libssm57.so, and build the issue-rate probe library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tag = ".tmp%d" % os.getpid()
    objs = [os.path.splitext(s)[0] + tag + ".o" for s in SRCS]
    try:
        with ThreadPoolExecutor(len(SRCS) + 1) as ex:
            probe = ex.submit(_run, [hipcc] + FLAGS + ["-shared", PROBE_SRC, "-o", PROBE_LIB + tag], verbose)
            list(ex.map(lambda so: _run([hipcc] + FLAGS + ["-I", INC, "-c", so[0], "-o", so[1]], verbose),
                        zip(SRCS, objs)))
            probe.result()
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", LIB + tag], verbose)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    os.replace(LIB + tag, LIB)
    os.replace(PROBE_LIB + tag, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
