"""Build libmi355attn.so (gfx950) in-tree with hipcc.

    python -m long_context_exact_fwd_amd.build [--jobs N]

Every HIP source under csrc/ is compiled for gfx950 and linked into
long_context_exact_fwd_amd/libmi355attn.so. The same sources compiled with
-DATTN_DEBUG give libmi355attn_debug.so: the same C ABI, with every LDS
access made through the checked helpers bounds-checked on the device and a
synchronising check after each call (ATTN_ERR_DEBUG_CHECK). The measurement
probes under csrc/probe/ (not part of the attention library) go into
libmi355probe.so.
Packed fp32 VALU instructions are disabled (``-packed-fp32-ops``); hipcc's
host pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmi355attn.so")
DEBUG_LIB = os.path.join(PKG, "libmi355attn_debug.so")
PROBE_LIB = os.path.join(PKG, "libmi355probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(PKG, "..", "include"),
]


def _compile(job) -> str:
    src, debug = job
    obj = os.path.join(BUILD, os.path.basename(src) + (".debug.o" if debug else ".o"))
    cmd = [HIPCC, *CFLAGS, *(["-DATTN_DEBUG"] if debug else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(jobs: int = 0, debug: bool = True) -> str:
    """Builds libmi355attn.so and libmi355probe.so, and libmi355attn_debug.so unless debug is False."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probes = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))
    jobs_list = [(f, False) for f in srcs + probes] + ([(f, True) for f in srcs] if debug else [])
    jobs = jobs or min(8, len(jobs_list), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, jobs_list))
    n, m = len(srcs), len(srcs) + len(probes)
    _link(objs[:n], LIB)
    _link(objs[n:m], PROBE_LIB)
    if debug:
        _link(objs[m:], DEBUG_LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--no-debug", action="store_true", help="skip libmi355attn_debug.so")
    a = ap.parse_args(argv)
    print(build(a.jobs, debug=not a.no_debug))
    return 0


if __name__ == "__main__":
    sys.exit(main())
