"""Build the gfx950 shared library ``lib/libarfuse.so`` with hipcc, in-tree.

    python reduce_residual_rmsnorm_amd/build.py

(Run it as a file: importing the package loads the library it builds.)

The row-kernel instances are compiled per rank count N (``arfuse_rows.hip``
with ``-DARFUSE_N=1..8``) in parallel with the host ABI unit
(``arfuse.hip``), then linked into one library.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRC = os.path.join(CSRC, "arfuse.hip")
ROWS = os.path.join(CSRC, "arfuse_rows.hip")
DEVICE = os.path.join(CSRC, "arfuse_device.hpp")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libarfuse.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the rank sum must be plain IEEE adds in order; division and sqrt correctly rounded
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall",
    "-Wno-unused-function",
    # the arrival lambda captures the peer-row pointers by value for the
    # flag and sentinel instances; the plain instances leave them unused
    "-Wno-unused-lambda-capture",
]


def _jobs():
    units = [(SRC, [], "arfuse")]
    units += [(ROWS, ["-DARFUSE_N=%d" % n], "rows_n%d" % n) for n in range(1, 9)]
    return units


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="arfuse_build_") as tmpdir:
        procs = []
        for src, defs, name in _jobs():
            obj = os.path.join(tmpdir, name + ".o")
            cmd = [HIPCC, *FLAGS, *defs, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            # Each compiler writes its diagnostics to a file of its own: a pipe
            # that is read only after the earlier units finish fills up and
            # stalls its compiler, which turns the parallel build serial.
            log = open(os.path.join(tmpdir, name + ".log"), "w+")
            procs.append((subprocess.Popen(cmd, stdout=log, stderr=subprocess.STDOUT), log, obj))
        objs = []
        failed = False
        for p, log, obj in procs:
            p.wait()
            log.seek(0)
            out = log.read()
            log.close()
            if p.returncode != 0:
                sys.stderr.write(out)
                failed = True
            elif verbose and out:
                sys.stdout.write(out)
            objs.append(obj)
        if failed:
            raise RuntimeError("hipcc failed building %s" % CSRC)
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking %s" % LIB)
        os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [SRC, ROWS, DEVICE, os.path.join(INCLUDE, "arfuse.h")]
    return any(os.path.getmtime(p) > t for p in deps)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
