"""The C ABI used from plain C: `tests/c_abi/arfuse_c_demo.c` links only
libarfuse.so, the HIP runtime and the oracle (no Python, no PyTorch in its
process), runs fused calls on device buffers from hipMalloc and checks them
against the oracle. The CPU tests build it and compile the public header as
C99 and C++; the GPU test runs it."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "arfuse_c_demo.c")
LIBDIR = os.path.join(ROOT, "reduce_residual_rmsnorm_amd", "lib")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_demo(out: str) -> str:
    if not os.path.exists(os.path.join(LIBDIR, "libarfuse.so")):
        pytest.fail("libarfuse.so is not built (run reduce_residual_rmsnorm_amd/build.py)")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "oracle"), "-ffp-contract=off", SRC,
           os.path.join(ROOT, "oracle", "arfuse_oracle.c"), "-o", out,
           "-L", LIBDIR, "-larfuse", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def test_demo_builds_against_the_c_abi(tmp_path):
    build_demo(str(tmp_path / "arfuse_c_demo"))


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++11")])
def test_header_is_plain_c_and_cxx(tmp_path, lang, std):
    src = tmp_path / "h.c"
    src.write_text('#include "arfuse.h"\nint main(void) { return arfuse_version() == ARFUSE_VERSION ? 0 : 1; }\n')
    comp = "gcc" if lang == "c" else "g++"
    r = subprocess.run([comp, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-x", lang, "-I", os.path.join(ROOT, "include"), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.gpu
def test_demo_runs_on_the_gpu(tmp_path):
    exe = build_demo(str(tmp_path / "arfuse_c_demo"))
    print("[gpu-case] c demo", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "[c-demo] ok" in r.stdout
