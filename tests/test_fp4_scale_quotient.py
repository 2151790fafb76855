"""The kernel's block-scale quotient equals IEEE division by 6 (no GPU).

The FP4 scale is E4M3(fl32(blockmax / 6)). The kernel forms the quotient as
q0 = fl32(x * fl32(1/6)), then q = fma(fma(-q0, 6, x), fl32(1/6), q0): one
correction from the exact remainder. This test runs a small C program over
every finite non-negative binary32 x (about 2^31 patterns, some 20 s): q
must equal the IEEE quotient x / 6 for every x >= 6 * 2^-126, and below that
both must be smaller than 2^-10, half the smallest E4M3 step, so the scale
code is 0 either way."""

import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
int main(void) {
  const float c = 1.0f / 6.0f;
  unsigned long long bad = 0, small = 0;
  for (uint32_t u = 0; u < 0x7F800000u; ++u) {
    float x, w, q;
    memcpy(&x, &u, 4);
    w = x / 6.0f;
    const float q0 = x * c;
    q = fmaf(fmaf(-q0, 6.0f, x), c, q0);
    uint32_t a, b;
    memcpy(&a, &q, 4);
    memcpy(&b, &w, 4);
    if (u >= 0x01400000u) {
      if (a != b) ++bad;
    } else if (!(q < 0x1p-10f && w < 0x1p-10f)) {
      ++small;
    }
  }
  printf("%llu %llu\n", bad, small);
  return 0;
}
"""


def _has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_div6_equals_ieee_quotient(tmp_path):
    src = tmp_path / "div6.c"
    exe = tmp_path / "div6"
    src.write_text(SRC)
    # -ffp-contract=off: only the explicit fmaf calls fuse; -mfma makes them
    # the hardware instruction (glibc's software fmaf is exact too, slower)
    flags = ["-O2", "-ffp-contract=off", "-fno-fast-math"] + (["-mfma"] if _has_fma() else [])
    subprocess.run(["gcc", *flags, "-o", str(exe), str(src), "-lm"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True,
                         timeout=1200, env=dict(os.environ)).stdout.split()
    assert out == ["0", "0"], out
