"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

A small C driver calls every oracle entry point on buffers allocated to
their exact sizes (so a read or write one element past a tensor is caught),
over rank counts 1..8, ragged row widths, t = 0, every fusion pattern, FP4
and FP8, the LL unpack and the sentinel count, and the bad-argument returns.
It is built with gcc, -fsanitize=address,undefined and no recovery: any
finding aborts the run. Host code only: nothing here touches the GPU
library."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "arfuse_oracle.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)st; }
static float frand(void) { return ((int32_t)(rnd() & 0xFFFFFF) - 0x800000) / 1048576.0f; }

static uint16_t* bf16_tensor(int64_t n) {
  uint16_t* p = (uint16_t*)malloc((size_t)(n ? n : 1) * 2);
  for (int64_t i = 0; i < n; ++i) p[i] = oracle_bf16_rne(frand());
  return p;
}

static int run_case(int n, int64_t t, int64_t d, int residual, int gamma, int fp4, int fp8) {
  const int64_t e = t * d;
  const uint16_t* parts[8];
  uint16_t* own[8];
  for (int i = 0; i < n; ++i) { own[i] = bf16_tensor(e); parts[i] = own[i]; }
  uint16_t* res = residual ? bf16_tensor(e) : NULL;
  float* g = NULL;
  if (gamma) { g = (float*)malloc((size_t)d * 4); for (int64_t j = 0; j < d; ++j) g[j] = 0.5f + (rnd() & 1023) / 1024.0f; }
  size_t ee = (size_t)(e ? e : 1);
  uint16_t* rout = (uint16_t*)malloc(ee * 2);
  float* y32 = gamma ? (float*)malloc(ee * 4) : NULL;
  uint16_t* out = gamma ? (uint16_t*)malloc(ee * 2) : NULL;
  uint8_t* codes = (gamma && fp4) ? (uint8_t*)malloc(ee / 2 + 1) : NULL;
  uint8_t* scales = (gamma && fp4) ? (uint8_t*)malloc(ee / 16 + 1) : NULL;
  uint8_t* f8 = (gamma && fp8) ? (uint8_t*)malloc(ee) : NULL;
  int rc = oracle_fused(parts, n, res, g, 1e-5f, t, d, rout, y32, out, codes, scales, f8, 3.0f);
  if (rc == 0 && gamma && res) {
    rc |= oracle_allreduce_rmsnorm(parts, n, res, g, 1e-5f, t, d, rout, y32, out, codes, scales);
    float* h = (float*)malloc(ee * 4);
    rc |= oracle_rank_sum_residual(parts, n, res, t, d, h);
    rc |= oracle_rmsnorm_rows(h, g, 1e-5f, t, d, y32);
    free(h);
  }
  for (int i = 0; i < n; ++i) free(own[i]);
  free(res); free(g); free(rout); free(y32); free(out); free(codes); free(scales); free(f8);
  return rc;
}

int main(void) {
  const int64_t ds[] = {16, 48, 1040};
  const int64_t ts[] = {0, 1, 3};
  int cases = 0;
  for (int n = 1; n <= 8; ++n)
    for (int a = 0; a < 3; ++a)
      for (int b = 0; b < 3; ++b)
        for (int pat = 0; pat < 6; ++pat) {
          const int residual = pat != 1, gamma = pat != 2, fp4 = pat == 3, fp8 = pat == 4;
          if (run_case(n, ts[b], ds[a], residual, gamma, fp4, fp8) != 0) {
            fprintf(stderr, "case n=%d t=%lld d=%lld pattern %d failed\n", n, (long long)ts[b],
                    (long long)ds[a], pat);
            return 1;
          }
          ++cases;
        }
  /* bad arguments are refused, and touch nothing */
  const uint16_t* none[1] = {NULL};
  uint16_t r1[16];
  if (oracle_fused(none, 0, NULL, NULL, 1e-5f, 1, 16, r1, NULL, NULL, NULL, NULL, NULL, 1.0f) != -1) return 2;
  if (oracle_fused(none, 9, NULL, NULL, 1e-5f, 1, 16, r1, NULL, NULL, NULL, NULL, NULL, 1.0f) != -1) return 3;
  /* element helpers and the quantizers on exact-size arrays */
  float* y = (float*)malloc(64 * 4);
  for (int i = 0; i < 64; ++i) y[i] = frand() * 37.0f;
  uint8_t* c = (uint8_t*)malloc(32); uint8_t* s = (uint8_t*)malloc(4); uint8_t* q = (uint8_t*)malloc(64);
  uint16_t* b = (uint16_t*)malloc(64 * 2);
  oracle_quantize_fp4(y, 2, 32, c, s);
  oracle_quantize_fp8(y, 4, 16, 0.5f, q);
  oracle_bf16_rne_array(y, 64, b);
  oracle_e4m3_rne_array(y, 64, q);
  for (int i = 0; i < 64; ++i) y[i] = y[i] < 0 ? -y[i] : y[i];
  oracle_e2m1_rne_array(y, 64, q);
  /* LL unpack: 16 elements = 4 words of 16 bytes */
  uint8_t* words = (uint8_t*)malloc(64);
  for (int w = 0; w < 4; ++w) { uint64_t f = (w == 2) ? 6 : 5; memset(words + 16 * w, w, 8); memcpy(words + 16 * w + 8, &f, 8); }
  if (oracle_ll_unpack(words, 16, 5, b) != 1) return 4;
  for (int i = 0; i < 16; ++i) b[i] = (i == 9) ? 0xFFFF : 0x3F80;
  if (oracle_sentinel_pending(b, 16, 0xFFFF) != 1) return 5;
  free(y); free(c); free(s); free(q); free(b); free(words);
  printf("%d\n", cases);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    src = tmp_path / "driver.c"
    exe = tmp_path / "driver"
    src.write_text(DRIVER)
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", ORACLE, "-o", str(exe), str(src), os.path.join(ORACLE, "arfuse_oracle.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert int(r.stdout.split()[0]) == 8 * 3 * 3 * 6
