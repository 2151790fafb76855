"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

The ABI unit (`csrc/arfuse.hip`) is built for the host with
-fsanitize=address,undefined (device code untouched), linked with row-kernel
selectors that select nothing, so no row kernel is ever launched, and driven
by a C++ program through argument validation and launch choice: every
documented argument error, t = 0 no-ops, split and layout choices over many
shapes, and valid calls, which pass validation and stop at the empty
selector (ARFUSE_ERR_UNSUPPORTED). Buffer addresses are fake and never
dereferenced: the host checks only ranges and alignment. Any sanitizer
finding aborts the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduce_residual_rmsnorm_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

STUB = r"""
// Row-kernel selectors that select nothing: this build checks the host
// ABI's validation and launch choices, and never launches a row kernel.
#include "arfuse_device.hpp"
namespace arfuse_detail {
RowFn select_row_kernel_n1(int, int, int, int) { return nullptr; }
RowFn select_row_kernel_n2(int, int, int, int) { return nullptr; }
RowFn select_row_kernel_n3(int, int, int, int) { return nullptr; }
RowFn select_row_kernel_n4(int, int, int, int) { return nullptr; }
RowFn select_row_kernel_n5(int, int, int, int) { return nullptr; }
RowFn select_row_kernel_n6(int, int, int, int) { return nullptr; }
RowFn select_row_kernel_n7(int, int, int, int) { return nullptr; }
RowFn select_row_kernel_n8(int, int, int, int) { return nullptr; }
}  // namespace arfuse_detail
"""

DRIVER = r"""
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include "arfuse.h"

static int fails = 0;
#define EXPECT(expr, want)                                                    \
  do {                                                                        \
    const int got_ = (expr);                                                  \
    if (got_ != (want)) {                                                     \
      std::printf("line %d: %s = %d, want %d\n", __LINE__, #expr, got_, want); \
      ++fails;                                                                \
    }                                                                         \
  } while (0)

static void* A(int i) { return (void*)(uintptr_t)(0x100000000ull * (uint64_t)(i + 1)); }

int main() {
  const int OK = ARFUSE_OK, INV = ARFUSE_ERR_INVALID_ARG, UNS = ARFUSE_ERR_UNSUPPORTED;
  const void* parts[8];
  for (int i = 0; i < 8; ++i) parts[i] = A(i);
  void* res = A(8); float* g = (float*)A(9); void* out = A(10); void* rout = A(11);
  uint8_t* c4 = (uint8_t*)A(12); uint8_t* s4 = (uint8_t*)A(13);

  // launch choice over shapes, layouts, splits and epilogues
  arfuse_launch_info info;
  int nq = 0;
  for (int n = 1; n <= 8; ++n)
    for (int64_t t : {0, 1, 3, 8, 64, 255, 256, 512, 1024, 4096})
      for (int64_t d : {16, 48, 1040, 4096, 8192, 16384, 65536})
        for (int layout = 0; layout <= 2; ++layout)
          for (uint32_t split : {0u, 2u, 4u, 8u, ARFUSE_SPLIT_AUTO})
            for (int epi : {0, 1, 2, 3, 4, 5}) {
              arfuse_opts o;
              std::memset(&o, 0, sizeof o);
              o.layout = layout;
              o.split = split;
              const int rc = arfuse_query_launch(n, t, d, epi, &o, &info);
              if (rc != OK && rc != INV && rc != UNS) { std::printf("query rc %d\n", rc); ++fails; }
              if (rc == OK && (info.block < 64 || info.block > 1024 || info.block % 64 ||
                               info.split < 1 || info.split > 8)) { std::printf("bad launch\n"); ++fails; }
              ++nq;
            }
  EXPECT(arfuse_query_launch(8, 4096, 8192, 1, nullptr, nullptr), INV);
  EXPECT(arfuse_query_launch(0, 1, 8192, 1, nullptr, &info), INV);
  EXPECT(arfuse_query_launch(9, 1, 8192, 1, nullptr, &info), INV);
  EXPECT(arfuse_query_launch(8, 1, 8200, 1, nullptr, &info), INV);
  EXPECT(arfuse_query_launch(8, 1, 8192, 6, nullptr, &info), UNS);  // FP4 with FP8

  // argument errors of the fused call
  EXPECT(arfuse_rmsnorm(nullptr, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 0, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 9, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4100, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 2, res, g, -1.0f, out, rout, nullptr, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 2, res, g, NAN, out, rout, nullptr, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 2, res, g, 1e-5f, out, rout, c4, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 2, res, nullptr, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 2, (char*)res + 8, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 2, res, g, 1e-5f, out, (char*)out + 16, nullptr, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 2, res, g, 1e-5f, (void*)parts[1], rout, nullptr, nullptr, 4, 4096, nullptr), INV);
  EXPECT(arfuse_rmsnorm(parts, 2, res, g, 1e-5f, out, (char*)res + 16, nullptr, nullptr, 4, 4096, nullptr), INV);
  // t = 0: nothing is touched, buffers may be NULL
  EXPECT(arfuse_rmsnorm(nullptr, 2, nullptr, nullptr, 1e-5f, nullptr, nullptr, nullptr, nullptr, 0, 4096, nullptr), OK);
  // valid calls pass validation and stop at the empty selector
  EXPECT(arfuse_rmsnorm(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr), UNS);
  EXPECT(arfuse_rmsnorm(parts, 8, res, g, 1e-5f, out, res, c4, s4, 4096, 8192, nullptr), UNS);
  EXPECT(arfuse_rmsnorm(parts, 8, res, nullptr, 1e-5f, nullptr, rout, nullptr, nullptr, 8, 8192, nullptr), UNS);

  // options
  arfuse_opts o;
  std::memset(&o, 0, sizeof o);
  o.layout = 3;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  std::memset(&o, 0, sizeof o);
  o.reserved2 = 1;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  std::memset(&o, 0, sizeof o);
  o.max_polls = ARFUSE_MAX_POLLS + 1;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  std::memset(&o, 0, sizeof o);
  o.layout = ARFUSE_LAYOUT_SENTINEL;
  o.sentinel = 0x10000;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  std::memset(&o, 0, sizeof o);
  void* slots[2] = {A(14), A(15)};
  o.reset = slots;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  o.layout = ARFUSE_LAYOUT_SENTINEL;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  o.status = (arfuse_ll_status*)A(18);
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), UNS);
  std::memset(&o, 0, sizeof o);
  o.fp8_out = (uint8_t*)A(16);
  o.fp8_inv_scale = INFINITY;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  std::memset(&o, 0, sizeof o);
  o.split = 3;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  o.split = 4;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  o.workspace = (char*)A(17) + 8;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  o.workspace = A(17);
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);
  o.status = (arfuse_ll_status*)A(18);
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), UNS);
  o.status = nullptr;
  o.split = 8;
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 64, 4096, nullptr, &o), UNS);
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 33, 4096, nullptr, &o), UNS);
  o.status = (arfuse_ll_status*)((char*)A(18) + 4);
  EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 4096, nullptr, &o), INV);

  // every call that can wait needs a status word (the only report of a
  // bounded wait that gave up); with one, each passes validation
  {
    arfuse_ll_status* st = (arfuse_ll_status*)A(18);
    const int lay[3] = {ARFUSE_LAYOUT_LL, ARFUSE_LAYOUT_SENTINEL, ARFUSE_LAYOUT_PLAIN};
    const uint32_t spl[3] = {0u, 0u, 4u};
    for (int c = 0; c < 3; ++c) {
      std::memset(&o, 0, sizeof o);
      o.layout = lay[c];
      o.split = spl[c];
      o.workspace = spl[c] ? A(17) : nullptr;
      EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 8192, nullptr, &o), INV);
      o.status = st;
      EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 8192, nullptr, &o), UNS);
    }
    // the library's own choice: n = 2, t = 4, d = 8192 splits 4 ways
    std::memset(&o, 0, sizeof o);
    o.split = ARFUSE_SPLIT_AUTO;
    o.workspace = A(17);
    EXPECT(arfuse_query_launch(2, 4, 8192, 1, &o, &info), OK);
    EXPECT(info.split, 4);
    EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 8192, nullptr, &o), INV);
    o.status = st;
    EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 8192, nullptr, &o), UNS);
    // the all-reduce alone never waits: no status needed, split or not
    std::memset(&o, 0, sizeof o);
    o.split = 4;
    EXPECT(arfuse_rmsnorm_ex(parts, 2, res, nullptr, 1e-5f, nullptr, rout, nullptr, nullptr, 4, 8192, nullptr, &o), UNS);
    // t = 0 stays a no-op
    std::memset(&o, 0, sizeof o);
    o.layout = ARFUSE_LAYOUT_LL;
    EXPECT(arfuse_rmsnorm_ex(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 0, 8192, nullptr, &o), OK);
  }

  // the allocation-free entry refuses a caller workspace before anything else
  std::memset(&o, 0, sizeof o);
  o.split = 4;
  o.workspace = A(17);
  o.status = (arfuse_ll_status*)A(18);
  EXPECT(arfuse_rmsnorm_noalloc(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 4, 8192, nullptr, &o), INV);
  EXPECT(arfuse_rmsnorm_noalloc(parts, 2, res, g, 1e-5f, out, rout, nullptr, nullptr, 0, 8192, nullptr, &o), INV);

  // auxiliary entries: argument errors and no-op sizes only (no launch)
  EXPECT(arfuse_quantize_fp4_ll(nullptr, 1, 16, c4, s4, nullptr), INV);
  EXPECT(arfuse_quantize_fp4_ll(g, 1, 24, c4, s4, nullptr), INV);
  EXPECT(arfuse_quantize_fp4_ll(g, 1, 16, c4 + 1, s4, nullptr), INV);
  EXPECT(arfuse_quantize_fp4_ll(g, 1, 64, (uint8_t*)g + 16, s4, nullptr), INV);
  EXPECT(arfuse_quantize_fp4_ll(g, 0, 16, nullptr, nullptr, nullptr), OK);
  {
    const void* ins[2] = {A(19), A(20)};
    void* outs[2] = {A(21), A(22)};
    void* bad_outs[2] = {A(21), (char*)A(19) + 16};
    EXPECT(arfuse_stream_mix(ins, 0, outs, 1, 4, 4096, nullptr), INV);
    EXPECT(arfuse_stream_mix(ins, 10, outs, 1, 4, 4096, nullptr), INV);
    EXPECT(arfuse_stream_mix(ins, 2, outs, 4, 4, 4096, nullptr), INV);
    EXPECT(arfuse_stream_mix(ins, 2, outs, 2, 4, 4104, nullptr), INV);
    EXPECT(arfuse_stream_mix(ins, 2, bad_outs, 2, 4, 4096, nullptr), INV);
    EXPECT(arfuse_stream_mix(ins, 2, outs, 2, 4, 65536 + 16, nullptr), UNS);
    EXPECT(arfuse_stream_mix(nullptr, 2, nullptr, 2, 0, 4096, nullptr), OK);
  }
  EXPECT(arfuse_quantize_fp4(nullptr, 1, 16, c4, s4, nullptr), INV);
  EXPECT(arfuse_quantize_fp4(g, 1, 24, c4, s4, nullptr), INV);
  EXPECT(arfuse_stream_copy(A(19), A(20), 24, nullptr), INV);
  EXPECT(arfuse_stream_copy(A(19), (char*)A(19) + 16, 64, nullptr), INV);
  EXPECT(arfuse_stream_copy(A(19), A(20), 0, nullptr), OK);
  EXPECT(arfuse_round_bf16((float*)A(21), 3, (uint16_t*)A(22), nullptr), INV);
  EXPECT(arfuse_round_fp8((float*)A(21), 6, (uint8_t*)A(22), nullptr), INV);
  EXPECT(arfuse_round_fp4((float*)A(21), 3, (uint8_t*)A(22), nullptr), INV);
  EXPECT(arfuse_round_fp4((float*)((char*)A(21) + 4), 2, (uint8_t*)A(22), nullptr), INV);
  EXPECT(arfuse_round_fp4((float*)A(21), 0, nullptr, nullptr), OK);
  EXPECT(arfuse_launch_floor(0, 1, 8192, 1, nullptr, nullptr), INV);
  for (int code = 0; code < 8; ++code)
    if (!arfuse_status_string(code | (3 << 8))) { std::printf("no status string\n"); ++fails; }
  EXPECT(arfuse_version(), ARFUSE_VERSION);
  std::printf("%d %d\n", nq, fails);
  return fails ? 1 : 0;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_host_abi_clean_under_asan_and_ubsan(tmp_path):
    stub = tmp_path / "stub.hip"
    drv = tmp_path / "driver.cpp"
    exe = tmp_path / "abi_sanitized"
    stub.write_text(STUB)
    drv.write_text(DRIVER)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "arfuse.hip"), str(stub), str(drv), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    nq, fails = map(int, run.stdout.split()[-2:])
    assert fails == 0 and nq == 8 * 10 * 7 * 3 * 5 * 6
