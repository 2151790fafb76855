"""HIP path vs the CPU oracle, element by element, on the same seeded inputs.

Covers every workload shape (single decode token, Llama-3-8B and
Llama-3.1-70B decode steps, the prefill bandwidth shapes at full size, the
FP4 shapes), ragged and extreme widths, every rank count, launch overrides,
in-place residual, t = 0, determinism, and the FP4 entry on the oracle's own
fp32 values (bit-exact, including sweeps around every rounding tie)."""

import numpy as np
import pytest
import torch

import oracle_pins
import reduce_residual_rmsnorm_amd as arf
import seeded_inputs as si
from gpu_util import (Dev, assert_fp4_close, assert_residual_exact, assert_y_close, dev_f32,
                      host_u16, note)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    arch = torch.cuda.get_device_properties(0).gcnArchName
    note("device %s" % arch)
    assert arch.startswith("gfx950"), arch


def check_call(ci, fp4=False, out=True, **opts):
    orc = __import__("oracle").default()
    ref = orc.allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps, fp4=fp4)
    note("n=%d t=%d d=%d fp4=%s out=%s opts=%s" % (ci.n, ci.t, ci.d, fp4, out, opts))
    got = Dev(ci, fp4=fp4, out=out).run(**opts).fetch()
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    stats = {}
    if out:
        stats = assert_y_close(got["out"], ref["y32"], ref["out"])
    if fp4:
        stats.update(assert_fp4_close(got["codes"], got["scales"], ref["codes"], ref["scales"]))
    return stats


@pytest.mark.parametrize("name", ["decode_n2_t1_d4096", "decode_n8_t8_d4096_chain64",
                                  "decode_n4_t8_d8192_chain160", "decode_n8_t8_d8192_chain160",
                                  "prefill_n8_t512_d8192", "prefill_n8_t4096_d8192"])
def test_workload_bf16(name):
    ci = si.make_workload(name)
    stats = check_call(ci)
    # the fp64 norm reproduces the oracle's rounding essentially everywhere
    assert stats["bf16_equal_frac"] > 0.9999, stats


@pytest.mark.parametrize("name", ["fp4_n4_t1_d8192", "fp4_n4_t8_d8192", "fp4_n4_t64_d8192",
                                  "fp4_n4_t512_d8192"])
def test_workload_fp4(name):
    ci = si.make_workload(name)
    check_call(ci, fp4=True, out=False)


def test_workload_fp4_with_bf16_out():
    check_call(si.make_workload("fp4_n4_t64_d8192"), fp4=True, out=True)


@pytest.mark.parametrize("n,t,d", [(1, 3, 16), (3, 5, 48), (5, 7, 1040), (6, 3, 8208),
                                   (7, 2, 16384), (8, 2, 65536), (2, 3, 65520), (4, 9, 4112),
                                   (8, 33, 8192), (2, 65, 2048)])
def test_ragged_and_extreme_shapes(n, t, d):
    ci = si.make_call(n, t, d, seed=1000 + n * 7 + d, outlier_frac=0.1)
    check_call(ci, fp4=True, out=True)


@pytest.mark.parametrize("block,vpt", [(256, 4), (512, 2), (1024, 1), (128, 8), (576, 2)])
def test_launch_overrides(block, vpt):
    ci = si.make_call(8, 6, 8192, seed=77)
    info = arf.arfuse_query_launch(8, 6, 8192, block_threads=block, vpt=vpt)
    assert (info.block, info.vpt) == (block, vpt)
    check_call(ci, fp4=True, block_threads=block, vpt=vpt)


@pytest.mark.parametrize("n", range(1, 9))
def test_every_rank_count(n):
    check_call(si.make_call(n, 4, 4096, seed=n))


# every lane reads its residual elements before it stores residual_out over
# them, at decode and at prefill-like row counts
@pytest.mark.parametrize("t,d", [(8, 8192), (300, 4096)])
def test_residual_in_place(t, d):
    ci = si.make_call(4, t, d, seed=5)
    orc = __import__("oracle").default()
    ref = orc.allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps)
    dv = Dev(ci)
    dv.residual_out = dv.residual  # in place
    note("in-place residual t=%d d=%d" % (t, d))
    got = dv.run().fetch()
    assert_residual_exact(got["residual_out"], ref["residual_out"])
    assert_y_close(got["out"], ref["y32"])


def test_t_zero_with_empty_tensors():
    e = torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda:0")
    g = torch.ones(4096, dtype=torch.float32, device="cuda:0")
    note("t=0")
    arf.arfuse_rmsnorm([e, e], e, g, 1e-5, e, e)
    torch.cuda.synchronize()


def test_deterministic():
    ci = si.make_workload("prefill_n8_t512_d8192")
    note("determinism")
    dv = Dev(ci, fp4=True)
    a = dv.run().fetch()
    b = dv.run().fetch()
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_eps_zero_and_large():
    for eps in (np.float32(0.0), np.float32(1.0)):
        ci = si.make_call(4, 5, 1024, seed=9)
        ci.eps = eps
        check_call(ci, fp4=True)


def test_zero_and_constant_rows():
    d = 4096
    ci = si.make_call(4, 3, d, seed=10)
    ci.partials[:, 0, :] = 0
    ci.residual[0, :] = 0
    ci.partials[:, 1, :] = si.to_bf16_bits(np.full(d, 0.75, np.float32))
    ci.residual[1, :] = 0
    stats = check_call(ci, fp4=True)
    assert stats["code_mismatch"] == 0


# ------------------------------------------------ FP4 entry, bit-exact

# The FP4 epilogue comes in two lane geometries: plain and sentinel rows hold
# 8 contiguous elements per lane, a block in a lane pair (fp4_pair,
# arfuse_quantize_fp4); LL rows hold 4-element groups, a block in a lane quad
# (fp4_quad, arfuse_quantize_fp4_ll). Each test runs both.
GEOMETRIES = pytest.mark.parametrize("ll", [False, True], ids=["pair", "quad"])


def quant_gpu(y, ll=False):
    t, d = y.shape
    yd = dev_f32(y)
    codes = torch.empty((t, d // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((t, d // 16), dtype=torch.uint8, device="cuda:0")
    (arf.arfuse_quantize_fp4_ll if ll else arf.arfuse_quantize_fp4)(yd, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@GEOMETRIES
def test_quantize_bit_exact_on_oracle_y(ll):
    orc = __import__("oracle").default()
    ci = si.make_workload("fp4_n4_t64_d8192")
    ref = orc.allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps, fp4=True)
    note("quantize oracle y32 ll=%s" % ll)
    c, s = quant_gpu(ref["y32"], ll)
    assert np.array_equal(s, ref["scales"])
    assert np.array_equal(c, ref["codes"])


def _tie_blocks():
    """The oracle pins' near-tie blocks: every E4M3 scale x every E2M1
    threshold +-1 ulp, and block maxima around every E4M3 midpoint x 6."""
    from fractions import Fraction as Fr
    E4 = oracle_pins.E4M3
    E2 = oracle_pins.E2M1
    ths = [(E2[i] + E2[i + 1]) / 2 for i in range(7)]
    blocks = []
    for sc in range(1, 127):
        s = E4[sc]
        vals = []
        for th in ths:
            vals += oracle_pins.ulp_steps(np.float32(float(s * th)), 2)
        for j in range(0, len(vals), 15):
            chunk = vals[j:j + 15]
            chunk += [np.float32(0)] * (15 - len(chunk))
            sign = -1 if (sc + j) % 3 == 0 else 1
            blocks.append([np.float32(float(6 * s))] + [np.float32(sign * v) for v in chunk])
    for i in range(len(E4) - 1):
        mid6 = 6 * (E4[i] + E4[i + 1]) / 2
        for v in oracle_pins.ulp_steps(np.float32(float(mid6)), 6):
            blocks.append([v] + [np.float32(0)] * 15)
    y = np.array(blocks, np.float32)
    pad = (-len(y)) % 4
    y = np.concatenate([y, np.zeros((pad, 16), np.float32)])
    return y.reshape(-1, 64)  # 4 blocks per row


@GEOMETRIES
def test_quantize_bit_exact_near_ties(ll):
    """Every value of these blocks lies within 2 ulps of s * (an E2M1
    decision point), so the hardware conversion's envelope leaves each one
    open and the exact comparison fallback decides every code."""
    orc = __import__("oracle").default()
    y = _tie_blocks()
    wc, ws = orc.quantize_fp4(y)
    note("quantize near-tie sweep rows=%d ll=%s" % (y.shape[0], ll))
    c, s = quant_gpu(y, ll)
    assert np.array_equal(s, ws)
    assert np.array_equal(c, wc)


@GEOMETRIES
def test_quantize_bit_exact_random_octaves(ll):
    orc = __import__("oracle").default()
    rng = np.random.default_rng(12)
    y = (rng.standard_normal((300, 1024)) * np.exp2(rng.uniform(-14, 8, (300, 1)))).astype(np.float32)
    y[::5, ::3] = -0.0
    y[7] = 0
    wc, ws = orc.quantize_fp4(y)
    note("quantize random octaves ll=%s" % ll)
    c, s = quant_gpu(y, ll)
    assert np.array_equal(s, ws) and np.array_equal(c, wc)


@GEOMETRIES
def test_quantize_ragged_rows(ll):
    """Row counts and widths whose blocks leave part of the last workgroup
    idle (the idle lanes clamp to the last block and store nothing)."""
    orc = __import__("oracle").default()
    rng = np.random.default_rng(13)
    for (t, d) in [(1, 16), (3, 48), (7, 1040), (5, 4112)]:
        y = rng.standard_normal((t, d)).astype(np.float32)
        wc, ws = orc.quantize_fp4(y)
        note("quantize t=%d d=%d ll=%s" % (t, d, ll))
        c, s = quant_gpu(y, ll)
        assert np.array_equal(s, ws) and np.array_equal(c, wc)


def test_kernel_fp8_conversion_on_every_tie_pattern():
    """The fused kernel's FP8 conversion (gfx950's E4M3 convert after a clamp
    to +-448) equals the oracle's sign | E4M3 round-to-nearest-even with
    saturation, on every 16-bit prefix combined with each tie and near-tie low
    half (E4M3 ties and their neighbours all fall on these patterns), and on
    random patterns."""
    orc = __import__("oracle").default()
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    pats = (hi[:, None] | lows[None, :]).reshape(-1)
    rnd = np.random.default_rng(15).integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([pats, rnd]).view(np.float32)
    x = x[np.isfinite(x)]
    x = x[: x.size // 4 * 4]
    want = orc.e4m3_rne(np.abs(x)) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    xd = dev_f32(x)
    out = torch.empty(x.size, dtype=torch.uint8, device="cuda:0")
    note("fp8 conversion sweep n=%d" % x.size)
    arf.arfuse_round_fp8(xd, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "fp8 conversion differs at %s: got %s want %s" % (
        x[bad[:4]].view(np.uint32), got[bad[:4]], want[bad[:4]])


def test_kernel_fp4_conversion_around_every_decision_point():
    """gfx950's FP4 conversion, as the fused kernel's fast FP4 path uses it
    (scale 1), equals the oracle's E2M1 rounding (nearest even, saturating,
    sign kept) at every value within 4096 ulps of each E2M1 value and
    decision point, both signs, on specials and on random values. The
    kernel keeps its codes only where both ends of its reciprocal envelope
    agree, so it relies on this equality near the decision points."""
    orc = __import__("oracle").default()
    pts = np.array([0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0,
                    7.0, 8.0], np.float32)
    u = (pts.view(np.int32)[:, None] + np.arange(-4096, 4097, dtype=np.int32)[None, :]).reshape(-1)
    u = u[(u >= 0) & (u < 0x7F800000)]
    a = u.view(np.float32)
    specials = np.array([1e-30, 1e-40, 6.0001, 6.5, 1e3, 1e30, 3.4e38, 0.0], np.float32)
    rnd = np.random.default_rng(16).standard_normal(1 << 20).astype(np.float32)
    rnd *= np.exp2(np.random.default_rng(17).integers(-8, 8, rnd.size)).astype(np.float32)
    x = np.concatenate([a, -a, specials, -specials, rnd]).astype(np.float32)
    x = x[: x.size // 2 * 2]
    want = orc.e2m1_rne(np.abs(x)) | np.where(np.signbit(x), 8, 0).astype(np.uint8)
    xd = dev_f32(x)
    out = torch.empty(x.size // 2, dtype=torch.uint8, device="cuda:0")
    note("fp4 conversion sweep n=%d" % x.size)
    arf.arfuse_round_fp4(xd, out)
    torch.cuda.synchronize()
    b = out.cpu().numpy()
    got = np.empty(x.size, np.uint8)
    got[0::2] = b & 0xF
    got[1::2] = b >> 4
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "fp4 conversion differs at %s: got %s want %s" % (
        x[bad[:4]], got[bad[:4]], want[bad[:4]])


def test_kernel_bf16_rounding_on_every_tie_pattern():
    """The fused kernel's fp32 -> bf16 conversion (gfx950's packed convert)
    equals the oracle's round-to-nearest-even on every 16-bit prefix combined
    with each tie and near-tie low half, and on random patterns."""
    orc = __import__("oracle").default()
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    pats = (hi[:, None] | lows[None, :]).reshape(-1)
    rnd = np.random.default_rng(14).integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([pats, rnd]).view(np.float32)
    x = x[np.isfinite(x)]
    x = x[: x.size // 2 * 2]
    want = orc.bf16_rne(x)
    xd = dev_f32(x)
    out = torch.empty(x.size, dtype=torch.int16, device="cuda:0")
    note("bf16 rounding sweep n=%d" % x.size)
    arf.arfuse_round_bf16(xd, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "bf16 rounding differs at %s" % x[bad[:4]].view(np.uint32)
