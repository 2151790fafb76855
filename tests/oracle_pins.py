"""Pins of the CPU oracle against things other than itself.

Every ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with:
  * a library routine that implements a special case (PyTorch's CPU bf16 and
    float8_e4m3fn conversions, ``torch.nn.functional.rms_norm`` in float64,
    ``math.fsum`` for the exact sum),
  * brute force in exact rational arithmetic (``fractions.Fraction``) on small
    inputs and on sweeps around every rounding tie,
  * closed forms and invariants of RMSNorm,
  * figures the pages print (tests/golden/page_figures.json).

The same functions run against deliberately broken copies of the oracle in
test_oracle_mutants.py, to show that each plausible mistake fails a pin.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import torch

import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------- helpers

def f32(x) -> np.float32:
    return np.float32(x)


def ulp_steps(x: np.float32, k: int):
    """fp32 neighbours of x, k steps each way (x included)."""
    out = [np.float32(x)]
    up = dn = np.float32(x)
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        out += [up, dn]
    return out


def e4m3_table_exact():
    """Positive finite E4M3 values from the OCP bit fields (bias 7, 3-bit
    mantissa, exponent field 0 subnormal), code 0..126, as Fractions."""
    vals = []
    for c in range(127):
        e, m = c >> 3, c & 7
        v = Fr(m, 8) * Fr(1, 64) if e == 0 else (1 + Fr(m, 8)) * Fr(2) ** (e - 7)
        vals.append(v)
    return vals


def e2m1_table_exact():
    """E2M1 magnitudes from the bit fields (bias 1, 1-bit mantissa)."""
    vals = []
    for c in range(8):
        e, m = c >> 1, c & 1
        v = Fr(m, 2) if e == 0 else (1 + Fr(m, 2)) * Fr(2) ** (e - 1)
        vals.append(v)
    return vals


E4M3 = e4m3_table_exact()
E2M1 = e2m1_table_exact()


def nearest_even(x: Fr, table) -> int:
    """Index of the table value nearest to x; equal distance -> even index."""
    best, bestd = 0, None
    for i, v in enumerate(table):
        dist = abs(x - v)
        if bestd is None or dist < bestd or (dist == bestd and i % 2 == 0 and best % 2 == 1):
            best, bestd = i, dist
    return best


# ------------------------------------------------------------ bf16 pins

def pin_bf16_vs_torch(orc, n=1 << 20, seed=1):
    """bf16 round-to-nearest-even equals PyTorch's CPU float32->bfloat16 on
    random finite bit patterns, on exact ties of both parities and on their
    neighbours, and on subnormals."""
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 1 << 16, size=n // 4, dtype=np.uint64).astype(np.uint32) << 16)
    pats = np.concatenate([u, ties | 0x8000, ties | 0x7FFF, ties | 0x8001,
                           ties & 0x807FFFFF, np.array([0x7F7F8000, 0x7F7FFFFF, 0x7F7F7FFF,
                                                        0x00008000, 0x80018000], np.uint32)])
    x = pats.view(np.float32)
    x = x[np.isfinite(x)]
    want = si.to_bf16_bits(x)
    got = orc.bf16_rne(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "bf16 mismatch at %s: got %s want %s" % (
        x[bad[:4]].view(np.uint32), got[bad[:4]], want[bad[:4]])


# ------------------------------------------------------------ E4M3 pins

def pin_e4m3_decode_vs_torch(orc):
    """Decoding every E4M3 code equals PyTorch's float8_e4m3fn decoding."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.e4m3_value(c) for c in range(256)])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), "E4M3 decode differs at codes %s" % np.nonzero(~same)[0][:8]


def _e4m3_sweep_points():
    pts = []
    for i in range(len(E4M3) - 1):
        mid = (E4M3[i] + E4M3[i + 1]) / 2
        pts += ulp_steps(f32(float(mid)), 3)
        pts += ulp_steps(f32(float(E4M3[i])), 1)
    pts += [f32(448), f32(449), f32(463.9), f32(464), f32(1000), f32(2.0 ** -10),
            f32(2.0 ** -12), f32(0)]
    # saturation over the whole fp32 range: every power of two above 448, its
    # neighbours, and the largest finite float
    for e in range(9, 128):
        pts += ulp_steps(f32(2.0 ** e), 1)
    pts += [np.float32(np.finfo(np.float32).max)]
    return np.array([v for v in pts if not np.signbit(v)], np.float32)


def pin_e4m3_rne_exact(orc):
    """E4M3 rounding equals brute-force nearest-even in exact rationals around
    every tie and value, and PyTorch's float8_e4m3fn conversion below 464
    (where PyTorch does not turn the value into NaN)."""
    x = _e4m3_sweep_points()
    got = orc.e4m3_rne(x)
    want = np.array([nearest_even(Fr(float(v)), E4M3) for v in x], np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "E4M3 rne vs exact: x=%s got %s want %s" % (x[bad[:4]], got[bad[:4]], want[bad[:4]])
    lib_ok = x < 464
    tref = torch.from_numpy(x[lib_ok]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[lib_ok], tref), "E4M3 rne vs torch float8_e4m3fn"


# ------------------------------------------------------------ E2M1 pins

def pin_e2m1_rne_exact(orc):
    """E2M1 rounding equals brute-force nearest-even in exact rationals around
    every tie and value, and saturates to 6 above it."""
    pts = []
    for i in range(7):
        pts += ulp_steps(f32(float((E2M1[i] + E2M1[i + 1]) / 2)), 4)
        pts += ulp_steps(f32(float(E2M1[i])), 1)
    pts += [f32(6), f32(6.5), f32(7), f32(100), f32(0), np.float32(np.inf)]
    # far above 6, where fp64 distances to the grid can no longer tell the
    # grid values apart
    pts += [f32(2.0 ** 52), f32(2.0 ** 56), f32(1e30), f32(3.4e38)]
    q = np.array([p for p in pts if p >= 0], np.float32)
    got = orc.e2m1_rne(q)
    want = np.array([7 if np.isinf(v) else nearest_even(Fr(float(v)), E2M1) for v in q], np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "E2M1 rne: q=%s got %s want %s" % (q[bad[:4]], got[bad[:4]], want[bad[:4]])
    for c in range(8):
        assert orc.e2m1_value(c) == float(E2M1[c]), "E2M1 value table at %d" % c


# ------------------------------------------------------- FP4 block pins

def fp4_block_exact(y16):
    """Block quantization in exact rationals: s = nearest-even E4M3 of
    blockmax/6, code = sign | nearest-even E2M1 of |y|/s (0 when s == 0)."""
    bm = max(abs(Fr(float(v))) for v in y16)
    sc = nearest_even(bm / 6, E4M3)
    s = E4M3[sc]
    codes = []
    for v in y16:
        mag = 0 if s == 0 else nearest_even(abs(Fr(float(v))) / s, E2M1)
        codes.append((8 if math.copysign(1.0, float(v)) < 0 else 0) | mag)
    return sc, codes


def _pack_codes(codes):
    return [codes[2 * k] | (codes[2 * k + 1] << 4) for k in range(len(codes) // 2)]


def pin_fp4_code_ties(orc):
    """For every positive E4M3 scale s and every E2M1 decision threshold T,
    elements within a few fp32 ulps of s*T quantize as exact rational
    rounding of |y|/s says (the block max 6s fixes the scale to s)."""
    ths = [(E2M1[i] + E2M1[i + 1]) / 2 for i in range(7)]
    blocks = []
    for sc in range(1, 127):
        s = E4M3[sc]
        vals = []
        for th in ths:
            vals += ulp_steps(f32(float(s * th)), 1)
        vals = vals[:len(vals) // 15 * 15] if len(vals) >= 15 else vals
        for j in range(0, len(vals), 15):
            chunk = vals[j:j + 15]
            if len(chunk) < 15:
                chunk = chunk + [f32(0)] * (15 - len(chunk))
            sign = -1 if (sc + j) % 3 == 0 else 1
            blocks.append([f32(float(6 * s))] + [f32(sign * v) for v in chunk])
    y = np.array(blocks, np.float32)
    codes, scales = orc.quantize_fp4(y)
    for b in range(y.shape[0]):
        sc, want = fp4_block_exact(y[b])
        assert scales[b, 0] == sc, "scale of block %d: %d vs %d" % (b, scales[b, 0], sc)
        packed = _pack_codes(want)
        if list(codes[b]) != packed:
            raise AssertionError("codes of block %d: %s vs %s (y=%s)" % (b, list(codes[b]), packed, y[b]))


def pin_fp4_scale_ties(orc):
    """Block maxima within a few fp32 ulps of 6 x (every E4M3 rounding
    midpoint) pick the scale that exact rational rounding of blockmax/6 picks."""
    blocks = []
    for i in range(len(E4M3) - 1):
        mid6 = 6 * (E4M3[i] + E4M3[i + 1]) / 2
        for v in ulp_steps(f32(float(mid6)), 6):
            blocks.append([v] + [f32(0)] * 15)
    y = np.array(blocks, np.float32)
    codes, scales = orc.quantize_fp4(y)
    for b in range(y.shape[0]):
        sc, want = fp4_block_exact(y[b])
        assert scales[b, 0] == sc, "scale tie block %d bm=%r: %d vs %d" % (b, y[b, 0], scales[b, 0], sc)
        assert list(codes[b]) == _pack_codes(want)


def pin_fp4_small_random_blocks(orc, nblocks=400, seed=2):
    """Brute force on small random blocks with magnitudes over many octaves."""
    rng = np.random.default_rng(seed)
    mags = np.exp2(rng.uniform(-16, 7, size=(nblocks, 1))).astype(np.float32)
    y = (rng.standard_normal((nblocks, 16)).astype(np.float32) * mags).astype(np.float32)
    y[::7, 3] = -0.0
    y[::11, :] = 0.0
    codes, scales = orc.quantize_fp4(y)
    for b in range(nblocks):
        sc, want = fp4_block_exact(y[b])
        assert scales[b, 0] == sc and list(codes[b]) == _pack_codes(want), "random block %d" % b


def pin_fp4_invariants(orc):
    """Layout and sign invariants: element 2k in the low nibble, the sign bit
    of -0.0 kept, an all-zero block gives scale 0 and codes 0, and with a
    normal scale the block maximum always encodes to magnitude 6 (code 7)."""
    y = np.zeros((3, 16), np.float32)
    y[0, 0], y[0, 1] = 6.0, -1.0             # s = 1.0 -> codes 7 and 0xA
    y[0, 2] = -0.0
    # block max 3e-3: blockmax/6 = 5e-4 < 2^-10, half the smallest E4M3
    # subnormal, so the scale is 0 and every magnitude is 0 (signs kept)
    y[2, :] = np.float32(3e-3) * np.where(np.arange(16) % 2, -1, 1).astype(np.float32)
    codes, scales = orc.quantize_fp4(y)
    assert scales[0, 0] == 0x38, "scale of 6/6 should be E4M3 1.0 (0x38)"
    assert codes[0, 0] == 0xA7, "nibble order / sign: got 0x%02x" % codes[0, 0]
    assert codes[0, 1] == 0x08, "-0.0 keeps its sign bit: got 0x%02x" % codes[0, 1]
    assert scales[1, 0] == 0 and not codes[1].any()
    assert scales[2, 0] == 0 and np.all(codes[2] == 0x80), "zero scale: %s" % list(codes[2])
    rng = np.random.default_rng(3)
    yb = (rng.standard_normal((2000, 16)) * np.exp2(rng.uniform(-3, 6, (2000, 1)))).astype(np.float32)
    codes, scales = orc.quantize_fp4(yb)
    lo = codes & 0xF
    hi = codes >> 4
    allc = np.empty((2000, 16), np.uint8)
    allc[:, 0::2], allc[:, 1::2] = lo, hi
    jmax = np.argmax(np.abs(yb), axis=1)
    normal = scales >= 0x08
    assert np.all((allc[np.arange(2000), jmax] & 7)[normal[:, 0]] == 7)


# ------------------------------------------------- sum / residual pins

def _bf16(v):
    return si.to_bf16_bits(np.array(v, np.float32))


def pin_rank_order(orc):
    """Rank-ordered fp32 sum with the residual added last.
    p = [2^24, 1, -2^24], r = 0 gives 0 (in rank order 2^24 + 1 rounds back
    to 2^24); any other order, or a wider accumulator, gives 1.
    p = [2^24, 1], r = -2^24 gives 0 (residual last), not 1 (residual first).
    An all -0.0 input keeps its sign."""
    P = [_bf16([[2.0 ** 24]]), _bf16([[1.0]]), _bf16([[-(2.0 ** 24)]])]
    h = orc.rank_sum_residual(P, _bf16([[0.0]]))
    assert h[0, 0] == 0.0, "rank order probe 1 gave %r" % h[0, 0]
    h = orc.rank_sum_residual(P[:2], _bf16([[-(2.0 ** 24)]]))
    assert h[0, 0] == 0.0, "residual-last probe gave %r" % h[0, 0]
    z = _bf16([[-0.0]])
    h = orc.rank_sum_residual([z, z], z)
    assert math.copysign(1.0, float(h[0, 0])) < 0, "sign of -0 + -0 + -0 lost"
    # the fused entry writes bf16(h): the same probe through residual_out
    r = orc.allreduce_rmsnorm(P, _bf16([[0.0]]), np.ones(1, np.float32), np.float32(1e-5))
    assert r["residual_out"][0, 0] == 0, "fused rank-order probe gave 0x%04x" % r["residual_out"][0, 0]


def pin_summation_bound(orc, seed=4):
    """|fp32 rank sum - exact sum| <= gamma_n * sum|x_i| (the standard
    summation bound the pages quote for fp32), with the exact sum from
    math.fsum; and the golden coefficient gamma_64 = 3.8e-6."""
    g = golden("page_figures.json")["fp32_sum_error_coefficient_64"]
    u = 2.0 ** -24

    def gamma(n):
        return n * u / (1 - n * u)

    assert abs(gamma(64) - g["value"]) <= g["rel_tol"] * g["value"]
    rng = np.random.default_rng(seed)
    for n in (1, 2, 8, 63):
        t, d = 4, 64
        parts = [si.to_bf16_bits(rng.standard_normal((t, d)).astype(np.float32) * np.float32(
            10.0 ** rng.uniform(-3, 3))) for _ in range(n)]
        res = si.to_bf16_bits(rng.standard_normal((t, d)).astype(np.float32))
        h = orc.rank_sum_residual(parts, res)
        xs = [si.bf16_bits_to_f32(p).astype(np.float64) for p in parts] + [si.bf16_bits_to_f32(res).astype(np.float64)]
        X = np.stack(xs)
        for e in range(t * d):
            col = X[:, e // d, e % d]
            exact = math.fsum(col)
            bound = gamma(n) * math.fsum(abs(v) for v in col)
            err = abs(float(h.flat[e]) - exact)
            assert err <= bound, "n=%d element %d: err %g > bound %g" % (n, e, err, bound)
        if n == 1:
            want = si.bf16_bits_to_f32(parts[0]) + si.bf16_bits_to_f32(res)
            assert np.array_equal(h, want), "N=1 must be p0 + residual"


def pin_residual_out_is_bf16_of_h(orc, seed=5):
    """residual_out = bf16(h) with h the rank-ordered fp32 sum + residual,
    and bf16 rounding agreeing with PyTorch's conversion."""
    ci = si.make_call(4, 3, 48, seed=seed)
    r = orc.allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps)
    h = orc.rank_sum_residual(ci.partials, ci.residual)
    assert np.array_equal(r["residual_out"], si.to_bf16_bits(h))


# ------------------------------------------------------------ RMSNorm pins

def pin_rmsnorm_vs_torch_f64(orc, seed=6):
    """y32 equals torch.nn.functional.rms_norm evaluated in float64 on the
    fp32 h (eps inside the root, mean over the full row, times gamma), then
    rounded to fp32: at most one fp32 ulp apart, and nearly always equal."""
    rng = np.random.default_rng(seed)
    for (t, d, scale, eps) in [(5, 4096, 1.0, 1e-5), (3, 48, 1e-3, 1e-5), (2, 8192, 30.0, 1e-6),
                               (4, 16, 1e-2, 1e-2)]:
        ci = si.make_call(3, t, d, seed=int(rng.integers(1 << 30)))
        h = orc.rank_sum_residual(ci.partials, ci.residual) * np.float32(scale)
        g = ci.gamma
        y = orc.rmsnorm_rows(h, g, np.float32(eps))
        ref = torch.nn.functional.rms_norm(torch.from_numpy(h).double(), (d,),
                                           weight=torch.from_numpy(g).double(),
                                           eps=float(np.float32(eps))).float().numpy()
        ulps = np.abs(y.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1, "rms_norm differs by %d ulps (t=%d d=%d)" % (ulps.max(), t, d)
        assert (ulps == 0).mean() > 0.99


def pin_fused_uses_fp32_h(orc, seed=7):
    """The fused call normalizes the fp32 h, not bf16(residual_out): its y32
    matches rms_norm of the fp32 h in float64 within one ulp."""
    ci = si.make_call(8, 4, 1024, seed=seed)
    r = orc.allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps)
    h = orc.rank_sum_residual(ci.partials, ci.residual)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h).double(), (1024,),
                                       weight=torch.from_numpy(ci.gamma).double(),
                                       eps=float(ci.eps)).float().numpy()
    ulps = np.abs(r["y32"].view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    assert np.array_equal(r["out"], si.to_bf16_bits(r["y32"]))


def pin_closed_forms(orc):
    """Closed forms: a constant row c gives y = c / sqrt(c^2 + eps) * gamma;
    a row with one nonzero a gives y = a / sqrt(a^2/d + eps) * gamma there
    and 0 elsewhere; a zero row gives y = 0 and FP4 scale/codes 0; with
    gamma = 1 a row's RMS is sqrt(ms / (ms + eps))."""
    d = 4096
    eps = np.float32(1e-5)
    rng = np.random.default_rng(8)
    g = rng.uniform(0.5, 1.5, d).astype(np.float32)
    # constant row: 4 partials of 0.75 sum exactly to 3
    P = [_bf16(np.full((1, d), 0.75)) for _ in range(4)]
    res = _bf16(np.zeros((1, d)))
    r = orc.allreduce_rmsnorm(P, res, g, eps)
    c = 3.0
    want = (np.float64(c) * (1.0 / math.sqrt(c * c + float(eps))) * g.astype(np.float64)).astype(np.float32)
    ulps = np.abs(r["y32"][0].view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, "constant-row closed form off by %d ulps" % ulps.max()
    # single spike
    a = 5.0
    p0 = np.zeros((1, d), np.float32)
    p0[0, 123] = a
    r = orc.allreduce_rmsnorm([_bf16(p0), _bf16(np.zeros((1, d)))], res, g, eps, fp4=True)
    want = a / math.sqrt(a * a / d + float(eps)) * float(g[123])
    assert abs(float(r["y32"][0, 123]) - want) <= 1e-6 * abs(want)
    assert np.count_nonzero(r["y32"][0]) == 1
    # zero row
    z = _bf16(np.zeros((1, d)))
    r = orc.allreduce_rmsnorm([z, z], z, g, eps, fp4=True)
    assert not r["y32"].any() and not r["scales"].any() and not r["codes"].any()
    # unit RMS with gamma = 1, residual 0
    ci = si.make_call(4, 6, d, seed=9)
    ones = np.ones(d, np.float32)
    r = orc.allreduce_rmsnorm(ci.partials, z.repeat(6, axis=0), ones, eps)
    h = orc.rank_sum_residual(ci.partials, z.repeat(6, axis=0)).astype(np.float64)
    ms = (h * h).mean(axis=1)
    rms_y = np.sqrt((r["y32"].astype(np.float64) ** 2).mean(axis=1))
    assert np.all(np.abs(rms_y - np.sqrt(ms / (ms + float(eps)))) <= 2e-7)


def pin_scale_invariance(orc):
    """Scaling partials and residual by 2^k scales residual_out by exactly 2^k;
    with eps = 0, y32 is bit-identical."""
    ci = si.make_call(4, 3, 512, seed=10)
    base = orc.allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, np.float32(0.0))
    for k in (-6, 5):
        s = np.float32(2.0 ** k)
        P = [si.to_bf16_bits(si.bf16_bits_to_f32(p) * s) for p in ci.partials]
        R = si.to_bf16_bits(si.bf16_bits_to_f32(ci.residual) * s)
        r = orc.allreduce_rmsnorm(P, R, ci.gamma, np.float32(0.0))
        ro = si.bf16_bits_to_f32(r["residual_out"])
        assert np.array_equal(ro, si.bf16_bits_to_f32(base["residual_out"]) * s)
        assert np.array_equal(r["y32"], base["y32"]), "y not invariant under 2^%d scaling" % k


# ------------------------------------------------------------- LL pins

def pin_ll_roundtrip(orc):
    """LL words: the payload of every 16-byte word is four bf16 elements in
    order, the last 8 bytes the flag; unpack restores the partial and counts
    the words whose flag differs from the expected one."""
    ci = si.make_call(1, 3, 64, seed=11)
    p = ci.partials[0]
    flag = ci.ll_base + 7
    w = si.ll_pack(p, flag)
    out, bad = orc.ll_unpack(w, p.size, flag)
    assert bad == 0 and np.array_equal(out, p.reshape(-1))
    si.ll_set_flag(w, [0, 5, 47], flag - 1)
    out, bad = orc.ll_unpack(w, p.size, flag)
    assert bad == 3 and np.array_equal(out, p.reshape(-1))
    out, bad = orc.ll_unpack(w, p.size, flag + 1)
    assert bad == p.size // 4


# ------------------------------------------------------------- FP8 pins

def pin_fp8_exact(orc):
    """FP8 output: code = sign | E4M3(|fl32(y * inv_scale)|), checked by
    exact-rational nearest-even around every E4M3 tie (both signs), against
    PyTorch's float8_e4m3fn below 464, and saturating to 448 above."""
    pts = _e4m3_sweep_points()
    y = np.concatenate([pts, -pts, np.array([-0.0, 0.0, 1e6, -1e6, 500.0], np.float32)])
    y = y.astype(np.float32).reshape(1, -1)
    got = orc.quantize_fp8(y, np.float32(1.0))[0]
    for v, c in zip(y[0], got):
        mag = 0x7E if abs(float(v)) > 448 else nearest_even(abs(Fr(float(v))), E4M3)
        want = (0x80 if math.copysign(1.0, float(v)) < 0 else 0) | mag
        assert c == want, "fp8 of %r: 0x%02x vs 0x%02x" % (float(v), c, want)
    ok = np.abs(y[0]) < 464
    tref = torch.from_numpy(y[0][ok].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[ok], tref)
    # the scale is one fp32 multiply before rounding
    rng = np.random.default_rng(15)
    y = rng.standard_normal((4, 64)).astype(np.float32) * np.float32(3)
    inv = np.float32(37.5)
    got = orc.quantize_fp8(y, inv)
    want = orc.quantize_fp8((y * inv).astype(np.float32), np.float32(1.0))
    assert np.array_equal(got, want)


# ------------------------------------------------------ pattern pins

def pin_patterns(orc):
    """Without a residual the fused call normalizes the rank sum itself
    (rank-order probe, summation bound, rms_norm of the sum); without gamma
    it is the plain all-reduce: residual_out = bf16 of the rank-ordered sum,
    and the residual, when given, added last."""
    P = [_bf16([[2.0 ** 24]]), _bf16([[1.0]]), _bf16([[-(2.0 ** 24)]])]
    r = orc.fused(P, None, None, 0.0)
    assert r["residual_out"][0, 0] == 0
    r = orc.fused(P[:2], _bf16([[-(2.0 ** 24)]]), None, 0.0)
    assert r["residual_out"][0, 0] == 0
    z = _bf16([[-0.0]])
    r = orc.fused([z, z, z], None, None, 0.0)
    assert r["residual_out"][0, 0] == 0x8000, "the sum starts from p0: -0 + -0 + -0 is -0"
    ci = si.make_call(4, 3, 256, seed=16)
    r = orc.fused(ci.partials, None, ci.gamma, ci.eps)
    zero = np.zeros_like(ci.residual)
    h = orc.rank_sum_residual(ci.partials, zero)     # + 0.0 changes nothing here
    assert np.array_equal(r["residual_out"], si.to_bf16_bits(h))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h).double(), (256,),
                                       weight=torch.from_numpy(ci.gamma).double(),
                                       eps=float(ci.eps)).float().numpy()
    ulps = np.abs(r["y32"].view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    full = orc.allreduce_rmsnorm(ci.partials, ci.residual, ci.gamma, ci.eps, fp4=True)
    r = orc.fused(ci.partials, ci.residual, None, ci.eps)
    assert np.array_equal(r["residual_out"], full["residual_out"]) and r["y32"] is None
    r = orc.fused(ci.partials, ci.residual, ci.gamma, ci.eps, fp4=True, fp8_inv_scale=2.0)
    assert np.array_equal(r["codes"], full["codes"]) and np.array_equal(r["y32"], full["y32"])
    assert np.array_equal(r["fp8"], orc.quantize_fp8(full["y32"], np.float32(2.0)))


# ----------------------------------------------------------- sentinel pins

def pin_sentinel_pending(orc):
    """A 16-byte vector (8 elements) is pending while any of its elements
    still holds the sentinel pattern; brute force on small arrays."""
    rng = np.random.default_rng(17)
    for sentinel in (0xFFFF, 0x8000):
        for _ in range(20):
            a = si.to_bf16_bits(rng.standard_normal(64).astype(np.float32))
            a[a == sentinel] = 0
            hits = rng.choice(64, size=int(rng.integers(0, 12)), replace=False)
            a[hits] = sentinel
            want = len({int(h) // 8 for h in hits})
            assert orc.sentinel_pending(a, sentinel) == want


# ------------------------------------------------------------ chain pins

def _const_rows(values, d):
    """bf16 [len(values)][d] whose row i is the constant values[i]."""
    return si.to_bf16_bits(np.repeat(np.array(values, np.float32)[:, None], d, axis=1))


def pin_chain(orc):
    """The chained replay (call c takes call c-1's residual_out as its
    residual) against closed forms. Every row of every partial is a constant
    integer, so each call's sums are exact (integers below 256 are exact in
    bf16 and fp32): after calls 0..c a row's residual is r0 + s_0 + ... + s_c
    with s_i that call's rank sum, and each call's y on a constant row h is
    h / sqrt(h^2 + eps) * gamma (0 on a zero row). With one shared set every
    call adds the same s, including when the rank count equals the number of
    calls; with one set per call, call c adds its own s_c, all different, so
    reading another call's set, or not handing the residual on, changes some
    call's residual_out."""
    d = 16
    gamma = np.linspace(0.5, 1.5, d).astype(np.float32)
    eps = np.float32(1e-5)
    r0 = [3.0, -2.0]

    def check(results, sums, what):
        assert len(results) == len(sums), what
        h = np.array(r0, np.float64)
        for c, r in enumerate(results):
            h = h + np.array(sums[c], np.float64)
            assert np.array_equal(r["residual_out"], _const_rows(h, d)), \
                "%s: call %d residual_out is not the running sum %s" % (what, c, h)
            want = (h / np.sqrt(h * h + float(eps)))[:, None] * gamma.astype(np.float64)[None, :]
            assert np.allclose(r["y32"].astype(np.float64), want, rtol=1e-6, atol=0), \
                "%s: call %d y" % (what, c)

    # one shared set of 4 ranks, 4 calls (row sums 2 and 1; row 1 passes 0)
    ranks = [[2.0, -1.0], [-1.0, 3.0], [1.0, 0.0], [0.0, -1.0]]
    shared = [_const_rows(v, d) for v in ranks]
    check(orc.chain(shared, _const_rows(r0, d), gamma, eps, 4), [[2.0, 1.0]] * 4, "shared set")
    # one set of 3 ranks per call, call c sums to (c + 1, -(2c + 1))
    k = 5
    sets, sums = [], []
    for c in range(k):
        sets.append([_const_rows(v, d) for v in ([c + 1.0, -(2.0 * c + 1)], [1.0, 1.0], [-1.0, -1.0])])
        sums.append([c + 1.0, -(2.0 * c + 1)])
    check(orc.chain(sets, _const_rows(r0, d), gamma, eps, k, per_call=True), sums, "per-call sets")
    # a one-call chain is the fused call itself
    one = orc.chain(sets[:1], _const_rows(r0, d), gamma, eps, 1, per_call=True)
    full = orc.allreduce_rmsnorm(sets[0], _const_rows(r0, d), gamma, eps)
    assert np.array_equal(one[0]["residual_out"], full["residual_out"])
    assert np.array_equal(one[0]["y32"], full["y32"])


ALL_PINS = [
    pin_bf16_vs_torch, pin_e4m3_decode_vs_torch, pin_e4m3_rne_exact, pin_e2m1_rne_exact,
    pin_fp4_code_ties, pin_fp4_scale_ties, pin_fp4_small_random_blocks, pin_fp4_invariants,
    pin_rank_order, pin_summation_bound, pin_residual_out_is_bf16_of_h,
    pin_rmsnorm_vs_torch_f64, pin_fused_uses_fp32_h, pin_closed_forms, pin_scale_invariance,
    pin_ll_roundtrip, pin_fp8_exact, pin_patterns, pin_sentinel_pending, pin_chain,
]
