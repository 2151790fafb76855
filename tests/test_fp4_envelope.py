"""The kernel's fast FP4 path equals the oracle wherever it is taken (no GPU).

The kernel converts y * r_lo and y * r_hi with gfx950's FP4 conversion,
where r_lo and r_hi are the hardware reciprocal of the block scale s (within
one ulp) moved 2^-20 down and up; where the two codes agree it keeps them,
else it falls back to exact comparisons. The conversion rounds to nearest
even with saturation and keeps the sign (a GPU probe found it equal to the
oracle's rounding around every decision point); this test takes that
rounding as the oracle's own and checks the envelope: for every positive
E4M3 scale, every decision point +-4096 ulps, both signs, and the three
reciprocals a 1-ulp instruction may return, agreement of the two codes
implies the oracle's code, and the fallback is rare away from the decision
points. s = 0 uses r = 0: every magnitude 0, sign kept."""

import numpy as np

T = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
STRICT = [True, False, True, False, True, False, True]


def rne_e2m1(q):
    """sign | E2M1 magnitude of fl32 q: ties to the even code, saturating."""
    a = np.abs(q)
    mag = np.zeros(q.shape, np.int64)
    for t, strict in zip(T, STRICT):
        mag += (a > t) if strict else (a >= t)
    return (np.signbit(q).astype(np.int64) << 3) | mag


def e4m3_positive():
    out = []
    for c in range(1, 127):
        e, m = c >> 3, c & 7
        out.append(np.float32(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)))
    return out


def envelope_codes(y, r):
    r_lo = np.float32(r * np.float32(1.0 - 2.0 ** -20))
    r_hi = np.float32(r * np.float32(1.0 + 2.0 ** -20))
    return rne_e2m1((y * r_lo).astype(np.float32)), rne_e2m1((y * r_hi).astype(np.float32))


def test_envelope_agreement_implies_the_oracle_code():
    win = 1 << 12
    checked = fallbacks = 0
    for s in e4m3_positive():
        r0 = np.float32(np.float32(1.0) / s)
        rcps = [r0, np.nextafter(r0, np.float32(0)), np.nextafter(r0, np.float32(np.inf))]
        for t in T:
            c = np.float32(s * t)
            a = (c.view(np.int32) + np.arange(-win, win + 1, dtype=np.int32)).view(np.float32)
            a = a[np.isfinite(a) & (a >= 0)]
            y = np.concatenate([a, -a]).astype(np.float32)
            want = rne_e2m1((y / s).astype(np.float32))
            for r in rcps:
                lo, hi = envelope_codes(y, r)
                agree = lo == hi
                assert np.array_equal(lo[agree], want[agree]), (s, t, r)
                checked += int(agree.sum())
                fallbacks += int((~agree).sum())
    assert checked > 40_000_000
    # inside +-4096 ulps of every decision point the fallback covers about
    # 2^-20 / 2^-23 ulps each side
    assert fallbacks < 0.01 * checked


def test_envelope_is_rarely_left_on_ordinary_values():
    rng = np.random.default_rng(3)
    y = (rng.standard_normal(1 << 20) * 3).astype(np.float32)
    for s in (np.float32(0.25), np.float32(1.125), np.float32(7.5)):
        r = np.float32(np.float32(1.0) / s)
        lo, hi = envelope_codes(y, r)
        agree = lo == hi
        assert np.array_equal(lo[agree], rne_e2m1((y / s).astype(np.float32))[agree])
        assert (~agree).mean() < 1e-4


def test_zero_scale_keeps_the_sign_only():
    y = np.array([0.0, -0.0, 1.0, -1.0, 1e-30, -1e-30, 3e38, -3e38], np.float32)
    lo, hi = envelope_codes(y, np.float32(0.0))
    assert np.array_equal(lo, hi)
    assert np.array_equal(lo, np.signbit(y).astype(np.int64) << 3)
