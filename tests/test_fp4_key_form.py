"""The kernel's packed 16-bit E2M1 decision equals the oracle's (no GPU).

The kernel compares |y| with the exact thresholds s*T through 16-bit keys:
with A the high half of |y|'s binary32 pattern, L its low half and K the
high half of s*T (whose low half is zero: s*T has at most 7 significant
bits), |y| >= s*T is A >= K and |y| > s*T is A + (L != 0) > K; A + (L != 0)
is the high half of the pattern plus 0xFFFF. Three levels of such
comparisons (t3, then t1 or t5, then t0, t2, t4 or t6) give the magnitude.

This test runs that procedure in numpy, written from the description above,
against the oracle's rule, rounding q = fl32(|y| / s) (IEEE binary32
division) to the E2M1 grid, for every positive E4M3 scale and every
threshold over +-4096 ulps of s*T, both signs, and for s = 0."""

import numpy as np

T = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
STRICT = [True, False, True, False, True, False, True]  # ties round down at .25, 1.25, 2.5, 5


def e4m3_positive():
    out = []
    for c in range(1, 127):
        e, m = c >> 3, c & 7
        out.append(np.float32(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)))
    return out


def by_quotient(y, s):
    """The oracle's rule: sign bit, then E2M1 rounding of fl32(|y| / s)."""
    a = np.abs(y)
    mag = np.zeros(y.shape, np.int64)
    if s != 0:
        q = (a / np.float32(s)).astype(np.float32)
        for t, strict in zip(T, STRICT):
            mag += (q > np.float32(t)) if strict else (q >= np.float32(t))
    return (np.signbit(y).astype(np.int64) << 3) | mag


def by_keys(y, s):
    """The kernel's procedure on 16-bit keys."""
    u = y.view(np.uint32).astype(np.int64)
    a16 = (u >> 16) & 0x7FFF
    ac16 = ((u + 0xFFFF) >> 16) & 0x7FFF
    ss = np.float32(s) if s != 0 else np.float32(np.inf)
    k = [int(np.float32(ss * np.float32(t)).view(np.uint32)) >> 16 for t in T]
    for t in T:
        low = int(np.float32(ss * np.float32(t)).view(np.uint32)) & 0xFFFF
        assert low == 0, "s*T must have a zero low half"
    b2 = a16 >= k[3]
    mid = np.where(b2, k[5], k[1])
    b1 = a16 >= mid
    tl = np.where(b2, np.where(b1, k[6], k[4]), np.where(b1, k[2], k[0]))
    b0 = ac16 > tl
    sign = (u >> 31) & 1
    return (sign << 3) | (b2.astype(np.int64) << 2) | (b1.astype(np.int64) << 1) | b0


def test_key_form_equals_quotient_rounding():
    win = 1 << 12
    checked = 0
    for s in e4m3_positive():
        for t in T:
            c = np.float32(s * np.float32(t))
            a = (c.view(np.int32) + np.arange(-win, win + 1, dtype=np.int32)).view(np.float32)
            a = a[np.isfinite(a) & (a >= 0)]
            y = np.concatenate([a, -a]).astype(np.float32)
            assert np.array_equal(by_keys(y, s), by_quotient(y, s)), (s, t)
            checked += y.size
    assert checked > 14_000_000


def test_key_form_zero_scale_and_extremes():
    y = np.array([0.0, -0.0, 1e-30, -1e-30, 3.4e38, -3.4e38, 1.0, -7.5], np.float32)
    got = by_keys(y, 0.0)
    assert np.array_equal(got, (np.signbit(y).astype(np.int64) << 3)), got
    # largest scale: everything past 5 * 448 saturates to magnitude 7
    s = np.float32(448.0)
    y = np.array([2240.0, 2240.0001, 3.0e38, -2500.0], np.float32)
    assert np.array_equal(by_keys(y, s), by_quotient(y, s))


def test_key_form_catches_a_dropped_sticky_bit():
    """The sticky term matters: without it a value just above a strict
    threshold (a tie that rounds down) would keep the lower code."""
    s = np.float32(1.0)
    y = np.array([np.nextafter(np.float32(1.25), np.float32(2))], np.float32)
    u = y.view(np.uint32).astype(np.int64)
    assert ((u + 0xFFFF) >> 16) != (u >> 16)
    assert by_keys(y, s)[0] == 3 and by_quotient(y, s)[0] == 3
