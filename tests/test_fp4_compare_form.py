"""The kernel's division-free E2M1 decision equals the oracle's (no GPU).

The oracle rounds q = fl32(|y| / s) (IEEE binary32 division) to the E2M1
grid: magnitude = [q > .25] + [q >= .75] + [q > 1.25] + [q >= 1.75] +
[q > 2.5] + [q >= 3.5] + [q > 5] (ties to the even code). The kernel compares
|y| with the products s*T instead, which are exact in binary32 (s has 4
significant bits, T at most 3). Both decisions can only differ where the
quotient's rounding (at most half an ulp, 2^-24 relative) carries it across
T, i.e. for |y| within a couple of ulps of s*T. This test checks every
positive E4M3 scale and every threshold over +-4096 ulps of s*T with numpy's
IEEE float32 division: a window far wider than the region where a
difference is possible, so the two decisions agree for every finite |y|."""

import numpy as np

THRESHOLDS = [(0.25, True), (0.75, False), (1.25, True), (1.75, False), (2.5, True), (3.5, False),
              (5.0, True)]  # (T, strict): strict means q > T (a tie rounds down to the even code)


def e4m3_positive():
    out = []
    for c in range(1, 127):
        e, m = c >> 3, c & 7
        out.append(np.float32(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)))
    return out


def test_compare_form_equals_quotient_rounding():
    win = 1 << 12
    checked = 0
    for s in e4m3_positive():
        for th, strict in THRESHOLDS:
            c = np.float32(s * np.float32(th))
            assert float(c) == float(s) * th, "s*T must be exact"
            a = (c.view(np.int32) + np.arange(-win, win + 1, dtype=np.int32)).view(np.float32)
            a = a[np.isfinite(a) & (a >= 0)]
            q = a / s
            by_quotient = (q > np.float32(th)) if strict else (q >= np.float32(th))
            by_compare = (a > c) if strict else (a >= c)
            assert np.array_equal(by_quotient, by_compare), (s, th)
            checked += a.size
    assert checked > 7_000_000
