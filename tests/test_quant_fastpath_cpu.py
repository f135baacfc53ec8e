"""The INT8 quantisers' quotient shortcut (host check of its arithmetic).

The device quantisers (quant_codes in csrc/moe_device.h) take each quotient
x / s as t = x * r with r = 1/s correctly rounded, and fall back to the
division for any group in which some t lies within 6e-5 of a half-integer.
This checks, in IEEE binary32 on the host, that the shortcut's rint(t) equals
rint of the correctly rounded quotient whenever the fallback is not taken,
for every bf16 value |x| <= amax, over amax drawn as the quantisers meet it
(the row maximum of bf16 values) -- so that a wrong bound or threshold fails
here rather than as a rare code mismatch on the GPU.  It tests the kernel's
arithmetic, not the oracle's (which divides).
"""
import numpy as np

THRESH = np.float32(6e-5)


def _all_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def _check(amax, xs):
    amax = np.float32(amax)
    s = np.float32(amax / np.float32(127.0))
    assert np.float32(2.0 ** -125) <= s <= np.float32(2.0 ** 125)
    r = np.float32(np.float32(1.0) / s)
    x = xs[np.abs(xs) <= amax]
    exact = np.rint(x / s)                      # float32 / float32: correctly rounded
    t = (x * r).astype(np.float32)
    near = np.abs(t - np.floor(t) - np.float32(0.5)) < THRESH
    fast = np.rint(t)
    bad = ~near & (fast != exact)
    assert not bad.any(), (amax, x[bad][:4])
    return near.sum(), x.size


def test_quotient_shortcut_matches_division():
    xs = _all_bf16()
    g = np.random.default_rng(7)
    pos = xs[(xs > 0) & (xs >= np.float32(2.0 ** -118)) & (xs <= np.float32(2.0 ** 120))]
    picks = list(g.choice(pos, 160, replace=False))
    # edges: powers of two, 127 times powers of two, values that give exact ties
    picks += [np.float32(2.0 ** e) for e in (-118, -60, -8, 0, 1, 7, 60, 120)]
    picks += [np.float32(127.0 * 2.0 ** e) for e in (-100, -3, 0, 5, 100)]
    picks += [np.float32(v) for v in (1.0, 2.5, 63.5, 254.0, 3.0e38 / 1e8)]
    slow = total = 0
    for amax in picks:
        n, m = _check(amax, xs)
        slow += n
        total += m
    assert total > 1_000_000
    assert slow < total * 1e-3  # the fallback stays rare
