"""The divisionless rule the 2-bit value encoder uses, against fp32 division.

The encoder finds q = clamp(rint(fl32(d / s)), 0, 3) (d = fl32(v - z16), s the
stored fp16 scale, rint ties to even) as the number of three per-group
thresholds that d reaches: the least floats d with d / s > 1/2 + 2^-25,
d / s >= 3/2 - 2^-24 and d / s > 5/2 + 2^-23, each product formed exactly in
fp64.  This checks that rule, written out here in numpy, against numpy's
correctly rounded fp32 division for every positive finite fp16 scale, at the
floats around every threshold and rounding boundary, at random d and at the
special values.  (The GPU tests check the encoder's codes bit for bit against
the oracle.)  Each boundary is an odd 25-bit number over a power of two, so its
product with an fp16 scale is never a float: d never sits exactly on one, and
whether a threshold is the least float >= or > the product makes no difference.
"""

import numpy as np

f32, f64 = np.float32, np.float64


def _next_up(t):
    return (t.view(np.uint32) + np.uint32(1)).view(f32)


def _least_ge(p):
    t = p.astype(f32)
    return np.where(t.astype(f64) < p, _next_up(t), t)


def _least_gt(p):
    t = p.astype(f32)
    return np.where(t.astype(f64) <= p, _next_up(t), t)


def _by_division(d, s):
    with np.errstate(all="ignore"):
        r = (d / s).astype(f32)
        q = np.clip(np.rint(r), 0, 3)
    return np.where(np.isnan(q), 0, q).astype(np.int32)


def test_threshold_rule_equals_division():
    s = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(f32)[:, None]
    s64 = s.astype(f64)
    t1 = _least_gt((0.5 + 2.0 ** -25) * s64)
    t2 = _least_ge((1.5 - 2.0 ** -24) * s64)
    t3 = _least_gt((2.5 + 2.0 ** -23) * s64)

    def rule(d):
        return (d >= t1).astype(np.int32) + (d >= t2) + (d >= t3)

    rng = np.random.default_rng(11)
    probes = []
    for p in (t1, t2, t3, (0.5 * s64).astype(f32), (1.5 * s64).astype(f32),
              (2.5 * s64).astype(f32)):
        u = p.view(np.uint32).astype(np.int64)
        probes.append((u + np.arange(-4, 5)).astype(np.uint32).view(f32))
    probes.append((rng.uniform(-0.5, 3.6, size=(s.shape[0], 48)) * s64).astype(f32))
    probes.append(np.broadcast_to(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45,
                                            3e38], f32), (s.shape[0], 8)))
    for d in probes:
        bad = np.argwhere(rule(d) != _by_division(d, s))
        assert bad.size == 0, f"s={s[bad[0][0], 0]!r} d={d[tuple(bad[0])]!r}"
