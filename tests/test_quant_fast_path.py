"""The rule behind the quantisers' encoding by reciprocal (csrc/quant.hip,
DivQuant), checked on the CPU with IEEE fp32 arithmetic.

The quantisers must produce the E4M3 code of v / s rounded to fp32 (the
oracle's division).  The kernels instead form y = v * r with r = 1 / s
rounded once, and encode y directly when it is zero, or when
2^-6 <= |y| < 464 and fp32 fraction bits 19..0 of y are more than 5 from
0x80000 (an E4M3 rounding midpoint); otherwise they divide.  The claim: y is
within 3 ulps of the rounded quotient, so wherever the rule says "direct"
both give the same code.  These tests sample quotients close to every
midpoint, under scales across the fp32 range, and check the claim, and that
the window is needed (outside it the codes do differ for some values).
"""
import numpy as np

import oracle

F32 = np.float32


def grid():
    vals = [c / 512.0 for c in range(8)]
    vals += [(1 + f / 8.0) * 2.0 ** (e - 7) for e in range(1, 16) for f in range(8) if not (e == 15 and f == 7)]
    return np.array(vals)


def direct(y):
    au = y.view(np.uint32) & np.uint32(0x7FFFFFFF)
    in_range = (au >= 0x3C800000) & (au < 0x43E80000)
    far = np.abs((au & np.uint32(0xFFFFF)).astype(np.int64) - 0x80000) > 5
    return (au == 0) | (in_range & far)


def samples(scale, rng, n_random=20000):
    g = grid()
    mids = (g[:-1] + g[1:]) / 2
    base = np.concatenate([mids, g]) * scale
    b = base.astype(F32)
    b = b[np.isfinite(b) & (b > 0)].view(np.int32)
    near = np.concatenate([(b + u).view(F32) for u in range(-12, 13)])
    rand = (rng.standard_normal(n_random) * 100 * scale).astype(F32)
    v = np.concatenate([near, -near, rand])
    return v[np.isfinite(v)]


def check_scale(s, rng):
    s = F32(s)
    r = F32(1) / s
    v = samples(float(s), rng)
    y = (v * r).astype(F32)
    q = (v / s).astype(F32)
    d = direct(y)
    enc_y, enc_q = oracle.enc_e4m3(y), oracle.enc_e4m3(q)
    assert np.array_equal(enc_y[d], enc_q[d]), (float(s), v[d][enc_y[d] != enc_q[d]][:5])
    # the product stays within 3 ulps of the quotient where both are normal and finite
    ok = np.isfinite(q) & (np.abs(q) >= F32(2.0 ** -126))
    ulps = np.abs(y[ok].view(np.int32).astype(np.int64) - q[ok].view(np.int32).astype(np.int64))
    return int(np.sum(enc_y[~d] != enc_q[~d])), int(ulps.max(initial=0))


def test_reciprocal_rule_gives_the_division_code():
    rng = np.random.default_rng(7)
    scales = [1.3, 0.0071, 97.31, 2.0, 3.0e-30, 1.0, 448.0 / 3.0, 2.0 ** 100 * 1.7, 2.0 ** -120 * 1.1]
    scales += list(np.exp(rng.uniform(np.log(2.0 ** -120), np.log(2.0 ** 110), 40)))
    differ, worst = 0, 0
    for s in scales:
        d, w = check_scale(s, rng)
        differ += d
        worst = max(worst, w)
    assert worst <= 3, worst
    # the window is not vacuous: some values near midpoints do encode differently
    assert differ > 0
