"""Pin of the oracle's fp32 exponential, the one inside SiLU
(DeepSeek开源TileKernels walk-through, §3.3: SiLU is g / (1 + exp(-g))).

The oracle reads that exponential as e^x rounded once to the nearest fp32 value.
The reference here is Python's decimal module, whose exp() is correctly rounded
to the context precision (60 digits): the expected fp32 value is the candidate
nearest to that decimal, compared exactly. No step shares code with the oracle.
"""
from decimal import Decimal, localcontext

import numpy as np
import pytest

import oracle

# Halfway between FLT_MAX = 2^128 - 2^104 and 2^128: at or above it, rounding
# to nearest overflows (FLT_MAX has an odd significand, so the tie goes up).
OVERFLOW_MID = Decimal(2) ** 128 - Decimal(2) ** 103


def cr_exp_f32(x):
    """The fp32 value nearest to e^x, from a 60-digit correctly rounded decimal."""
    with localcontext() as ctx:
        ctx.prec = 60
        e = Decimal(float(x)).exp()
        if e >= OVERFLOW_MID:
            return np.float32(np.inf)
        with np.errstate(over="ignore"):
            f0 = np.float32(float(e))
        cands = [f0, np.nextafter(f0, np.float32(-np.inf)), np.nextafter(f0, np.float32(np.inf))]
        cands = [c for c in cands if np.isfinite(c) and c >= 0]
        return min(cands, key=lambda c: abs(Decimal(float(c)) - e))


def bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def check(xs):
    xs = np.asarray(xs, dtype=np.float32)
    got = oracle.exp_f32(xs)
    want = np.array([cr_exp_f32(x) for x in xs], dtype=np.float32)
    bad = np.nonzero(bits(got) != bits(want))[0]
    assert bad.size == 0, [(float(xs[i]), float(got[i]), float(want[i])) for i in bad[:5]]


def test_exp_special_values():
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    xs = np.array([0.0, -0.0, tiny, -tiny, 1.0, -1.0, 0.5, 2.0, 10.0, -10.0], np.float32)
    got = oracle.exp_f32(xs)
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 and got[3] == 1.0
    check(xs)
    # Limits: e^+inf overflows, e^-inf is 0, NaN stays NaN.
    lim = oracle.exp_f32(np.array([np.inf, -np.inf, np.nan], np.float32))
    assert np.isposinf(lim[0]) and lim[1] == 0.0 and np.isnan(lim[2])


def test_exp_overflow_and_underflow_edges():
    # ln(FLT_MAX + 2^103) = 88.72283906...; ln(2^-150) = -103.97207708...
    # The fp32 neighbours of both thresholds straddle them.
    hi = np.float32(88.72283)
    lo = np.float32(-103.97209)
    xs = [hi]
    for _ in range(4):
        xs.append(np.nextafter(xs[-1], np.float32(np.inf)))
    ys = [lo]
    for _ in range(4):
        ys.append(np.nextafter(ys[-1], np.float32(np.inf)))
    xs = np.array(xs + ys, np.float32)
    got = oracle.exp_f32(xs)
    assert np.isfinite(got[0]) and np.isposinf(got[4])  # crosses into overflow
    assert got[5] == 0.0 and got[9] > 0.0                # crosses out of underflow to 0
    check(xs)


def test_exp_seeded_sample_over_the_range():
    """20,000 fp32 inputs drawn uniformly over the bit patterns of [-104, 89]:
    every binade from the subnormals up is sampled."""
    rng = np.random.default_rng(20260)
    n = 20_000
    neg_hi = np.float32(104.0).view(np.uint32)
    pos_hi = np.float32(89.0).view(np.uint32)
    neg = rng.integers(0, neg_hi, n // 2, dtype=np.uint32).view(np.float32) * np.float32(-1)
    pos = rng.integers(0, pos_hi, n - n // 2, dtype=np.uint32).view(np.float32)
    check(np.concatenate([neg, pos]))


def test_exp_inputs_next_to_rounding_midpoints():
    """The inputs whose e^x lies closest to a midpoint between two fp32 values
    (found among 4M seeded inputs in the SiLU range) are where an exponential
    that is accurate to within an ulp, but not correctly rounded, goes wrong."""
    rng = np.random.default_rng(77)
    x = rng.uniform(-40.0, 40.0, 1 << 22).astype(np.float32)
    d = np.exp(x.astype(np.float64))
    f = d.astype(np.float32).astype(np.float64)
    up = d > f
    nb = np.where(up, np.nextafter(f.astype(np.float32), np.float32(np.inf)),
                  np.nextafter(f.astype(np.float32), np.float32(0))).astype(np.float64)
    mid = 0.5 * (f + nb)
    rel = np.abs(d - mid) / mid
    rel[d == f] = np.inf
    near = x[np.argsort(rel)[:300]]
    check(near)


@pytest.mark.parametrize("g", [-30.0, -3.0, -0.25, 0.0, 0.25, 3.0, 30.0])
def test_silu_uses_this_exponential(g):
    """The SwiGLU oracle's SiLU(g) * 1 is g / (1 + exp_f32(-g)) in single fp32
    operations (u = 1, no weight): the pinned exponential is the one it uses."""
    gb = np.float32(g)
    h = np.array([[gb.view(np.uint32) >> 16, np.float32(1.0).view(np.uint32) >> 16]],
                 dtype=np.uint32).astype(np.uint16)
    v = oracle.swiglu_values(h)
    e = oracle.exp_f32(np.array([-gb], np.float32))[0]
    expect = np.float32(gb / (np.float32(1.0) + e))
    assert bits(v[0, 0]) == bits(expect)
