"""Pins of the oracle's number formats against sources other than itself.

E4M3 ("fn", OCP FP8): decoded against torch's float8_e4m3fn; encoded against
torch's cast and a brute-force nearest-value search. E2M1 (OCP MX FP4): its
eight magnitudes are the format's definition (0, 0.5, 1, 1.5, 2, 3, 4, 6), and
its encoder is checked against a brute-force search. The walk-through page
"DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限", §3.1, names the
two output types float8_e4m3fn and float4_e2m1fn.
"""
import numpy as np
import pytest
import torch

import oracle

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_magnitudes_from_torch():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e5m2_magnitudes_from_torch():
    codes = torch.arange(0, 0x7C, dtype=torch.uint8)
    return codes.view(torch.float8_e5m2).to(torch.float64).numpy()


def magnitudes(fmt):
    return {"e4m3": e4m3_magnitudes_from_torch, "e5m2": e5m2_magnitudes_from_torch,
            "e2m1": lambda: E2M1_MAGNITUDES}[fmt]()


def brute_force_encode(y, magnitudes, sign_bit):
    """Nearest representable magnitude by exhaustive distance, ties to the even
    code, saturating at the largest magnitude; sign from the sign bit."""
    y = np.asarray(y, np.float32)
    a = np.abs(y.astype(np.float64))
    d = np.abs(a[:, None] - magnitudes[None, :])
    best = d.min(axis=1, keepdims=True)
    tied = d == best
    even = (np.arange(len(magnitudes)) % 2 == 0)[None, :]
    idx = np.where(tied.sum(1) > 1, np.argmax(tied & even, axis=1), np.argmin(d, axis=1))
    idx = np.where(a >= magnitudes[-1], len(magnitudes) - 1, idx)
    return (idx | np.where(np.signbit(y), sign_bit, 0)).astype(np.uint8)


def structured_fp32_sweep(max_exp_field, min_exp_field=0):
    """fp32 patterns of both signs over a range of exponent fields, with the
    top 11 mantissa bits exhaustive and the low 12 bits from a set that hits
    exact midpoints and their neighbours."""
    lows = np.array([0, 1, 0x7FF, 0x800, 0x801, 0xFFF], np.uint32)
    k = np.arange(2048, dtype=np.uint32) << 12
    e = np.arange(min_exp_field, max_exp_field + 1, dtype=np.uint32) << 23
    mant = (k[:, None] | lows[None, :]).ravel()
    bits = (e[:, None] | mant[None, :]).ravel()
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


# ---------------------------------------------------------------- decoding

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode("e4m3", codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(theirs)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), theirs[~nan].view(np.uint32))


def test_e5m2_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode("e5m2", codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float32).numpy()
    nan = np.isnan(theirs)
    assert nan.sum() == 6 and np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), theirs[~nan].view(np.uint32))
    assert np.isinf(ours[0x7C]) and ours[0x7C] > 0 and ours[0xFC] < 0
    assert oracle.format_max("e5m2") == 57344.0 and oracle.decode("e5m2", 0x01) == 2.0 ** -16


def test_e4m3_landmarks():
    # max 448, min normal 2^-6, min subnormal 2^-9 (OCP E4M3)
    assert oracle.decode("e4m3", 0x7E) == 448.0
    assert oracle.decode("e4m3", 0x08) == 2.0 ** -6
    assert oracle.decode("e4m3", 0x01) == 2.0 ** -9
    assert oracle.format_max("e4m3") == 448.0


def test_e2m1_decode_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    ours = oracle.decode("e2m1", codes).astype(np.float64)
    assert np.array_equal(ours[:8], E2M1_MAGNITUDES)
    assert np.array_equal(ours[8:], -E2M1_MAGNITUDES)
    assert np.signbit(ours[8])  # code 8 is -0
    assert oracle.format_max("e2m1") == 6.0


# ---------------------------------------------------------------- encoding

@pytest.mark.parametrize("fmt,ncodes,nan_codes", [("e4m3", 256, {0x7F, 0xFF}), ("e2m1", 16, set()),
                                                   ("e5m2", 256, {0x7C, 0x7D, 0x7E, 0x7F, 0xFC,
                                                                  0xFD, 0xFE, 0xFF})])
def test_encode_decode_roundtrip(fmt, ncodes, nan_codes):
    codes = np.array([c for c in range(ncodes) if c not in nan_codes], np.uint8)
    vals = oracle.decode(fmt, codes)
    assert np.array_equal(oracle.encode(fmt, vals), codes)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e5m2"])
def test_midpoints_tie_to_even_and_neighbours_round_to_nearer(fmt):
    mags = magnitudes(fmt)
    sign_bit = 0x08 if fmt == "e2m1" else 0x80
    lo, hi = mags[:-1], mags[1:]
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # exact in fp32
    c_lo = np.arange(len(lo))
    even = np.where(c_lo % 2 == 0, c_lo, c_lo + 1).astype(np.uint8)
    assert np.array_equal(oracle.encode(fmt, mid), even)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(oracle.encode(fmt, below), c_lo.astype(np.uint8))
    assert np.array_equal(oracle.encode(fmt, above), (c_lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.encode(fmt, -mid), even | sign_bit)


def test_e2m1_midpoint_table():
    # ties go to the even code: 0.25->0 (0), 0.75->1.0 (2), 1.25->1.0 (2),
    # 1.75->2 (4), 2.5->2 (4), 3.5->4 (6), 5->4 (6)
    y = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert oracle.encode("e2m1", y).tolist() == [0, 2, 2, 4, 4, 6, 6]


def test_e4m3_examples():
    y = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 464.0, 448.0, 224.0], np.float32)
    assert oracle.encode("e4m3", y).tolist() == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0x7E, 0x76]


@pytest.mark.parametrize("fmt,maxcode", [("e4m3", 0x7E), ("e2m1", 0x7), ("e5m2", 0x7B)])
def test_saturation(fmt, maxcode):
    m = np.float32(oracle.format_max(fmt))
    big = np.array([np.nextafter(m, np.float32(np.inf)), m * 1.5, 1e30, np.finfo(np.float32).max,
                    np.inf], np.float32)
    sign_bit = 0x08 if fmt == "e2m1" else 0x80
    assert (oracle.encode(fmt, big) == maxcode).all()
    assert (oracle.encode(fmt, -big) == (maxcode | sign_bit)).all()


@pytest.mark.parametrize("fmt,neg0,tiny", [("e4m3", 0x80, 0.0009), ("e2m1", 0x08, 0.2),
                                           ("e5m2", 0x80, 2.0 ** -18)])
def test_signed_zero(fmt, neg0, tiny):
    # `tiny` is below half the smallest nonzero magnitude (2^-10 for E4M3,
    # 0.25 for E2M1, 2^-17 for E5M2), so it rounds to a zero of its own sign
    y = np.array([0.0, -0.0, 1e-45, -1e-45, -1e-39, -tiny], np.float32)
    assert oracle.encode(fmt, y).tolist() == [0, neg0, 0, neg0, neg0, neg0]


def test_e4m3_encode_matches_torch_cast_on_sweep():
    # torch's float8_e4m3fn cast rounds to nearest even but does not saturate:
    # it is an independent reference for |y| < 464 (above, it returns NaN).
    y = structured_fp32_sweep(max_exp_field=135)  # |y| < 2^9
    rng = np.random.default_rng(7)
    rand = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    y = np.concatenate([y, rand])
    y = y[np.isfinite(y) & (np.abs(y) < 464)]
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode("e4m3", y), theirs)


def test_e4m3_encode_matches_brute_force():
    rng = np.random.default_rng(11)
    y = np.concatenate([
        (rng.standard_normal(100_000) * 10.0 ** rng.uniform(-4, 2.7, 100_000)).astype(np.float32),
        rng.uniform(-500, 500, 20_000).astype(np.float32),
    ])
    mags = e4m3_magnitudes_from_torch()
    assert np.array_equal(oracle.encode("e4m3", y), brute_force_encode(y, mags, 0x80))


def test_e2m1_encode_matches_brute_force_dense():
    # every fp32 pattern on a dense grid over [-8, 8] plus the neighbours of
    # every midpoint
    y = np.linspace(-8, 8, 400_001, dtype=np.float32)
    mids = ((E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 9)])
    y = np.concatenate([y, near, -near, structured_fp32_sweep(130, 100)])
    y = y[np.isfinite(y)]
    assert np.array_equal(oracle.encode("e2m1", y), brute_force_encode(y, E2M1_MAGNITUDES, 0x08))


def test_e5m2_encode_matches_torch_cast_on_sweep():
    # torch's float8_e5m2 cast rounds to nearest even; above 59392 (the
    # midpoint between 57344 and the infinity code) it would overflow, so the
    # comparison stays below it.
    y = structured_fp32_sweep(max_exp_field=142)  # |y| < 2^16
    rng = np.random.default_rng(8)
    rand = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    y = np.concatenate([y, rand])
    y = y[np.isfinite(y) & (np.abs(y) < 59392)]
    theirs = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode("e5m2", y), theirs)


def test_e5m2_encode_matches_brute_force():
    rng = np.random.default_rng(12)
    y = (rng.standard_normal(100_000) * 10.0 ** rng.uniform(-6, 4.8, 100_000)).astype(np.float32)
    assert np.array_equal(oracle.encode("e5m2", y), brute_force_encode(y, magnitudes("e5m2"), 0x80))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(13)
    bits = np.concatenate([
        rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32),
        # exact ties and their neighbours: low 16 bits 0x8000, 0x7FFF, 0x8001
        (rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint64).astype(np.uint32) << 16)[:, None]
        + np.array([0x7FFF, 0x8000, 0x8001], np.uint32)[None, :],
    ], axis=None).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.f32_to_bf16(f)
    theirs = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
