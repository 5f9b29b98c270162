"""Pins of the oracle's casts: closed forms, invariants, identities between
the casts, and brute force on tiny inputs.

Pages (cited by title and section):
  walk  = "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限"
          §3.1 (clamp_min_value), §3.2 (per-token cast: group abs-max, scale
          and inverse, x * sf_inv), §3.3 (SwiGLU fused with the cast)
  split = "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工"
          §二 (per_block_cast, per_channel_cast (+transpose))
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from precision_quantization_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMAX = {"e4m3": 448.0, "e2m1": 6.0, "e5m2": 57344.0}
MAXCODE = {"e4m3": 0x7E, "e2m1": 0x7, "e5m2": 0x7B}
SIGN = {"e4m3": 0x80, "e2m1": 0x08, "e5m2": 0x80}


def f32(x):
    return np.float32(x)


def bf16(values):
    """fp32 values -> bf16 bit patterns (round to nearest even via torch)."""
    return workloads.bf16_bits(torch.tensor(np.asarray(values, np.float32)).to(torch.bfloat16))


def bf16_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def unpack_e2m1(q):
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def spacing(fmt, a):
    """Distance between adjacent representable magnitudes around |y| = a."""
    a = np.asarray(a, np.float64)
    if fmt == "e4m3":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
        return 2.0 ** (e - 3)
    return np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))


# ------------------------------------------------------------ page facts

def test_page_facts_floors_and_shapes():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    assert oracle.default_floor("e4m3") == f32(facts["clamp_min_value"]["e4m3"])
    p = facts["clamp_min_value"]["e2m1_max_times_pow2"]
    assert oracle.default_floor("e2m1") == f32(np.ldexp(oracle.format_max("e2m1"), p))
    api = facts["api_example"]
    x = np.zeros(api["x_shape"], np.uint16)
    q, sf = oracle.per_token(x, "e4m3", api["num_per_channels"])
    assert list(q.shape) == api["out_shape"] and list(sf.shape) == api["out_sf_shape"]


# ------------------------------------------------------------ scale

@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e5m2"])
def test_scale_closed_form(fmt):
    # sf = RN(a / M) and sf_inv = RN(1 / sf): computing the quotient in double
    # and rounding once to fp32 gives the correctly rounded fp32 quotient
    # (53 >= 2*24 + 2), so it pins the oracle's fp32 divisions.
    rng = np.random.default_rng(3)
    amax = np.concatenate([
        (10.0 ** rng.uniform(-6, 4, 3000)).astype(np.float32),
        bf16_to_f32(rng.integers(0x3000, 0x7F00, 3000).astype(np.uint16)),
    ])
    floor = oracle.default_floor(fmt)
    for a in amax:
        sf, inv = oracle.scale(fmt, a)
        aa = max(float(a), float(floor))
        assert sf == f32(aa / FMAX[fmt])
        assert inv == f32(1.0 / float(sf))


def test_zero_group_scales():
    # floor / max: E4M3 1e-4f/448 = 0x346FACAD; E2M1 6*2^-126/6 = 2^-126
    sf, _ = oracle.scale("e4m3", 0.0)
    assert np.array([sf], np.float32).view(np.uint32)[0] == 0x346FACAD
    sf, inv = oracle.scale("e2m1", 0.0)
    assert np.array([sf], np.float32).view(np.uint32)[0] == 0x00800000
    assert inv == f32(2.0 ** 126)


def test_custom_floor_replaces_default():
    sf, _ = oracle.scale("e4m3", 1e-9, clamp_min=0.5)
    assert sf == f32(0.5 / 448.0)
    sf, _ = oracle.scale("e4m3", 2.0, clamp_min=0.5)   # amax above the floor wins
    assert sf == f32(2.0 / 448.0)


# ------------------------------------------------------------ per-token cast

def small_rows(seed, rows, cols, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g) * scale
    x *= torch.exp(torch.randn(rows, 1, generator=g) * 3)  # rows over many binades
    return workloads.bf16_bits(x.to(torch.bfloat16))


@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e4m3", 32), ("e4m3", 64), ("e2m1", 32),
                                       ("e2m1", 128), ("e5m2", 128), ("e5m2", 32)])
def test_per_token_against_brute_force(fmt, group):
    """Brute force: scale from the abs-max in double, every element encoded by
    exhaustive nearest search (test_oracle_codec pins that search)."""
    from test_oracle_codec import brute_force_encode, magnitudes
    x = small_rows(5, 6, 256)
    q, sf = oracle.per_token(x, fmt, group)
    xf = bf16_to_f32(x).reshape(6, 256 // group, group)
    amax = np.abs(xf).max(axis=2).astype(np.float64)
    a = np.maximum(amax, float(oracle.default_floor(fmt)))
    sf_ref = (a / FMAX[fmt]).astype(np.float32)
    assert np.array_equal(sf.view(np.uint32), sf_ref.view(np.uint32))
    inv = (1.0 / sf_ref.astype(np.float64)).astype(np.float32)
    y = (xf.astype(np.float64) * inv[..., None].astype(np.float64)).astype(np.float32)
    codes = brute_force_encode(y.ravel(), magnitudes(fmt), SIGN[fmt]).reshape(6, 256)
    got = unpack_e2m1(q) if fmt == "e2m1" else q
    assert np.array_equal(got, codes)


@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e2m1", 32), ("e5m2", 128)])
def test_amax_element_maps_to_format_max(fmt, group):
    x = small_rows(8, 64, 512)
    q, sf = oracle.per_token(x, fmt, group)
    codes = unpack_e2m1(q) if fmt == "e2m1" else q
    xf = bf16_to_f32(x).reshape(64, -1, group)
    c = codes.reshape(64, -1, group)
    arg = np.abs(xf).argmax(axis=2)
    top = np.take_along_axis(c, arg[..., None], axis=2)[..., 0]
    sign = np.take_along_axis(xf, arg[..., None], axis=2)[..., 0] < 0
    assert np.array_equal(top, np.where(sign, MAXCODE[fmt] | SIGN[fmt], MAXCODE[fmt]))


@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e2m1", 32)])
def test_error_bound(fmt, group):
    """|x - dec(q)*sf| <= spacing(|y|)/2 * sf + 2^-21 |x| for every element."""
    x = small_rows(9, 32, 1024)
    q, sf = oracle.per_token(x, fmt, group)
    deq = oracle.dequant_per_token(q, sf, 1024, fmt, group).astype(np.float64)
    xf = bf16_to_f32(x).astype(np.float64)
    s = np.repeat(sf.astype(np.float64), group, axis=1)
    y = np.abs(xf) / s
    bound = spacing(fmt, y) / 2 * s + 2.0 ** -21 * np.abs(xf)
    assert (np.abs(xf - deq) <= bound).all()


@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e2m1", 32), ("e5m2", 128)])
def test_dequantize_requantize_idempotent(fmt, group):
    x = small_rows(10, 4, 256)
    # add a floor-active group
    x[0, :group] = bf16(np.linspace(-5e-5, 5e-5, group))
    q, sf = oracle.per_token(x, fmt, group)
    deq = oracle.dequant_per_token(q, sf, 256, fmt, group)
    q2, sf2 = oracle.per_token_f32(deq, fmt, group)
    assert np.array_equal(q2, q)
    ulp = np.abs(sf2.view(np.int32) - sf.view(np.int32))
    assert ulp.max() <= 1


@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e2m1", 32), ("e5m2", 128)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_cast_back(fmt, group, out_dtype):
    """fp32: decode(q) * sf, the product taken exactly in double and rounded
    once (both factors are fp32, so the double product is exact); bf16: that
    fp32 value through torch's float32 -> bfloat16 conversion."""
    x = small_rows(14, 8, 256)
    q, sf = oracle.per_token(x, fmt, group)
    out = oracle.cast_back(q, sf, 256, fmt, group, out_dtype)
    codes = q if fmt != "e2m1" else unpack_e2m1(q)
    dec = oracle.decode(fmt, codes).astype(np.float64)
    ref = (dec * np.repeat(sf.astype(np.float64), group, axis=1)).astype(np.float32)
    if out_dtype == "f32":
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    else:
        theirs = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(out, theirs)


def test_zero_and_negative_zero_groups():
    x = np.zeros((2, 256), np.uint16)
    x[1] = 0x8000  # -0.0
    q, sf = oracle.per_token(x, "e4m3", 128)
    assert (q[0] == 0).all() and (q[1] == 0x80).all()
    assert (sf.view(np.uint32) == 0x346FACAD).all()
    q, sf = oracle.per_token(x, "e2m1", 32)
    assert (q[0] == 0).all() and (q[1] == 0x88).all()
    assert (sf.view(np.uint32) == 0x00800000).all()
    q, sf = oracle.per_token(x, "e5m2", 128)
    assert (q[0] == 0).all() and (q[1] == 0x80).all()
    assert (sf == np.float32(np.float32(1e-4) / np.float32(57344.0))).all()


def test_power_of_two_scale_groups_hit_midpoints():
    # amax = 448 * 2^k gives sf = 2^k and sf_inv = 2^-k exactly, so x = m * 2^k
    # lands on the exact code midpoint m, which must round to the even code.
    mids = np.array([1.0625, 1.1875, 17.0, 50.0, 3 * 2.0 ** -10, 2.0 ** -10], np.float32)
    for k in (-3, 0, 5):
        row = np.zeros(128, np.float32)
        row[0] = 448.0 * 2.0 ** k
        row[1:1 + len(mids)] = mids * 2.0 ** k
        row[10:10 + len(mids)] = -mids * 2.0 ** k
        q, sf = oracle.per_token(bf16(row[None, :]), "e4m3", 128)
        assert sf[0, 0] == f32(2.0 ** k)
        expect = oracle.encode("e4m3", mids)
        assert expect.tolist() == [0x38, 0x3A, 0x58, 0x64, 0x02, 0x00]
        assert np.array_equal(q[0, 1:1 + len(mids)], expect)
        assert np.array_equal(q[0, 10:10 + len(mids)], expect | 0x80)


def test_e2m1_hand_example_and_nibble_order():
    # amax 6 -> sf = 1; codes 0.5->1, -1->0xA, 6->7, -3->0xD, 1.75->4 (tie to
    # even), 0.25->0 (tie to even); the low nibble holds the even column
    row = np.zeros(32, np.float32)
    row[:6] = [0.5, -1.0, 6.0, -3.0, 1.75, 0.25]
    q, sf = oracle.per_token(bf16(row[None, :]), "e2m1", 32)
    assert sf[0, 0] == 1.0
    assert q[0, :3].tolist() == [0x1 | (0xA << 4), 0x7 | (0xD << 4), 0x4 | (0x0 << 4)]


def test_e2m1_denormal_bf16_with_floor_active():
    # The E2M1 floor 6*2^-126 gives sf = 2^-126 and sf_inv = 2^126, so a bf16
    # subnormal 2^-127 becomes y = 0.5, code 1; fp32 denormals must be kept.
    row = np.zeros(32, np.float32)
    row[0] = 2.0 ** -127
    row[1] = -(2.0 ** -127)
    row[2] = 2.0 ** -125   # 2.0 -> code 4
    q, sf = oracle.per_token(bf16(row[None, :]), "e2m1", 32)
    assert sf[0, 0] == f32(2.0 ** -126)
    assert q[0, 0] == 0x1 | (0x9 << 4)
    assert q[0, 1] & 0xF == 0x4


def test_largest_bf16_value():
    row = np.zeros(128, np.float32)
    big = bf16_to_f32(np.array([0x7F7F], np.uint16))[0]  # ~3.39e38
    row[0], row[1] = big, -big / 2
    q, sf = oracle.per_token(bf16(row[None, :]), "e4m3", 128)
    assert q[0, 0] == 0x7E and q[0, 1] == 0xF6  # -224 -> 0xF6
    assert sf[0, 0] == f32(float(big) / 448.0)


# ------------------------------------------------------------ per-channel + transpose, per-block

def test_per_channel_T_equals_per_token_of_transpose():
    x = small_rows(12, 256, 96)
    qT, sfT = oracle.per_channel_T(x, "e4m3", 128)
    q, sf = oracle.per_token(np.ascontiguousarray(x.T), "e4m3", 128)
    assert qT.shape == (96, 256) and sfT.shape == (96, 2)
    assert np.array_equal(qT, q) and np.array_equal(sfT.view(np.uint32), sf.view(np.uint32))


def test_per_block_scale_is_max_of_row_scales_and_codes_follow():
    x = small_rows(13, 256, 384)   # 2 x 3 blocks, not square
    q, sf = oracle.per_block(x, "e4m3", 128)
    assert sf.shape == (2, 3)
    _, sf_rows = oracle.per_token(x, "e4m3", 128)  # [256, 3]
    # RN is monotone, so the block's scale is the largest of its rows' scales
    expect = sf_rows.reshape(2, 128, 3).max(axis=1)
    assert np.array_equal(sf.view(np.uint32), expect.view(np.uint32))
    xf = bf16_to_f32(x).reshape(2, 128, 3, 128)
    inv = (1.0 / sf.astype(np.float64)).astype(np.float32)
    y = (xf * inv[:, None, :, None]).astype(np.float32).reshape(256, 384)
    assert np.array_equal(q, oracle.encode("e4m3", y))


# ------------------------------------------------------------ SwiGLU

def swiglu_h(g, u):
    return bf16(np.concatenate([np.asarray(g, np.float32), np.asarray(u, np.float32)], axis=1))


def test_swiglu_large_gate_passes_through_and_negative_gate_vanishes():
    # For g >= 17, exp(-g) < 2^-24, so 1 + exp(-g) rounds to 1 and SiLU(g) = g
    # exactly; for g <= -89 exp(-g) overflows fp32 and SiLU(g) = -0.
    g = np.array([[20.0, 100.0, -110.0, 0.0, 17.0, -200.0]], np.float32)
    u = np.array([[1.0, 3.0, 2.0, 5.0, -1.0, -4.0]], np.float32)
    v = oracle.swiglu_values(swiglu_h(g, u))
    assert v.tolist() == [[20.0, 300.0, -0.0, 0.0, -17.0, 0.0]]
    assert np.signbit(v[0, 2]) and not np.signbit(v[0, 5])


def test_swiglu_known_values():
    # SiLU(x) = x * sigmoid(x): SiLU(1) = 0.7310585786, SiLU(-1) = -0.2689414214,
    # SiLU(2) = 1.7615941560 (textbook values)
    g = np.array([[1.0, -1.0, 2.0, 1.0]], np.float32)
    u = np.array([[1.0, 1.0, 1.0, 2.0]], np.float32)
    v = oracle.swiglu_values(swiglu_h(g, u))[0].astype(np.float64)
    ref = np.array([0.7310585786, -0.2689414214, 1.7615941560, 1.4621171573])
    assert np.allclose(v, ref, rtol=3e-7, atol=0)


def test_swiglu_identity_silu_x_minus_silu_neg_x():
    # SiLU(x) - SiLU(-x) = x for every x
    rng = np.random.default_rng(4)
    gv = bf16_to_f32(bf16(rng.standard_normal(2048) * 4))
    g = np.stack([gv, -gv])
    u = np.ones_like(g)
    v = oracle.swiglu_values(swiglu_h(g, u)).astype(np.float64)
    assert np.allclose(v[0] - v[1], gv, rtol=0, atol=4e-7 * np.maximum(1, np.abs(gv)).max())


def test_swiglu_weight_scales_its_own_row():
    rng = np.random.default_rng(5)
    g = rng.standard_normal((3, 256)).astype(np.float32)
    u = rng.standard_normal((3, 256)).astype(np.float32)
    h = swiglu_h(g, u)
    w = np.array([0.25, 0.5, 2.0], np.float32)   # powers of two: exact scaling
    v1 = oracle.swiglu_values(h)
    vw = oracle.swiglu_values(h, w)
    assert np.array_equal(vw, v1 * w[:, None])


def test_swiglu_zero_weight_gives_signed_zero_codes_and_floor_scale():
    rng = np.random.default_rng(6)
    g = rng.standard_normal((2, 256)).astype(np.float32)
    u = rng.standard_normal((2, 256)).astype(np.float32)
    h = swiglu_h(g, u)
    w = np.zeros(2, np.float32)
    q, sf = oracle.swiglu_per_token(h, w)
    s = oracle.swiglu_values(h)
    assert np.array_equal(q, np.where(np.signbit(s), 0x80, 0x00).astype(np.uint8))
    assert (sf.view(np.uint32) == 0x346FACAD).all()


def test_swiglu_cast_equals_per_token_of_values():
    wl = workloads.swiglu_input(seed=21, rows=16, cols=256)
    h = workloads.bf16_bits(wl.x)
    w = wl.w.numpy()
    q, sf = oracle.swiglu_per_token(h, w)
    v = oracle.swiglu_values(h, w)
    q2, sf2 = oracle.per_token_f32(v, "e4m3", 128)
    assert np.array_equal(q, q2) and np.array_equal(sf, sf2)


def test_swiglu_fp32_path_close_to_double_restatement():
    """In double precision the codes may differ only where v sits within a few
    fp32 ulps of a code midpoint: far fewer than 0.1% of the elements."""
    wl = workloads.swiglu_input(seed=22, rows=64, cols=2048)
    h = workloads.bf16_bits(wl.x)
    w = wl.w.numpy().astype(np.float64)
    hf = bf16_to_f32(h).astype(np.float64)
    g, u = hf[:, :2048], hf[:, 2048:]
    vd = g / (1.0 + np.exp(-g)) * u * w[:, None]
    v = oracle.swiglu_values(h, wl.w.numpy()).astype(np.float64)
    assert np.all(np.abs(v - vd) <= 2.0 ** -21 * np.abs(vd) + 1e-45)
    q, _ = oracle.swiglu_per_token(h, wl.w.numpy())
    qd, _ = oracle.per_token_f32(vd.astype(np.float32), "e4m3", 128)
    assert (q != qd).mean() < 1e-3


# ------------------------------------------------------------ scale-factor layouts

def pow2_ceil(sf):
    """Smallest power of two >= sf and >= 2^-126 (closed form via frexp)."""
    m, e = np.frexp(sf.astype(np.float64))
    p = np.where(m == 0.5, sf.astype(np.float64), np.ldexp(1.0, e))
    return np.maximum(p, 2.0 ** -126).astype(np.float32)


@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e2m1", 32), ("e5m2", 64)])
def test_round_sf_is_the_next_power_of_two_and_codes_follow(fmt, group):
    from test_oracle_codec import brute_force_encode, magnitudes
    x = small_rows(20, 6, 512)
    x[0, :group] = 0                                     # a floor-only group
    _, sf_plain = oracle.per_token(x, fmt, group)
    q, sf = oracle.per_token_sf(x, fmt, group, sf_flags=oracle.SF_ROUND_POW2)
    assert np.array_equal(sf, pow2_ceil(sf_plain))
    assert (sf >= sf_plain).all() and (sf < 2 * sf_plain + 2.0 ** -126).all()
    xf = bf16_to_f32(x).reshape(6, -1, group).astype(np.float64)
    y = (xf / sf[..., None].astype(np.float64)).astype(np.float32)   # exact: sf is 2^k
    assert (np.abs(y) <= FMAX[fmt]).all()                # nothing saturates
    codes = brute_force_encode(y.ravel(), magnitudes(fmt), SIGN[fmt]).reshape(6, 512)
    got = unpack_e2m1(q) if fmt == "e2m1" else q
    assert np.array_equal(got, codes)


def test_col_major_layout_is_the_padded_transpose():
    x = small_rows(21, 7, 512)                           # 7 rows -> padded to 8
    _, sf_row = oracle.per_token_sf(x, "e4m3", 128, sf_flags=0)
    _, sf_col = oracle.per_token_sf(x, "e4m3", 128, sf_flags=oracle.SF_COL_MAJOR, sf_fill=-1.0)
    assert sf_col.shape == (4, 8)
    assert np.array_equal(sf_col[:, :7], sf_row.T)
    assert (sf_col[:, 7] == -1.0).all()                 # padding untouched


def test_packed_ue8m0_hand_example_and_layouts():
    # groups with amax 448, 896, 224 and 0 give sf = 1, 2, 0.5 and the floor
    # 1e-4/448 rounded up to 2^-22: exponent bytes 127, 128, 126, 105.
    row = np.zeros(512, np.float32)
    row[0], row[128], row[256] = 448.0, 896.0, -224.0
    x = bf16(np.stack([row, row * 2]))
    _, w = oracle.per_token_sf(x, "e4m3", 128, sf_flags=oracle.SF_PACKED_UE8M0)
    assert w.shape == (2, 1) and w.dtype == np.uint32
    assert w[0, 0] == 127 | (128 << 8) | (126 << 16) | (105 << 24)
    assert w[1, 0] == 128 | (129 << 8) | (127 << 16) | (105 << 24)
    _, wc = oracle.per_token_sf(x, "e4m3", 128,
                                sf_flags=oracle.SF_PACKED_UE8M0 | oracle.SF_COL_MAJOR, sf_fill=7)
    assert wc.shape == (1, 4) and np.array_equal(wc[0, :2], w[:, 0]) and (wc[0, 2:] == 7).all()
    # packed bytes are the exponents of the round_sf scales
    x = small_rows(22, 5, 1024)
    _, sf = oracle.per_token_sf(x, "e4m3", 128, sf_flags=oracle.SF_ROUND_POW2)
    _, w = oracle.per_token_sf(x, "e4m3", 128, sf_flags=oracle.SF_PACKED_UE8M0)
    bytes_ = w.view(np.uint8).reshape(5, 8)
    assert np.array_equal(bytes_.astype(np.float64), np.log2(sf.astype(np.float64)) + 127)


def test_packed_requires_groups_divisible_by_four():
    with pytest.raises(oracle.OracleError):
        oracle.per_token_sf(small_rows(23, 2, 384), "e4m3", 128,
                            sf_flags=oracle.SF_PACKED_UE8M0)


def test_swiglu_sf_layouts_agree_with_plain_swiglu():
    wl = workloads.swiglu_input(seed=24, rows=12, cols=512)
    h, w = workloads.bf16_bits(wl.x), wl.w.numpy()
    q0, sf0 = oracle.swiglu_per_token(h, w)
    q1, sf1 = oracle.swiglu_per_token_sf(h, w, sf_flags=0)
    assert np.array_equal(q0, q1) and np.array_equal(sf0, sf1)
    _, sfc = oracle.swiglu_per_token_sf(h, w, sf_flags=oracle.SF_COL_MAJOR)
    assert np.array_equal(sfc[:, :12], sf0.T)
    qr, sfr = oracle.swiglu_per_token_sf(h, w, sf_flags=oracle.SF_ROUND_POW2)
    assert np.array_equal(sfr, pow2_ceil(sf0))
