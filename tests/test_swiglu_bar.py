"""The SwiGLU bar helper (tests/swiglu_bar.py) on the CPU: it accepts the
oracle's own outputs, accepts the one-step differences the bar allows, and
rejects each kind of mistake planted in a copy of the oracle's outputs."""
import numpy as np
import pytest

import oracle
from precision_quantization_amd import workloads
from swiglu_bar import check_swiglu_bar, element_codes

FORMATS = [("e4m3", 128), ("e5m2", 64), ("e2m1", 32), ("e5m6", 128)]


def case(fmt, group, flags=0, rows=16, cols=512, seed=5):
    wl = workloads.swiglu_input(seed=seed, rows=rows, cols=cols)
    hb = workloads.bf16_bits(wl.x)
    w = wl.w.numpy()
    v = oracle.swiglu_values(hb, w)
    q, sf = oracle.swiglu_per_token_sf(hb, w, fmt, group, sf_flags=flags)
    return q, sf, v


def bump(q, fmt, row, col, steps):
    """Move the code of element (row, col) by `steps` magnitude steps away from zero."""
    q = q.copy()
    if fmt == "e2m1":
        b = q[row, col // 2]
        nib = (b >> (4 * (col % 2))) & 0xF
        nib = (nib & 0x8) | min((nib & 0x7) + steps, 7)
        q[row, col // 2] = (b & ~(0xF << (4 * (col % 2)))) | (nib << (4 * (col % 2)))
    elif fmt == "e5m6":
        codes = element_codes(q, fmt, q.shape[1] // 3 * 2)
        c = int(codes[row, col])
        c = (c & 0x800) | min((c & 0x7FF) + steps, 0x7BF)
        # re-pack the row's bit stream
        bits = 12 * col
        r = q[row]
        for b in range(12):
            byte, off = divmod(bits + b, 8)
            r[byte] = (r[byte] & ~(1 << off)) | (((c >> b) & 1) << off)
    else:
        c = int(q[row, col])
        q[row, col] = (c & 0x80) | min((c & 0x7F) + steps, 0x7E if fmt == "e4m3" else 0x7B)
    return q


@pytest.mark.parametrize("fmt,group", FORMATS)
def test_the_oracle_meets_the_bar_against_itself(fmt, group):
    q, sf, v = case(fmt, group)
    assert check_swiglu_bar(q, sf, q.copy(), sf.copy(), v, fmt, group) == 0.0


@pytest.mark.parametrize("fmt,group", FORMATS)
def test_one_step_on_one_code_passes_two_steps_fail(fmt, group):
    q, sf, v = case(fmt, group, rows=64, cols=2048)      # 131072 codes: 131 may differ
    # a small-magnitude element, so that one step stays inside the dequantized bound
    r, c = np.unravel_index(np.argmin(np.abs(v) + (v == 0)), v.shape)
    check_swiglu_bar(bump(q, fmt, r, c, 1), sf, q, sf, v, fmt, group)
    with pytest.raises(AssertionError, match="steps apart"):
        check_swiglu_bar(bump(q, fmt, r, c, 2), sf, q, sf, v, fmt, group)


def test_too_many_differing_codes_fail():
    q, sf, v = case("e4m3", 128, rows=8, cols=256)      # 2048 codes: at most 2 may differ
    small = np.argsort((np.abs(v) + (v == 0)).ravel())[:3]
    q2 = q
    for k in small[:2]:
        q2 = bump(q2, "e4m3", *np.unravel_index(k, v.shape), 1)
    check_swiglu_bar(q2, sf, q, sf, v)
    q3 = bump(q2, "e4m3", *np.unravel_index(small[2], v.shape), 1)
    with pytest.raises(AssertionError, match="of codes differ"):
        check_swiglu_bar(q3, sf, q, sf, v)


def test_a_scale_off_by_more_than_1e6_fails():
    q, sf, v = case("e4m3", 128)
    sf2 = sf.copy()
    sf2[3, 1] *= 1 + 2e-6
    with pytest.raises(AssertionError, match="scale relative error"):
        check_swiglu_bar(q, sf2, q, sf, v)
    sf2 = sf.copy()
    sf2[3, 1] = np.nextafter(sf2[3, 1], np.float32(1))       # one ulp: within the bar
    check_swiglu_bar(q, sf2, q, sf, v)


def test_a_large_code_step_breaks_the_dequantized_bound():
    # E5M2: a one-step move of the group's largest code is within 2^-2 of amax,
    # but rebinding the bar to E5M6's 2^-6 rejects it
    q, sf, v = case("e5m2", 64)
    r, c = np.unravel_index(np.argmax(np.abs(v[:, :64])), (v.shape[0], 64))
    q2 = bump(q, "e5m2", r, c, -1)
    check_swiglu_bar(q2, sf, q, sf, v, "e5m2", 64)
    import swiglu_bar
    saved = swiglu_bar.MANTISSA_BITS["e5m2"]
    swiglu_bar.MANTISSA_BITS["e5m2"] = 6
    try:
        with pytest.raises(AssertionError, match="dequantized"):
            check_swiglu_bar(q2, sf, q, sf, v, "e5m2", 64)
    finally:
        swiglu_bar.MANTISSA_BITS["e5m2"] = saved


@pytest.mark.parametrize("flags", [1 | 2, 4, 4 | 2])
def test_power_of_two_layouts(flags):
    q, sf, v = case("e4m3", 128, flags)
    check_swiglu_bar(q, sf, q.copy(), sf.copy(), v, "e4m3", 128, flags)
    # a scale a whole power of two off, where the unrounded scale is nowhere
    # near a power of two, is refused
    sf2 = sf.copy()
    if flags & 4:
        sf2.view(np.uint8).reshape(-1)[0] += 1
    else:
        sf2.reshape(-1)[0] *= 2
    with pytest.raises(AssertionError, match="power-of-two scale"):
        check_swiglu_bar(q, sf2, q, sf, v, "e4m3", 128, flags)
