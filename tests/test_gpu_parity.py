"""GPU parity: the HIP casts against the CPU oracle on the same seeded inputs.

Pure casts (per-token E4M3/E2M1, per-block, per-channel transposed) must be
bit-exact in every code byte and every fp32 scale. The SwiGLU-fused cast uses
the hardware exponential and reciprocal, so it is held to the tolerance of
tests/swiglu_bar.py: codes at most one step apart on at most 0.1% of the
elements, scales within a relative 1e-6, dequantized values within one step
at the group abs-max (2^-3 of it for E4M3).

Every call goes through the C ABI (the ctypes binding), with outputs
poisoned beforehand so that an unwritten byte cannot pass.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_amd as pq
from precision_quantization_amd import workloads
from swiglu_bar import check_swiglu_bar

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def codes_np(t):
    return t.view(torch.uint8).cpu().numpy()


def sf_bits(t):
    return t.cpu().numpy().view(np.uint32)


def poisoned(shape, dtype, dev, byte):
    t = torch.empty(shape, dtype=dtype, device=dev)
    t.view(torch.uint8).fill_(byte)
    return t


def gpu_cast(op, x, dev, fmt="e4m3", group=128, w=None, poison=0xAA):
    """Run one cast on the GPU with poisoned outputs; numpy codes + scales."""
    xd = x.to(dev)
    rows, cols = x.shape
    code_dt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}.get(fmt, torch.uint8)
    if op == "per_token" or op == "e2m1":
        qs = (rows, cols // 2) if fmt == "e2m1" else (rows, cols)
        out = poisoned(qs, code_dt, dev, poison)
        sf = poisoned((rows, cols // group), torch.float32, dev, poison)
        if op == "e2m1":
            pq.qcast_e2m1(xd, group, out=out, out_sf=sf)
        else:
            pq.qcast_per_token(xd, fmt, group, out=out, out_sf=sf)
    elif op == "swiglu_per_token":
        n = cols // 2
        out = poisoned((rows, n), code_dt, dev, poison)
        sf = poisoned((rows, n // group), torch.float32, dev, poison)
        pq.qcast_swiglu_per_token(xd, None if w is None else w.to(dev), fmt, group, out=out,
                                  out_sf=sf)
    elif op == "per_block":
        out = poisoned((rows, cols), code_dt, dev, poison)
        sf = poisoned((rows // group, cols // group), torch.float32, dev, poison)
        pq.qcast_per_block(xd, fmt, group, out=out, out_sf=sf)
    elif op == "per_channel_T":
        out = poisoned((cols, rows), code_dt, dev, poison)
        sf = poisoned((cols, rows // group), torch.float32, dev, poison)
        pq.qcast_per_channel_T(xd, fmt, group, out=out, out_sf=sf)
    else:
        raise ValueError(op)
    torch.cuda.synchronize()
    return codes_np(out), sf.cpu().numpy()


def oracle_cast(op, x, fmt="e4m3", group=128, w=None):
    """The oracle's codes and scales for one cast on the CPU."""
    xb = workloads.bf16_bits(x)
    if op == "per_token":
        return oracle.per_token(xb, fmt, group)
    if op == "e2m1":
        return oracle.e2m1(xb, group)
    if op == "swiglu_per_token":
        return oracle.swiglu_per_token(xb, None if w is None else w.numpy(), fmt, group)
    if op == "per_block":
        return oracle.per_block(xb, fmt, group)
    if op == "per_channel_T":
        return oracle.per_channel_T(xb, fmt, group)
    raise ValueError(op)


def assert_exact(op, x, dev, fmt="e4m3", group=128, poisons=(0xAA,)):
    q_ref, sf_ref = oracle_cast(op, x, fmt, group)
    for p in poisons:
        q, sf = gpu_cast(op, x, dev, fmt, group, poison=p)
        bad = np.nonzero(q != q_ref)
        assert bad[0].size == 0, (
            f"{op} {fmt} g{group} {tuple(x.shape)}: {bad[0].size} code bytes differ, first at "
            f"{tuple(int(b[0]) for b in bad)}: gpu {q[tuple(b[0] for b in bad)]:#x} "
            f"oracle {q_ref[tuple(b[0] for b in bad)]:#x}")
        assert np.array_equal(sf.view(np.uint32), sf_ref.view(np.uint32)), \
            f"{op}: {(sf.view(np.uint32) != sf_ref.view(np.uint32)).sum()} scales differ"


# ------------------------------------------------------------ full-size workloads

def test_full_per_token_small(dev):
    wl = workloads.per_token_small()
    assert_exact("per_token", wl.x, dev, poisons=(0xAA, 0x55))


def test_full_per_token_hidden(dev):
    wl = workloads.per_token_hidden()
    assert_exact("per_token", wl.x, dev)


def test_full_e2m1(dev):
    wl = workloads.student_t()
    # the default E2M1 floor (6 * 2^-126) and a floor of 1e-4 give the same
    # result here only if no group has amax below 1e-4
    amax = wl.x.float().abs().view(wl.rows, -1, 32).amax(dim=2)
    assert (amax >= 1e-4).all()
    assert_exact("e2m1", wl.x, dev, "e2m1", 32)


def test_full_per_block(dev):
    wl = workloads.weight_block()
    assert_exact("per_block", wl.x, dev)


def test_full_per_channel_T(dev):
    wl = workloads.activation_channel()
    assert_exact("per_channel_T", wl.x, dev)


def swiglu_tolerance_check(wl, dev, q, sf, fmt="e4m3", group=128):
    """The SwiGLU bar (tests/swiglu_bar.py) against the oracle on wl."""
    q_ref, sf_ref = oracle_cast("swiglu_per_token", wl.x, fmt, group, w=wl.w)
    v = oracle.swiglu_values(workloads.bf16_bits(wl.x), None if wl.w is None else wl.w.numpy())
    return check_swiglu_bar(q, sf, q_ref, sf_ref, v, fmt, group)


def test_full_swiglu(dev):
    wl = workloads.swiglu_input()
    q, sf = gpu_cast("swiglu_per_token", wl.x, dev, w=wl.w)
    frac = swiglu_tolerance_check(wl, dev, q, sf)
    print(f"swiglu full: {frac:.5%} of codes differ from the oracle")


# ------------------------------------------------------------ small, ragged, all groups

@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e4m3", 64), ("e4m3", 32),
                                       ("e2m1", 32), ("e2m1", 64), ("e2m1", 128)])
@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 384), (127, 7168), (257, 1024)])
def test_per_token_shapes(dev, fmt, group, rows, cols):
    g = torch.Generator().manual_seed(rows * 1000 + cols)
    x = torch.randn(rows, cols, generator=g) * torch.exp(torch.randn(rows, 1, generator=g) * 4)
    assert_exact("per_token", x.to(torch.bfloat16), dev, fmt, group)


@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 384), (384, 1152), (128, 256), (640, 1280)])
def test_per_block_shapes(dev, rows, cols):
    g = torch.Generator().manual_seed(rows + cols)
    x = torch.randn(rows, cols, generator=g)
    # a different magnitude per 128 x 128 block
    x = x * torch.exp(torch.randn(rows // 128, 1, cols // 128, 1, generator=g) * 3).expand(
        rows // 128, 128, cols // 128, 128).reshape(rows, cols)
    assert_exact("per_block", x.to(torch.bfloat16), dev)


@pytest.mark.parametrize("rows,cols", [(128, 8), (128, 64), (256, 200), (384, 136), (1024, 7168)])
def test_per_channel_T_shapes(dev, rows, cols):
    g = torch.Generator().manual_seed(rows * 7 + cols)
    x = torch.randn(rows, cols, generator=g) * torch.exp(torch.randn(1, cols, generator=g) * 3)
    assert_exact("per_channel_T", x.to(torch.bfloat16), dev)


@pytest.mark.parametrize("group", [128, 64, 32])
@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("rows,cols", [(1, 128), (5, 384), (130, 2048)])
def test_swiglu_shapes(dev, group, weighted, rows, cols):
    wl = workloads.swiglu_input(seed=rows + cols, rows=rows, cols=cols, with_weight=weighted)
    q, sf = gpu_cast("swiglu_per_token", wl.x, dev, group=group, w=wl.w)
    swiglu_tolerance_check(wl, dev, q, sf, group=group)


# ------------------------------------------------------------ edge cases

def rows_of(values, cols=128):
    """bf16 tensor whose rows are `values` (each padded/cycled to `cols`)."""
    x = np.zeros((len(values), cols), np.float32)
    for r, v in enumerate(values):
        v = np.asarray(v, np.float32).ravel()
        x[r, :len(v)] = v[:cols]
    return torch.from_numpy(x).to(torch.bfloat16)


def edge_rows():
    rng = np.random.default_rng(0)
    big = float(torch.tensor([0x7F7F], dtype=torch.int16).view(torch.bfloat16).float())
    mids = np.array([1.0625, 1.1875, 17.0, 50.0, 3 * 2.0 ** -10, 2.0 ** -10], np.float32)
    return [
        np.zeros(128),                                   # zero group
        -np.zeros(128),                                  # -0 group
        np.linspace(-5e-5, 5e-5, 128),                   # floor-active (amax < 1e-4)
        np.r_[3.0, np.zeros(127)],                       # single nonzero
        np.r_[-448.0 * 4, mids * 4, -mids * 4],          # power-of-two scale: exact midpoints
        np.r_[448.0 / 8, mids / 8, -mids / 8],
        -np.abs(rng.standard_normal(128)) * 1e-3,        # tiny negatives
        np.r_[big, -big / 2, 1.0, -1.0],                 # largest bf16
        rng.standard_normal(128) * 1e30,
        rng.standard_normal(128) * 1e-30,
    ]


def test_edge_cases_per_token_e4m3(dev):
    x = rows_of(edge_rows())
    # -0.0 survives the conversion to bf16
    assert (x[1].view(torch.int16) == -32768).all()
    assert_exact("per_token", x, dev, "e4m3", 128, poisons=(0xAA, 0x55))


def test_edge_cases_per_token_e2m1(dev):
    rows = edge_rows() + [
        np.r_[2.0 ** -127, -(2.0 ** -127), 2.0 ** -125, np.zeros(29)],   # bf16 subnormals, floor active
        np.r_[2.0 ** -133, 3 * 2.0 ** -133, np.zeros(30)],
    ]
    x = rows_of(rows, 128)
    assert_exact("per_token", x, dev, "e2m1", 32, poisons=(0xAA, 0x55))
    assert_exact("per_token", x, dev, "e2m1", 128)


def test_edge_cases_other_casts(dev):
    x = rows_of(edge_rows() * 13, 256)[:128]     # 128 token rows x 256 channels
    assert_exact("per_block", x, dev)
    assert_exact("per_channel_T", x, dev)
    assert_exact("per_channel_T", x.T.contiguous()[:, :128], dev)


def test_swiglu_extremes(dev):
    g = np.array([[100.0, -100.0, -89.0, 0.0, 20.0, -3.0, 1.0, -200.0] * 16], np.float32)
    u = np.array([[1.0, 5.0, -2.0, 7.0, -1.0, 4.0, 3.0, -6.0] * 16], np.float32)
    h = torch.from_numpy(np.concatenate([g, u], axis=1)).to(torch.bfloat16)
    for w in (None, torch.tensor([0.0]), torch.tensor([0.37])):
        q, sf = gpu_cast("swiglu_per_token", h, dev, w=w)
        q_ref, sf_ref = oracle_cast("swiglu_per_token", h, w=w)
        assert np.array_equal(q, q_ref), (w, q, q_ref)
        assert np.array_equal(sf.view(np.uint32), sf_ref.view(np.uint32)), w


# ------------------------------------------------------------ exhaustive encoder sweeps

def test_every_bf16_below_448_encodes_like_the_oracle(dev):
    # A group whose abs-max is 448 has sf = 1 and sf_inv = 1 exactly, so the
    # other 127 elements are encoded as they are: this sweeps the hardware
    # conversion over every finite bf16 value of magnitude <= 448.
    bits = np.arange(0, 0x43E1, dtype=np.uint16)               # +0 .. 448
    vals = np.concatenate([bits, bits | 0x8000])
    n = len(vals)
    per_row = 127
    nrows = (n + per_row - 1) // per_row
    x = np.zeros((nrows, 128), np.uint16)
    x[:, 0] = 0x43E0                                           # 448
    flat = np.zeros(nrows * per_row, np.uint16)
    flat[:n] = vals
    x[:, 1:] = flat.reshape(nrows, per_row)
    assert_exact("per_token", workloads.bits_to_bf16(x), dev, "e4m3", 128)


def test_every_bf16_below_6_encodes_like_the_oracle_e2m1(dev):
    bits = np.arange(0, 0x40C1, dtype=np.uint16)               # +0 .. 6
    vals = np.concatenate([bits, bits | 0x8000])
    n = len(vals)
    per_row = 31
    nrows = (n + per_row - 1) // per_row
    x = np.zeros((nrows, 32), np.uint16)
    x[:, 0] = 0x40C0                                           # 6.0
    flat = np.zeros(nrows * per_row, np.uint16)
    flat[:n] = vals
    x[:, 1:] = flat.reshape(nrows, per_row)
    assert_exact("per_token", workloads.bits_to_bf16(x), dev, "e2m1", 32)


# ------------------------------------------------------------ API behaviour

def test_page_api_shapes(dev):
    # per_token_cast(x, fmt='e4m3', num_per_channels=128) on bf16 [1024, 4096]
    x = torch.randn(1024, 4096, dtype=torch.bfloat16, device=dev)
    out, out_sf = pq.per_token_cast(x, fmt="e4m3", num_per_channels=128)
    assert out.shape == (1024, 4096) and out.dtype == torch.float8_e4m3fn
    assert out_sf.shape == (1024, 32) and out_sf.dtype == torch.float32


def test_empty_input_is_a_no_op(dev):
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=dev)
    out, sf = pq.qcast_per_token(x)
    assert out.shape == (0, 256) and sf.shape == (0, 2)


def test_every_entry_point_accepts_empty_inputs(dev):
    bf = torch.bfloat16
    e = lambda r, c: torch.empty(r, c, dtype=bf, device=dev)
    assert pq.qcast_e2m1(e(0, 256), 32)[0].shape == (0, 128)
    assert pq.qcast_per_token(e(0, 256), "e5m6", 128)[0].shape == (0, 384)
    assert pq.qcast_per_token_sf(e(0, 512), "e4m3", 32, sf_flags=pq.SF_PACKED_UE8M0)[0].shape == (0, 512)
    assert pq.qcast_per_block(e(0, 256))[0].shape == (0, 256)
    assert pq.qcast_per_channel_T(e(0, 64))[0].shape == (64, 0)
    assert pq.qcast_per_channel_T(e(128, 0))[0].shape == (0, 128)
    assert pq.qcast_per_channel(e(0, 64))[0].shape == (0, 64)
    count = torch.full((1,), 7, dtype=torch.int64, device=dev)
    w = torch.empty(0, device=dev)
    assert pq.qcast_swiglu_per_token(e(0, 512), w)[0].shape == (0, 256)
    assert pq.qcast_swiglu_per_token_ex(e(0, 512), w, swiglu_clamp=1.0,
                                        clamp_count=count)[0].shape == (0, 256)
    assert pq.qcast_swiglu_per_channel_T(e(0, 512), w, swiglu_clamp=1.0,
                                         clamp_count=count)[0].shape == (256, 0)
    assert pq.qcast_swiglu_backward_per_token(e(0, 512), e(0, 256), w)[0].shape == (0, 512)
    q = torch.empty(0, 256, dtype=torch.float8_e4m3fn, device=dev)
    assert pq.qcast_cast_back(q, torch.empty(0, 2, device=dev)).shape == (0, 256)
    torch.cuda.synchronize()
    assert int(count.item()) == 7                        # untouched


def test_side_stream_and_repeat_determinism(dev):
    wl = workloads.per_token_hidden(rows=512)
    x = wl.x.to(dev)
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        a, asf = pq.qcast_per_token(x)
    s.synchronize()
    b, bsf = pq.qcast_per_token(x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)) and torch.equal(asf, bsf)


def test_binding_errors_raise(dev):
    x = torch.zeros(4, 200, dtype=torch.bfloat16, device=dev)
    with pytest.raises(pq.QcastError):
        pq.qcast_per_token(x, group=128)
    with pytest.raises(pq.QcastError):
        pq.qcast_per_block(torch.zeros(128, 128, dtype=torch.bfloat16, device=dev), block=64)


@pytest.mark.parametrize("op", ["per_token", "per_channel_T"])
def test_cu_override_does_not_change_results(dev, op):
    # The override sizes the capped grids of the counting SwiGLU casts that
    # run without a count workspace (the only launches that read it): 1, 3
    # and 256 CUs give codes and scales equal to the device's own count, bit
    # for bit, and the exact clamp count.
    wl = workloads.swiglu_input(seed=33, rows=1024, cols=2048)
    h, w = wl.x.to(dev), wl.w.to(dev)
    _, n_ref = oracle.swiglu_values_ex(workloads.bf16_bits(wl.x), wl.w.numpy(), swiglu_clamp=3.0)
    fn = pq.qcast_swiglu_per_token_ex if op == "per_token" else pq.qcast_swiglu_per_channel_T

    def run(n_cus):
        count = torch.zeros(1, dtype=torch.int64, device=dev)
        try:
            pq.qcast_set_num_cus(n_cus)
            q, sf = fn(h, w, "e4m3", 128, swiglu_clamp=3.0, clamp_count=count,
                       count_workspace=False)
        finally:
            pq.qcast_set_num_cus(0)
        torch.cuda.synchronize()
        return codes_np(q), sf.cpu().numpy().view(np.uint32), int(count.item())

    q0, sf0, n0 = run(0)
    assert n0 == n_ref > 0
    for n_cus in (1, 3, 256):
        q, sf, n = run(n_cus)
        assert np.array_equal(q, q0) and np.array_equal(sf, sf0) and n == n_ref, n_cus


def test_bench_copy_helper(dev):
    src = torch.randint(0, 256, ((1 << 20) + 48,), dtype=torch.uint8, device=dev)
    dst = torch.zeros_like(src)
    pq.qcast_bench_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


# ------------------------------------------------------------ the scale routine

@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_scale_routine_equals_ieee_division_on_every_positive_fp32(dev, fmt):
    # The kernels' short FMA sequences (and their IEEE fallback) against the
    # IEEE quotients a / fmt_max and 1 / sf, for all 2^31 - 2^23 - 1 positive
    # finite fp32 abs-maxima.
    assert pq.qcast_bench_check_scale(fmt, 1, 0x7F7FFFFF) == (0, 0)


@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e2m1", 32)])
def test_every_bf16_abs_max(dev, fmt, group):
    # One group per positive finite bf16 value v (subnormals included), with
    # v, v/2 and -v/3 in it: every abs-max a bf16 input can produce.
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    v = (bits.astype(np.uint32) << 16).view(np.float32)
    x = np.zeros((len(v), group), np.float32)
    x[:, 0] = v
    x[:, 1] = v / 2
    x[:, 2] = -v / 3
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert (xt.float().abs().amax(dim=1).numpy() == v).all()
    assert_exact("per_token", xt, dev, fmt, group)
    assert_exact("per_token", -xt, dev, fmt, group)


# Floors below fmt_max * 2^-126 take the IEEE-division fallback of the scale
# routine (3e-36 for E4M3, 5e-38 for E2M1); they are still large enough for
# 1 / sf to stay finite.
@pytest.mark.parametrize("fmt,group,clamp_min", [
    ("e4m3", 128, 0.5), ("e4m3", 128, 1e-30), ("e4m3", 128, 3e-36),
    ("e2m1", 32, 0.5), ("e2m1", 32, 1e-30), ("e2m1", 32, 5e-38)])
def test_custom_floor(dev, fmt, group, clamp_min):
    g = torch.Generator().manual_seed(17)
    x = torch.randn(64, 256, generator=g) * torch.exp(torch.randn(64, 1, generator=g) * 10)
    x[:8] = 0.0
    x = x.to(torch.bfloat16)
    q_ref, sf_ref = oracle.per_token(workloads.bf16_bits(x), fmt, group, clamp_min)
    xd = x.to(dev)
    q, sf = pq.qcast_per_token(xd, fmt, group, clamp_min=clamp_min)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(q), q_ref)
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), sf_ref.view(np.uint32))



# ------------------------------------------------------------ E5M2

@pytest.mark.parametrize("op,shape", [("per_token", (127, 7168)), ("per_block", (256, 384)),
                                      ("per_channel_T", (384, 200))])
def test_e5m2_casts(dev, op, shape):
    g = torch.Generator().manual_seed(31)
    x = torch.randn(*shape, generator=g) * torch.exp(torch.randn(shape[0], 1, generator=g) * 3)
    assert_exact(op, x.to(torch.bfloat16), dev, "e5m2", 128)


def test_e5m2_full_per_token_hidden(dev):
    assert_exact("per_token", workloads.per_token_hidden().x, dev, "e5m2", 128)


def test_every_bf16_below_57344_encodes_like_the_oracle_e5m2(dev):
    bits = np.arange(0, 0x4761, dtype=np.uint16)               # +0 .. 57344
    vals = np.concatenate([bits, bits | 0x8000])
    per_row = 127
    nrows = (len(vals) + per_row - 1) // per_row
    x = np.zeros((nrows, 128), np.uint16)
    x[:, 0] = 0x4760                                           # 57344
    flat = np.zeros(nrows * per_row, np.uint16)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(nrows, per_row)
    assert_exact("per_token", workloads.bits_to_bf16(x), dev, "e5m2", 128)


def test_e5m2_swiglu(dev):
    wl = workloads.swiglu_input(seed=40, rows=256, cols=2048)
    q, sf = gpu_cast("swiglu_per_token", wl.x, dev, "e5m2", w=wl.w)
    swiglu_tolerance_check(wl, dev, q, sf, "e5m2")


def test_scale_routine_e5m2(dev):
    assert pq.qcast_bench_check_scale("e5m2", 1, 0x7F7FFFFF) == (0, 0)


# ------------------------------------------------------------ cast_back

@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e5m2", 128), ("e2m1", 32), ("e4m3", 64)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_cast_back_parity(dev, fmt, group, out_dtype):
    g = torch.Generator().manual_seed(41)
    x = (torch.randn(257, 1024, generator=g) * torch.exp(torch.randn(257, 1, generator=g) * 4)).to(
        torch.bfloat16)
    q_ref, sf_ref = oracle.per_token(workloads.bf16_bits(x), fmt, group)
    name = "bf16" if out_dtype == torch.bfloat16 else "f32"
    ref = oracle.cast_back(q_ref, sf_ref, 1024, fmt, group, name)
    code_dt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}.get(fmt, torch.uint8)
    qd = torch.from_numpy(q_ref).to(dev).view(code_dt)
    out = torch.empty(257, 1024, dtype=out_dtype, device=dev)
    out.view(torch.uint8).fill_(0xAA)
    pq.qcast_cast_back(qd, torch.from_numpy(sf_ref).to(dev), fmt, group, out_dtype, out=out)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16 if name == "bf16" else torch.int32).numpy()
    assert np.array_equal(got.view(ref.dtype), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1"])
def test_cast_back_every_code(dev, fmt):
    # every code of the format (NaN / infinity codes excluded) with scale 1
    # and with a non-power-of-two scale
    if fmt == "e2m1":
        codes = np.arange(16, dtype=np.uint8)
        q = np.tile((codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), 4).reshape(1, 32)
        cols, group = 64, 32
    else:
        bad = {0x7F, 0xFF} if fmt == "e4m3" else set(range(0x7C, 0x80)) | set(range(0xFC, 0x100))
        codes = np.array([c for c in range(256) if c not in bad] * 4, np.uint8)[:512]
        q = codes.reshape(4, 128)
        cols, group = 128, 128
    rows = q.shape[0]
    for s in (1.0, 0.3371):
        sf = np.full((rows, cols // group), s, np.float32)
        code_dt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}.get(fmt, torch.uint8)
        out = pq.qcast_cast_back(torch.from_numpy(q).to(dev).view(code_dt),
                                 torch.from_numpy(sf).to(dev), fmt, group, torch.float32)
        torch.cuda.synchronize()
        ref = oracle.cast_back(q, sf, cols, fmt, group, "f32")
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e2m1", 32)])
def test_cast_back_round_trip_full_size(dev, fmt, group):
    # the GPU's own codes of the hidden-size workload, dequantized on the GPU
    # and by the oracle (the shapes and launches bench.py times)
    wl = workloads.per_token_hidden()
    x = wl.x.to(dev)
    q, sf = pq.qcast_per_token(x, fmt, group)
    out = pq.qcast_cast_back(q, sf, fmt, group)
    torch.cuda.synchronize()
    ref = oracle.cast_back(codes_np(q), sf.cpu().numpy(), 7168, fmt, group, "bf16")
    assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16), ref)



# ------------------------------------------------------------ scale-factor layouts

SF_FLAG_SETS = [0, pq.SF_ROUND_POW2, pq.SF_COL_MAJOR, pq.SF_ROUND_POW2 | pq.SF_COL_MAJOR,
                pq.SF_PACKED_UE8M0, pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR]


def gpu_sf_cast(x, dev, fmt, group, flags, swiglu_w=None, swiglu=False, poison=0x5A):
    rows = x.shape[0]
    cols = x.shape[1] // 2 if swiglu else x.shape[1]
    shape, dt = pq.sf_layout_shape(rows, cols, group, flags)
    sf = torch.empty(shape, dtype=dt, device=dev)
    sf.view(torch.uint8).fill_(poison)
    if swiglu:
        q, _ = pq.qcast_swiglu_per_token_sf(x.to(dev), None if swiglu_w is None else swiglu_w.to(dev),
                                            fmt, group, sf_flags=flags, out_sf=sf)
    else:
        q, _ = pq.qcast_per_token_sf(x.to(dev), fmt, group, sf_flags=flags, out_sf=sf)
    torch.cuda.synchronize()
    return codes_np(q), sf.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("flags", SF_FLAG_SETS)
@pytest.mark.parametrize("fmt,group,rows,cols", [("e4m3", 128, 127, 7168), ("e4m3", 64, 6, 1024),
                                                 ("e2m1", 32, 33, 1024), ("e5m2", 128, 5, 512)])
def test_per_token_sf_layouts(dev, flags, fmt, group, rows, cols):
    g = torch.Generator().manual_seed(rows + cols + flags)
    x = (torch.randn(rows, cols, generator=g) * torch.exp(torch.randn(rows, 1, generator=g) * 6))
    x[0, :group] = 0.0
    x = x.to(torch.bfloat16)
    q_ref, sf_ref = oracle.per_token_sf(workloads.bf16_bits(x), fmt, group, sf_flags=flags,
                                        sf_fill=0x5A5A5A5A if flags & pq.SF_PACKED_UE8M0 else
                                        np.array([0x5A5A5A5A], np.uint32).view(np.float32)[0])
    q, sf = gpu_sf_cast(x, dev, fmt, group, flags)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(sf, sf_ref.view(np.uint32))      # padding still poisoned


@pytest.mark.parametrize("group,flags", [
    (128, pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR), (32, pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR),
    (32, pq.SF_COL_MAJOR), (128, pq.SF_COL_MAJOR), (128, pq.SF_ROUND_POW2)])
def test_per_token_sf_full_size_layouts(dev, group, flags):
    """Every scale word of the 4096 x 7168 workload in each layout (no padding rows)."""
    wl = workloads.per_token_hidden()
    q_ref, sf_ref = oracle.per_token_sf(workloads.bf16_bits(wl.x), "e4m3", group, sf_flags=flags)
    q, sf = gpu_sf_cast(wl.x, dev, "e4m3", group, flags, poison=0)
    assert np.array_equal(q, q_ref) and np.array_equal(sf, sf_ref.view(np.uint32))


@pytest.mark.parametrize("flags", [pq.SF_ROUND_POW2 | pq.SF_COL_MAJOR,
                                   pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR, pq.SF_PACKED_UE8M0])
def test_swiglu_sf_layouts(dev, flags):
    wl = workloads.swiglu_input(seed=50, rows=130, cols=2048)
    q_ref, sf_ref = oracle.swiglu_per_token_sf(workloads.bf16_bits(wl.x), wl.w.numpy(),
                                               sf_flags=flags)
    q, sf = gpu_sf_cast(wl.x, dev, "e4m3", 128, flags, swiglu_w=wl.w, swiglu=True, poison=0)
    v = oracle.swiglu_values(workloads.bf16_bits(wl.x), wl.w.numpy())
    check_swiglu_bar(q, sf, q_ref, sf_ref.view(np.uint32), v, "e4m3", 128, flags,
                     what=f"swiglu layout {flags}")


# ------------------------------------------------------------ timing helper

def test_time_next_records_the_kernel(dev):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    a, b = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipEventCreateWithFlags(ctypes.byref(a), 0) == 0
    assert hip.hipEventCreateWithFlags(ctypes.byref(b), 0) == 0
    x = workloads.per_token_hidden().x.to(dev)
    torch.cuda.synchronize()
    pq.qcast_bench_time_next(a, b)
    q, sf = pq.qcast_per_token(x)
    q2, sf2 = pq.qcast_per_token(x)      # not timed: the events were taken
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    # the events bracket the kernel: 89 MB cannot move in under 2 us (44 TB/s,
    # beyond HBM and the last-level cache alike, which may hold the fresh input)
    assert 0.002 <= ms.value < 10.0
    assert torch.equal(q.view(torch.uint8), q2.view(torch.uint8))
    hip.hipEventDestroy(a)
    hip.hipEventDestroy(b)


@pytest.mark.parametrize("rows,cols", [(256, 192), (1024, 512), (16384, 7168)])
def test_per_channel_T_traffic_moves_every_vector_once(dev, rows, cols):
    # the measurement helper loads and stores what the cast does: with whole
    # channel tiles every loaded 16-byte vector lands in exactly one stored
    # one, so the XOR over all vectors is preserved; nothing past qT is written
    g = torch.Generator().manual_seed(rows + cols)
    x = torch.randn(rows, cols, generator=g).to(torch.bfloat16)
    big = torch.full((cols * rows + 4096,), 0xA5, dtype=torch.uint8, device=dev)
    out = big[:cols * rows].view(cols, rows)
    pq.qcast_bench_per_channel_T_traffic(x.to(dev), out=out)
    torch.cuda.synchronize()
    xv = x.contiguous().view(torch.int32).numpy().reshape(-1, 4)
    ov = out.view(torch.int32).cpu().numpy().reshape(-1, 4)
    assert np.array_equal(np.bitwise_xor.reduce(xv, axis=0), np.bitwise_xor.reduce(ov, axis=0))
    assert bool((big[cols * rows:] == 0xA5).all())
