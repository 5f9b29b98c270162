"""GPU parity of every code format on the casts besides the per-token one.

The page "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工" (§四 A)
lists the SwiGLU cast in E4M3 / E5M2 / E2M1 / E5M6, per-token and
per-channel, with a matching backward; the TileKernels overview of
"DeepSeek 的 GPU 内核帝国" lists FP8 / FP4 / E5M6 at per-token, per-block and
per-channel granularity. Here the packed formats (E2M1, E5M6) go through
the per-block, per-channel (both layouts), SwiGLU (per-token, clamp and
counter, scale layouts, backward, per-channel + transpose) casts against
the oracle on the same seeded inputs:

* pure casts: every code byte and every fp32 scale bit-exact;
* SwiGLU casts: the SwiGLU bar of tests/swiglu_bar.py, clamp counts exact.

Outputs are poisoned before every call, so an unwritten byte cannot pass;
the full-size cases use the workload shapes of the hot path.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_amd as pq
from precision_quantization_amd import workloads
from swiglu_bar import check_swiglu_bar

pytestmark = pytest.mark.gpu

PACKED = ["e2m1", "e5m6"]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def bits(t):
    return workloads.bf16_bits(t)


def poisoned(shape, dtype, dev, byte=0xA5):
    t = torch.empty(shape, dtype=dtype, device=dev)
    t.view(torch.uint8).fill_(byte)
    return t


def codes_np(t):
    return t.view(torch.uint8).cpu().numpy()


def spread_rows(seed, rows, cols, col_scales=False):
    """N(0,1) scaled per row (or per column) over many binades, bf16."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g)
    shape = (1, cols) if col_scales else (rows, 1)
    x = x * torch.exp(torch.randn(*shape, generator=g) * 3)
    return x.to(torch.bfloat16)


def assert_exact(q, sf, q_ref, sf_ref, what):
    assert q.shape == q_ref.shape, what
    assert np.array_equal(q, q_ref), f"{what}: {np.mean(q != q_ref):.4%} code bytes differ"
    assert np.array_equal(sf.view(np.uint32), sf_ref.view(np.uint32)), f"{what}: scales differ"


# ------------------------------------------------------------------ per-block

def gpu_per_block(x, dev, fmt):
    rows, cols = x.shape
    q = poisoned(pq.code_shape(fmt, rows, cols), torch.uint8, dev)
    sf = poisoned((rows // 128, cols // 128), torch.float32, dev)
    pq.qcast_per_block(x.to(dev), fmt, 128, out=q, out_sf=sf)
    torch.cuda.synchronize()
    return codes_np(q), sf.cpu().numpy()


@pytest.mark.parametrize("fmt", PACKED)
@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 384), (384, 1152), (640, 1280)])
def test_per_block_shapes(dev, fmt, rows, cols):
    g = torch.Generator().manual_seed(rows + cols + len(fmt))
    x = torch.randn(rows, cols, generator=g)
    x = x * torch.exp(torch.randn(rows // 128, 1, cols // 128, 1, generator=g) * 3).expand(
        rows // 128, 128, cols // 128, 128).reshape(rows, cols)
    x[:128, :128] = 0.0                      # a floor-only block
    x = x.to(torch.bfloat16)
    q, sf = gpu_per_block(x, dev, fmt)
    assert_exact(q, sf, *oracle.per_block(bits(x), fmt, 128), f"per_block {fmt} {rows}x{cols}")


def test_per_block_e2m1_full_size(dev):
    wl = workloads.weight_block()            # W [7168, 18432]
    q, sf = gpu_per_block(wl.x, dev, "e2m1")
    assert_exact(q, sf, *oracle.per_block(bits(wl.x), "e2m1", 128), "per_block e2m1 full")


def test_per_block_e5m6_full_size_sampled(dev):
    # every 7th row of 128 x 128 blocks, and the last, of the full weight
    wl = workloads.weight_block()
    rows = wl.x.shape[0]
    q, sf = gpu_per_block(wl.x, dev, "e5m6")
    brows = np.unique(np.r_[np.arange(0, rows // 128, 7), rows // 128 - 1])
    sel = (brows[:, None] * 128 + np.arange(128)[None, :]).ravel()
    q_ref, sf_ref = oracle.per_block(bits(wl.x[sel]), "e5m6", 128)
    assert_exact(q[sel], sf[brows], q_ref, sf_ref, "per_block e5m6 full, sampled")


# ---------------------------------------------------------- per-channel (T)

def gpu_per_channel_T(x, dev, fmt, byte=0xA5):
    rows, cols = x.shape
    q = poisoned(pq.code_shape(fmt, cols, rows), torch.uint8, dev, byte)
    sf = poisoned((cols, rows // 128), torch.float32, dev, byte)
    pq.qcast_per_channel_T(x.to(dev), fmt, 128, out=q, out_sf=sf)
    torch.cuda.synchronize()
    return codes_np(q), sf.cpu().numpy()


def gpu_per_channel(x, dev, fmt):
    rows, cols = x.shape
    q = poisoned(pq.code_shape(fmt, rows, cols), torch.uint8, dev)
    sf = poisoned((rows // 128, cols), torch.float32, dev)
    pq.qcast_per_channel(x.to(dev), fmt, 128, out=q, out_sf=sf)
    torch.cuda.synchronize()
    return codes_np(q), sf.cpu().numpy()


@pytest.mark.parametrize("fmt", PACKED)
@pytest.mark.parametrize("rows,cols", [(128, 8), (128, 64), (256, 200), (384, 136),
                                       (1024, 7168), (2048, 520)])
def test_per_channel_T_shapes(dev, fmt, rows, cols):
    x = spread_rows(rows * 7 + cols, rows, cols, col_scales=True)
    x[:128, 0] = 0.0                         # a floor-only group
    for byte in (0xA5, 0x5A):
        q, sf = gpu_per_channel_T(x, dev, fmt, byte)
        assert_exact(q, sf, *oracle.per_channel_T(bits(x), fmt, 128),
                     f"per_channel_T {fmt} {rows}x{cols}")


def test_per_channel_T_e2m1_full_size(dev):
    wl = workloads.activation_channel()      # A [16384, 7168]
    q, sf = gpu_per_channel_T(wl.x, dev, "e2m1")
    assert_exact(q, sf, *oracle.per_channel_T(bits(wl.x), "e2m1", 128), "per_channel_T e2m1 full")


def test_per_channel_T_e5m6_full_size_sampled(dev):
    # every channel of 1 in 61, and the last one, at the full shape
    wl = workloads.activation_channel()
    rows, cols = wl.x.shape
    q, sf = gpu_per_channel_T(wl.x, dev, "e5m6")
    chans = np.unique(np.r_[np.arange(0, cols, 61), cols - 1])
    q_ref, sf_ref = oracle.per_channel_T(bits(wl.x[:, chans]), "e5m6", 128)
    assert_exact(q[chans], sf[chans], q_ref, sf_ref, "per_channel_T e5m6 full, sampled")


def test_per_channel_e2m1_full_size(dev):
    wl = workloads.activation_channel()      # A [16384, 7168], codes in the input layout
    q, sf = gpu_per_channel(wl.x, dev, "e2m1")
    assert_exact(q, sf, *oracle.per_channel(bits(wl.x), "e2m1", 128), "per_channel e2m1 full")


@pytest.mark.parametrize("fmt", PACKED)
@pytest.mark.parametrize("rows,cols", [(128, 8), (256, 264), (384, 1024), (1024, 7168)])
def test_per_channel_shapes(dev, fmt, rows, cols):
    x = spread_rows(rows * 3 + cols, rows, cols, col_scales=True)
    q, sf = gpu_per_channel(x, dev, fmt)
    assert_exact(q, sf, *oracle.per_channel(bits(x), fmt, 128), f"per_channel {fmt} {rows}x{cols}")


# ------------------------------------------------------------- SwiGLU casts

def gpu_swiglu_ex(wl, dev, fmt, group, clamp=0.0, flags=0, count=None, ws=None):
    rows, n = wl.rows, wl.cols
    q = poisoned(pq.code_shape(fmt, rows, n), torch.uint8, dev)
    shape, dt = pq.sf_layout_shape(rows, n, group, flags)
    sf = poisoned(shape, dt, dev)
    pq.qcast_swiglu_per_token_ex(wl.x.to(dev), None if wl.w is None else wl.w.to(dev), fmt,
                                 group, sf_flags=flags, swiglu_clamp=clamp, clamp_count=count,
                                 out=q, out_sf=sf, count_workspace=ws)
    torch.cuda.synchronize()
    return codes_np(q), sf.cpu().numpy()


@pytest.mark.parametrize("fmt,group", [("e2m1", 32), ("e2m1", 64), ("e2m1", 128),
                                       ("e5m6", 128), ("e5m6", 32)])
@pytest.mark.parametrize("rows,cols,weighted", [(1, 128, True), (5, 384, False),
                                                (130, 2048, True), (67, 1920, False)])
def test_swiglu_per_token_shapes(dev, fmt, group, rows, cols, weighted):
    wl = workloads.swiglu_input(seed=rows + cols + group, rows=rows, cols=cols,
                                with_weight=weighted)
    w = None if wl.w is None else wl.w.numpy()
    q, sf = gpu_swiglu_ex(wl, dev, fmt, group)
    q_ref, sf_ref = oracle.swiglu_per_token(bits(wl.x), w, fmt, group)
    v = oracle.swiglu_values(bits(wl.x), w)
    check_swiglu_bar(q, sf, q_ref, sf_ref, v, fmt, group, what=f"swiglu {fmt} g{group}")


@pytest.mark.parametrize("fmt,group", [("e2m1", 32), ("e5m6", 128)])
def test_swiglu_per_token_full_size(dev, fmt, group):
    wl = workloads.swiglu_input()             # H [8192, 4096] -> [8192, 2048]
    q, sf = gpu_swiglu_ex(wl, dev, fmt, group)
    q_ref, sf_ref = oracle.swiglu_per_token(bits(wl.x), wl.w.numpy(), fmt, group)
    v = oracle.swiglu_values(bits(wl.x), wl.w.numpy())
    frac = check_swiglu_bar(q, sf, q_ref, sf_ref, v, fmt, group, what=f"swiglu {fmt} full")
    print(f"swiglu {fmt} g{group} full: {frac:.5%} of codes differ from the oracle")


@pytest.mark.parametrize("fmt,group,flags", [
    ("e2m1", 32, pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR), ("e2m1", 32, pq.SF_ROUND_POW2),
    ("e5m6", 128, pq.SF_COL_MAJOR), ("e2m1", 64, pq.SF_PACKED_UE8M0)])
@pytest.mark.parametrize("ws", [None, False])
def test_swiglu_clamp_count_and_layouts(dev, fmt, group, flags, ws):
    wl = workloads.swiglu_input(seed=77, rows=257, cols=1024)
    clamp = 3.0
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    q, sf = gpu_swiglu_ex(wl, dev, fmt, group, clamp, flags, count, ws)
    q_ref, sf_ref, n_ref = oracle.swiglu_per_token_ex(bits(wl.x), wl.w.numpy(), fmt, group,
                                                      sf_flags=flags, swiglu_clamp=clamp)
    assert int(count.item()) == n_ref > 0
    v, _ = oracle.swiglu_values_ex(bits(wl.x), wl.w.numpy(), swiglu_clamp=clamp)
    check_swiglu_bar(q, sf, q_ref, sf_ref, v, fmt, group, flags,
                     what=f"swiglu clamp {fmt} g{group} flags {flags}")


def gpu_swiglu_T(wl, dev, fmt, clamp=0.0, count=None, ws=None):
    rows, n = wl.rows, wl.cols
    q = poisoned(pq.code_shape(fmt, n, rows), torch.uint8, dev)
    sf = poisoned((n, rows // 128), torch.float32, dev)
    pq.qcast_swiglu_per_channel_T(wl.x.to(dev), None if wl.w is None else wl.w.to(dev), fmt,
                                  128, swiglu_clamp=clamp, clamp_count=count, out=q, out_sf=sf,
                                  count_workspace=ws)
    torch.cuda.synchronize()
    return codes_np(q), sf.cpu().numpy()


@pytest.mark.parametrize("fmt", PACKED)
@pytest.mark.parametrize("clamp", [0.0, 2.5])
@pytest.mark.parametrize("ws", [None, False])
@pytest.mark.parametrize("rows,cols,weighted", [(128, 8, True), (256, 200, False),
                                                (384, 136, True), (1024, 2048, True)])
def test_swiglu_per_channel_T_shapes(dev, fmt, clamp, ws, rows, cols, weighted):
    wl = workloads.swiglu_input(seed=rows + 3 * cols, rows=rows, cols=cols, with_weight=weighted)
    w = None if wl.w is None else wl.w.numpy()
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    q, sf = gpu_swiglu_T(wl, dev, fmt, clamp, count, ws)
    q_ref, sf_ref = oracle.swiglu_per_channel_T(bits(wl.x), w, fmt, 128, swiglu_clamp=clamp)
    v, n_ref = oracle.swiglu_values_ex(bits(wl.x), w, swiglu_clamp=clamp)
    check_swiglu_bar(q, sf, q_ref, sf_ref, v.T, fmt, 128,
                     what=f"swiglu_T {fmt} c{clamp} {rows}x{cols}")
    assert int(count.item()) == n_ref


@pytest.mark.parametrize("fmt", PACKED)
def test_swiglu_per_channel_T_full_size(dev, fmt):
    wl = workloads.swiglu_input()
    q, sf = gpu_swiglu_T(wl, dev, fmt)
    q_ref, sf_ref = oracle.swiglu_per_channel_T(bits(wl.x), wl.w.numpy(), fmt, 128)
    v = oracle.swiglu_values(bits(wl.x), wl.w.numpy())
    frac = check_swiglu_bar(q, sf, q_ref, sf_ref, v.T, fmt, 128, what=f"swiglu_T {fmt} full")
    print(f"swiglu + transpose {fmt} full: {frac:.5%} of codes differ from the oracle")


@pytest.mark.parametrize("fmt,group", [("e2m1", 32), ("e2m1", 128), ("e5m6", 128),
                                       ("e5m6", 64)])
@pytest.mark.parametrize("clamp", [0.0, 3.0])
@pytest.mark.parametrize("rows,cols", [(1, 128), (130, 2048)])
def test_swiglu_backward_shapes(dev, fmt, group, clamp, rows, cols):
    h, dv, w = workloads.swiglu_grad(seed=rows + cols + group, rows=rows, cols=cols)
    q = poisoned(pq.code_shape(fmt, rows, 2 * cols), torch.uint8, dev)
    sf = poisoned((rows, 2 * cols // group), torch.float32, dev)
    pq.qcast_swiglu_backward_per_token(h.to(dev), dv.to(dev), w.to(dev), fmt, group,
                                       swiglu_clamp=clamp, out=q, out_sf=sf)
    torch.cuda.synchronize()
    q_ref, sf_ref = oracle.swiglu_backward_per_token(bits(h), bits(dv), w.numpy(), fmt, group,
                                                     swiglu_clamp=clamp)
    v = oracle.swiglu_backward_values(bits(h), bits(dv), w.numpy(), swiglu_clamp=clamp)
    check_swiglu_bar(codes_np(q), sf.cpu().numpy(), q_ref, sf_ref, v, fmt, group,
                     what=f"backward {fmt} g{group} c{clamp}")


def test_swiglu_backward_e2m1_full_size(dev):
    # the 8192 x 2048 gradient in E2M1 with 1 x 32 groups and clamp 6
    h, dv, w = workloads.swiglu_grad()
    rows, cols = dv.shape
    q = poisoned(pq.code_shape("e2m1", rows, 2 * cols), torch.uint8, dev)
    sf = poisoned((rows, 2 * cols // 32), torch.float32, dev)
    pq.qcast_swiglu_backward_per_token(h.to(dev), dv.to(dev), w.to(dev), "e2m1", 32,
                                       swiglu_clamp=6.0, out=q, out_sf=sf)
    torch.cuda.synchronize()
    q_ref, sf_ref = oracle.swiglu_backward_per_token(bits(h), bits(dv), w.numpy(), "e2m1", 32,
                                                     swiglu_clamp=6.0)
    v = oracle.swiglu_backward_values(bits(h), bits(dv), w.numpy(), swiglu_clamp=6.0)
    frac = check_swiglu_bar(codes_np(q), sf.cpu().numpy(), q_ref, sf_ref, v, "e2m1", 32,
                            what="backward e2m1 g32 full")
    print(f"swiglu backward e2m1 full: {frac:.5%} of codes differ from the oracle")
