"""GPU parity of the SwiGLU variants and of the per-channel cast without
transpose, against the CPU oracle on the same seeded inputs.

* per-channel cast (input layout): bit-exact codes and scales.
* clamp counter: exactly the oracle's count (it is decided by comparisons of
  the bf16 inputs with the bound).
* SwiGLU forward with clamp, SwiGLU backward, SwiGLU + per-channel +
  transpose: these use the hardware exponential and reciprocal, so they are
  held to the SwiGLU bar of tests/swiglu_bar.py: codes at most one step apart
  on at most 0.1% of the elements, scales within a relative 1e-6,
  dequantized values within one step at the group abs-max.

Every call goes through the C ABI with poisoned outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_amd as pq
from precision_quantization_amd import workloads
from swiglu_bar import check_swiglu_bar

pytestmark = pytest.mark.gpu

CODE_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def poisoned(shape, dtype, dev, byte=0xA5):
    t = torch.empty(shape, dtype=dtype, device=dev)
    t.view(torch.uint8).fill_(byte)
    return t


def codes_np(t):
    return t.view(torch.uint8).cpu().numpy()




def bits(t):
    return workloads.bf16_bits(t)


# ------------------------------------------------- per-channel, input layout

def gpu_per_channel(x, dev, fmt):
    rows, cols = x.shape
    out = poisoned((rows, cols), CODE_DT[fmt], dev)
    sf = poisoned((rows // 128, cols), torch.float32, dev)
    pq.qcast_per_channel(x.to(dev), fmt, 128, out=out, out_sf=sf)
    torch.cuda.synchronize()
    return codes_np(out), sf.cpu().numpy()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols", [(128, 8), (128, 256), (256, 200), (384, 136),
                                       (128, 264), (1024, 7168)])
def test_per_channel_shapes(dev, fmt, rows, cols):
    g = torch.Generator().manual_seed(rows * 3 + cols)
    # per-channel magnitudes spread over many octaves, one channel all zero
    x = torch.randn(rows, cols, generator=g) * torch.exp(torch.randn(1, cols, generator=g) * 3)
    x[:, 0] = 0.0
    x = x.to(torch.bfloat16)
    q_ref, sf_ref = oracle.per_channel(bits(x), fmt)
    q, sf = gpu_per_channel(x, dev, fmt)
    assert np.array_equal(q, q_ref), f"{(q != q_ref).sum()} codes differ"
    assert np.array_equal(sf.view(np.uint32), sf_ref.view(np.uint32))


def test_per_channel_full_size(dev):
    wl = workloads.activation_channel()
    q_ref, sf_ref = oracle.per_channel(bits(wl.x))
    q, sf = gpu_per_channel(wl.x, dev, "e4m3")
    assert np.array_equal(q, q_ref)
    assert np.array_equal(sf.view(np.uint32), sf_ref.view(np.uint32))


def test_per_channel_equals_transpose_of_per_channel_T_on_gpu(dev):
    wl = workloads.activation_channel(seed=9, rows=512, cols=1024)
    xd = wl.x.to(dev)
    q, sf = pq.qcast_per_channel(xd)
    qT, sfT = pq.qcast_per_channel_T(xd)
    assert torch.equal(q.view(torch.uint8), qT.view(torch.uint8).t())
    assert torch.equal(sf, sfT.t())


# ------------------------------------------------- SwiGLU forward with clamp

# How the clamp count reaches the counter: through the binding's own
# workspace per stream (the default), with one atomic per workgroup of a
# capped grid (no workspace), or through a workspace the caller passes.
WS_MODES = ["default", "direct", "caller"]


def count_workspace(mode, dev):
    if mode == "default":
        return None
    if mode == "direct":
        return False
    return torch.zeros(pq.COUNT_WS_BYTES // 8, dtype=torch.int64, device=dev)


def gpu_swiglu_ex(wl, dev, clamp, flags=0, fmt="e4m3", group=128, count=None, ws=None):
    rows, n = wl.rows, wl.cols
    out = poisoned((rows, n), CODE_DT[fmt], dev)
    shape, dt = pq.sf_layout_shape(rows, n, group, flags)
    sf = poisoned(shape, dt, dev)
    pq.qcast_swiglu_per_token_ex(wl.x.to(dev), None if wl.w is None else wl.w.to(dev), fmt,
                                 group, sf_flags=flags, swiglu_clamp=clamp, clamp_count=count,
                                 out=out, out_sf=sf, count_workspace=ws)
    torch.cuda.synchronize()
    return codes_np(out), sf.cpu().numpy()


@pytest.mark.parametrize("ws_mode", WS_MODES)
@pytest.mark.parametrize("clamp", [1.5, 4.0, 7.0])
@pytest.mark.parametrize("weighted", [True, False])
def test_swiglu_clamp_parity_and_count(dev, clamp, weighted, ws_mode):
    wl = workloads.swiglu_input(seed=71, rows=257, cols=1024, with_weight=weighted)
    w = None if wl.w is None else wl.w.numpy()
    q_ref, sf_ref, n_ref = oracle.swiglu_per_token_ex(bits(wl.x), w, swiglu_clamp=clamp)
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = count_workspace(ws_mode, dev)
    q, sf = gpu_swiglu_ex(wl, dev, clamp, count=count, ws=ws)
    assert int(count.item()) == n_ref > 0
    v, _ = oracle.swiglu_values_ex(bits(wl.x), w, swiglu_clamp=clamp)
    check_swiglu_bar(q, sf, q_ref, sf_ref, v, what=f"clamp {clamp}")
    # the counter accumulates over calls
    gpu_swiglu_ex(wl, dev, clamp, count=count, ws=ws)
    assert int(count.item()) == 2 * n_ref
    if ws_mode == "caller":
        assert not ws.any()              # left zeroed


def test_count_workspace_over_calls_of_different_sizes(dev):
    # one workspace through a large call, a small one (fewer workgroups than
    # slots), the fused transpose, and a large one again: each count exact,
    # the workspace zero after each
    ws = count_workspace("caller", dev)
    cases = [(workloads.swiglu_input(seed=91, rows=2048, cols=2048), 3.0, "token"),
             (workloads.swiglu_input(seed=92, rows=3, cols=128), 1.0, "token"),
             (workloads.swiglu_input(seed=93, rows=384, cols=136), 2.0, "channel"),
             (workloads.swiglu_input(seed=94, rows=128, cols=8), 2.0, "channel"),
             (workloads.swiglu_input(seed=95, rows=2048, cols=2048, with_weight=False), 0.5,
              "token")]
    for wl, clamp, kind in cases:
        w = None if wl.w is None else wl.w.numpy()
        _, n_ref = oracle.swiglu_values_ex(bits(wl.x), w, swiglu_clamp=clamp)
        count = torch.zeros(1, dtype=torch.int64, device=dev)
        if kind == "token":
            gpu_swiglu_ex(wl, dev, clamp, count=count, ws=ws)
        else:
            gpu_swiglu_T(wl, dev, clamp=clamp, count=count, ws=ws)
        assert int(count.item()) == n_ref > 0, (wl.rows, wl.cols, kind)
        assert not ws.any(), (wl.rows, wl.cols, kind)


def test_count_workspace_is_checked(dev):
    wl = workloads.swiglu_input(seed=96, rows=4, cols=128)
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    small = torch.zeros(16, dtype=torch.int64, device=dev)
    with pytest.raises(pq.QcastError):
        gpu_swiglu_ex(wl, dev, 1.0, count=count, ws=small)
    offset = torch.zeros(pq.COUNT_WS_BYTES // 8 + 8, dtype=torch.int64, device=dev)[1:]
    with pytest.raises(pq.QcastError):           # 8-byte, not 128-byte aligned
        gpu_swiglu_ex(wl, dev, 1.0, count=count, ws=offset)


def test_swiglu_clamp_off_matches_plain_swiglu_exactly(dev):
    wl = workloads.swiglu_input(seed=72, rows=64, cols=2048)
    count = torch.full((1,), 5, dtype=torch.int64, device=dev)
    q, sf = gpu_swiglu_ex(wl, dev, 0.0, count=count)
    q2, sf2 = pq.qcast_swiglu_per_token(wl.x.to(dev), wl.w.to(dev))
    assert np.array_equal(q, codes_np(q2))
    assert np.array_equal(sf.view(np.uint32), sf2.cpu().numpy().view(np.uint32))
    assert int(count.item()) == 5          # untouched without a clamp
    q3, _ = gpu_swiglu_ex(wl, dev, float("inf"), count=count)
    assert np.array_equal(q3, q) and int(count.item()) == 5


def test_swiglu_clamp_full_size_with_layout(dev):
    wl = workloads.swiglu_input()
    flags = pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR
    q_ref, sf_ref, n_ref = oracle.swiglu_per_token_ex(bits(wl.x), wl.w.numpy(), sf_flags=flags,
                                                      swiglu_clamp=5.0)
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    q, sf = gpu_swiglu_ex(wl, dev, 5.0, flags=flags, count=count)
    assert int(count.item()) == n_ref
    count.zero_()
    gpu_swiglu_ex(wl, dev, 5.0, flags=flags, count=count, ws=False)
    assert int(count.item()) == n_ref
    v, _ = oracle.swiglu_values_ex(bits(wl.x), wl.w.numpy(), swiglu_clamp=5.0)
    check_swiglu_bar(q, sf, q_ref, sf_ref, v, sf_flags=flags, what="clamp full, packed col-major")


# ------------------------------------------------------------ SwiGLU backward

def gpu_backward(h, dv, w, dev, fmt="e4m3", group=128, clamp=0.0):
    rows, two_n = h.shape
    out = poisoned((rows, two_n), CODE_DT[fmt], dev)
    sf = poisoned((rows, two_n // group), torch.float32, dev)
    pq.qcast_swiglu_backward_per_token(h.to(dev), dv.to(dev), None if w is None else w.to(dev),
                                       fmt, group, swiglu_clamp=clamp, out=out, out_sf=sf)
    torch.cuda.synchronize()
    return codes_np(out), sf.cpu().numpy()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("group", [128, 64, 32])
@pytest.mark.parametrize("clamp", [0.0, 3.0])
@pytest.mark.parametrize("rows,cols,weighted", [(1, 128, True), (5, 384, False),
                                                (130, 2048, True)])
def test_swiglu_backward_shapes(dev, fmt, group, clamp, rows, cols, weighted):
    h, dv, w = workloads.swiglu_grad(seed=rows + cols, rows=rows, cols=cols,
                                     with_weight=weighted)
    q_ref, sf_ref = oracle.swiglu_backward_per_token(
        bits(h), bits(dv), None if w is None else w.numpy(), fmt, group, swiglu_clamp=clamp)
    q, sf = gpu_backward(h, dv, w, dev, fmt, group, clamp)
    v = oracle.swiglu_backward_values(bits(h), bits(dv), None if w is None else w.numpy(),
                                      swiglu_clamp=clamp)
    check_swiglu_bar(q, sf, q_ref, sf_ref, v, fmt, group, what=f"backward {fmt} g{group} c{clamp}")
    if clamp > 0:
        hf = h.float().numpy()
        n = cols
        # clamped positions carry an exact zero gradient
        assert np.all(q[:, :n][hf[:, :n] > clamp] == 0)
        assert np.all(q[:, n:][np.abs(hf[:, n:]) > clamp] == 0)


def test_swiglu_backward_full_size(dev):
    h, dv, w = workloads.swiglu_grad()
    q_ref, sf_ref = oracle.swiglu_backward_per_token(bits(h), bits(dv), w.numpy(),
                                                     swiglu_clamp=6.0)
    q, sf = gpu_backward(h, dv, w, dev, clamp=6.0)
    v = oracle.swiglu_backward_values(bits(h), bits(dv), w.numpy(), swiglu_clamp=6.0)
    frac = check_swiglu_bar(q, sf, q_ref, sf_ref, v, what="backward full")
    print(f"swiglu backward full: {frac:.5%} of codes differ from the oracle")


# ------------------------------------------- SwiGLU + per-channel + transpose

def gpu_swiglu_T(wl, dev, fmt="e4m3", clamp=0.0, count=None, ws=None):
    rows, n = wl.rows, wl.cols
    out = poisoned((n, rows), CODE_DT[fmt], dev)
    sf = poisoned((n, rows // 128), torch.float32, dev)
    pq.qcast_swiglu_per_channel_T(wl.x.to(dev), None if wl.w is None else wl.w.to(dev), fmt, 128,
                                  swiglu_clamp=clamp, clamp_count=count, out=out, out_sf=sf,
                                  count_workspace=ws)
    torch.cuda.synchronize()
    return codes_np(out), sf.cpu().numpy()


@pytest.mark.parametrize("ws_mode", WS_MODES)
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("clamp", [0.0, 2.5])
@pytest.mark.parametrize("rows,cols,weighted", [(128, 8, True), (256, 200, False),
                                                (384, 136, True), (1024, 2048, True)])
def test_swiglu_per_channel_T_shapes(dev, fmt, clamp, rows, cols, weighted, ws_mode):
    wl = workloads.swiglu_input(seed=rows + 2 * cols, rows=rows, cols=cols, with_weight=weighted)
    w = None if wl.w is None else wl.w.numpy()
    q_ref, sf_ref = oracle.swiglu_per_channel_T(bits(wl.x), w, fmt, swiglu_clamp=clamp)
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = count_workspace(ws_mode, dev)
    q, sf = gpu_swiglu_T(wl, dev, fmt, clamp, count, ws)
    v, n_ref = oracle.swiglu_values_ex(bits(wl.x), w, swiglu_clamp=clamp)
    # groups run along tokens: the per-token bar on the transposed values
    check_swiglu_bar(q, sf, q_ref, sf_ref, v.T, fmt, 128, what=f"swiglu_T {fmt} c{clamp} {rows}x{cols}")
    assert int(count.item()) == n_ref
    if ws_mode == "caller":
        assert not ws.any()


def test_swiglu_per_channel_T_full_size(dev):
    wl = workloads.swiglu_input()
    q_ref, sf_ref = oracle.swiglu_per_channel_T(bits(wl.x), wl.w.numpy())
    q, sf = gpu_swiglu_T(wl, dev)
    v = oracle.swiglu_values(bits(wl.x), wl.w.numpy())
    frac = check_swiglu_bar(q, sf, q_ref, sf_ref, v.T, what="swiglu_T full")
    print(f"swiglu + transpose full: {frac:.5%} of codes differ from the oracle")



def test_count_workspaces_per_stream_under_concurrency(dev):
    # two streams at once, each with the binding's own workspace for it:
    # every count exact, both workspaces zero afterwards
    wls = [workloads.swiglu_input(seed=97 + i, rows=2048, cols=2048) for i in range(2)]
    clamps = [2.0, 3.0]
    refs = [oracle.swiglu_values_ex(bits(wl.x), wl.w.numpy(), swiglu_clamp=c)[1]
            for wl, c in zip(wls, clamps)]
    ins = [(wl.x.to(dev), wl.w.to(dev)) for wl in wls]
    streams = [torch.cuda.Stream(dev) for _ in wls]
    counts = [torch.zeros(1, dtype=torch.int64, device=dev) for _ in wls]
    torch.cuda.synchronize()
    for _ in range(3):
        for (h, w), c, s, n in zip(ins, clamps, streams, counts):
            with torch.cuda.stream(s):
                pq.qcast_swiglu_per_token_ex(h, w, "e4m3", 128, swiglu_clamp=c, clamp_count=n)
                pq.qcast_swiglu_per_channel_T(h, w, "e4m3", 128, swiglu_clamp=c, clamp_count=n)
    torch.cuda.synchronize()
    for n, ref in zip(counts, refs):
        assert int(n.item()) == 6 * ref > 0
    for s in streams:
        ws = pq._count_ws_cache[(dev, s.cuda_stream)]
        assert not ws.any()
