"""No cast writes outside its outputs: every code and scale tensor is a view
into the middle of a larger buffer whose 4 KiB on either side are poisoned,
and after the call those bytes must be unchanged. The shapes are ragged
(partial tiles, odd tile columns, single rows, padded column-major scales)
so that the kernels' edge handling is what is checked."""
import numpy as np
import pytest
import torch

import precision_quantization_amd as pq
from precision_quantization_amd import workloads

pytestmark = pytest.mark.gpu

GUARD = 4096
POISON = 0x5A


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


class Guarded:
    """Tensors carved out of poisoned buffers with guard bands."""

    def __init__(self, dev):
        self.dev = dev
        self.bufs = []

    def make(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((GUARD + n + GUARD,), POISON, dtype=torch.uint8, device=self.dev)
        self.bufs.append((buf, n))
        return buf[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        for i, (buf, n) in enumerate(self.bufs):
            head = buf[:GUARD].cpu().numpy()
            tail = buf[GUARD + n:].cpu().numpy()
            assert (head == POISON).all() and (tail == POISON).all(), f"{what}: buffer {i}"


def code_dtype(fmt):
    return {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}.get(fmt, torch.uint8)


def bf16(rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(rows, cols, generator=g) * 3).to(torch.bfloat16)


@pytest.mark.parametrize("fmt,group,flags", [("e4m3", 128, 0), ("e2m1", 32, 0), ("e5m6", 64, 0),
                                             ("e4m3", 32, pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR),
                                             ("e5m2", 128, pq.SF_COL_MAJOR)])
@pytest.mark.parametrize("rows", [1, 5, 257])
def test_per_token_and_swiglu_stay_inside(dev, fmt, group, flags, rows):
    cols = 512
    g = Guarded(dev)
    x = bf16(rows, cols, rows).to(dev)
    q = g.make(pq.code_shape(fmt, rows, cols), code_dtype(fmt))
    shape, dt = pq.sf_layout_shape(rows, cols, group, flags)
    sf = g.make(shape, dt)
    pq.qcast_per_token_sf(x, fmt, group, sf_flags=flags, out=q, out_sf=sf)
    g.check(f"per_token {fmt} g{group} flags {flags} rows {rows}")
    h = bf16(rows, 2 * cols, rows + 1).to(dev)
    w = torch.rand(rows, device=dev)
    qs = g.make(pq.code_shape(fmt, rows, cols), code_dtype(fmt))
    ss = g.make(shape, dt)
    count = g.make((1,), torch.int64)
    count.zero_()
    pq.qcast_swiglu_per_token_ex(h, w, fmt, group, sf_flags=flags, swiglu_clamp=2.0,
                                 clamp_count=count, out=qs, out_sf=ss)
    g.check(f"swiglu {fmt} g{group} flags {flags} rows {rows}")
    # without a counter: the launch whose grid is padded to whole XCD ranges
    qp = g.make(pq.code_shape(fmt, rows, cols), code_dtype(fmt))
    sp = g.make(shape, dt)
    pq.qcast_swiglu_per_token_sf(h, w, fmt, group, sf_flags=flags, out=qp, out_sf=sp)
    g.check(f"swiglu, no counter, {fmt} g{group} flags {flags} rows {rows}")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e5m6"])
@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 384), (384, 256)])
def test_per_block_stays_inside(dev, fmt, rows, cols):
    g = Guarded(dev)
    x = bf16(rows, cols, 7).to(dev)
    q = g.make(pq.code_shape(fmt, rows, cols), code_dtype(fmt))
    sf = g.make((rows // 128, cols // 128), torch.float32)
    pq.qcast_per_block_sf(x, fmt, 128, sf_flags=pq.SF_ROUND_POW2, out=q, out_sf=sf)
    g.check(f"per_block {fmt} {rows}x{cols}")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e5m6"])
@pytest.mark.parametrize("flags", [0, pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR, pq.SF_COL_MAJOR])
@pytest.mark.parametrize("rows,cols", [(512, 72), (512, 200), (1024, 8)])
def test_transposed_casts_stay_inside(dev, fmt, flags, rows, cols):
    g = Guarded(dev)
    x = bf16(rows, cols, 11).to(dev)
    q = g.make(pq.code_shape(fmt, cols, rows), code_dtype(fmt))
    shape, dt = pq.sf_layout_shape(cols, rows, 128, flags)
    sf = g.make(shape, dt)
    pq.qcast_per_channel_T_sf(x, fmt, 128, sf_flags=flags, out=q, out_sf=sf)
    g.check(f"per_channel_T {fmt} flags {flags} {rows}x{cols}")
    h = bf16(rows, 2 * cols, 12).to(dev)
    w = torch.rand(rows, device=dev)
    qs = g.make(pq.code_shape(fmt, cols, rows), code_dtype(fmt))
    ss = g.make(shape, dt)
    count = g.make((1,), torch.int64)
    count.zero_()
    pq.qcast_swiglu_per_channel_T_sf(h, w, fmt, 128, sf_flags=flags, swiglu_clamp=2.0,
                                     clamp_count=count, out=qs, out_sf=ss)
    g.check(f"swiglu_per_channel_T {fmt} flags {flags} {rows}x{cols}")
    qc = g.make(pq.code_shape(fmt, rows, cols), code_dtype(fmt))
    sc = g.make((rows // 128, cols), torch.float32)
    pq.qcast_per_channel_sf(x, fmt, 128, sf_flags=pq.SF_ROUND_POW2 if flags else 0, out=qc,
                            out_sf=sc)
    g.check(f"per_channel {fmt} {rows}x{cols}")


@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e2m1", 32), ("e5m6", 64)])
@pytest.mark.parametrize("flags", [0, pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR])
@pytest.mark.parametrize("rows", [1, 7, 130])
def test_backward_and_cast_back_stay_inside(dev, fmt, group, flags, rows):
    cols = 4 * group
    g = Guarded(dev)
    hh, dv, w = workloads.swiglu_grad(seed=rows, rows=rows, cols=cols)
    q = g.make(pq.code_shape(fmt, rows, 2 * cols), code_dtype(fmt))
    shape, dt = pq.sf_layout_shape(rows, 2 * cols, group, flags)
    sf = g.make(shape, dt)
    pq.qcast_swiglu_backward_per_token_sf(hh.to(dev), dv.to(dev), w.to(dev), fmt, group,
                                          sf_flags=flags, swiglu_clamp=3.0, out=q, out_sf=sf)
    g.check(f"backward {fmt} g{group} flags {flags} rows {rows}")
    x = bf16(rows, cols, rows + 5).to(dev)
    q0, sf0 = pq.qcast_per_token(x, fmt, group)
    for dtype in (torch.bfloat16, torch.float32):
        out = g.make((rows, cols), dtype)
        pq.qcast_cast_back(q0, sf0, fmt, group, out_dtype=dtype, out=out)
        g.check(f"cast_back {fmt} g{group} rows {rows} {dtype}")
