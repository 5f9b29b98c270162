"""GPU parity of the scale-factor options on the casts other than the
per-token ones, against the oracle:

* the transposed per-channel cast (every layout, every format): bit-exact;
* SwiGLU + per-channel + transpose (every layout, clamp and counter): the
  SwiGLU bar, exact clamp counts;
* the SwiGLU backward (every layout): the SwiGLU bar;
* round_sf on the per-block and input-layout per-channel casts: bit-exact.

Outputs are poisoned with two byte patterns beforehand, and the oracle's
unwritten padding holds the same pattern, so whole arrays compare equal only
if every byte the cast owns was written and no other byte was touched.

Pages (cited by title and section): "DeepSeek开源TileKernels：用Python写的GPU
算子逼近硬件性能上限", §3.1 (round_sf); "TileKernels 与 DeepGEMM 的分界线：
DeepSeek 开源内核栈的分工", §四 C (layouts written while quantizing or
re-arranging).
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_amd as pq
from precision_quantization_amd import workloads
from swiglu_bar import check_swiglu_bar

pytestmark = pytest.mark.gpu

LAYOUTS = [pq.SF_ROUND_POW2, pq.SF_COL_MAJOR, pq.SF_ROUND_POW2 | pq.SF_COL_MAJOR,
           pq.SF_PACKED_UE8M0, pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR]
POISONS = (0xAA, 0x55)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def bits(t):
    return workloads.bf16_bits(t)


def poisoned(shape, dtype, dev, byte):
    t = torch.empty(shape, dtype=dtype, device=dev)
    t.view(torch.uint8).fill_(byte)
    return t


def fill_of(flags, byte):
    """The oracle's padding value with the bit pattern of the poison."""
    word = np.uint32(int.from_bytes(bytes([byte]) * 4, "little"))
    return word if flags & pq.SF_PACKED_UE8M0 else word.view(np.float32)


def sf_tensor(rows, cols, group, flags, dev, byte):
    shape, dt = pq.sf_layout_shape(rows, cols, group, flags)
    return poisoned(shape, dt, dev, byte)


def code_tensor(fmt, rows, cols, dev, byte):
    f = oracle.fmt_id(fmt)
    dt = {1: torch.float8_e4m3fn, 3: torch.float8_e5m2}.get(f, torch.uint8)
    return poisoned(pq.code_shape(f, rows, cols), dt, dev, byte)


def u8(t):
    return t.view(torch.uint8).cpu().numpy()


def u32(t):
    return t.cpu().view(torch.int32).numpy().view(np.uint32)


def spread_input(seed, rows, cols):
    """Channels (columns) over many binades, one channel all zero."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g) * torch.exp(torch.randn(1, cols, generator=g) * 3)
    x[:, 1] = 0.0
    return x.to(torch.bfloat16)


# --------------------------------------------------------------- per-channel + T

@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1", "e5m6"])
@pytest.mark.parametrize("flags", LAYOUTS)
@pytest.mark.parametrize("rows,cols", [(512, 200), (2048, 72)])
def test_per_channel_T_layouts(dev, fmt, flags, rows, cols):
    x = spread_input(rows + cols + flags, rows, cols)
    for p in POISONS:
        q_ref, sf_ref = oracle.per_channel_T_sf(bits(x), fmt, 128, sf_flags=flags,
                                                sf_fill=fill_of(flags, p))
        out = code_tensor(fmt, cols, rows, dev, p)
        sf = sf_tensor(cols, rows, 128, flags, dev, p)
        pq.qcast_per_channel_T_sf(x.to(dev), fmt, 128, sf_flags=flags, out=out, out_sf=sf)
        torch.cuda.synchronize()
        q = u8(out)
        assert np.array_equal(q, q_ref), f"{(q != q_ref).sum()} code bytes differ"
        assert np.array_equal(u32(sf), sf_ref.view(np.uint32))


def test_per_channel_T_without_options_equals_the_plain_entry_point(dev):
    x = spread_input(3, 1024, 136).to(dev)
    q0, sf0 = pq.qcast_per_channel_T(x)
    q1, sf1 = pq.qcast_per_channel_T_sf(x, sf_flags=0)
    assert torch.equal(q0.view(torch.uint8), q1.view(torch.uint8))
    assert torch.equal(sf0.view(torch.int32), sf1.view(torch.int32))


@pytest.mark.parametrize("flags", [pq.SF_COL_MAJOR,
                                   pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR])
def test_per_channel_T_layouts_full_size(dev, flags):
    # 16384 tokens x 7168 channels: the layout's scales follow the plain
    # cast's (a transpose; a power of two's exponent), and the codes of 64
    # channels spread over the tensor equal the oracle's on those channels.
    wl = workloads.activation_channel()
    x = wl.x.to(dev)
    rows, cols = wl.x.shape
    q0, sf0 = pq.qcast_per_channel_T(x)
    out = code_tensor("e4m3", cols, rows, dev, 0xAA)
    sf = sf_tensor(cols, rows, 128, flags, dev, 0xAA)
    pq.qcast_per_channel_T_sf(x, sf_flags=flags, out=out, out_sf=sf)
    torch.cuda.synchronize()
    plain = sf0.cpu().numpy()
    if flags & pq.SF_PACKED_UE8M0:
        m, e = np.frexp(plain.astype(np.float64))
        expo = np.where(m == 0.5, e - 1, e) + 127          # biased exponent of the power above
        got = u32(sf).T.copy().view(np.uint8).reshape(cols, rows // 128)
        assert np.array_equal(got, expo.astype(np.uint8))
    else:
        assert np.array_equal(u32(sf).T, plain.view(np.uint32))
        assert torch.equal(out.view(torch.uint8), q0.view(torch.uint8))
    chans = np.linspace(0, cols - 8, 8).astype(int) // 8 * 8
    q = u8(out)
    xb = bits(wl.x)
    for c0 in chans:
        q_ref, _ = oracle.per_channel_T_sf(np.ascontiguousarray(xb[:, c0:c0 + 8]), "e4m3", 128,
                                           sf_flags=flags)
        assert np.array_equal(q[c0:c0 + 8], q_ref), f"channels {c0}..{c0 + 7}"


# ------------------------------------------------------- SwiGLU + per-channel + T

@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e5m6"])
@pytest.mark.parametrize("flags", LAYOUTS)
def test_swiglu_per_channel_T_layouts(dev, fmt, flags):
    rows, cols = 1024, 200
    wl = workloads.swiglu_input(seed=60 + flags, rows=rows, cols=cols)
    h, w = bits(wl.x), wl.w.numpy()
    clamp = 3.0
    q_ref, sf_ref = oracle.swiglu_per_channel_T_sf(h, w, fmt, 128, sf_flags=flags,
                                                   swiglu_clamp=clamp, sf_fill=fill_of(flags, 0xAA))
    v, n_ref = oracle.swiglu_values_ex(h, w, swiglu_clamp=clamp)
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    out = code_tensor(fmt, cols, rows, dev, 0xAA)
    sf = sf_tensor(cols, rows, 128, flags, dev, 0xAA)
    pq.qcast_swiglu_per_channel_T_sf(wl.x.to(dev), wl.w.to(dev), fmt, 128, sf_flags=flags,
                                     swiglu_clamp=clamp, clamp_count=count, out=out, out_sf=sf)
    torch.cuda.synchronize()
    assert int(count.item()) == n_ref > 0
    check_swiglu_bar(u8(out), sf.cpu().numpy(), q_ref, sf_ref, v.T, fmt, 128, sf_flags=flags,
                     what=f"swiglu_T {fmt} flags {flags}")


# ------------------------------------------------------------------ SwiGLU backward

@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e4m3", 32), ("e2m1", 32),
                                       ("e5m6", 64)])
@pytest.mark.parametrize("flags", LAYOUTS)
@pytest.mark.parametrize("rows", [7, 300])
def test_swiglu_backward_layouts(dev, fmt, group, flags, rows):
    cols = 4 * group if rows == 7 else 8 * group
    h, dv, w = workloads.swiglu_grad(seed=70 + rows + flags, rows=rows, cols=cols)
    clamp = 4.0 if rows == 300 else 0.0
    q_ref, sf_ref = oracle.swiglu_backward_per_token_sf(
        bits(h), bits(dv), w.numpy(), fmt, group, sf_flags=flags, swiglu_clamp=clamp,
        sf_fill=fill_of(flags, 0x55))
    out = code_tensor(fmt, rows, 2 * cols, dev, 0x55)
    sf = sf_tensor(rows, 2 * cols, group, flags, dev, 0x55)
    pq.qcast_swiglu_backward_per_token_sf(h.to(dev), dv.to(dev), w.to(dev), fmt, group,
                                          sf_flags=flags, swiglu_clamp=clamp, out=out, out_sf=sf)
    torch.cuda.synchronize()
    v = oracle.swiglu_backward_values(bits(h), bits(dv), w.numpy(), swiglu_clamp=clamp)
    sfn = sf.cpu().numpy()
    check_swiglu_bar(u8(out), sfn, q_ref, sf_ref, v, fmt, group, sf_flags=flags,
                     what=f"backward {fmt} g{group} flags {flags} rows {rows}")
    if flags & pq.SF_COL_MAJOR:                             # row padding untouched
        rows_pad = (rows + 3) // 4 * 4
        assert (sfn.view(np.uint32)[:, rows:rows_pad] == 0x55555555).all()


# ------------------------------------------ round_sf on per-block and per-channel

@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1", "e5m6"])
@pytest.mark.parametrize("rows,cols", [(256, 384), (384, 256)])
def test_per_block_round_sf(dev, fmt, rows, cols):
    x = spread_input(80 + rows, rows, cols)
    q_ref, sf_ref = oracle.per_block_sf(bits(x), fmt, 128, sf_flags=pq.SF_ROUND_POW2)
    for p in POISONS:
        out = code_tensor(fmt, rows, cols, dev, p)
        sf = poisoned((rows // 128, cols // 128), torch.float32, dev, p)
        pq.qcast_per_block_sf(x.to(dev), fmt, 128, sf_flags=pq.SF_ROUND_POW2, out=out, out_sf=sf)
        torch.cuda.synchronize()
        assert np.array_equal(u8(out), q_ref)
        assert np.array_equal(u32(sf), sf_ref.view(np.uint32))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1", "e5m6"])
@pytest.mark.parametrize("rows,cols", [(256, 200), (384, 264)])
def test_per_channel_round_sf(dev, fmt, rows, cols):
    x = spread_input(90 + cols, rows, cols)
    q_ref, sf_ref = oracle.per_channel_sf(bits(x), fmt, 128, sf_flags=pq.SF_ROUND_POW2)
    for p in POISONS:
        out = code_tensor(fmt, rows, cols, dev, p)
        sf = poisoned((rows // 128, cols), torch.float32, dev, p)
        pq.qcast_per_channel_sf(x.to(dev), fmt, 128, sf_flags=pq.SF_ROUND_POW2, out=out,
                                out_sf=sf)
        torch.cuda.synchronize()
        assert np.array_equal(u8(out), q_ref)
        assert np.array_equal(u32(sf), sf_ref.view(np.uint32))


def test_per_block_round_sf_full_size(dev):
    # the 7168 x 18432 weight: every scale is the power of two above the plain
    # cast's scale, and rows 0..127 of tile row 31 match the oracle bit for bit
    wl = workloads.weight_block()
    x = wl.x.to(dev)
    _, sf0 = pq.qcast_per_block(x)
    q, sf = pq.qcast_per_block_sf(x, sf_flags=pq.SF_ROUND_POW2)
    plain = sf0.cpu().numpy().astype(np.float64)
    m, e = np.frexp(plain)
    assert np.array_equal(sf.cpu().numpy().astype(np.float64),
                          np.where(m == 0.5, plain, np.ldexp(1.0, e)))
    xb = bits(wl.x)
    band = np.ascontiguousarray(xb[31 * 128:32 * 128])
    q_ref, _ = oracle.per_block_sf(band, "e4m3", 128, sf_flags=pq.SF_ROUND_POW2)
    assert np.array_equal(u8(q)[31 * 128:32 * 128], q_ref)


def test_swiglu_backward_layouts_full_size(dev):
    # 8192 x 2048 gradient, packed UE8M0 column-major scales: 32 rows spread
    # over the tensor held to the SwiGLU bar against the oracle on those rows
    h, dv, w = workloads.swiglu_grad()
    flags = pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR
    rows, cols = dv.shape
    out = code_tensor("e4m3", rows, 2 * cols, dev, 0xAA)
    sf = sf_tensor(rows, 2 * cols, 128, flags, dev, 0xAA)
    pq.qcast_swiglu_backward_per_token_sf(h.to(dev), dv.to(dev), w.to(dev), "e4m3", 128,
                                          sf_flags=flags, swiglu_clamp=6.0, out=out, out_sf=sf)
    torch.cuda.synchronize()
    q = u8(out)
    words = u32(sf)                                       # [groups/4][rows]
    picks = np.linspace(0, rows - 1, 32).astype(int)
    hb, db, wn = bits(h), bits(dv), w.numpy()
    for r in picks:
        sl = slice(r, r + 1)
        q_ref, sf_ref = oracle.swiglu_backward_per_token_sf(
            np.ascontiguousarray(hb[sl]), np.ascontiguousarray(db[sl]), wn[sl], "e4m3", 128,
            sf_flags=pq.SF_PACKED_UE8M0, swiglu_clamp=6.0)
        v = oracle.swiglu_backward_values(np.ascontiguousarray(hb[sl]),
                                          np.ascontiguousarray(db[sl]), wn[sl],
                                          swiglu_clamp=6.0)
        got_sf = np.ascontiguousarray(words[:, r:r + 1].T)  # this row's words, row-major
        check_swiglu_bar(q[sl], got_sf, q_ref, sf_ref, v, "e4m3", 128,
                         sf_flags=pq.SF_PACKED_UE8M0, what=f"backward full, row {r}")


def test_swiglu_per_channel_T_layouts_full_size(dev):
    # 8192 tokens x 2048 outputs, round_sf column-major scales, clamp 5 with a
    # counter: 64 channels spread over the output held to the SwiGLU bar
    # against the oracle on those channels; the clamp count is exact
    wl = workloads.swiglu_input()
    rows, n = wl.rows, wl.cols
    flags = pq.SF_ROUND_POW2 | pq.SF_COL_MAJOR
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    out = code_tensor("e4m3", n, rows, dev, 0x55)
    sf = sf_tensor(n, rows, 128, flags, dev, 0x55)
    pq.qcast_swiglu_per_channel_T_sf(wl.x.to(dev), wl.w.to(dev), "e4m3", 128, sf_flags=flags,
                                     swiglu_clamp=5.0, clamp_count=count, out=out, out_sf=sf)
    torch.cuda.synchronize()
    hb, wn = bits(wl.x), wl.w.numpy()
    _, n_ref = oracle.swiglu_values_ex(hb, wn, swiglu_clamp=5.0)
    assert int(count.item()) == n_ref
    q, sfn = u8(out), sf.cpu().numpy()
    for c0 in np.linspace(0, n - 8, 8).astype(int) // 8 * 8:
        sub = np.ascontiguousarray(np.concatenate([hb[:, c0:c0 + 8], hb[:, n + c0:n + c0 + 8]],
                                                  axis=1))
        q_ref, sf_ref = oracle.swiglu_per_channel_T_sf(sub, wn, "e4m3", 128, sf_flags=flags,
                                                       swiglu_clamp=5.0)
        v, _ = oracle.swiglu_values_ex(sub, wn, swiglu_clamp=5.0)
        got_sf = np.ascontiguousarray(sfn[:, c0:c0 + 8])   # [groups][channels of the slice]
        check_swiglu_bar(q[c0:c0 + 8], got_sf, q_ref, sf_ref, v.T, "e4m3", 128, sf_flags=flags,
                         what=f"swiglu_T full, channels {c0}..{c0 + 7}")
