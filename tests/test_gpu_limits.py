"""GPU parity at the largest shapes the kernels' 32-bit indexing allows
(include/qcast.h states the limits; one step past them is refused on the
CPU, see test_abi_cpu.py). The inputs are a few GB, so the oracle checks a
sample: the first and last channels / blocks (the ends of the 32-bit offset
range) and random ones in between.
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


def big_input(dev, rows, cols, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    x = torch.randn(rows, cols, generator=g, device=dev, dtype=torch.float32)
    x.mul_(torch.exp(torch.randn(1, cols, generator=g, device=dev) * 2))
    return x.to(torch.bfloat16)


def sample(n, k, step, seed):
    """k sorted distinct indices in [0, n) that are multiples of `step`:
    the first, the last and random ones."""
    rng = np.random.default_rng(seed)
    idx = rng.choice(n // step, size=k - 2, replace=False) * step
    return np.unique(np.concatenate([[0, (n - 1) // step * step], idx]))


def bits_of(t):
    return workloads.bf16_bits(t.cpu())


def test_per_channel_T_at_the_column_limit(dev):
    rows, cols = 128, (1 << 24) - 8          # 128 * cols just below 2^31; ragged last tile
    x = big_input(dev, rows, cols, 101)
    qT, sf = pq.qcast_per_channel_T(x)
    chans = np.concatenate([sample(cols, 62, 1, 1), np.arange(cols - 8, cols)])
    chans = np.unique(chans)
    ci = torch.from_numpy(chans).to(dev)
    q_ref, sf_ref = oracle.per_channel_T(bits_of(x.index_select(1, ci)))
    assert np.array_equal(qT.index_select(0, ci).view(torch.uint8).cpu().numpy(), q_ref)
    assert np.array_equal(sf.index_select(0, ci).cpu().numpy().view(np.uint32),
                          sf_ref.view(np.uint32))
    del x, qT, sf
    torch.cuda.empty_cache()


def test_per_channel_at_the_column_limit(dev):
    rows, cols = 128, (1 << 24) - 8
    x = big_input(dev, rows, cols, 102)
    q, sf = pq.qcast_per_channel(x)
    chans = np.unique(np.concatenate([sample(cols, 62, 1, 2), np.arange(cols - 8, cols)]))
    ci = torch.from_numpy(chans).to(dev)
    q_ref, sf_ref = oracle.per_channel(bits_of(x.index_select(1, ci)))
    assert np.array_equal(q.index_select(1, ci).view(torch.uint8).cpu().numpy(), q_ref)
    assert np.array_equal(sf.index_select(1, ci).cpu().numpy().view(np.uint32),
                          sf_ref.view(np.uint32))
    del x, q, sf
    torch.cuda.empty_cache()


# 128 * cols just below 2^31, with an odd and an even number of tile columns
@pytest.mark.parametrize("cols", [(1 << 24) - 128, (1 << 24) - 256])
def test_per_block_at_the_column_limit(dev, cols):
    rows = 256
    x = big_input(dev, rows, cols, 103)
    q, sf = pq.qcast_per_block(x)
    for b in sample(cols // 128, 24, 1, 3):
        c = slice(128 * int(b), 128 * int(b) + 128)
        q_ref, sf_ref = oracle.per_block(bits_of(x[:, c]))
        assert np.array_equal(q[:, c].view(torch.uint8).cpu().numpy(), q_ref), b
        assert np.array_equal(sf[:, int(b):int(b) + 1].cpu().numpy().view(np.uint32),
                              sf_ref.view(np.uint32)), b
    del x, q, sf
    torch.cuda.empty_cache()


def test_swiglu_per_channel_T_at_the_column_limit(dev):
    rows, cols = 128, (1 << 23) - 8          # 256 * cols just below 2^31
    h = big_input(dev, rows, 2 * cols, 104)
    w = torch.rand(rows, device=dev)
    qT, sf = pq.qcast_swiglu_per_channel_T(h, w)
    chans = np.unique(np.concatenate([sample(cols, 30, 1, 4), np.arange(cols - 8, cols)]))
    ci = torch.from_numpy(chans).to(dev)
    hs = torch.cat([h.index_select(1, ci), h.index_select(1, ci + cols)], dim=1)
    q_ref, sf_ref = oracle.swiglu_per_channel_T(bits_of(hs), w.cpu().numpy())
    q = qT.index_select(0, ci).view(torch.uint8).cpu().numpy()
    s = sf.index_select(0, ci).cpu().numpy()
    v = oracle.swiglu_values(bits_of(hs), w.cpu().numpy())
    check_swiglu_bar(q, s, q_ref, sf_ref, v.T, what="swiglu_T column limit")
    del h, qT, sf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("op", ["forward", "backward"])
def test_swiglu_rows_at_the_length_limit(dev, op):
    rows, cols = 3, (1 << 19) - 128          # cols / 8 just below 2^16
    g = torch.Generator().manual_seed(105)
    h = (torch.randn(rows, 2 * cols, generator=g) * 2).to(torch.bfloat16)
    w = torch.rand(rows, generator=g)
    if op == "forward":
        q, sf = pq.qcast_swiglu_per_token(h.to(dev), w.to(dev))
        q_ref, sf_ref = oracle.swiglu_per_token(workloads.bf16_bits(h), w.numpy())
        v = oracle.swiglu_values(workloads.bf16_bits(h), w.numpy())
    else:
        dv = torch.randn(rows, cols, generator=g).to(torch.bfloat16)
        q, sf = pq.qcast_swiglu_backward_per_token(h.to(dev), dv.to(dev), w.to(dev))
        q_ref, sf_ref = oracle.swiglu_backward_per_token(workloads.bf16_bits(h),
                                                         workloads.bf16_bits(dv), w.numpy())
        v = oracle.swiglu_backward_values(workloads.bf16_bits(h), workloads.bf16_bits(dv),
                                          w.numpy())
    check_swiglu_bar(q.view(torch.uint8).cpu().numpy(), sf.cpu().numpy(), q_ref, sf_ref, v,
                     what=f"{op} at the row-length limit")


@pytest.mark.parametrize("ws", [None, False])
def test_swiglu_clamp_count_over_several_launches(dev, ws):
    # 66,536 rows of 2048 outputs: past the 2^24 chunks of one launch, so the
    # cast runs as two launches that count through the same workspace (or,
    # with ws=False, on capped grids); the count is additive over rows, so
    # the oracle counts slabs of rows
    rows, cols, clamp = 65536 + 1000, 2048, 3.0
    g = torch.Generator().manual_seed(107)
    h = (torch.randn(rows, 2 * cols, generator=g) * 2).to(torch.bfloat16)
    w = torch.rand(rows, generator=g)
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    q, sf = pq.qcast_swiglu_per_token_ex(h.to(dev), w.to(dev), "e4m3", 128, swiglu_clamp=clamp,
                                         clamp_count=count, count_workspace=ws)
    torch.cuda.synchronize()
    hb = workloads.bf16_bits(h)
    wn = w.numpy()
    n_ref = 0
    for r0 in range(0, rows, 8192):
        n_ref += oracle.swiglu_values_ex(hb[r0:r0 + 8192], wn[r0:r0 + 8192],
                                         swiglu_clamp=clamp)[1]
    assert int(count.item()) == n_ref > 0
    # codes and scales of sampled rows in both launches
    for r in sample(rows, 12, 1, 108):
        r = int(r)
        q_ref, sf_ref, _ = oracle.swiglu_per_token_ex(hb[r:r + 1], wn[r:r + 1],
                                                      swiglu_clamp=clamp)
        v, _ = oracle.swiglu_values_ex(hb[r:r + 1], wn[r:r + 1], swiglu_clamp=clamp)
        check_swiglu_bar(q[r:r + 1].view(torch.uint8).cpu().numpy(), sf[r:r + 1].cpu().numpy(),
                         q_ref, sf_ref, v, what=f"row {r}")
    del q, sf
    torch.cuda.empty_cache()
