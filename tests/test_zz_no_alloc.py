"""qcast_swiglu_per_token_noalloc (the counting SwiGLU cast for callers that
cannot allocate: its count slots are the library's own device array) against
qcast_swiglu_per_token_ex with a caller's count workspace, through the C ABI:
codes and scales bit-equal, counts equal and equal to the oracle's, on two
calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_amd as pq
from precision_quantization_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def poisoned(shape, dtype, dev, byte):
    t = torch.empty(shape, dtype=dtype, device=dev)
    t.view(torch.uint8).fill_(byte)
    return t


def bits(t):
    return t.view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("fmt,group,flags", [
    ("e4m3", 128, 0), ("e2m1", 32, pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR),
    ("e5m2", 64, pq.SF_ROUND_POW2)])
def test_noalloc_equals_the_workspace_entry_point(dev, fmt, group, flags):
    clamp = 3.0
    # two calls in a row, the second smaller (fewer workgroups than slots)
    for rows, cols, seed in [(4096, 2048, 81), (37, 512, 82)]:
        print(f"noalloc {fmt} g{group} flags {flags}: {rows} x {cols}", flush=True)
        wl = workloads.swiglu_input(seed=seed, rows=rows, cols=cols)
        h, w = wl.x.to(dev), wl.w.to(dev)
        qshape = pq.code_shape(fmt, rows, cols)
        sshape, sdt = pq.sf_layout_shape(rows, cols, group, flags)
        ws = torch.zeros(pq.COUNT_WS_BYTES // 8, dtype=torch.int64, device=dev)
        n_ws = torch.zeros(1, dtype=torch.int64, device=dev)
        qdt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}.get(fmt, torch.uint8)
        q_ws = poisoned(qshape, qdt, dev, 0x5A)
        s_ws = poisoned(sshape, sdt, dev, 0x5A)
        pq.qcast_swiglu_per_token_ex(h, w, fmt, group, sf_flags=flags, swiglu_clamp=clamp,
                                     clamp_count=n_ws, out=q_ws, out_sf=s_ws,
                                     count_workspace=ws)
        n = torch.zeros(1, dtype=torch.int64, device=dev)
        q = poisoned(qshape, qdt, dev, 0xA5)
        s = poisoned(sshape, sdt, dev, 0xA5)
        pq.qcast_swiglu_per_token_noalloc(h, w, fmt, group, sf_flags=flags, swiglu_clamp=clamp,
                                          clamp_count=n, out=q, out_sf=s)
        torch.cuda.synchronize()
        assert np.array_equal(bits(q), bits(q_ws))
        # column-major scales: the padding entries (poisoned differently) are not written
        used = rows * 4 if flags & pq.SF_COL_MAJOR else None
        assert np.array_equal(bits(s)[:, :used], bits(s_ws)[:, :used])
        _, n_ref = oracle.swiglu_values_ex(workloads.bf16_bits(wl.x), wl.w.numpy(),
                                           swiglu_clamp=clamp)
        assert int(n.item()) == int(n_ws.item()) == n_ref > 0
        assert not ws.any()


def test_noalloc_accumulates_and_runs_without_a_counter(dev):
    wl = workloads.swiglu_input(seed=83, rows=512, cols=1024)
    h, w = wl.x.to(dev), wl.w.to(dev)
    n = torch.zeros(1, dtype=torch.int64, device=dev)
    q1, s1 = pq.qcast_swiglu_per_token_noalloc(h, w, swiglu_clamp=2.0, clamp_count=n)
    q2, s2 = pq.qcast_swiglu_per_token_noalloc(h, w, swiglu_clamp=2.0, clamp_count=n)
    q3, s3 = pq.qcast_swiglu_per_token_noalloc(h, w, swiglu_clamp=2.0)   # no counter
    torch.cuda.synchronize()
    _, n_ref = oracle.swiglu_values_ex(workloads.bf16_bits(wl.x), wl.w.numpy(), swiglu_clamp=2.0)
    assert int(n.item()) == 2 * n_ref
    for q, s in ((q2, s2), (q3, s3)):
        assert np.array_equal(bits(q), bits(q1)) and np.array_equal(bits(s), bits(s1))
