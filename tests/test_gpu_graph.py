"""The casts under HIP graph capture: a graph of one pass of the five casts
(through the C ABI, on torch's capture stream) is replayed several times,
with eager casts and synchronizations between the replays, and every replay
must equal the eager result bit for bit. The library allocates nothing and
records no memset, so its launches are capturable as they are.
"""
import pytest
import torch

import precision_quantization_amd as pq
from precision_quantization_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def five_casts(ins, outs):
    x, h, w, wt, a, xt = ins
    pq.qcast_per_token(x, "e4m3", 128, out=outs[0], out_sf=outs[1])
    pq.qcast_swiglu_per_token(h, w, "e4m3", 128, out=outs[2], out_sf=outs[3])
    pq.qcast_per_block(wt, "e4m3", 128, out=outs[4], out_sf=outs[5])
    pq.qcast_per_channel_T(a, "e4m3", 128, out=outs[6], out_sf=outs[7])
    pq.qcast_e2m1(xt, 32, out=outs[8], out_sf=outs[9])


def test_graph_replays_match_eager(dev):
    ins = (workloads.per_token_hidden(rows=256).x.to(dev),
           workloads.swiglu_input(rows=512).x.to(dev), workloads.swiglu_input(rows=512).w.to(dev),
           workloads.weight_block(rows=512, cols=1024).x.to(dev),
           workloads.activation_channel(rows=1024, cols=512).x.to(dev),
           workloads.student_t(rows=512, cols=1024).x.to(dev))
    x, h, w, wt, a, xt = ins
    f8 = torch.float8_e4m3fn

    def alloc():
        return [torch.empty(256, 7168, dtype=f8, device=dev),
                torch.empty(256, 56, device=dev),
                torch.empty(512, 2048, dtype=f8, device=dev),
                torch.empty(512, 16, device=dev),
                torch.empty(512, 1024, dtype=f8, device=dev),
                torch.empty(4, 8, device=dev),
                torch.empty(512, 1024, dtype=f8, device=dev),
                torch.empty(512, 8, device=dev),
                torch.empty(512, 512, dtype=torch.uint8, device=dev),
                torch.empty(512, 32, device=dev)]

    eager = alloc()
    five_casts(ins, eager)
    torch.cuda.synchronize()
    ref = [t.view(torch.uint8).clone() for t in eager]

    graph_outs = alloc()
    for t in graph_outs:
        t.view(torch.uint8).fill_(0xA5)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):          # warm-up on the capture stream
        five_casts(ins, graph_outs)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        five_casts(ins, graph_outs)
    for replay in range(4):
        for t in graph_outs:
            t.view(torch.uint8).fill_(0x5A + replay)
        torch.cuda.synchronize()
        g.replay()
        five_casts(ins, eager)               # eager work between the replays
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(graph_outs, ref)):
            assert torch.equal(t.view(torch.uint8), r), (replay, i)
        for t, r in zip(eager, ref):
            assert torch.equal(t.view(torch.uint8), r)


def test_graph_replays_count_through_a_workspace(dev):
    # the clamp counters under capture: every replay adds the same count, and
    # the workspace the counting kernels share is zero again after each
    wl = workloads.swiglu_input(rows=1024, cols=2048)
    h, w = wl.x.to(dev), wl.w.to(dev)
    ws = torch.zeros(pq.COUNT_WS_BYTES // 8, dtype=torch.int64, device=dev)
    f8 = torch.float8_e4m3fn
    q = torch.empty(1024, 2048, dtype=f8, device=dev)
    sf = torch.empty(1024, 16, device=dev)
    qt = torch.empty(2048, 1024, dtype=f8, device=dev)
    sft = torch.empty(2048, 8, device=dev)
    counts = torch.zeros(2, dtype=torch.int64, device=dev)

    def counted():
        pq.qcast_swiglu_per_token_ex(h, w, "e4m3", 128, swiglu_clamp=3.0,
                                     clamp_count=counts[0:1], out=q, out_sf=sf,
                                     count_workspace=ws)
        pq.qcast_swiglu_per_channel_T(h, w, "e4m3", 128, swiglu_clamp=3.0,
                                      clamp_count=counts[1:2], out=qt, out_sf=sft,
                                      count_workspace=ws)

    counted()
    torch.cuda.synchronize()
    per_call = counts.clone()
    assert per_call[0] == per_call[1] > 0          # the same values are clamped
    ref = [q.view(torch.uint8).clone(), sf.clone(), qt.view(torch.uint8).clone(), sft.clone()]
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        counted()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        counted()
    counts.zero_()
    torch.cuda.synchronize()
    for replay in range(1, 5):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(counts, replay * per_call), replay
        assert not ws.any(), replay
        got = [q.view(torch.uint8), sf, qt.view(torch.uint8), sft]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), replay


def test_graph_replays_of_the_other_casts(dev):
    # every other entry point under capture: cast_back, E5M6 and its
    # cast_back, packed column-major scales, the SwiGLU backward, the
    # per-channel cast in the input layout and the fused SwiGLU transpose
    x = workloads.per_token_hidden(rows=256).x.to(dev)
    h = workloads.swiglu_input(rows=256, cols=1024).x.to(dev)
    w = workloads.swiglu_input(rows=256, cols=1024).w.to(dev)
    hg, dv, wg = workloads.swiglu_grad(rows=256, cols=1024)
    hg, dv, wg = hg.to(dev), dv.to(dev), wg.to(dev)
    a = workloads.activation_channel(rows=512, cols=384).x.to(dev)
    q8, sf8 = pq.qcast_per_token(x)
    q6, sf6 = pq.qcast_per_token(x, "e5m6", 128)
    torch.cuda.synchronize()
    flags = pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR
    sshape, sdt = pq.sf_layout_shape(256, 7168, 32, flags)
    f8 = torch.float8_e4m3fn

    def alloc():
        return [torch.empty(256, 7168, dtype=torch.bfloat16, device=dev),
                torch.empty(256, 7168, dtype=torch.bfloat16, device=dev),
                torch.empty(256, 7168, dtype=f8, device=dev),
                torch.empty(sshape, dtype=sdt, device=dev),
                torch.empty(256, 2048, dtype=f8, device=dev),
                torch.empty(256, 16, device=dev),
                torch.empty(512, 384, dtype=f8, device=dev),
                torch.empty(4, 384, device=dev),
                torch.empty(1024, 256, dtype=f8, device=dev),
                torch.empty(1024, 2, device=dev)]

    def casts(o):
        pq.qcast_cast_back(q8, sf8, "e4m3", 128, out=o[0])
        pq.qcast_cast_back(q6, sf6, "e5m6", 128, out=o[1])
        pq.qcast_per_token_sf(x, "e4m3", 32, sf_flags=flags, out=o[2], out_sf=o[3])
        pq.qcast_swiglu_backward_per_token(hg, dv, wg, "e4m3", 128, swiglu_clamp=6.0,
                                           out=o[4], out_sf=o[5])
        pq.qcast_per_channel(a, "e4m3", 128, out=o[6], out_sf=o[7])
        pq.qcast_swiglu_per_channel_T(h, w, "e4m3", 128, out=o[8], out_sf=o[9])

    eager = alloc()
    casts(eager)
    torch.cuda.synchronize()
    ref = [t.view(torch.uint8).clone() for t in eager]
    graph_outs = alloc()
    for t in graph_outs:
        t.view(torch.uint8).fill_(0xA5)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        casts(graph_outs)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        casts(graph_outs)
    for replay in range(4):
        for t in graph_outs:
            t.view(torch.uint8).fill_(0x5A + replay)
        torch.cuda.synchronize()
        g.replay()
        casts(eager)                       # eager work between the replays
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(graph_outs, ref)):
            assert torch.equal(t.view(torch.uint8), r), (replay, i)


def test_graph_replays_of_the_scale_option_casts(dev):
    # the _sf entry points of the transposed, backward, per-block and
    # per-channel casts under capture; the packed words of the transposed
    # cast are written one byte per token group, by four different tiles
    a = workloads.activation_channel(rows=1024, cols=384).x.to(dev)
    h = workloads.swiglu_input(rows=512, cols=512).x.to(dev)
    w = workloads.swiglu_input(rows=512, cols=512).w.to(dev)
    hg, dv, wg = workloads.swiglu_grad(rows=256, cols=1024)
    hg, dv, wg = hg.to(dev), dv.to(dev), wg.to(dev)
    wt = workloads.weight_block(rows=256, cols=512).x.to(dev)
    pc = pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR
    rc = pq.SF_ROUND_POW2 | pq.SF_COL_MAJOR
    f8 = torch.float8_e4m3fn
    s_t, d_t = pq.sf_layout_shape(384, 1024, 128, pc)
    s_s, d_s = pq.sf_layout_shape(512, 512, 128, rc)
    s_b, d_b = pq.sf_layout_shape(256, 2048, 128, pq.SF_PACKED_UE8M0)

    def alloc():
        return [torch.empty(384, 1024, dtype=f8, device=dev),
                torch.empty(s_t, dtype=d_t, device=dev),
                torch.empty(pq.code_shape("e2m1", 512, 512), dtype=torch.uint8, device=dev),
                torch.empty(s_s, dtype=d_s, device=dev),
                torch.empty(256, 2048, dtype=f8, device=dev),
                torch.empty(s_b, dtype=d_b, device=dev),
                torch.empty(pq.code_shape("e5m6", 256, 512), dtype=torch.uint8, device=dev),
                torch.empty(2, 4, device=dev),
                torch.empty(1024, 384, dtype=f8, device=dev),
                torch.empty(8, 384, device=dev)]

    def casts(o):
        pq.qcast_per_channel_T_sf(a, "e4m3", 128, sf_flags=pc, out=o[0], out_sf=o[1])
        pq.qcast_swiglu_per_channel_T_sf(h, w, "e2m1", 128, sf_flags=rc, out=o[2], out_sf=o[3])
        pq.qcast_swiglu_backward_per_token_sf(hg, dv, wg, "e4m3", 128,
                                              sf_flags=pq.SF_PACKED_UE8M0, swiglu_clamp=6.0,
                                              out=o[4], out_sf=o[5])
        pq.qcast_per_block_sf(wt, "e5m6", 128, sf_flags=pq.SF_ROUND_POW2, out=o[6], out_sf=o[7])
        pq.qcast_per_channel_sf(a, "e4m3", 128, sf_flags=pq.SF_ROUND_POW2, out=o[8],
                                out_sf=o[9])

    eager = alloc()
    casts(eager)
    torch.cuda.synchronize()
    ref = [t.view(torch.uint8).clone() for t in eager]
    graph_outs = alloc()
    for t in graph_outs:
        t.view(torch.uint8).fill_(0xA5)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        casts(graph_outs)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        casts(graph_outs)
    for replay in range(4):
        for t in graph_outs:
            t.view(torch.uint8).fill_(0x5A + replay)
        torch.cuda.synchronize()
        g.replay()
        casts(eager)                       # eager work between the replays
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(graph_outs, ref)):
            assert torch.equal(t.view(torch.uint8), r), (replay, i)
