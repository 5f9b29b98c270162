"""Entry points called from several host threads at once, each thread on its
own stream: every result equals the one the same call gives alone (the
library's host-side state is atomic or per thread)."""
import threading

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


def same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_two_threads_two_streams(dev):
    inputs = [workloads.activation_channel(seed=30 + i, rows=1024, cols=1024).x.to(dev)
              for i in range(2)]
    hs = [workloads.swiglu_input(seed=40 + i, rows=512, cols=512) for i in range(2)]
    hs = [(wl.x.to(dev), wl.w.to(dev)) for wl in hs]
    # results of each call made alone
    alone = []
    for x, (h, w) in zip(inputs, hs):
        alone.append((pq.qcast_per_token(x), pq.qcast_per_channel_T(x),
                      pq.qcast_swiglu_per_token(h, w)))
    torch.cuda.synchronize()

    rounds = 25
    results = [[None] * rounds for _ in range(2)]
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream(device=dev)
            x, (h, w) = inputs[i], hs[i]
            with torch.cuda.stream(s):
                for r in range(rounds):
                    results[i][r] = (pq.qcast_per_token(x, stream=s),
                                     pq.qcast_per_channel_T(x, stream=s),
                                     pq.qcast_swiglu_per_token(h, w, stream=s))
            s.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(rounds):
            for (q, sf), (q0, sf0) in zip(results[i][r], alone[i]):
                assert same(q, q0) and same(sf, sf0), (i, r)
