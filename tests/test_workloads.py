"""The seeded input recipes: determinism and the structure each one promises."""
import json
import os

import numpy as np
import torch

from precision_quantization_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_same_seed_same_bytes():
    a = workloads.per_token_hidden(rows=64)
    b = workloads.per_token_hidden(rows=64)
    assert workloads.sha256(a.x) == workloads.sha256(b.x)
    c = workloads.per_token_hidden(seed=99, rows=64)
    assert workloads.sha256(a.x) != workloads.sha256(c.x)


def test_per_token_small_structure():
    wl = workloads.per_token_small()
    assert wl.x.shape == (128, 512) and wl.x.dtype == torch.bfloat16
    row_amax = wl.x.float().abs().amax(dim=1)
    hot = sorted(wl.recipe["hot_rows"])
    assert len(set(hot)) == 2
    assert (row_amax[hot] > 50).all()
    others = [r for r in range(128) if r not in hot]
    assert (row_amax[others] < 10).all()


def test_per_token_hidden_structure_small():
    wl = workloads.per_token_hidden(rows=1000, cols=1024)
    x = wl.x.float()
    zero_rows = (x == 0).all(dim=1)
    assert zero_rows.sum().item() == 10            # round(1% of 1000)
    assert (x[zero_rows].view(torch.int32) == 0).all()   # +0.0
    assert wl.recipe["outliers"] == round(0.001 * 1000 * 1024)
    big = (x.abs() > 8).sum().item()
    assert 0.5 * wl.recipe["outliers"] < big <= wl.recipe["outliers"] + 5


def test_swiglu_input_halves_and_weight():
    wl = workloads.swiglu_input(rows=512, cols=256)
    assert wl.x.shape == (512, 512) and wl.w.shape == (512,) and wl.w.dtype == torch.float32
    assert 0 <= wl.w.min() and wl.w.max() < 1
    std = wl.x.float().std().item()
    assert 1.9 < std < 2.1
    assert wl.cols == 256


def test_student_t_heavy_tail():
    wl = workloads.student_t(rows=256, cols=1024)
    x = wl.x.float()
    # t(3) has infinite kurtosis: far more mass beyond 5 scale units than a normal
    assert (x.abs() > 2.5).float().mean() > 1e-3
    med = x.abs().median().item()
    assert 0.3 < med < 0.45        # 0.5 * median|t3| = 0.5 * 0.765


def test_algorithmic_bytes_match_the_configured_sizes():
    # Bytes = inputs once + codes + fp32 scales, at the full workload shapes
    def fake(op, shape, fmt="e4m3", group=128, w=False):
        x = torch.empty(shape, dtype=torch.bfloat16)
        return workloads.Workload(op, op, x, fmt, group, w=torch.empty(shape[0]) if w else None)
    assert fake("per_token", (128, 512)).algorithmic_bytes() == 198_656
    assert fake("per_token", (4096, 7168)).algorithmic_bytes() == 88_997_888
    assert fake("swiglu_per_token", (8192, 4096), w=True).algorithmic_bytes() == 84_443_136
    assert fake("per_block", (7168, 18432)).algorithmic_bytes() == 396_393_984
    assert fake("per_channel_T", (16384, 7168)).algorithmic_bytes() == 355_991_552
    assert fake("e2m1", (16384, 7168), "e2m1", 32).algorithmic_bytes() == 308_281_344
