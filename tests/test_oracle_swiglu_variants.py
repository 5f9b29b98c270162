"""Pins of the oracle's SwiGLU variants and of the per-channel cast without
transpose.

Pages (cited by title and section):
  walk  = "DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限"
          §3.3 (SwiGLU with an optional clamp of the gate from above and of
          the up value to [-c, c], and a counter of clamped values)
  split = "TileKernels 与 DeepGEMM 的分界线：DeepSeek 开源内核栈的分工"
          §二 (swiglu_backward_and_per_token_cast; per_channel_cast with and
          without transpose)
  news  = "DeepSeek open-sources TileKernels" item 2 (SwiGLU fused with the
          cast and the transpose)

The backward is pinned against float64 automatic differentiation of the
forward; the clamp against a NumPy clip of the inputs and counts fixed by
construction; the fused and transposed forms against the plain per-token cast
of the transposed values.
"""
import numpy as np
import pytest
import torch

import oracle
from precision_quantization_amd import workloads


def bf16(values):
    return workloads.bf16_bits(torch.tensor(np.asarray(values, np.float32)).to(torch.bfloat16))


def bf16_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def unpack_e2m1(q):
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def small_grad(seed=11, rows=64, cols=256, std=2.0, weighted=True):
    h, dv, w = workloads.swiglu_grad(seed=seed, rows=rows, cols=cols, std=std,
                                     with_weight=weighted)
    return (workloads.bf16_bits(h), workloads.bf16_bits(dv), None if w is None else w.numpy())


# ------------------------------------------------------------------ clamp

def test_clamp_counts_fixed_by_construction():
    rows, cols, c = 4, 128, 3.0
    g = np.zeros((rows, cols), np.float32) + 0.5
    u = np.zeros((rows, cols), np.float32) - 0.25
    g[0, :7] = 3.5          # 7 gates above c
    g[1, :5] = -50.0        # very negative gates: one-sided clamp, not counted
    u[2, :3] = 4.0          # 3 up values above c
    u[3, :11] = -8.0        # 11 up values below -c
    g[3, 20] = 3.0          # exactly c: unchanged, not counted
    u[3, 21] = -3.0
    h = bf16(np.concatenate([g, u], axis=1))
    v, n = oracle.swiglu_values_ex(h, swiglu_clamp=c)
    assert n == 7 + 3 + 11
    _, n0 = oracle.swiglu_values_ex(h, swiglu_clamp=0.0)
    assert n0 == 0
    # The counter of the fused cast is the same count.
    _, _, n_cast = oracle.swiglu_per_token_ex(h, swiglu_clamp=c)
    assert n_cast == 21


@pytest.mark.parametrize("c", [0.75, 2.0, 5.0])
@pytest.mark.parametrize("weighted", [False, True])
def test_clamp_equals_unclamped_swiglu_of_clipped_input(c, weighted):
    # c is a bf16 value, so clipping the bf16 inputs gives bf16 inputs.
    wl = workloads.swiglu_input(seed=21, rows=32, cols=256, with_weight=weighted)
    h = workloads.bf16_bits(wl.x)
    w = None if wl.w is None else wl.w.numpy()
    hf = bf16_to_f32(h)
    n = hf.shape[1] // 2
    gate, up = hf[:, :n], hf[:, n:]
    clipped = np.concatenate([np.minimum(gate, c), np.clip(up, -c, c)], axis=1)
    expect = oracle.swiglu_values(bf16(clipped), w)
    got, count = oracle.swiglu_values_ex(h, w, swiglu_clamp=c)
    np.testing.assert_array_equal(got.view(np.uint32), expect.view(np.uint32))
    assert count == int((gate > c).sum() + (np.abs(up) > c).sum())


@pytest.mark.parametrize("sf_flags", [0, oracle.SF_ROUND_POW2,
                                      oracle.SF_PACKED_UE8M0 | oracle.SF_COL_MAJOR])
def test_clamped_cast_is_per_token_of_clamped_values(sf_flags):
    wl = workloads.swiglu_input(seed=22, rows=20, cols=1024)
    h, w = workloads.bf16_bits(wl.x), wl.w.numpy()
    q, sf, n = oracle.swiglu_per_token_ex(h, w, sf_flags=sf_flags, swiglu_clamp=1.5)
    v, n_v = oracle.swiglu_values_ex(h, w, swiglu_clamp=1.5)
    assert n == n_v > 0
    # Unclamped through the same entry point == the plain layout cast.
    q0, sf0, n0 = oracle.swiglu_per_token_ex(h, w, sf_flags=sf_flags)
    q1, sf1 = oracle.swiglu_per_token_sf(h, w, sf_flags=sf_flags)
    assert n0 == 0
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(sf0, sf1)
    if sf_flags == 0:
        qv, sfv = oracle.per_token_f32(v)
        np.testing.assert_array_equal(q, qv)
        np.testing.assert_array_equal(sf, sfv)


# --------------------------------------------------------------- backward

def autograd_backward(h_bits, dv_bits, w, c):
    """[dg | du] by float64 automatic differentiation of
    v = silu(min(g, c)) * clamp(u, -c, c) * w."""
    hf = torch.from_numpy(bf16_to_f32(h_bits).astype(np.float64))
    n = hf.shape[1] // 2
    g = hf[:, :n].clone().requires_grad_(True)
    u = hf[:, n:].clone().requires_grad_(True)
    gc = torch.clamp(g, max=c) if c > 0 else g
    uc = torch.clamp(u, -c, c) if c > 0 else u
    v = torch.nn.functional.silu(gc) * uc
    if w is not None:
        v = v * torch.from_numpy(w.astype(np.float64))[:, None]
    v.backward(torch.from_numpy(bf16_to_f32(dv_bits).astype(np.float64)))
    return torch.cat([g.grad, u.grad], dim=1).numpy()


@pytest.mark.parametrize("c", [0.0, 3.0])
@pytest.mark.parametrize("weighted", [False, True])
def test_backward_matches_float64_autograd(c, weighted):
    h, dv, w = small_grad(seed=31 + int(c), weighted=weighted)
    got = oracle.swiglu_backward_values(h, dv, w, swiglu_clamp=c).astype(np.float64)
    ref = autograd_backward(h, dv, w, c)
    # fp32 evaluation of a few operations: a few ulps of the largest terms.
    scale = np.abs(ref).max()
    np.testing.assert_allclose(got, ref, rtol=2e-6, atol=scale * 1e-6)
    # Clamped positions carry no gradient at all.
    if c > 0:
        hf = bf16_to_f32(h)
        n = hf.shape[1] // 2
        assert np.all(got[:, :n][hf[:, :n] > c] == 0)
        assert np.all(got[:, n:][np.abs(hf[:, n:]) > c] == 0)
        assert (hf[:, :n] > c).any() and (np.abs(hf[:, n:]) > c).any()


def test_backward_special_values():
    # g = 0: sigmoid = 1/2 exactly, silu = 0, derivative of silu = 1/2.
    n = 128
    g = np.zeros((1, n), np.float32)
    u = np.linspace(-3, 3, n).astype(np.float32)[None, :]
    h = bf16(np.concatenate([g, u], axis=1))
    dv = bf16(np.full((1, n), 2.0, np.float32))
    out = oracle.swiglu_backward_values(h, dv, np.array([0.5], np.float32))
    uf = bf16_to_f32(h)[:, n:]
    np.testing.assert_array_equal(out[:, :n], (1.0 * uf * 0.5).astype(np.float32))
    assert np.all(out[:, n:] == 0)
    # Large gate: sigmoid -> 1, silu -> g, derivative -> 1.
    h = bf16(np.concatenate([np.full((1, n), 40.0, np.float32), u], axis=1))
    out = oracle.swiglu_backward_values(h, bf16(np.ones((1, n), np.float32)))
    np.testing.assert_array_equal(out[:, :n], uf)
    np.testing.assert_array_equal(out[:, n:], np.full((1, n), 40.0, np.float32))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("group", [32, 128])
def test_backward_cast_is_per_token_of_backward_values(fmt, group):
    h, dv, w = small_grad(seed=41, rows=24, cols=512)
    q, sf = oracle.swiglu_backward_per_token(h, dv, w, fmt=fmt, group=group, swiglu_clamp=4.0)
    vals = oracle.swiglu_backward_values(h, dv, w, swiglu_clamp=4.0)
    qv, sfv = oracle.per_token_f32(vals, fmt=fmt, group=group)
    np.testing.assert_array_equal(q, qv)
    np.testing.assert_array_equal(sf, sfv)
    assert q.shape == (24, 1024) and sf.shape == (24, 1024 // group)


@pytest.mark.parametrize("fmt", ["e2m1", "e5m6"])
def test_backward_cast_in_the_packed_formats_is_per_token_of_backward_values(fmt):
    h, dv, w = small_grad(seed=42, rows=8, cols=256)
    q, sf = oracle.swiglu_backward_per_token(h, dv, w, fmt=fmt, group=32, swiglu_clamp=4.0)
    vals = oracle.swiglu_backward_values(h, dv, w, swiglu_clamp=4.0)
    qv, sfv = oracle.per_token_f32(vals, fmt=fmt, group=32)
    np.testing.assert_array_equal(q, qv)
    np.testing.assert_array_equal(sf, sfv)


# ------------------------------------------------- fused SwiGLU + transpose

@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e5m2", 128), ("e4m3", 64),
                                       ("e2m1", 32)])
def test_swiglu_per_channel_T_is_per_token_of_transposed_values(fmt, group):
    wl = workloads.swiglu_input(seed=51, rows=256, cols=192)
    h, w = workloads.bf16_bits(wl.x), wl.w.numpy()
    qT, sf = oracle.swiglu_per_channel_T(h, w, fmt=fmt, group=group, swiglu_clamp=5.0)
    v, _ = oracle.swiglu_values_ex(h, w, swiglu_clamp=5.0)
    q_ref, sf_ref = oracle.per_token_f32(np.ascontiguousarray(v.T), fmt=fmt, group=group)
    np.testing.assert_array_equal(qT, q_ref)
    np.testing.assert_array_equal(sf, sf_ref)


# -------------------------------------------- per-channel without transpose

@pytest.mark.parametrize("fmt,group", [("e4m3", 128), ("e5m2", 128), ("e4m3", 32),
                                       ("e2m1", 32)])
def test_per_channel_is_transpose_of_per_channel_T(fmt, group):
    wl = workloads.activation_channel(seed=61, rows=384, cols=320)
    x = workloads.bf16_bits(wl.x)
    q, sf = oracle.per_channel(x, fmt=fmt, group=group)
    qT, sfT = oracle.per_channel_T(x, fmt=fmt, group=group)
    if fmt == "e2m1":
        q, qT = unpack_e2m1(q), unpack_e2m1(qT)
    np.testing.assert_array_equal(q, qT.T)
    np.testing.assert_array_equal(sf, sfT.T)
    # ... and of the per-token cast of the transpose.
    qt2, sft2 = oracle.per_token(np.ascontiguousarray(x.T), fmt=fmt, group=group)
    if fmt == "e2m1":
        qt2 = unpack_e2m1(qt2)
    np.testing.assert_array_equal(q, qt2.T)
    np.testing.assert_array_equal(sf, sft2.T)


def test_per_channel_scale_hand_example():
    # One channel whose 128 tokens peak at 448 * 2: scale 2, codes of x / 2.
    x = np.zeros((128, 2), np.float32)
    x[:, 0] = np.linspace(-1, 1, 128)
    x[5, 0] = 896.0
    x[:, 1] = 0.0
    q, sf = oracle.per_channel(bf16(x))
    assert sf.shape == (1, 2)
    assert sf[0, 0] == np.float32(2.0)
    assert sf[0, 1] == np.float32(1e-4) / np.float32(448.0)
    assert q[5, 0] == 0x7E
    assert np.all(q[:, 1] == 0)
