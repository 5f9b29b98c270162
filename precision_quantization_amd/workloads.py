"""Seeded synthetic inputs for the quantization casts.

This module only draws random numbers: it holds none of the casts'
arithmetic, and both the GPU tests and the CPU oracle take their inputs from
it. Every recipe samples in fp32 with a CPU ``torch.Generator`` seeded from the
recipe, applies its structure (scaling, zeroing) in fp32, and rounds to bf16
once (round-to-nearest-even). Standard deviations are written ``std``.

The shapes default to DeepSeek-V3 MoE sizes (hidden 7168, expert
intermediate 2048, a 7168 x 18432 weight); every recipe also takes smaller
shapes so the same structure can be exercised at sizes the oracle finishes in
seconds.
"""
from dataclasses import dataclass, field
import hashlib

import numpy as np
import torch


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def bf16_bits(t):
    """bf16 tensor (CPU) -> numpy uint16 array of its bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(a):
    """numpy uint16 bit patterns -> bf16 CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16)


def sha256(t):
    """SHA-256 of a tensor's (or array's) bytes."""
    if isinstance(t, torch.Tensor):
        t = t.contiguous().view(torch.uint8).numpy()
    return hashlib.sha256(np.ascontiguousarray(t).tobytes()).hexdigest()


@dataclass
class Workload:
    """One cast's inputs plus the parameters the cast is called with."""
    name: str
    op: str                      # per_token | swiglu_per_token | per_block | per_channel_T | e2m1
    x: torch.Tensor              # bf16 input (CPU)
    fmt: str = "e4m3"
    group: int = 128
    w: torch.Tensor = None       # fp32 per-row weight (SwiGLU only)
    recipe: dict = field(default_factory=dict)

    @property
    def rows(self):
        return self.x.shape[0]

    @property
    def cols(self):
        """Logical output columns of the cast (half of H's width for SwiGLU)."""
        return self.x.shape[1] // 2 if self.op == "swiglu_per_token" else self.x.shape[1]

    def algorithmic_bytes(self):
        """Bytes the cast must move: its inputs once, its codes and scales once."""
        r, c = self.x.shape
        inp = r * c * 2 + (r * 4 if self.w is not None else 0)
        n_out = self.rows * self.cols
        if self.op == "per_block":
            codes, scales = n_out, (r // self.group) * (c // self.group) * 4
        elif self.op == "per_channel_T":
            codes, scales = n_out, (r // self.group) * c * 4
        elif self.fmt == "e2m1":
            codes, scales = n_out // 2, n_out // self.group * 4
        else:
            codes, scales = n_out, n_out // self.group * 4
        return inp + codes + scales


def per_token_small(seed=1, rows=128, cols=512, hot_rows=2, hot_scale=100.0):
    """X ~ N(0, 1) with `hot_rows` distinct rows scaled by `hot_scale`."""
    g = _gen(seed)
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    hot = torch.randperm(rows, generator=g)[:hot_rows]
    x[hot] *= hot_scale
    return Workload("per_token_small", "per_token", x.to(torch.bfloat16), "e4m3", 128,
                    recipe=dict(seed=seed, rows=rows, cols=cols, dist="N(0,1)",
                                hot_rows=hot.tolist(), hot_scale=hot_scale))


def per_token_hidden(seed=2, rows=4096, cols=7168, outlier_frac=0.001, outlier_scale=100.0,
                     zero_row_frac=0.01):
    """X ~ N(0, 1); round(outlier_frac * numel) distinct positions scaled by
    `outlier_scale`; round(zero_row_frac * rows) distinct rows set to +0."""
    g = _gen(seed)
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    n_out = int(round(outlier_frac * rows * cols))
    pos = torch.randperm(rows * cols, generator=g)[:n_out]
    x.view(-1)[pos] *= outlier_scale
    n_zero = int(round(zero_row_frac * rows))
    zrows = torch.randperm(rows, generator=g)[:n_zero]
    x[zrows] = 0.0
    return Workload("per_token_hidden", "per_token", x.to(torch.bfloat16), "e4m3", 128,
                    recipe=dict(seed=seed, rows=rows, cols=cols, dist="N(0,1)",
                                outliers=n_out, outlier_scale=outlier_scale, zero_rows=n_zero))


def swiglu_input(seed=3, rows=8192, cols=2048, std=2.0, with_weight=True):
    """H = [gate | up], each [rows, cols], entries N(0, std); w ~ U(0, 1) in
    fp32 (not rounded to bf16)."""
    g = _gen(seed)
    h = torch.randn(rows, 2 * cols, generator=g, dtype=torch.float32) * std
    w = torch.rand(rows, generator=g, dtype=torch.float32) if with_weight else None
    return Workload("swiglu_per_token", "swiglu_per_token", h.to(torch.bfloat16), "e4m3", 128,
                    w=w, recipe=dict(seed=seed, rows=rows, cols=cols, dist=f"N(0,{std})",
                                     weight="U(0,1) fp32" if with_weight else None))


def swiglu_grad(seed=7, rows=8192, cols=2048, std=2.0, grad_std=1.0, with_weight=True):
    """Inputs of the SwiGLU backward: H = [gate | up] N(0, std) and the
    gradient dV [rows, cols] N(0, grad_std), both bf16; w ~ U(0, 1) fp32 or
    None. Returns (h, dv, w)."""
    g = _gen(seed)
    h = torch.randn(rows, 2 * cols, generator=g, dtype=torch.float32) * std
    dv = torch.randn(rows, cols, generator=g, dtype=torch.float32) * grad_std
    w = torch.rand(rows, generator=g, dtype=torch.float32) if with_weight else None
    return h.to(torch.bfloat16), dv.to(torch.bfloat16), w


def weight_block(seed=4, rows=7168, cols=18432, std=0.02):
    """W ~ N(0, std), cast with one scale per 128 x 128 block."""
    g = _gen(seed)
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32) * std
    return Workload("per_block", "per_block", x.to(torch.bfloat16), "e4m3", 128,
                    recipe=dict(seed=seed, rows=rows, cols=cols, dist=f"N(0,{std})"))


def activation_channel(seed=5, rows=16384, cols=7168, std=1.0):
    """A ~ N(0, std) [tokens, channels], cast per channel per 128 tokens and
    written transposed."""
    g = _gen(seed)
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    if std != 1.0:
        x *= std
    return Workload("per_channel_T", "per_channel_T", x.to(torch.bfloat16), "e4m3", 128,
                    recipe=dict(seed=seed, rows=rows, cols=cols, dist=f"N(0,{std})"))


def student_t(seed=6, rows=16384, cols=7168, nu=3, scale=0.5):
    """X = scale * Z / sqrt(chi2_nu / nu), chi2_nu a sum of nu squared
    standard normals drawn after Z; cast to E2M1 with groups of 32."""
    g = _gen(seed)
    z = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    chi2 = torch.zeros(rows, cols, dtype=torch.float32)
    for _ in range(nu):
        n = torch.randn(rows, cols, generator=g, dtype=torch.float32)
        chi2.addcmul_(n, n)
        del n
    x = z.mul_(scale).div_(chi2.div_(nu).sqrt_())
    del chi2
    return Workload("e2m1", "e2m1", x.to(torch.bfloat16), "e2m1", 32,
                    recipe=dict(seed=seed, rows=rows, cols=cols, dist=f"{scale}*t(nu={nu})"))


# The five workloads the casts are measured on, at their full sizes.
FULL = {
    "per_token_small": per_token_small,
    "per_token_hidden": per_token_hidden,
    "swiglu_per_token": swiglu_input,
    "per_block": weight_block,
    "per_channel_T": activation_channel,
    "e2m1": student_t,
}
