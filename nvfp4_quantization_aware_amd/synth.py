"""Seeded synthetic inputs for the QAD hot path.

This module only draws random numbers; it holds none of the quantizer's or
the loss's arithmetic.  The CPU oracle (in the tests) and the HIP library read
the very same bytes produced here.  Every generator takes a seed and a torch
device; on a GPU the draws come from the device's own counter-based generator
(the full-size workloads are too large to draw on the host in a benchmark), on
the CPU from torch's CPU generator -- a given (seed, device) pair always gives
the same tensor.

Workloads (stand-ins for real weights, activations and logits; no dataset is
used):
  * one fp32 tensor 256 x 1024, N(0,1), 0.1 % of the elements (distinct
    positions) multiplied by 50;
  * a MoE layer: E expert matrices [2048][4096] bf16 ~ N(0, 0.02^2), 16
    distinct input columns per expert multiplied by 20, and an upstream
    gradient of the same shape ~ N(0, (1e-3)^2);
  * W4A4 activations: [tokens][4096] bf16, Student-t with 3 degrees of freedom
    (unit scale, drawn as Z / sqrt(chi2_3 / 3)), 8 distinct channels multiplied
    by 30, gradient ~ N(0, (1e-3)^2);
  * a square weight 8192 x 8192 bf16 ~ N(0, 0.02^2) for the frozen-scale path;
  * logits: teacher bf16 ~ N(0, 3^2); student = bf16(float(teacher) + N(0, 0.5^2)).
"""
from __future__ import annotations

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, std=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def outlier_tensor_f32(rows=256, cols=1024, frac=0.001, factor=50.0, seed=1, device="cpu"):
    """fp32 [rows][cols] ~ N(0,1); round(frac*n) distinct elements scaled by factor."""
    g = _gen(seed, device)
    x = _randn((rows, cols), g, device)
    n = rows * cols
    k = int(round(frac * n))
    if k:
        idx = torch.randperm(n, generator=g, device=device)[:k]
        flat = x.view(-1)
        flat[idx] = flat[idx] * factor
    return x


def moe_weights_bf16(experts=128, rows=2048, cols=4096, std=0.02, n_outlier_cols=16,
                     factor=20.0, grad_std=1e-3, seed=2, device="cpu", with_grad=True):
    """Expert weights [E][rows][cols] bf16 with outlier input columns, plus a bf16 gradient."""
    g = _gen(seed, device)
    w = _randn((experts, rows, cols), g, device, std)
    if n_outlier_cols:
        cols_sel = torch.argsort(torch.rand((experts, cols), generator=g, device=device), dim=1)
        cols_sel = cols_sel[:, :n_outlier_cols]
        mult = torch.ones((experts, cols), device=device, dtype=torch.float32)
        mult.scatter_(1, cols_sel, factor)
        w.mul_(mult[:, None, :])
    wb = w.to(torch.bfloat16)
    del w
    grad = None
    if with_grad:
        grad = _randn((experts, rows, cols), g, device, grad_std).to(torch.bfloat16)
    return wb, grad


def student_t_activations_bf16(tokens=32768, hidden=4096, nu=3, n_outlier_ch=8, factor=30.0,
                               grad_std=1e-3, seed=3, device="cpu", with_grad=True):
    """Activations [tokens][hidden] bf16, iid Student-t(nu) with outlier channels."""
    g = _gen(seed, device)
    z = _randn((tokens, hidden), g, device)
    chi2 = torch.zeros((tokens, hidden), device=device, dtype=torch.float32)
    for _ in range(nu):
        e = _randn((tokens, hidden), g, device)
        chi2.addcmul_(e, e)
        del e
    z.div_(torch.sqrt(chi2.div_(float(nu))))
    del chi2
    if n_outlier_ch:
        ch = torch.randperm(hidden, generator=g, device=device)[:n_outlier_ch]
        z[:, ch] = z[:, ch] * factor
    xb = z.to(torch.bfloat16)
    del z
    grad = None
    if with_grad:
        grad = _randn((tokens, hidden), g, device, grad_std).to(torch.bfloat16)
    return xb, grad


def gaussian_weight_bf16(rows=8192, cols=8192, std=0.02, seed=4, device="cpu"):
    g = _gen(seed, device)
    return _randn((rows, cols), g, device, std).to(torch.bfloat16)


def logits_bf16(tokens=8192, vocab=131072, teacher_std=3.0, noise_std=0.5, seed=5, device="cpu"):
    """Teacher logits bf16 ~ N(0, teacher_std^2); student = bf16(teacher + noise)."""
    g = _gen(seed, device)
    t = _randn((tokens, vocab), g, device, teacher_std).to(torch.bfloat16)
    s = _randn((tokens, vocab), g, device, noise_std)
    s.add_(t.float())
    s = s.to(torch.bfloat16)
    return t, s


def bf16_bits(t: torch.Tensor):
    """Raw uint16 bit patterns of a bf16 tensor as a CPU numpy array."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")


def f32_array(t: torch.Tensor):
    return t.detach().contiguous().cpu().numpy()
