"""Helpers shared by the GPU parity tests (conversion of device tensors to the
numpy forms the oracle takes, and the comparison rules)."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def gpu_device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from nvfp4_quantization_aware_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from nvfp4_quantization_aware_amd import build
        build.build()
    return torch.device("cuda:0")


def announce(msg):
    """Name the case before a GPU step (so a fault can be traced to it)."""
    print("[gpu-case] " + msg, file=sys.stderr, flush=True)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in the oracle's representation (bf16 as uint16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_ulp(a: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at magnitude |a| (8 significant bits)."""
    a = np.maximum(np.abs(a), 2.0**-133)
    e = np.floor(np.log2(a))
    return np.maximum(2.0 ** (e - 7), 2.0**-133)


def prob_scale(t_bits: np.ndarray, s_bits: np.ndarray, T: float, grad_scale: float, kept=None):
    """Per row, the size of the probabilities whose difference the gradient
    is: max_v and L2 over v of (p_v + q_v) grad_scale / T, in binary64 from the
    inputs (bf16 bits or float32).  `kept` (bool, the shape of the inputs):
    the probabilities renormalized over the kept entries of each row, as the
    top-k and top-p losses take them."""
    f = lambda a: ((a.astype(np.uint32) << 16).view(np.float32) if a.dtype == np.uint16 else a).astype(np.float64)
    def softmax(x):
        x = x / T
        if kept is not None:
            x = np.where(kept, x, -np.inf)
        e = np.exp(x - x.max(axis=-1, keepdims=True))
        return e / e.sum(axis=-1, keepdims=True)
    ps = (softmax(f(t_bits)) + softmax(f(s_bits))) * grad_scale / T
    return ps.max(axis=-1), np.linalg.norm(ps, axis=-1)


def assert_kl_grad_close(g_dev: np.ndarray, g_ref: np.ndarray, rel=1e-5, zero_row_scale=0.0, floor=None):
    """Gradient rule: per row, |g - g_ref| <= rel * max_row |g_ref| for a
    float32 gradient; for bf16, the bf16 rounding of a value within that band
    (so additionally half a bf16 ulp).  A row whose reference gradient is 0
    everywhere (p and q equal, e.g. a single kept entry) has no relative
    scale; there `zero_row_scale` (grad_scale / T, the bound of |q - p| times
    the factor) stands in for max_row |g_ref|.  `floor` = prob_scale(...):
    the fp32 floor of a difference of probabilities, 1e-6 of the row's
    largest (p + q) grad_scale / T (and 1e-6 of its L2 for the L2 rule); it
    only matters on rows whose gradient is far smaller than the
    probabilities themselves (near one-hot rows where teacher and student
    agree)."""
    g_ref = np.asarray(g_ref, np.float64)
    row_max = np.abs(g_ref).max(axis=-1, keepdims=True)
    tol = rel * np.where(row_max > 0, row_max, zero_row_scale)
    if floor is not None:
        tol = np.maximum(tol, 1e-6 * np.asarray(floor[0])[:, None])
    if g_dev.dtype == np.uint16:
        g = (g_dev.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        bound = tol + 0.5 * bf16_ulp(np.abs(g_ref) + tol)
    else:
        g = g_dev.astype(np.float64)
        bound = tol
        l2 = np.linalg.norm(g - g_ref, axis=-1)
        l2_ref = np.linalg.norm(g_ref, axis=-1)
        l2_tol = rel * np.where(l2_ref > 0, l2_ref, zero_row_scale * np.sqrt(g_ref.shape[-1]))
        if floor is not None:
            l2_tol = np.maximum(l2_tol, 1e-6 * np.asarray(floor[1]))
        assert np.all(l2 <= l2_tol), l2.max()
    err = np.abs(g - g_ref)
    bad = err > bound
    assert not bad.any(), "worst excess %g at %s" % ((err - bound).max(), np.argwhere(bad)[:3])
