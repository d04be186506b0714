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


def f32_ulp(a: np.ndarray) -> np.ndarray:
    """Spacing of binary32 numbers at magnitude |a| (2^-149 below 2^-126)."""
    a = np.maximum(np.abs(np.asarray(a, np.float64)), 2.0**-126)
    return 2.0 ** (np.floor(np.log2(a)) - 23)


def _f64(a: np.ndarray) -> np.ndarray:
    return ((a.astype(np.uint32) << 16).view(np.float32) if a.dtype == np.uint16 else a).astype(np.float64)


def kl_probs(t_bits: np.ndarray, s_bits: np.ndarray, T: float, kept=None):
    """binary64 teacher and student probabilities p = softmax(t/T), q =
    softmax(s/T) of each row (inputs as bf16 bits or float32); `kept` (bool,
    the inputs' shape): renormalised over the kept entries, 0 elsewhere, as
    the top-k and top-p losses take them."""
    def softmax(x):
        x = x / T
        if kept is not None:
            x = np.where(kept, x, -np.inf)
        e = np.exp(x - x.max(axis=-1, keepdims=True))
        return e / e.sum(axis=-1, keepdims=True)
    return softmax(_f64(t_bits)), softmax(_f64(s_bits))


def assert_kl_grad_close(g_dev: np.ndarray, g_ref: np.ndarray, probs, grad_scale: float, T: float, rel=1e-5):
    """Gradient rule, element by element: with p, q = probs (kl_probs),
        |g - g_ref| <= rel |g_ref| + 1e-6 (p + q) grad_scale / T
    -- 1e-5 of the element itself, and 1e-6 of the two probabilities whose
    difference it is (a binary32 probability carries a few units in its last
    place) -- plus the output format's own rounding: one binary32 ulp of
    g_ref (2^-149 below 2^-126) for an fp32 gradient, half a bf16 ulp of
    |g_ref| + that band for a bf16 one.  Per row, for fp32: the L2 error
    within rel ||g_ref|| + 1e-6 ||p + q|| grad_scale / T."""
    g_ref = np.asarray(g_ref, np.float64)
    p, q = probs
    pq = (p + q) * (grad_scale / T)
    tol = rel * np.abs(g_ref) + 1e-6 * pq
    if g_dev.dtype == np.uint16:
        g = _f64(g_dev)
        bound = tol + 0.5 * bf16_ulp(np.abs(g_ref) + tol)
    else:
        g = g_dev.astype(np.float64)
        bound = tol + f32_ulp(g_ref)
        l2 = np.linalg.norm(g - g_ref, axis=-1)
        l2_tol = rel * np.linalg.norm(g_ref, axis=-1) + 1e-6 * np.linalg.norm(pq, axis=-1)
        assert np.all(l2 <= l2_tol), (l2 / l2_tol).max()
    err = np.abs(g - g_ref)
    bad = err > bound
    assert not bad.any(), "worst err/bound %g at %s" % ((err / bound).max(), np.argwhere(bad)[:3])


# A row whose exact KL is 0 (teacher and student distributions equal, e.g. a
# single kept entry) has no relative scale; the library's term-wise sum then
# holds only the second-order rounding of its log-ratios (|x| ~ 1e-7 gives
# psi(x) ~ 1e-15).
ZERO_KL_TOL = 1e-12


def assert_kl_loss_close(val, ref, rel=1e-5):
    """Loss rule (one mean or per-row losses): |val - ref| <= rel |ref|; where
    ref is exactly 0, |val| <= ZERO_KL_TOL."""
    val = np.asarray(val, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = np.where(ref == 0.0, ZERO_KL_TOL, rel * np.abs(ref))
    err = np.abs(val - ref)
    assert np.all(err <= bound), "worst err/bound %g at %s (val %s ref %s)" % (
        (err / bound).max(), np.argmax(err / bound), val.ravel()[np.argmax(err / bound)],
        ref.ravel()[np.argmax(err / bound)])
