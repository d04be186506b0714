"""Pins of the oracle's teacher-top-k KL.

Page 'Model-Optimizer 实战 ... W4A4 NVFP4 精度' (nlpx.cn), section '3. QAD': the
distillation run restricts the KD loss to the teacher's top-4096 vocabulary
entries.  The page gives no tie rule and no normalisation; the oracle keeps
every entry tied with the k-th largest teacher logit and renormalises both
softmaxes over the kept set.

Pins: a hand-derived row (tests/golden/kl_topk_worked_example.json); k >= V
equals the full-vocabulary KL; equality with the full KL applied to the kept
sub-vectors, the kept set found independently by a numpy sort; the tie rule
on constructed ties; KL(p||p) = 0 and KL >= 0; the gradient is 0 outside the
set and sums to 0 over it; central finite differences of the loss.
"""
import json
import math
import os

import numpy as np
import pytest

from nvfp4_quantization_aware_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_worked_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "kl_topk_worked_example.json")))
    t = np.array([g["teacher"]], np.float32)
    s = np.array([g["student"]], np.float32)
    loss, row, grad, cnt = orc.kl_topk_fwd_bwd(t, s, 2, grad_scale=1.0)
    assert cnt[0] == g["k2"]["count"]
    assert abs(loss - (math.log(1 + math.e ** 2) - 1 - math.log(2))) < 1e-14
    assert np.allclose(grad[0], g["k2"]["grad"], rtol=0, atol=1e-15)
    _, _, _, cnt3 = orc.kl_topk_fwd_bwd(t, s, 3)
    assert cnt3[0] == g["k3_count"]


@pytest.mark.parametrize("T", [1.0, 0.5])
def test_k_at_least_vocab_is_full_kl(orc, T):
    t, s = synth.logits_bf16(tokens=5, vocab=777 * 8, seed=11)
    tb, sb = synth.bf16_bits(t), synth.bf16_bits(s)
    full = orc.kl_fwd_bwd(tb, sb, T=T)
    for k in (tb.shape[1], tb.shape[1] + 5):
        top = orc.kl_topk_fwd_bwd(tb, sb, k, T=T)
        assert top[0] == full[0]
        assert np.array_equal(top[1], full[1]) and np.array_equal(top[2], full[2])
        assert np.all(top[3] == tb.shape[1])


@pytest.mark.parametrize("k", [1, 7, 64, 1000])
def test_equals_full_kl_on_kept_subvectors(orc, k):
    rng = np.random.default_rng(3)
    V = 2048
    t = np.round(rng.normal(0, 3, (4, V)) * 8) / 8          # coarse grid: many ties
    s = t + rng.normal(0, 0.5, (4, V))
    t, s = t.astype(np.float32), s.astype(np.float32)
    loss, row, grad, cnt = orc.kl_topk_fwd_bwd(t, s, k, grad_scale=1.0)
    for r in range(4):
        tau = np.sort(t[r])[::-1][k - 1]
        keep = t[r] >= tau
        assert cnt[r] == keep.sum() >= k
        sub = orc.kl_fwd_bwd(t[r:r + 1, keep], s[r:r + 1, keep], grad_scale=1.0)
        assert abs(row[r] - sub[1][0]) <= 1e-12 * max(1.0, abs(sub[1][0]))
        assert np.allclose(grad[r, keep], sub[2][0], rtol=0, atol=1e-15)
        assert np.all(grad[r, ~keep] == 0.0)


def test_ties_at_the_boundary_are_kept(orc):
    t = np.array([[5, 4, 4, 4, 4, 1, 0, 4]], np.float32)
    s = np.zeros_like(t)
    for k, want in ((1, 1), (2, 6), (5, 6), (6, 6), (7, 7), (8, 8)):
        assert orc.kl_topk_fwd_bwd(t, s, k)[3][0] == want


def test_identical_and_nonnegative(orc):
    t, s = synth.logits_bf16(tokens=6, vocab=4096, seed=21)
    tb, sb = synth.bf16_bits(t), synth.bf16_bits(s)
    loss, row, grad, _ = orc.kl_topk_fwd_bwd(tb, tb, 100)
    assert loss == 0.0 and np.all(row == 0.0) and np.all(grad == 0.0)
    loss, row, grad, cnt = orc.kl_topk_fwd_bwd(tb, sb, 100, grad_scale=1.0)
    assert np.all(row > 0.0)
    assert np.all(np.abs(grad.sum(axis=1)) < 1e-14)
    assert np.all((grad != 0).sum(axis=1) <= cnt)


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_finite_differences(orc, T):
    rng = np.random.default_rng(5)
    V, k = 64, 9
    t = (np.round(rng.normal(0, 3, (2, V)) * 1024) / 1024).astype(np.float32)
    s = (np.round(rng.normal(0, 3, (2, V)) * 1024) / 1024).astype(np.float32)
    _, _, grad, cnt = orc.kl_topk_fwd_bwd(t, s, k, T=T, grad_scale=0.5)
    h = 2.0 ** -10
    for r in range(2):
        for v in range(V):
            sp, sm = s.copy(), s.copy()
            sp[r, v] += h
            sm[r, v] -= h
            lp = orc.kl_topk_fwd_bwd(t, sp, k, T=T)[0]
            lm = orc.kl_topk_fwd_bwd(t, sm, k, T=T)[0]
            fd = (lp - lm) / (2 * h)       # d(mean over 2 rows)/ds = grad with grad_scale 1/2
            assert abs(fd - grad[r, v]) <= 1e-6 * max(1.0, abs(grad[r, v])), (r, v, fd, grad[r, v])
