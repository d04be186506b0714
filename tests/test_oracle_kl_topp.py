"""Pins of the oracle's teacher-top-p (nucleus) KL.

Page 'Model-Optimizer 实战 ... W4A4 NVFP4 精度' (nlpx.cn), section '3. QAD':
after the top-k run the page suggests top-p next, with no definition.  The
reading: the nucleus of the teacher distribution, every entry at or above the
largest teacher value at which the accumulated teacher mass reaches top_p
(ties kept), both softmaxes renormalised over it.

Pins: a hand-derived row (tests/golden/kl_topp_worked_example.json); a row
whose probabilities are fixed by construction (logits ln w); brute force on
small rows with many ties (numpy sort and cumulative sums, written here
independently) for the threshold, the set size and the mass bounds, then the
loss and gradient against the top-k KL (itself pinned) on the same set;
top_p >= 1 equals the full-vocabulary KL; a tiny top_p keeps only the
argmax group; set sizes grow with top_p.
"""
import json
import math
import os

import numpy as np
import pytest

from nvfp4_quantization_aware_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_worked_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "kl_topp_worked_example.json")))
    t = np.array([g["teacher"]], np.float32)
    s = np.array([g["student"]], np.float32)
    loss, row, grad, cnt, tau, mass = orc.kl_topp_fwd_bwd(t, s, 0.5, grad_scale=1.0)
    assert cnt[0] == g["p05"]["count"] and tau[0] == g["p05"]["tau"]
    assert abs(loss - (math.log(1 + math.e ** 2) - 1 - math.log(2))) < 1e-14
    assert np.allclose(grad[0], g["p05"]["grad"], rtol=0, atol=1e-15)
    Z = 2 * math.e ** 2 + 2 * math.e + 1
    assert abs(mass[0, 0]) < 1e-15 and abs(mass[0, 1] - 2 * math.e ** 2 / Z) < 1e-14
    for key, p in (("p07", 0.7), ("p096", 0.96)):
        _, _, _, c, tt, _ = orc.kl_topp_fwd_bwd(t, s, p)
        assert c[0] == g[key]["count"] and tt[0] == g[key]["tau"]


def test_constructed_probabilities(orc):
    # t = ln w: p = w / sum(w) = (0.4, 0.3, 0.15, 0.1, 0.05) up to float32
    # rounding of the logits (~1e-7), far from every top_p used here
    w = np.array([4, 3, 1.5, 1, 0.5])
    t = np.log(w).astype(np.float32)[None, :]
    s = np.zeros_like(t)
    for p, want in ((0.3, 1), (0.5, 2), (0.8, 3), (0.9, 4), (0.97, 5)):
        _, _, _, c, tau, mass = orc.kl_topp_fwd_bwd(t, s, p)
        assert c[0] == want, (p, c[0])
        assert tau[0] == t[0, want - 1]
        assert abs(mass[0, 1] - np.cumsum(w / w.sum())[want - 1]) < 1e-6


def brute_nucleus(tv: np.ndarray, top_p: float, T: float):
    """(tau, |S|, mass above tau, mass at or above tau) by a plain walk."""
    x = tv.astype(np.float64) / T
    p = np.exp(x - x.max())
    p /= p.sum()
    vals = np.unique(tv.astype(np.float64))[::-1]
    acc = 0.0
    for v in vals:
        m = p[tv.astype(np.float64) == v].sum()
        if acc + m >= top_p or v == vals[-1]:
            return v, int((tv.astype(np.float64) >= v).sum()), acc, acc + m
        acc += m


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("top_p", [0.1, 0.5, 0.9, 0.99])
def test_brute_force_small_rows(orc, seed, top_p):
    rng = np.random.default_rng(seed)
    rows, V = 6, 48
    # few distinct values (many ties) in bf16
    t = synth.bf16_bits(__import__("torch").from_numpy(rng.integers(-6, 7, (rows, V)).astype(np.float32) * 0.75))
    s = synth.bf16_bits(__import__("torch").from_numpy(rng.standard_normal((rows, V)).astype(np.float32)))
    T = 0.7
    loss, row, grad, cnt, tau, mass = orc.kl_topp_fwd_bwd(t, s, top_p, T=T, grad_scale=0.5)
    tf = (t.astype(np.uint32) << 16).view(np.float32)
    for r in range(rows):
        bt, bc, ba, bi = brute_nucleus(tf[r], top_p, T)
        margin = min(abs(ba - top_p), abs(bi - top_p))
        assert margin > 1e-12
        assert tau[r] == bt and cnt[r] == bc
        assert abs(mass[r, 0] - ba) < 1e-12 and abs(mass[r, 1] - bi) < 1e-12
        assert mass[r, 0] < top_p <= mass[r, 1]
        # loss and gradient: the top-k KL on the same set (k = entries above
        # tau, plus one, keeps exactly the entries at or above tau)
        k = int((tf[r] > bt).sum()) + 1
        lk, rk, gk, ck = orc.kl_topk_fwd_bwd(t[r:r + 1], s[r:r + 1], k, T=T, grad_scale=0.5)
        assert ck[0] == bc
        assert row[r] == rk[0]
        assert np.array_equal(grad[r], gk[0])


@pytest.mark.parametrize("T", [1.0, 0.5])
def test_top_p_one_is_full_kl(orc, T):
    t, s = synth.logits_bf16(tokens=4, vocab=512, seed=9)
    tb, sb = synth.bf16_bits(t), synth.bf16_bits(s)
    loss, row, grad, cnt, tau, _ = orc.kl_topp_fwd_bwd(tb, sb, 1.0, T=T)
    lf, rf, gf = orc.kl_fwd_bwd(tb, sb, T=T)
    assert (cnt == 512).all()
    assert np.allclose(row, rf, rtol=1e-13, atol=1e-15)
    assert np.allclose(grad, gf, rtol=1e-12, atol=1e-18)
    assert abs(loss - lf) <= 1e-13 * abs(lf)


def test_tiny_top_p_keeps_the_argmax(orc):
    t, s = synth.logits_bf16(tokens=5, vocab=1024, seed=10)
    tb, sb = synth.bf16_bits(t), synth.bf16_bits(s)
    loss, row, grad, cnt, tau, _ = orc.kl_topp_fwd_bwd(tb, sb, 1e-9)
    tf = (tb.astype(np.uint32) << 16).view(np.float32)
    for r in range(5):
        assert tau[r] == tf[r].max()
        assert cnt[r] == (tf[r] == tf[r].max()).sum()
        if cnt[r] == 1:
            assert abs(row[r]) < 1e-15 and np.all(np.abs(grad[r]) < 1e-18)


def test_sizes_grow_with_top_p(orc):
    t, s = synth.logits_bf16(tokens=3, vocab=4096, seed=11)
    tb, sb = synth.bf16_bits(t), synth.bf16_bits(s)
    prev = np.zeros(3, np.int64)
    for p in (0.05, 0.2, 0.5, 0.8, 0.95, 0.999):
        _, _, g, cnt, tau, mass = orc.kl_topp_fwd_bwd(tb, sb, p)
        assert (cnt >= prev).all()
        assert (mass[:, 0] < p).all() and (mass[:, 1] >= p).all()
        assert np.all(np.abs(g.sum(axis=1)) < 1e-14)   # renormalised: the gradient sums to 0
        prev = cnt
