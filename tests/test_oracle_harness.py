"""The oracle's all-cores harness, its binary32 KL timing variant and MSE
grids beyond 4096 candidates (CPU).

* The OpenMP harness (oracle/oracle_omp.c) runs the unchanged oracle functions
  over tensors, rows or row ranges: its results must equal the
  single-threaded calls bit for bit.
* kl_fwd_bwd_f32 is a timing variant only (no parity test uses it); it is
  held to the binary64 oracle within binary32 accuracy, so that the CPU rate
  it gives is the rate of a correct computation.
* orc_mse_calibrate / orc_mse_calibrate_blocks take any number of
  candidates: with 5000 the k grid is still the exactly rounded one, the
  chosen scale the first minimum of the full candidate table, and the tensor
  call equal to the blockwise one.
"""
from fractions import Fraction

import numpy as np
import pytest

from nvfp4_quantization_aware_amd import synth


def test_omp_quantize_batch_and_tensor_equal_single_thread(orc):
    w, _ = synth.moe_weights_bf16(experts=6, rows=64, cols=256, seed=11, with_grad=False)
    wb = synth.bf16_bits(w)
    codes, scales, ts, y = orc.omp_quantize_batch(wb)
    for b in range(wb.shape[0]):
        rc, rs, rt, ry = orc.nvfp4_quantize(wb[b])
        assert np.array_equal(codes[b], rc) and np.array_equal(scales[b], rs)
        assert np.float32(ts[b]) == np.float32(rt) and np.array_equal(y[b], ry)
    x = orc.f32_from_bf16(wb[0]) * np.float32(3.0)
    c2, s2, t2, y2 = orc.omp_quantize_tensor(x)
    rc, rs, rt, ry = orc.nvfp4_quantize(x)
    assert np.array_equal(c2, rc) and np.array_equal(s2, rs) and np.float32(t2) == np.float32(rt)
    assert np.array_equal(y2, ry)
    c3, _, t3, y3 = orc.omp_quantize_tensor(x, rs, rt)              # frozen scales
    fc, _, _, fy = orc.nvfp4_quantize(x, rs, rt)
    assert np.array_equal(c3, fc) and np.array_equal(y3, fy) and t3 == np.float32(rt)


def test_omp_mse_equals_single_thread(orc):
    w = synth.bf16_bits(synth.gaussian_weight_bf16(rows=40, cols=512, seed=12))
    s1, t1 = orc.mse_calibrate(w)
    s2, t2 = orc.omp_mse_calibrate(w)
    assert np.array_equal(s1, s2) and t1 == t2


def test_omp_kl_equals_single_thread(orc):
    t, s = synth.logits_bf16(tokens=9, vocab=3000, seed=13)
    t, s = synth.bf16_bits(t), synth.bf16_bits(s)
    l1, r1, g1 = orc.kl_fwd_bwd(t, s, T=0.7)
    l2, r2, g2 = orc.omp_kl_fwd_bwd(t, s, T=0.7)
    assert l1 == l2 and np.array_equal(r1, r2) and np.array_equal(g1, g2)
    f1 = orc.kl_fwd_bwd_f32(t, s, T=0.7)
    f2 = orc.omp_kl_fwd_bwd_f32(t, s, T=0.7)
    assert f1[0] == f2[0] and np.array_equal(f1[1], f2[1]) and np.array_equal(f1[2], f2[2])


@pytest.mark.parametrize("T,noise", [(1.0, 0.5), (2.0, 1.0)])
def test_f32_kl_variant_within_binary32_accuracy(orc, T, noise):
    t, s = synth.logits_bf16(tokens=6, vocab=8192, noise_std=noise, seed=14)
    t, s = synth.bf16_bits(t), synth.bf16_bits(s)
    l64, r64, g64 = orc.kl_fwd_bwd(t, s, T=T)
    l32, r32, g32 = orc.kl_fwd_bwd_f32(t, s, T=T)
    # sums over 8192 terms in binary32: a few thousand ulps at most
    assert abs(l32 - l64) <= 2e-4 * abs(l64)
    assert np.all(np.abs(r32 - r64) <= 2e-4 * np.abs(r64))
    scale = np.abs(g64).max(axis=1, keepdims=True)
    assert np.all(np.abs(g32 - g64) <= 1e-4 * scale + 1e-3 * np.abs(g64))


def _nearest_f32(q: Fraction) -> np.float32:
    f = np.float32(float(q))
    best = f
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d, db = abs(Fraction(float(c)) - q), abs(Fraction(float(best)) - q)
        if d < db or (d == db and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best = c
    return best


def test_mse_grid_beyond_4096_candidates(orc):
    n = 5000
    k = orc.mse_kgrid(n, 0.5, 1.0)
    assert k.size == n
    for i in list(range(0, 40)) + list(range(4090, 4110)) + list(range(n - 40, n)):
        assert k[i] == _nearest_f32(Fraction(1, 2) + Fraction(i, 2 * (n - 1))), i
    w = synth.gaussian_weight_bf16(rows=4, cols=128, seed=15)
    x = orc.f32_from_bf16(synth.bf16_bits(w)).reshape(-1, 16)
    s_g = orc.tensor_scale(orc.amax(x))
    sc, err, cc, ce = orc.mse_calibrate_blocks(x, s_g, n_cand=n, detail=True)
    assert cc.shape == (x.shape[0], n)
    first = np.argmin(ce, axis=1)
    assert np.array_equal(sc, cc[np.arange(len(sc)), first]) and np.array_equal(err, ce.min(axis=1))
    # candidates past index 4096 take part in the minimum
    assert np.all(err <= ce[:, 4500]) and np.all(err <= ce[:, n - 1])
    st, tt = orc.mse_calibrate(x.reshape(4, 128), n_cand=n)
    assert np.array_equal(st.reshape(-1), sc) and tt == np.float32(s_g)
