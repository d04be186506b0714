"""CPU tests of the C ABI: the library loads, exports every function that
include/libqad.h declares, and rejects bad arguments on the host before any
launch (every call here fails validation, so nothing touches a GPU)."""
import ctypes as C
import os
import re

import pytest

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libqad.h")

OK, INVALID, SHAPE, DTYPE, ALIGN, WS = 0, 1, 2, 3, 4, 5
P = 0x10000      # a 16-byte-aligned fake device address (never dereferenced)
P_ODD = 0x10002  # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from nvfp4_quantization_aware_amd import build
        build.build()
    return q.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qad_\w+|nvfp4_\w+|fp8_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 20, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_exported_symbols_in_dynamic_table(L):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in declared_functions():
        assert n in exported, n


def test_status_strings_and_version(L):
    assert L.qad_abi_version() == 2
    for s in range(8):
        assert L.qad_status_string(s).startswith(b"QAD_")
    assert L.qad_status_string(99) == b"unknown qad_status_t"


def _record_bytes(B, rc):
    # per tensor: 32-word header, one 32-word line per 16 chunks, one 16-word
    # slot per chunk; chunks of 8192 fp32 elements (the most numerous case)
    P = -(-rc // 8192)
    words = 32 + 32 * (-(-P // 16)) + 16 * P
    words = (words + 31) // 32 * 32
    return -(-(B * words * 4) // 256) * 256


def test_workspace_sizes(L):
    for op in (q.QAD_OP_AMAX, q.QAD_OP_QUANTIZE, q.QAD_OP_MSE_CALIBRATE):
        for B, R, C_ in ((128, 2048, 4096), (1, 1, 16), (1, 8192, 8192), (3, 7, 48)):
            assert L.qad_workspace_bytes(op, B, R, C_) == _record_bytes(B, R * C_)
    # KL: per-row losses, then one record per row when a row spans 2..64
    # segments of 16384 logits (6 tagged 64-bit state words and three binary64
    # loss shares per segment, one flag word), then one binary64 partial sum
    # of the mean per 256 rows; each part starts on a 256-byte boundary
    r256 = lambda n: -(-n // 256) * 256
    for tokens, vocab in ((8192, 131072), (100, 4096), (7, 16384), (7, 16392), (3, 1 << 20), (3, (1 << 20) + 8),
                          (3, 1 << 22), (0, 131072)):
        W = -(-vocab // 16384)
        rec = ((19 * W + 1 + 31) // 32 * 32) * 4 if 1 < W <= 64 else 0
        expect = r256(tokens * 4) + r256(tokens * rec) + r256(-(-tokens // 256) * 8)
        assert L.qad_workspace_bytes(q.QAD_OP_KL, 1, tokens, vocab) == expect
    # top-k KL: the KL workspace, then one float per row (thresholds)
    for tokens, vocab in ((8192, 131072), (3, 8), (1000, 248320), (3, 1 << 22)):
        kl = L.qad_workspace_bytes(q.QAD_OP_KL, 1, tokens, vocab)
        assert L.qad_workspace_bytes(q.QAD_OP_KL_TOPK, 1, tokens, vocab) == kl + -(-(tokens * 4) // 256) * 256
        assert L.qad_workspace_bytes(q.QAD_OP_KL_TOPP, 1, tokens, vocab) == kl + -(-(tokens * 4) // 256) * 256
    assert L.qad_workspace_bytes(q.QAD_OP_QUANTIZE, -1, 2, 16) == 0
    for op in range(7):
        assert L.qad_workspace_bytes(op, 1, 1, 16) % 256 == 0


def test_quantize_rejects(L):
    f = L.nvfp4_quantize
    ws = 1 << 16
    # C not a multiple of 16
    assert f(P, 1, 1, 4, 24, None, None, None, None, None, P * 2, P * 3, ws, None) == SHAPE
    # negative size
    assert f(P, 1, -1, 4, 32, None, None, None, None, None, P * 2, P * 3, ws, None) == SHAPE
    # bad dtype
    assert f(P, 7, 1, 4, 32, None, None, None, None, None, P * 2, P * 3, ws, None) == DTYPE
    # no output at all
    assert f(P, 1, 1, 4, 32, None, None, None, None, None, None, P * 3, ws, None) == INVALID
    # scales without tensor scale
    assert f(P, 1, 1, 4, 32, P * 5, None, None, None, None, P * 2, None, 0, None) == INVALID
    # null input
    assert f(None, 1, 1, 4, 32, None, None, None, None, None, P * 2, P * 3, ws, None) == INVALID
    # misaligned input / output / codes
    assert f(P_ODD, 1, 1, 4, 32, None, None, None, None, None, P * 2, P * 3, ws, None) == ALIGN
    assert f(P, 1, 1, 4, 32, None, None, None, None, None, P * 2 + 8, P * 3, ws, None) == ALIGN
    assert f(P, 1, 1, 4, 32, None, None, P * 4 + 2, None, None, None, P * 3, ws, None) == ALIGN
    # workspace missing / too small (dynamic mode needs it)
    assert f(P, 1, 1, 4, 32, None, None, None, None, None, P * 2, None, 0, None) == WS
    assert f(P, 1, 1, 4, 32, None, None, None, None, None, P * 2, P * 3, 8, None) == WS
    assert f(P, 1, 1, 4, 32, None, None, None, None, None, P * 2, P * 3 + 16, ws, None) == ALIGN
    # output overlapping the input
    assert f(P, 1, 1, 4, 32, None, None, None, None, None, P + 16, P * 3, ws, None) == INVALID
    # empty tensor: nothing to do
    assert f(P, 1, 0, 4, 32, None, None, None, None, None, P * 2, P * 3, ws, None) == OK


def test_empty_tensors_accepted_without_launch(L):
    # R * C == 0: every buffer is empty and may be NULL; without a tensor
    # scale output nothing is launched, so these return on the host
    f = L.nvfp4_quantize
    assert f(None, 1, 3, 0, 64, None, None, None, None, None, None, None, 0, None) == OK
    assert f(None, 1, 3, 0, 64, None, P, None, None, None, None, None, 0, None) == OK      # frozen, no block scales
    assert f(None, 1, 3, 0, 64, P, None, None, None, None, None, None, 0, None) == INVALID  # block scales alone
    assert L.nvfp4_qdq_fwd(None, 1, 2, 0, 32, None, None, None, None, 0, None) == OK
    assert L.fp8_quantize(None, 0, 2, 5, 0, None, None, None, None, None, 0, None) == OK
    assert L.nvfp4_mse_calibrate(None, 1, 2, 0, 32, 64, 0.5, 1.0, None, None, None, 0, None) == OK
    # the batch count stays bounded even when every tensor is empty
    assert f(None, 1, 1 << 40, 0, 64, None, None, None, None, None, None, None, 0, None) == SHAPE


def test_batches_beyond_one_grid_rejected(L):
    # 2^31 tensors of 16 elements: 2^35 elements (allowed) but one workgroup
    # per tensor already exceeds a grid's 2^31 - 1 workgroups
    B = 1 << 31
    assert L.nvfp4_quantize(P, 1, B, 1, 16, None, None, None, None, None, P * 2, P * 3, 1 << 40, None) == SHAPE
    assert L.nvfp4_amax(P, 1, B, 1, 16, P * 2, P * 3, 1 << 40, None) == SHAPE
    assert L.nvfp4_mse_calibrate(P, 1, B, 1, 16, 64, 0.5, 1.0, P * 2, P * 3, P * 4, 1 << 40, None) == SHAPE
    assert L.fp8_quantize(P, 1, B, 1, 16, None, None, None, P * 2, P * 3, 1 << 40, None) == SHAPE


def test_fp8_quantize_rejects(L):
    f = L.fp8_quantize
    ws = 1 << 16
    assert f(P, 1, 1, 4, 12, None, None, None, P * 2, P * 3, ws, None) == SHAPE    # C % 8
    assert f(P, 7, 1, 4, 16, None, None, None, P * 2, P * 3, ws, None) == DTYPE
    assert f(P, 1, 1, 4, 16, None, None, None, None, P * 3, ws, None) == INVALID   # no output
    assert f(None, 1, 1, 4, 16, None, None, None, P * 2, P * 3, ws, None) == INVALID
    assert f(P, 1, 1, 4, 16, None, P * 4 + 4, None, None, P * 3, ws, None) == ALIGN  # codes 8-byte aligned
    assert f(P, 1, 1, 4, 16, None, None, None, P * 2, None, 0, None) == WS           # dynamic needs workspace
    assert f(P, 1, 1, 4, 16, None, None, None, P + 16, P * 3, ws, None) == INVALID   # y overlaps x
    assert f(P, 1, 0, 4, 16, None, None, None, P * 2, None, 0, None) == OK           # empty


def test_w4a4_linear_rejects(L):
    fw, bw = L.qad_w4a4_linear_fwd, L.qad_w4a4_linear_bwd
    ws = L.qad_workspace_bytes(q.QAD_OP_W4A4_LINEAR, 64, 32, 128)
    assert ws > 0 and ws % 256 == 0            # the quantizer's records only
    # (M, N, K) is no tensor: M N K may pass the tensor-size bound as long as
    # each operand (M x K, N x K) is within it; the records of the larger one
    for M, N, K in ((8200, 2048, 4096), (1 << 20, 4096, 8192), (64, 32, 128)):
        big = max(L.qad_workspace_bytes(q.QAD_OP_QUANTIZE, 1, M, K), L.qad_workspace_bytes(q.QAD_OP_QUANTIZE, 1, N, K))
        assert big > 0 and L.qad_workspace_bytes(q.QAD_OP_W4A4_LINEAR, M, N, K) == big
    assert L.qad_workspace_bytes(q.QAD_OP_W4A4_LINEAR, -1, 32, 128) == 0
    a = lambda **kw: [kw.get("x", P), kw.get("w", P * 2), kw.get("dt", 1), kw.get("M", 64), kw.get("N", 32),
                      kw.get("K", 128), kw.get("wsc", None), kw.get("wts", None), kw.get("y", P * 3),
                      kw.get("xq", P * 4), kw.get("wq", P * 5), kw.get("ws", P * 6), kw.get("wsb", ws), None]
    assert fw(*a(dt=5)) == DTYPE
    assert fw(*a(K=24)) == SHAPE and fw(*a(K=0)) == SHAPE and fw(*a(M=-1)) == SHAPE
    assert fw(*a(y=None)) == INVALID and fw(*a(x=None)) == INVALID
    assert fw(*a(wsc=P * 7)) == INVALID and fw(*a(wts=P * 8)) == INVALID   # frozen weight scales come in pairs
    assert fw(*a(xq=P * 4 + 8)) == ALIGN
    assert fw(*a(wsb=ws - 256)) == WS and fw(*a(ws=None)) == WS
    assert fw(*a(ws=P * 6 + 128)) == ALIGN
    assert fw(*a(y=P * 4)) == INVALID                 # y overlaps xq
    assert fw(*a(M=0, N=0)) == OK                     # nothing to do
    assert fw(*a(M=0, N=0, x=None, w=None, y=None, xq=None, wq=None)) == OK   # empty buffers may be NULL
    assert fw(*a(M=0, wq=None)) == INVALID            # wq is still written when only M is 0
    b = lambda **kw: [kw.get("gy", P), kw.get("xq", P * 2), kw.get("wq", P * 3), kw.get("M", 64), kw.get("N", 32),
                      kw.get("K", 128), kw.get("gx", P * 4), kw.get("gw", P * 5), kw.get("ws", P * 6),
                      kw.get("wsb", ws), None]
    assert bw(*b(gx=None, gw=None)) == INVALID
    assert bw(*b(M=0, N=0, gx=None, gw=None)) == OK
    assert bw(*b(K=8)) == SHAPE
    assert bw(*b(wq=None)) == INVALID                 # grad_x needs wq
    assert bw(*b(gx=P)) == INVALID                    # grad_x overlaps grad_y
    assert bw(*b(gw=P * 2)) == INVALID                # grad_w over xq


def test_qdq_fwd_bwd_reject(L):
    assert L.nvfp4_qdq_fwd(P, 1, 1, 4, 32, None, None, None, P * 3, 1 << 16, None) == INVALID
    assert L.nvfp4_qdq_bwd(P, P * 2, 5, 100, None) == DTYPE
    assert L.nvfp4_qdq_bwd(P, P * 2, 1, -3, None) == SHAPE
    assert L.nvfp4_qdq_bwd(None, P * 2, 1, 100, None) == INVALID
    assert L.nvfp4_qdq_bwd(P_ODD, P * 2, 1, 100, None) == ALIGN
    assert L.nvfp4_qdq_bwd(P, P + 64, 1, 100, None) == INVALID  # partial overlap
    # in place and empty are no-ops
    assert L.nvfp4_qdq_bwd(P, P, 1, 100, None) == OK
    assert L.nvfp4_qdq_bwd(P, P * 2, 1, 0, None) == OK


def test_qdq_bwd_clipped_rejects(L):
    f = L.nvfp4_qdq_bwd_clipped
    Q = 1 << 24   # far-apart fake addresses: grad_y, x, scales, tscale, grad_x

    def a(gy=P, gt=1, x=P + Q, xt=1, B=2, R=4, C=32, sc=P + 2 * Q, ts=P + 3 * Q, gx=P + 4 * Q):
        return gy, gt, x, xt, B, R, C, sc, ts, gx, None

    assert f(*a(gt=7)) == DTYPE
    assert f(*a(xt=7)) == DTYPE
    assert f(*a(C=24)) == SHAPE                      # C % 16
    assert f(*a(B=-1)) == SHAPE
    assert f(*a(B=1 << 31, R=1, C=16)) == SHAPE      # grid beyond 2^31 workgroups
    assert f(*a(x=None)) == INVALID
    assert f(*a(sc=None)) == INVALID
    assert f(*a(ts=None)) == INVALID
    assert f(*a(gx=None)) == INVALID
    assert f(*a(x=P_ODD)) == ALIGN
    assert f(*a(gx=P_ODD + 4 * Q)) == ALIGN
    assert f(*a(ts=P + 3 * Q + 2)) == ALIGN
    assert f(*a(gx=P + 64)) == INVALID               # partial overlap with grad_y
    assert f(*a(gx=P + Q)) == INVALID                # grad_x over x
    assert f(*a(gx=P + 2 * Q)) == INVALID            # grad_x over the scales
    assert f(*a(R=0)) == OK                          # empty: nothing launched


def test_frozen_sgd_step_rejects(L):
    f = L.nvfp4_frozen_sgd_step
    Q = 1 << 24   # far-apart fake addresses: w, grad, scales, tscale, w_out

    def a(w=P, wt=1, g=P + Q, gt=1, B=2, R=4, C=32, sc=P + 2 * Q, ts=P + 3 * Q, lr=0.5, cc=1.0, wo=P + 4 * Q):
        return w, wt, g, gt, B, R, C, sc, ts, lr, cc, wo, None

    assert f(*a(wt=7)) == DTYPE
    assert f(*a(gt=7)) == DTYPE
    assert f(*a(C=24)) == SHAPE                      # C % 16
    assert f(*a(B=-1)) == SHAPE
    assert f(*a(B=1 << 31, R=1, C=16)) == SHAPE      # grid beyond 2^31 workgroups
    assert f(*a(lr=float("nan"))) == INVALID
    assert f(*a(cc=float("inf"))) == INVALID
    assert f(*a(g=None)) == INVALID
    assert f(*a(sc=None)) == INVALID
    assert f(*a(ts=None)) == INVALID
    assert f(*a(wo=None)) == INVALID
    assert f(*a(w=P_ODD)) == ALIGN
    assert f(*a(wo=P_ODD + 4 * Q)) == ALIGN
    assert f(*a(ts=P + 3 * Q + 2)) == ALIGN
    assert f(*a(wo=P + 64)) == INVALID               # partial overlap with w
    assert f(*a(wo=P + Q)) == INVALID                # w_out over grad
    assert f(*a(wo=P + 2 * Q)) == INVALID            # w_out over the scales
    assert f(*a(R=0)) == OK                          # empty: nothing launched


def test_amax_rejects(L):
    ws = 1 << 16
    assert L.nvfp4_amax(P, 1, 1, 4, 12, P * 2, P * 4, ws, None) == SHAPE   # 24-byte rows
    assert L.nvfp4_amax(P, 2, 1, 4, 16, P * 2, P * 4, ws, None) == DTYPE
    assert L.nvfp4_amax(P, 1, 1, 4, 16, None, P * 4, ws, None) == INVALID
    assert L.nvfp4_amax(P_ODD, 1, 1, 4, 16, P * 2, P * 4, ws, None) == ALIGN
    assert L.nvfp4_amax(P, 1, 1, 4, 16, P * 2, None, 0, None) == WS
    assert L.nvfp4_amax(P, 1, 1, 4, 16, P * 2, P * 4, 16, None) == WS
    assert L.nvfp4_amax(P, 1, 1, 4, 16, P * 2, P * 4 + 64, ws, None) == ALIGN
    assert L.nvfp4_amax(P, 1, 0, 4, 16, None, None, 0, None) == OK


def test_mse_rejects(L):
    f = L.nvfp4_mse_calibrate
    args = lambda n, lo, hi: (P, 1, 1, 4, 32, n, lo, hi, P * 2, P * 3, P * 4, 1 << 16, None)
    assert f(*args(0, 0.5, 1.0)) == INVALID
    assert f(*args(64, 0.0, 1.0)) == INVALID
    assert f(*args(64, 0.8, 0.5)) == INVALID
    assert f(*args(4, 0.5, 1.0)) == INVALID          # step 1/6 > 0.5/16: could skip E4M3 codes
    assert f(*args(64, 0.5, float("inf"))) == INVALID
    assert f(P, 1, 1, 4, 24, 64, 0.5, 1.0, P * 2, P * 3, P * 4, 1 << 16, None) == SHAPE
    assert f(P, 1, 1, 4, 32, 64, 0.5, 1.0, None, P * 3, P * 4, 1 << 16, None) == INVALID
    assert f(P, 1, 1, 4, 32, 64, 0.5, 1.0, P * 2, P * 3, None, 0, None) == WS
    assert f(P, 1, 1, 4, 32, 64, 0.5, 1.0, P * 2, P * 3 + 2, P * 4, 1 << 16, None) == ALIGN
    assert f(P, 1, 1, 4, 32, 64, 0.5, 1.0, P * 2, P * 3, P * 4 + 32, 1 << 16, None) == ALIGN


def test_kl_rejects(L):
    f = L.qad_kl_fwd_bwd
    good = [P, P * 2, 1, 4, 64, 1.0, 0.25, P * 3, None, P * 4, 1, P * 5, 1 << 16, None]

    def call(**kw):
        a = list(good)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a2=9) == DTYPE
    assert call(a10=9) == DTYPE
    assert call(a4=60) == SHAPE                       # vocab % 8
    assert call(a3=-1) == SHAPE
    assert call(a5=0.0) == INVALID                    # temperature
    assert call(a5=float("nan")) == INVALID
    assert call(a6=float("inf")) == INVALID
    assert call(a7=None) == INVALID                   # loss_out
    assert call(a0=None) == INVALID
    assert call(a1=P_ODD) == ALIGN
    assert call(a9=P + 32) == INVALID                 # gradient overlaps the teacher
    assert call(a11=None, a12=0) == WS                # no workspace
    assert call(a12=16) == WS
    assert call(a11=P * 5 + 64) == ALIGN


def test_kl_topk_rejects(L):
    f = L.qad_kl_topk_fwd_bwd
    good = [P, P * 2, 1, 4, 64, 16, 1.0, 0.25, P * 3, None, P * 4, 1, P * 5, 1 << 16, None]

    def call(**kw):
        a = list(good)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a2=9) == DTYPE
    assert call(a11=9) == DTYPE
    assert call(a4=60) == SHAPE                       # vocab % 8
    assert call(a3=-1) == SHAPE
    assert call(a5=0) == INVALID                      # k
    assert call(a5=-3) == INVALID
    assert call(a6=0.0) == INVALID                    # temperature
    assert call(a7=float("nan")) == INVALID
    assert call(a8=None) == INVALID                   # loss_out
    assert call(a1=None) == INVALID
    assert call(a0=P_ODD) == ALIGN
    assert call(a10=P + 32) == INVALID                # gradient overlaps the teacher
    assert call(a12=None, a13=0) == WS                # no workspace
    assert call(a13=16) == WS
    assert call(a12=P * 5 + 64) == ALIGN


def test_kl_topp_rejects(L):
    f = L.qad_kl_topp_fwd_bwd
    good = [P, P * 2, 1, 4, 64, 0.9, 1.0, 0.25, P * 3, None, P * 4, 1, P * 6, P * 5, 1 << 16, None]

    def call(**kw):
        a = list(good)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a2=9) == DTYPE
    assert call(a11=9) == DTYPE
    assert call(a4=60) == SHAPE                       # vocab % 8
    assert call(a3=-1) == SHAPE
    assert call(a3=2, a4=0) == SHAPE                  # rows without a vocabulary
    assert call(a5=0.0) == INVALID                    # top_p
    assert call(a5=-0.5) == INVALID
    assert call(a5=float("nan")) == INVALID
    assert call(a5=float("inf")) == INVALID
    assert call(a6=0.0) == INVALID                    # temperature
    assert call(a7=float("nan")) == INVALID
    assert call(a8=None) == INVALID                   # loss_out
    assert call(a1=None) == INVALID
    assert call(a0=P_ODD) == ALIGN
    assert call(a12=P * 6 + 2) == ALIGN               # tau_out
    assert call(a10=P + 32) == INVALID                # gradient overlaps the teacher
    assert call(a12=P + 64) == INVALID                # thresholds over the teacher
    assert call(a12=P * 5 + 256) == INVALID           # thresholds inside the workspace
    assert call(a13=None, a14=0) == WS                # no workspace
    assert call(a14=16) == WS
    assert call(a13=P * 5 + 64) == ALIGN


def test_check_finite_rejects(L):
    assert L.qad_check_finite(P, -1, None) == SHAPE
    assert L.qad_check_finite(None, 3, None) == INVALID
    assert L.qad_check_finite(None, 0, None) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_binding_rejects_host_tensors():
    # host tensors never reach the library: their pointers would be read by
    # the kernels as device addresses
    import numpy as np
    import torch
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    t = torch.zeros(2, 64, dtype=torch.bfloat16)
    calls = [
        lambda: q.nvfp4_amax(x),
        lambda: q.nvfp4_quantize(x),
        lambda: q.nvfp4_qdq_fwd(x),
        lambda: q.nvfp4_qdq_bwd(x),
        lambda: q.nvfp4_qdq_bwd_clipped(x, x, torch.zeros(8, dtype=torch.uint8), torch.ones(1)),
        lambda: q.nvfp4_frozen_sgd_step(x, x, torch.zeros(8, dtype=torch.uint8), torch.ones(1), 0.1),
        lambda: q.nvfp4_mse_calibrate(x),
        lambda: q.fp8_quantize(x),
        lambda: q.qad_kl_fwd_bwd(t, t),
        lambda: q.qad_kl_topk_fwd_bwd(t, t, 4),
        lambda: q.qad_kl_topp_fwd_bwd(t, t, 0.9),
        lambda: q.qad_w4a4_linear_fwd(x, x),
        lambda: q.qad_w4a4_linear_bwd(x[:, :4].contiguous(), x, x, 32),
        lambda: q.qad_check_finite(torch.zeros(3)),
    ]
    for i, f in enumerate(calls):
        with pytest.raises(ValueError, match="must be on the GPU"):
            f()
    with pytest.raises(TypeError):
        q.nvfp4_quantize(np.zeros((4, 32), np.float32))


def test_wait_limit_setting(L):
    # host-only: the bound of the one-pass kernels' device waits
    prev = L.qad_set_wait_limit_us(-1)
    assert prev == 20000                       # default 20 ms
    try:
        assert L.qad_set_wait_limit_us(0) == 20000
        assert L.qad_set_wait_limit_us(-5) == 0  # query only
        assert q.set_wait_limit_us(1 << 50) == 0
        assert q.set_wait_limit_us(-1) == 1 << 40  # clamped
    finally:
        L.qad_set_wait_limit_us(prev)
    assert q.set_wait_limit_us(-1) == 20000


def test_plain_c_client(L, tmp_path):
    # the header is plain C (C99, no HIP include) and the library links into
    # a C program; host-only calls need no GPU
    import subprocess
    src = tmp_path / "client.c"
    src.write_text(
        '#include <stdio.h>\n#include <string.h>\n#include "libqad.h"\n'
        "int main(void) {\n"
        "  if (qad_abi_version() != 2) return 1;\n"
        '  if (strncmp(qad_status_string(QAD_ERR_SHAPE), "QAD_ERR_SHAPE", 13) != 0) return 2;\n'
        "  if (qad_workspace_bytes(QAD_OP_QUANTIZE, 1, 64, 64) % 256 != 0) return 3;\n"
        "  if (qad_set_wait_limit_us(-1) != 20000) return 4;\n"
        "  if (nvfp4_quantize(NULL, QAD_BF16, 1, 4, 24, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL)\n"
        "      != QAD_ERR_SHAPE) return 5;\n"
        '  printf("ok\\n");\n  return 0;\n}\n')
    exe = tmp_path / "client"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-lqad", "-Wl,-rpath," + libdir], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", (out.returncode, out.stdout, out.stderr)
