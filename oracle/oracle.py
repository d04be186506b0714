"""ctypes front-end of the C oracle (test infrastructure only).

Every function takes and returns numpy arrays; bf16 tensors travel as their
raw uint16 bit patterns.  No arithmetic of the method happens in this file:
it only builds ``liboracle.so`` from ``oracle.c`` and calls into it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SRC_OMP = os.path.join(_HERE, "oracle_omp.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (strict IEEE binary32/binary64, no fusion),
    with the OpenMP harness oracle_omp.c beside it."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-fopenmp", "-o", tmp, _SRC, _SRC_OMP, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = C.CDLL(_LIB_PATH)
        vp, i64, f32, f64, i32 = C.c_void_p, C.c_int64, C.c_float, C.c_double, C.c_int
        sig = {
            "orc_e2m1_encode": (C.c_uint8, [f32]),
            "orc_e2m1_decode": (f32, [C.c_uint8]),
            "orc_e4m3_encode": (C.c_uint8, [f32]),
            "orc_e4m3_decode": (f32, [C.c_uint8]),
            "orc_bf16_from_f32": (C.c_uint16, [f32]),
            "orc_f32_from_bf16": (f32, [C.c_uint16]),
            "orc_e2m1_encode_array": (None, [vp, i64, vp]),
            "orc_e4m3_encode_array": (None, [vp, i64, vp]),
            "orc_bf16_from_f32_array": (None, [vp, i64, vp]),
            "orc_amax": (f32, [vp, i32, i64]),
            "orc_nvfp4_quantize": (None, [vp, i32, i64, i64, vp, vp, vp, vp, vp, vp]),
            "orc_nvfp4_quantize_blocks": (None, [vp, i32, i64, f32, vp, vp, vp, vp]),
            "orc_tensor_scale": (f32, [f32]),
            "orc_mse_kgrid": (None, [i32, f32, f32, vp]),
            "orc_mse_calibrate": (None, [vp, i32, i64, i64, i32, f32, f32, vp, vp]),
            "orc_mse_calibrate_blocks": (None, [vp, i64, f32, i32, f32, f32, vp, vp, vp, vp]),
            "orc_fp8_quantize": (None, [vp, i32, i64, vp, vp, vp, vp]),
            "orc_nvfp4_qdq_bwd_clipped": (None, [vp, i32, vp, i32, i64, vp, f32, vp, vp]),
            "orc_nvfp4_frozen_sgd_step": (None, [vp, i32, vp, i32, i64, vp, f32, f32, f32, vp, vp]),
            "orc_kl_fwd_bwd": (f64, [vp, vp, i32, i64, i64, f64, f64, vp, vp]),
            "orc_kl_topk_fwd_bwd": (f64, [vp, vp, i32, i64, i64, i64, f64, f64, vp, vp, vp]),
            "orc_kl_topp_fwd_bwd": (f64, [vp, vp, i32, i64, i64, f64, f64, f64, vp, vp, vp, vp, vp]),
            "orc_kl_fwd_bwd_f32": (f32, [vp, vp, i32, i64, i64, f32, f32, vp, vp]),
            "orc_omp_threads": (i32, []),
            "orc_omp_quantize_batch": (None, [vp, i32, i64, i64, i64, vp, vp, vp, vp]),
            "orc_omp_quantize_tensor": (None, [vp, i32, i64, i64, vp, vp, vp, vp, vp, vp]),
            "orc_omp_mse_calibrate": (None, [vp, i32, i64, i64, i32, f32, f32, vp, vp]),
            "orc_omp_kl_fwd_bwd": (f64, [vp, vp, i32, i64, i64, f64, f64, vp, vp]),
            "orc_omp_kl_fwd_bwd_f32": (f32, [vp, vp, i32, i64, i64, f32, f32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or raw-bf16 uint16 arrays, got %s" % x.dtype)


# ---- scalar / array codecs ------------------------------------------------
def e2m1_encode(r: np.ndarray) -> np.ndarray:
    r = np.ascontiguousarray(r, dtype=np.float32)
    out = np.empty(r.shape, np.uint8)
    _load().orc_e2m1_encode_array(_ptr(r), r.size, _ptr(out))
    return out


def e2m1_decode(code: int) -> float:
    return float(_load().orc_e2m1_decode(int(code)))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_decode(code: int) -> float:
    return float(_load().orc_e4m3_decode(int(code)))


def e4m3_decode_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_e4m3_decode(c) for c in range(256)], np.float32)


def bf16_from_f32(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().orc_bf16_from_f32_array(_ptr(f), f.size, _ptr(out))
    return out


def f32_from_bf16(h: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to float32 (exact; a bit shift, not arithmetic)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# ---- NVFP4 tensor operations ----------------------------------------------
def amax(x: np.ndarray) -> float:
    x = np.ascontiguousarray(x)
    return float(_load().orc_amax(_ptr(x), _dtype_code(x), x.size))


def tensor_scale(a: float) -> float:
    return float(_load().orc_tensor_scale(float(a)))


def nvfp4_quantize(x: np.ndarray, scales_in: np.ndarray | None = None,
                   tscale_in: float | None = None):
    """Quantize one tensor [..., C] (C % 16 == 0); leading dims are rows.

    Returns (codes u8[R, C/2], scales u8[R, C/16], tscale float, y bf16-bits
    u16[R, C]).  Pass scales_in / tscale_in for the frozen variant.
    """
    x = np.ascontiguousarray(x)
    Cc = x.shape[-1]
    R = x.size // Cc if Cc else 0
    assert Cc % 16 == 0
    codes = np.empty((R, Cc // 2), np.uint8)
    scales = np.empty((R, Cc // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    y = np.empty((R, Cc), np.uint16)
    sin = None
    tin = None
    if scales_in is not None:
        sin = np.ascontiguousarray(scales_in, dtype=np.uint8).reshape(-1)
        assert sin.size == R * Cc // 16
        tin = np.array([tscale_in], np.float32)
    _load().orc_nvfp4_quantize(_ptr(x), _dtype_code(x), R, Cc, _ptr(sin), _ptr(tin),
                               _ptr(codes), _ptr(scales), _ptr(ts), _ptr(y))
    return codes, scales, float(ts[0]), y


def nvfp4_quantize_blocks(x: np.ndarray, s_g: float, scales_in: np.ndarray | None = None):
    """Quantize whole 16-element blocks of x (any shape, size % 16 == 0) under
    tensor scale s_g.  Returns (codes u8[nb, 8], scales u8[nb], y u16[nb, 16])."""
    x = np.ascontiguousarray(x)
    assert x.size % 16 == 0
    nb = x.size // 16
    codes = np.empty((nb, 8), np.uint8)
    scales = np.empty(nb, np.uint8)
    y = np.empty((nb, 16), np.uint16)
    sin = None if scales_in is None else np.ascontiguousarray(scales_in, dtype=np.uint8).reshape(-1)
    _load().orc_nvfp4_quantize_blocks(_ptr(x), _dtype_code(x), nb, float(s_g), _ptr(sin),
                                      _ptr(codes), _ptr(scales), _ptr(y))
    return codes, scales, y


def mse_kgrid(n: int = 64, k_min: float = 0.5, k_max: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    _load().orc_mse_kgrid(n, k_min, k_max, _ptr(out))
    return out


def mse_calibrate(x: np.ndarray, n_cand: int = 64, k_min: float = 0.5, k_max: float = 1.0):
    """MSE-calibrate one tensor: returns (E4M3 scales u8[R, C/16], tscale)."""
    x = np.ascontiguousarray(x)
    Cc = x.shape[-1]
    R = x.size // Cc if Cc else 0
    scales = np.empty((R, Cc // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    _load().orc_mse_calibrate(_ptr(x), _dtype_code(x), R, Cc, n_cand, k_min, k_max,
                              _ptr(scales), _ptr(ts))
    return scales, float(ts[0])


def mse_calibrate_blocks(blocks: np.ndarray, s_g: float, n_cand: int = 64,
                         k_min: float = 0.5, k_max: float = 1.0, detail: bool = False):
    """Calibrate independent 16-element fp32 blocks under tensor scale s_g.

    Returns scales u8[nb] and best errors f32[nb]; with detail=True also every
    candidate's E4M3 code u8[nb, n_cand] and error f32[nb, n_cand].
    """
    blocks = np.ascontiguousarray(blocks, dtype=np.float32).reshape(-1, 16)
    nb = blocks.shape[0]
    scales = np.empty(nb, np.uint8)
    err = np.empty(nb, np.float32)
    cc = np.empty((nb, n_cand), np.uint8) if detail else None
    ce = np.empty((nb, n_cand), np.float32) if detail else None
    _load().orc_mse_calibrate_blocks(_ptr(blocks), nb, float(s_g), n_cand, k_min, k_max,
                                     _ptr(scales), _ptr(err), _ptr(cc), _ptr(ce))
    if detail:
        return scales, err, cc, ce
    return scales, err


def fp8_quantize(x: np.ndarray, tscale: float | None = None):
    """FP8 (E4M3) per-tensor QDQ of one tensor (any shape).

    Returns (codes u8 like x, tensor scale f32, y bf16 bits u16 like x).
    tscale None: dynamic amax/448; else the given (frozen) scale.
    """
    x = np.ascontiguousarray(x)
    n = x.size
    codes = np.empty(x.shape, np.uint8)
    y = np.empty(x.shape, np.uint16)
    ts = np.empty(1, np.float32)
    tin = None if tscale is None else np.array([tscale], np.float32)
    _load().orc_fp8_quantize(_ptr(x), _dtype_code(x), n, _ptr(tin), _ptr(codes), _ptr(ts), _ptr(y))
    return codes, float(ts[0]), y


def nvfp4_qdq_bwd_clipped(grad_y: np.ndarray, x: np.ndarray, scales: np.ndarray, tscale: float):
    """Clipped straight-through backward of one tensor (x.size % 16 == 0):
    grad_y where |x| <= 6 * dec(scale) * tscale, +0 elsewhere.  grad_y and x
    are float32 or raw-bf16 uint16 arrays of the same size; scales holds one
    E4M3 code per 16 consecutive elements.  Returns (grad_x like grad_y,
    number of clipped elements)."""
    g = np.ascontiguousarray(grad_y)
    x = np.ascontiguousarray(x)
    sc = np.ascontiguousarray(scales, dtype=np.uint8)
    if g.size != x.size or x.size % 16 or sc.size != x.size // 16:
        raise ValueError("grad_y, x and scales sizes do not match")
    out = np.empty_like(g)
    nc = np.zeros(1, np.int64)
    _load().orc_nvfp4_qdq_bwd_clipped(_ptr(g), _dtype_code(g), _ptr(x), _dtype_code(x), x.size // 16,
                                      _ptr(sc), float(tscale), _ptr(out), _ptr(nc))
    return out, int(nc[0])


def nvfp4_frozen_sgd_step(w: np.ndarray, grad: np.ndarray, scales: np.ndarray, tscale: float, lr: float,
                          clip_coef: float):
    """Frozen-scale SGD step of one weight tensor (w.size % 16 == 0): w where
    |w| > 6 * dec(scale) * tscale, else round_w(fma32(-fl32(lr * clip_coef),
    g, w)).  w and grad are float32 or raw-bf16 uint16 arrays of the same
    size; scales holds one E4M3 code per 16 consecutive elements.  Returns
    (w' like w, number of weights the clip left unchanged)."""
    w = np.ascontiguousarray(w)
    g = np.ascontiguousarray(grad)
    sc = np.ascontiguousarray(scales, dtype=np.uint8)
    if g.size != w.size or w.size % 16 or sc.size != w.size // 16:
        raise ValueError("w, grad and scales sizes do not match")
    out = np.empty_like(w)
    nc = np.zeros(1, np.int64)
    _load().orc_nvfp4_frozen_sgd_step(_ptr(w), _dtype_code(w), _ptr(g), _dtype_code(g), w.size // 16, _ptr(sc),
                                      float(tscale), float(lr), float(clip_coef), _ptr(out), _ptr(nc))
    return out, int(nc[0])


def w4a4_linear_fwd(x: np.ndarray, w: np.ndarray, w_scales: np.ndarray | None = None,
                    w_tscale: float | None = None):
    """W4A4 fake-quant linear: y = QDQ(x) QDQ(w)^T in binary64 (numpy matmul of
    the oracle's NVFP4 QDQ outputs; w with frozen scales when given).
    Returns (y f64 [M][N], xq bf16 bits, wq bf16 bits)."""
    _, _, _, xq = nvfp4_quantize(x)
    _, _, _, wq = nvfp4_quantize(w, w_scales, w_tscale)
    xf = (xq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (wq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return xf @ wf.T, xq, wq


def w4a4_linear_bwd(grad_y: np.ndarray, xq: np.ndarray, wq: np.ndarray):
    """Straight-through backward in binary64: grad_x = grad_y wq, grad_w =
    grad_y^T xq (bf16 bit inputs)."""
    f = lambda b: (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g = f(grad_y)
    return g @ f(wq), g.T @ f(xq)


# ---- KL ---------------------------------------------------------------------
def kl_fwd_bwd(teacher: np.ndarray, student: np.ndarray, T: float = 1.0,
               grad_scale: float | None = None, want_grad: bool = True):
    """Binary64 KL(teacher || student) over the last dim.

    Returns (mean loss, row losses f64[rows], gradient f64[rows, V] or None).
    grad_scale defaults to 1/rows (gradient of the mean).
    """
    t = np.ascontiguousarray(teacher)
    s = np.ascontiguousarray(student)
    assert t.shape == s.shape and t.dtype == s.dtype
    V = t.shape[-1]
    rows = t.size // V if V else 0
    if grad_scale is None:
        grad_scale = 1.0 / rows if rows else 0.0
    row = np.empty(rows, np.float64)
    g = np.empty((rows, V), np.float64) if want_grad else None
    loss = _load().orc_kl_fwd_bwd(_ptr(t), _ptr(s), _dtype_code(t), rows, V, float(T),
                                  float(grad_scale), _ptr(row), _ptr(g))
    return float(loss), row, g


def kl_topk_fwd_bwd(teacher: np.ndarray, student: np.ndarray, k: int, T: float = 1.0,
                    grad_scale: float | None = None, want_grad: bool = True):
    """Binary64 KL restricted to the teacher's top-k entries of each row (all
    entries tied with the k-th largest kept), both softmaxes renormalised over
    that set; gradient 0 outside it.

    Returns (mean loss, row losses f64[rows], gradient f64[rows, V] or None,
    set sizes i64[rows]).
    """
    t = np.ascontiguousarray(teacher)
    s = np.ascontiguousarray(student)
    assert t.shape == s.shape and t.dtype == s.dtype and k >= 1
    V = t.shape[-1]
    rows = t.size // V if V else 0
    if grad_scale is None:
        grad_scale = 1.0 / rows if rows else 0.0
    row = np.empty(rows, np.float64)
    cnt = np.empty(rows, np.int64)
    g = np.empty((rows, V), np.float64) if want_grad else None
    loss = _load().orc_kl_topk_fwd_bwd(_ptr(t), _ptr(s), _dtype_code(t), rows, V, int(k), float(T),
                                       float(grad_scale), _ptr(row), _ptr(g), _ptr(cnt))
    return float(loss), row, g, cnt


def kl_topp_fwd_bwd(teacher: np.ndarray, student: np.ndarray, top_p: float, T: float = 1.0,
                    grad_scale: float | None = None, want_grad: bool = True):
    """Binary64 KL restricted to the teacher's nucleus of each row: the
    entries at or above tau, the largest teacher value at which the teacher
    mass of the entries at or above it reaches top_p (ties kept); both
    softmaxes renormalised over that set, gradient 0 outside it.

    Returns (mean loss, row losses f64[rows], gradient f64[rows, V] or None,
    set sizes i64[rows], tau f64[rows], masses f64[rows, 2] = (mass strictly
    above tau, mass at or above tau)).
    """
    t = np.ascontiguousarray(teacher)
    s = np.ascontiguousarray(student)
    assert t.shape == s.shape and t.dtype == s.dtype and top_p > 0
    V = t.shape[-1]
    rows = t.size // V if V else 0
    if grad_scale is None:
        grad_scale = 1.0 / rows if rows else 0.0
    row = np.empty(rows, np.float64)
    cnt = np.empty(rows, np.int64)
    tau = np.empty(rows, np.float64)
    mass = np.empty((rows, 2), np.float64)
    g = np.empty((rows, V), np.float64) if want_grad else None
    loss = _load().orc_kl_topp_fwd_bwd(_ptr(t), _ptr(s), _dtype_code(t), rows, V, float(top_p), float(T),
                                       float(grad_scale), _ptr(row), _ptr(g), _ptr(cnt), _ptr(tau), _ptr(mass))
    return float(loss), row, g, cnt, tau, mass


# ---- binary32 KL (timing variant) and the all-cores harness ----------------
def kl_fwd_bwd_f32(teacher: np.ndarray, student: np.ndarray, T: float = 1.0, grad_scale: float | None = None):
    """The KL loss and gradient in binary32 (a CPU timing variant, not a
    parity reference).  Returns (mean loss, row losses f32, grad f32)."""
    t = np.ascontiguousarray(teacher)
    s = np.ascontiguousarray(student)
    rows, V = t.shape
    gs = 1.0 / rows if grad_scale is None else grad_scale
    row = np.empty(rows, np.float32)
    grad = np.empty((rows, V), np.float32)
    loss = _load().orc_kl_fwd_bwd_f32(_ptr(t), _ptr(s), _dtype_code(t), rows, V, float(T), float(gs), _ptr(row), _ptr(grad))
    return float(loss), row, grad


def omp_threads() -> int:
    return int(_load().orc_omp_threads())


def omp_quantize_batch(x: np.ndarray):
    """orc_nvfp4_quantize of every tensor of x [B, R, C] on all cores.
    Returns (codes, scales, tscale [B], y bits)."""
    x = np.ascontiguousarray(x)
    B, R, C = x.shape
    codes = np.empty((B, R, C // 2), np.uint8)
    scales = np.empty((B, R, C // 16), np.uint8)
    ts = np.empty(B, np.float32)
    y = np.empty((B, R, C), np.uint16)
    _load().orc_omp_quantize_batch(_ptr(x), _dtype_code(x), B, R, C, _ptr(codes), _ptr(scales), _ptr(ts), _ptr(y))
    return codes, scales, ts, y


def omp_quantize_tensor(x: np.ndarray, scales_in: np.ndarray | None = None, tscale_in: float | None = None):
    """nvfp4_quantize of one [R, C] tensor on all cores (row ranges)."""
    x = np.ascontiguousarray(x)
    R, C = x.shape
    codes = np.empty((R, C // 2), np.uint8)
    scales = np.empty((R, C // 16), np.uint8)
    ts = np.empty(1, np.float32)
    y = np.empty((R, C), np.uint16)
    si = None if scales_in is None else np.ascontiguousarray(scales_in, dtype=np.uint8)
    ti = None if tscale_in is None else np.array([tscale_in], np.float32)
    _load().orc_omp_quantize_tensor(_ptr(x), _dtype_code(x), R, C, _ptr(si), _ptr(ti), _ptr(codes), _ptr(scales),
                                    _ptr(ts), _ptr(y))
    return codes, scales, float(ts[0]), y


def omp_mse_calibrate(x: np.ndarray, n_cand: int = 64, k_min: float = 0.5, k_max: float = 1.0):
    """mse_calibrate of one [R, C] tensor on all cores.  Returns (scales, tscale)."""
    x = np.ascontiguousarray(x)
    R, C = x.shape
    scales = np.empty((R, C // 16), np.uint8)
    ts = np.empty(1, np.float32)
    _load().orc_omp_mse_calibrate(_ptr(x), _dtype_code(x), R, C, int(n_cand), float(k_min), float(k_max),
                                  _ptr(scales), _ptr(ts))
    return scales, float(ts[0])


def omp_kl_fwd_bwd(teacher: np.ndarray, student: np.ndarray, T: float = 1.0, grad_scale: float | None = None):
    """kl_fwd_bwd on all cores, one row per call.  Returns (mean, rows, grad)."""
    t = np.ascontiguousarray(teacher)
    s = np.ascontiguousarray(student)
    rows, V = t.shape
    gs = 1.0 / rows if grad_scale is None else grad_scale
    row = np.empty(rows, np.float64)
    grad = np.empty((rows, V), np.float64)
    loss = _load().orc_omp_kl_fwd_bwd(_ptr(t), _ptr(s), _dtype_code(t), rows, V, float(T), float(gs), _ptr(row), _ptr(grad))
    return float(loss), row, grad


def omp_kl_fwd_bwd_f32(teacher: np.ndarray, student: np.ndarray, T: float = 1.0, grad_scale: float | None = None):
    """kl_fwd_bwd_f32 on all cores, one row per call.  Returns (mean, rows, grad)."""
    t = np.ascontiguousarray(teacher)
    s = np.ascontiguousarray(student)
    rows, V = t.shape
    gs = 1.0 / rows if grad_scale is None else grad_scale
    row = np.empty(rows, np.float32)
    grad = np.empty((rows, V), np.float32)
    loss = _load().orc_omp_kl_fwd_bwd_f32(_ptr(t), _ptr(s), _dtype_code(t), rows, V, float(T), float(gs), _ptr(row),
                                          _ptr(grad))
    return float(loss), row, grad


__all__ = [
    "build", "F32", "BF16", "e2m1_encode", "e2m1_decode", "e4m3_encode", "e4m3_decode",
    "e4m3_decode_table", "bf16_from_f32", "f32_from_bf16", "amax", "tensor_scale",
    "nvfp4_quantize", "nvfp4_quantize_blocks", "mse_kgrid", "mse_calibrate", "mse_calibrate_blocks", "kl_fwd_bwd",
    "kl_topk_fwd_bwd", "fp8_quantize", "w4a4_linear_fwd", "w4a4_linear_bwd", "nvfp4_qdq_bwd_clipped",
    "kl_topp_fwd_bwd", "nvfp4_frozen_sgd_step", "kl_fwd_bwd_f32", "omp_threads", "omp_quantize_batch",
    "omp_quantize_tensor", "omp_mse_calibrate", "omp_kl_fwd_bwd", "omp_kl_fwd_bwd_f32",
]
