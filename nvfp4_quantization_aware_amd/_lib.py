"""Thin ctypes binding of libqad (include/libqad.h).

Argument marshalling only: every step of the hot path runs in the HIP
library.  PyTorch supplies device memory (outputs and workspace are allocated
here with torch when the caller does not pass them) and the current stream.
If libqad.so has not been built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libqad.so")

QAD_F32, QAD_BF16 = 0, 1
QAD_OP_AMAX, QAD_OP_QUANTIZE, QAD_OP_MSE_CALIBRATE, QAD_OP_KL, QAD_OP_KL_TOPK, QAD_OP_W4A4_LINEAR, QAD_OP_KL_TOPP = \
    0, 1, 2, 3, 4, 5, 6
STATUS = {0: "QAD_OK", 1: "QAD_ERR_INVALID_ARG", 2: "QAD_ERR_SHAPE", 3: "QAD_ERR_DTYPE",
          4: "QAD_ERR_ALIGNMENT", 5: "QAD_ERR_WORKSPACE", 6: "QAD_ERR_NONFINITE", 7: "QAD_ERR_HIP"}

# every symbol include/libqad.h declares, with its ctypes signature
_vp, _i64, _f32, _i32, _sz, _int = C.c_void_p, C.c_int64, C.c_float, C.c_int32, C.c_size_t, C.c_int
SIGNATURES = {
    "qad_status_string": (C.c_char_p, [_int]),
    "qad_abi_version": (_int, []),
    "qad_set_wait_limit_us": (_i64, [_i64]),
    "qad_workspace_bytes": (_sz, [_int, _i64, _i64, _i64]),
    "qad_nvfp4_packed_bytes": (_sz, [_i64, _i64]),
    "nvfp4_amax": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "nvfp4_quantize": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_quantize_noalloc": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "nvfp4_qdq_fwd": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_qdq_bwd": (_int, [_vp, _vp, _int, _i64, _vp]),
    "nvfp4_qdq_bwd_clipped": (_int, [_vp, _int, _vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_frozen_sgd_step": (_int, [_vp, _int, _vp, _int, _i64, _i64, _i64, _vp, _vp, C.c_float, C.c_float, _vp,
                                     _vp]),
    "nvfp4_mse_calibrate": (_int, [_vp, _int, _i64, _i64, _i64, _i32, _f32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "qad_kl_fwd_bwd": (_int, [_vp, _vp, _int, _i64, _i64, _f32, _f32, _vp, _vp, _vp, _int, _vp, _sz, _vp]),
    "qad_w4a4_linear_fwd": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "qad_w4a4_linear_bwd": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _sz, _vp]),
    "fp8_quantize": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "qad_kl_topk_fwd_bwd": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _f32, _f32, _vp, _vp, _vp, _int, _vp, _sz,
                                   _vp]),
    "qad_kl_topp_fwd_bwd": (_int, [_vp, _vp, _int, _i64, _i64, _f32, _f32, _f32, _vp, _vp, _vp, _int, _vp, _vp,
                                   _sz, _vp]),
    "qad_check_finite": (_int, [_vp, _i64, _vp]),
}

_lock = threading.Lock()
_lib = None


class QadError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, STATUS.get(status, status)))


def lib() -> C.CDLL:
    """The loaded libqad (raises if it was never built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libqad.so is not built (%s); run `python -m "
                                   "nvfp4_quantization_aware_amd.build`" % LIB_PATH)
            h = C.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
        return _lib


def _check(status: int, where: str):
    if status != 0:
        raise QadError(status, where)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return QAD_F32
    if t.dtype == torch.bfloat16:
        return QAD_BF16
    raise TypeError("libqad takes float32 or bfloat16 tensors, got %s" % t.dtype)


def _p(t):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device):
    return torch.cuda.current_stream(dev).cuda_stream
# Every library call runs with the tensors' device current (torch.cuda.device):
# the library launches on the stream it is given, but keys its per-device
# state (CU count, occupancy, the no-workspace scratch address) by HIP's current
# device, and the two must agree.


def _gpu(t, name: str, dev: torch.device | None = None, dtype=None, numel: int | None = None) -> torch.Tensor:
    """Check a tensor argument before its pointer goes to the library: a
    contiguous tensor on the GPU (on `dev` when given), of `dtype` (one dtype
    or a tuple) and `numel` elements when given.  Raises ValueError or
    TypeError; the library itself cannot tell a host pointer or a short
    buffer from a good one."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got device %s" % (name, t.device))
    if dev is not None and t.device != dev:
        raise ValueError("%s is on %s, the other arguments on %s" % (name, t.device, dev))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s must hold %d elements, got %d" % (name, numel, t.numel()))
    return t


def _opt(t, name: str, dev: torch.device, dtype=None, numel: int | None = None):
    return None if t is None else _gpu(t, name, dev, dtype, numel)


_FLOAT = (torch.float32, torch.bfloat16)


def _ws(ws, dev: torch.device):
    """The caller's workspace: a uint8 GPU tensor (its size is checked by the library)."""
    return _opt(ws, "ws", dev, torch.uint8)


def _brc(x: torch.Tensor, name: str = "x"):
    _gpu(x, name, dtype=_FLOAT)
    if x.dim() == 2:
        return 1, x.shape[0], x.shape[1]
    if x.dim() == 3:
        return x.shape[0], x.shape[1], x.shape[2]
    raise ValueError("expected [R, C] or [B, R, C], got shape %s" % (tuple(x.shape),))


def _logits(teacher: torch.Tensor, student: torch.Tensor):
    """(tokens, vocab, device) of a teacher / student pair of one dtype and shape"""
    _gpu(teacher, "teacher", dtype=_FLOAT)
    _gpu(student, "student", teacher.device, teacher.dtype)
    if teacher.shape != student.shape or teacher.dim() != 2:
        raise ValueError("teacher and student must both be [tokens, vocab]")
    tokens, vocab = teacher.shape
    return tokens, vocab, teacher.device


def set_wait_limit_us(us: int) -> int:
    """Bound of the one-pass kernels' device-side waits in microseconds
    (default 20000; 0: every wait gives up at once and the workgroup computes
    what it waited for itself; negative: query).  Returns the previous bound."""
    return int(lib().qad_set_wait_limit_us(int(us)))


def qad_workspace_bytes(op: int, B: int, R: int, C_: int) -> int:
    return int(lib().qad_workspace_bytes(op, B, R, C_))


def workspace(op: int, B: int, R: int, C_: int, device) -> torch.Tensor | None:
    n = qad_workspace_bytes(op, B, R, C_)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def nvfp4_amax(x: torch.Tensor, amax_out: torch.Tensor | None = None,
               ws: torch.Tensor | None = None) -> torch.Tensor:
    B, R, Cc = _brc(x)
    amax_out = _opt(amax_out, "amax_out", x.device, torch.float32, B)
    ws = _ws(ws, x.device)
    if amax_out is None:
        amax_out = torch.empty(B, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(QAD_OP_AMAX, B, R, Cc, x.device)
    with torch.cuda.device(x.device):
        _check(lib().nvfp4_amax(_p(x), _dt(x), B, R, Cc, _p(amax_out), _p(ws), 0 if ws is None else ws.numel(),
                                _stream(x.device)), "nvfp4_amax")
    return amax_out


def nvfp4_quantize(x: torch.Tensor, scales_in=None, tscale_in=None, codes=True, scales_out=True,
                   tscale_out=True, y=True, ws: torch.Tensor | None = None):
    """Returns (codes u8[B,R,C/2], scales u8[B,R,C/16], tscale f32[B], y bf16[B,R,C]).

    Pass a tensor to write into it, True to have it allocated, None/False to
    skip that output.
    """
    B, R, Cc = _brc(x)
    dev = x.device
    n = B * R * Cc
    scales_in = _opt(scales_in, "scales_in", dev, torch.uint8, n // 16)
    tscale_in = _opt(tscale_in, "tscale_in", dev, torch.float32, B)
    ws = _ws(ws, dev)

    def out(arg, name, shape, dtype):
        if arg is True:
            return torch.empty(shape, dtype=dtype, device=dev)
        if arg is None or arg is False:
            return None
        return _gpu(arg, name, dev, dtype, shape[0] * shape[1] * shape[2] if len(shape) == 3 else shape[0])

    codes = out(codes, "codes", (B, R, Cc // 2), torch.uint8)
    scales_out = out(scales_out, "scales_out", (B, R, Cc // 16), torch.uint8)
    tscale_out = out(tscale_out, "tscale_out", (B,), torch.float32)
    y = out(y, "y", (B, R, Cc), torch.bfloat16)
    if ws is None and scales_in is None:
        ws = workspace(QAD_OP_QUANTIZE, B, R, Cc, dev)
    with torch.cuda.device(dev):
        _check(lib().nvfp4_quantize(_p(x), _dt(x), B, R, Cc, _p(scales_in), _p(tscale_in), _p(codes),
                                    _p(scales_out), _p(tscale_out), _p(y), _p(ws),
                                    0 if ws is None else ws.numel(), _stream(dev)), "nvfp4_quantize")
    return codes, scales_out, tscale_out, y


def nvfp4_quantize_noalloc(x: torch.Tensor, codes: torch.Tensor | None = None, scales_out: torch.Tensor | None = None,
                           tscale_out: torch.Tensor | None = None, y: torch.Tensor | None = None, scales_in=None,
                           tscale_in=None):
    """nvfp4_quantize without a workspace (the library's fixed scratch): the
    caller passes every output it wants (None skips it; nothing is allocated
    here).  Returns (codes, scales_out, tscale_out, y)."""
    B, R, Cc = _brc(x)
    dev = x.device
    n = B * R * Cc
    scales_in = _opt(scales_in, "scales_in", dev, torch.uint8, n // 16)
    tscale_in = _opt(tscale_in, "tscale_in", dev, torch.float32, B)
    codes = _opt(codes, "codes", dev, torch.uint8, n // 2)
    scales_out = _opt(scales_out, "scales_out", dev, torch.uint8, n // 16)
    tscale_out = _opt(tscale_out, "tscale_out", dev, torch.float32, B)
    y = _opt(y, "y", dev, torch.bfloat16, n)
    with torch.cuda.device(dev):
        _check(lib().nvfp4_quantize_noalloc(_p(x), _dt(x), B, R, Cc, _p(scales_in), _p(tscale_in), _p(codes),
                                            _p(scales_out), _p(tscale_out), _p(y), _stream(dev)),
               "nvfp4_quantize_noalloc")
    return codes, scales_out, tscale_out, y


def nvfp4_qdq_fwd(x: torch.Tensor, scales_in=None, tscale_in=None, y: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None) -> torch.Tensor:
    B, R, Cc = _brc(x)
    n = B * R * Cc
    scales_in = _opt(scales_in, "scales_in", x.device, torch.uint8, n // 16)
    tscale_in = _opt(tscale_in, "tscale_in", x.device, torch.float32, B)
    y = _opt(y, "y", x.device, torch.bfloat16, n)
    ws = _ws(ws, x.device)
    if y is None:
        y = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    if ws is None and scales_in is None:
        ws = workspace(QAD_OP_QUANTIZE, B, R, Cc, x.device)
    with torch.cuda.device(x.device):
        _check(lib().nvfp4_qdq_fwd(_p(x), _dt(x), B, R, Cc, _p(scales_in), _p(tscale_in), _p(y), _p(ws),
                                   0 if ws is None else ws.numel(), _stream(x.device)), "nvfp4_qdq_fwd")
    return y


def nvfp4_qdq_bwd(grad_y: torch.Tensor, grad_x: torch.Tensor | None = None) -> torch.Tensor:
    _gpu(grad_y, "grad_y", dtype=_FLOAT)
    grad_x = _opt(grad_x, "grad_x", grad_y.device, grad_y.dtype, grad_y.numel())
    if grad_x is None:
        grad_x = torch.empty_like(grad_y)
    with torch.cuda.device(grad_y.device):
        _check(lib().nvfp4_qdq_bwd(_p(grad_y), _p(grad_x), _dt(grad_y), grad_y.numel(),
                                   _stream(grad_y.device)), "nvfp4_qdq_bwd")
    return grad_x


def nvfp4_qdq_bwd_clipped(grad_y: torch.Tensor, x: torch.Tensor, scales: torch.Tensor, tscale: torch.Tensor,
                          grad_x: torch.Tensor | None = None) -> torch.Tensor:
    """Clipped straight-through backward with the forward's scales: grad_y
    where |x| <= 6 * s_eff, +0 elsewhere.  grad_y and x share the shape
    [R, C] or [B, R, C]; scales [.., C/16] u8, tscale [B] float32."""
    B, R, Cc = _brc(x)
    _gpu(grad_y, "grad_y", x.device, _FLOAT)
    if tuple(grad_y.shape) != tuple(x.shape):
        raise ValueError("grad_y and x shapes differ")
    _gpu(scales, "scales (uint8, one code per 16 elements)", x.device, torch.uint8, B * R * (Cc // 16))
    _gpu(tscale, "tscale (float32, one scale per tensor)", x.device, torch.float32, B)
    grad_x = _opt(grad_x, "grad_x", x.device, grad_y.dtype, grad_y.numel())
    if grad_x is None:
        grad_x = torch.empty_like(grad_y)
    with torch.cuda.device(x.device):
        _check(lib().nvfp4_qdq_bwd_clipped(_p(grad_y), _dt(grad_y), _p(x), _dt(x), B, R, Cc, _p(scales), _p(tscale),
                                           _p(grad_x), _stream(x.device)), "nvfp4_qdq_bwd_clipped")
    return grad_x


def nvfp4_frozen_sgd_step(w: torch.Tensor, grad: torch.Tensor, scales: torch.Tensor, tscale: torch.Tensor,
                          lr: float, clip_coef: float = 1.0, w_out: torch.Tensor | None = None) -> torch.Tensor:
    """Frozen-scale SGD step through the clipped straight-through gradient:
    w where |w| > 6 * s_eff, else round(fma32(-fl32(lr * clip_coef), grad, w)).
    w and grad share the shape [R, C] or [B, R, C]; scales [.., C/16] u8,
    tscale [B] float32.  w_out=w updates in place; None allocates."""
    B, R, Cc = _brc(w, "w")
    _gpu(grad, "grad", w.device, _FLOAT)
    if tuple(grad.shape) != tuple(w.shape):
        raise ValueError("grad and w shapes differ")
    _gpu(scales, "scales (uint8, one code per 16 elements)", w.device, torch.uint8, B * R * (Cc // 16))
    _gpu(tscale, "tscale (float32, one scale per tensor)", w.device, torch.float32, B)
    w_out = _opt(w_out, "w_out", w.device, w.dtype, w.numel())
    if w_out is None:
        w_out = torch.empty_like(w)
    with torch.cuda.device(w.device):
        _check(lib().nvfp4_frozen_sgd_step(_p(w), _dt(w), _p(grad), _dt(grad), B, R, Cc, _p(scales), _p(tscale),
                                           float(lr), float(clip_coef), _p(w_out), _stream(w.device)),
               "nvfp4_frozen_sgd_step")
    return w_out


def nvfp4_mse_calibrate(w: torch.Tensor, n_candidates: int = 64, k_min: float = 0.5, k_max: float = 1.0,
                        scales_out: torch.Tensor | None = None, tscale_out: torch.Tensor | None = None,
                        ws: torch.Tensor | None = None):
    B, R, Cc = _brc(w, "w")
    dev = w.device
    scales_out = _opt(scales_out, "scales_out", dev, torch.uint8, B * R * (Cc // 16))
    tscale_out = _opt(tscale_out, "tscale_out", dev, torch.float32, B)
    ws = _ws(ws, dev)
    if scales_out is None:
        scales_out = torch.empty((B, R, Cc // 16), dtype=torch.uint8, device=dev)
    if tscale_out is None:
        tscale_out = torch.empty(B, dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(QAD_OP_MSE_CALIBRATE, B, R, Cc, dev)
    with torch.cuda.device(dev):
        _check(lib().nvfp4_mse_calibrate(_p(w), _dt(w), B, R, Cc, n_candidates, k_min, k_max, _p(scales_out),
                                         _p(tscale_out), _p(ws), 0 if ws is None else ws.numel(),
                                         _stream(dev)), "nvfp4_mse_calibrate")
    return scales_out, tscale_out


def qad_kl_fwd_bwd(teacher: torch.Tensor, student: torch.Tensor, temperature: float = 1.0,
                   grad_scale: float | None = None, grad_dtype=torch.bfloat16, row_loss=False,
                   loss_out: torch.Tensor | None = None, grad: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None):
    """Returns (loss f32[1], row_loss f32[tokens] or None, grad or None)."""
    tokens, vocab, dev = _logits(teacher, student)
    loss_out = _opt(loss_out, "loss_out", dev, torch.float32, 1)
    grad = _opt(grad, "grad", dev, _FLOAT, tokens * vocab)
    ws = _ws(ws, dev)
    if grad_scale is None:
        grad_scale = 1.0 / tokens if tokens else 0.0
    if loss_out is None:
        loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    rows = torch.empty(tokens, dtype=torch.float32, device=dev) if row_loss is True else (
        _gpu(row_loss, "row_loss", dev, torch.float32, tokens) if isinstance(row_loss, torch.Tensor) else None)
    if grad is None and grad_dtype is not None:
        grad = torch.empty((tokens, vocab), dtype=grad_dtype, device=dev)
    gt = _dt(grad) if grad is not None else QAD_BF16
    if ws is None:
        ws = workspace(QAD_OP_KL, 1, tokens, vocab, dev)
    with torch.cuda.device(dev):
        _check(lib().qad_kl_fwd_bwd(_p(teacher), _p(student), _dt(teacher), tokens, vocab, temperature,
                                    grad_scale, _p(loss_out), _p(rows), _p(grad), gt, _p(ws),
                                    0 if ws is None else ws.numel(), _stream(dev)), "qad_kl_fwd_bwd")
    return loss_out, rows, grad


def fp8_quantize(x: torch.Tensor, tscale_in: torch.Tensor | None = None, codes=True, y=True,
                 tscale_out: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """FP8 (E4M3) per-tensor QDQ of x ([R, C] or [B, R, C]).  Dynamic scales
    (amax/448) unless tscale_in (float[B]) is given.  Returns (codes u8 like x
    or None, tscale f32[B], y bf16 like x or None)."""
    B, R, Cc = _brc(x)
    dev = x.device
    n = B * R * Cc
    tscale_in = _opt(tscale_in, "tscale_in", dev, torch.float32, B)
    tscale_out = _opt(tscale_out, "tscale_out", dev, torch.float32, B)
    ws = _ws(ws, dev)
    cd = torch.empty(x.shape, dtype=torch.uint8, device=dev) if codes is True else (
        _gpu(codes, "codes", dev, torch.uint8, n) if isinstance(codes, torch.Tensor) else None)
    yy = torch.empty(x.shape, dtype=torch.bfloat16, device=dev) if y is True else (
        _gpu(y, "y", dev, torch.bfloat16, n) if isinstance(y, torch.Tensor) else None)
    if tscale_out is None:
        tscale_out = torch.empty(B, dtype=torch.float32, device=dev)
    if ws is None and tscale_in is None:
        ws = workspace(QAD_OP_QUANTIZE, B, R, Cc, dev)
    with torch.cuda.device(dev):
        _check(lib().fp8_quantize(_p(x), _dt(x), B, R, Cc, _p(tscale_in), _p(cd), _p(tscale_out), _p(yy), _p(ws),
                                  0 if ws is None else ws.numel(), _stream(dev)), "fp8_quantize")
    return cd, tscale_out, yy


def nvfp4_packed_bytes(R: int, C: int) -> int:
    """Bytes of a packed NVFP4 tensor (codes, block scales, tensor scale) of R x C."""
    return int(lib().qad_nvfp4_packed_bytes(R, C))


def nvfp4_unpack(packed: torch.Tensor, R: int, C: int):
    """Views of a packed NVFP4 tensor: (codes u8 [R, C/2], scales u8 [R, C/16],
    tensor scale f32 [1])."""
    n = R * C
    toff = (n // 2 + n // 16 + 15) // 16 * 16
    return (packed[:n // 2].view(R, C // 2), packed[n // 2:n // 2 + n // 16].view(R, C // 16),
            packed[toff:toff + 4].view(torch.float32))


def qad_w4a4_linear_fwd(x: torch.Tensor, w: torch.Tensor, y=None, xq=None, wq=None, ws: torch.Tensor | None = None,
                        w_scales_in: torch.Tensor | None = None, w_tscale_in: torch.Tensor | None = None):
    """y = QDQ(x) QDQ(w)^T (bf16) for x [M, K], w [N, K]; w's scales are
    dynamic, or the frozen w_scales_in (u8 [N, K/16]) / w_tscale_in (f32 [1]).
    Returns (y, xq, wq): xq, wq the packed NVFP4 forms of x and w (uint8,
    nvfp4_packed_bytes each; nvfp4_unpack gives their parts)."""
    _gpu(x, "x", dtype=_FLOAT)
    _gpu(w, "w", x.device, x.dtype)
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x [M, K] and w [N, K] of one dtype")
    (M, K), N = x.shape, w.shape[0]
    dev = x.device
    bx, bw = nvfp4_packed_bytes(M, K), nvfp4_packed_bytes(N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else _gpu(y, "y", dev, torch.bfloat16, M * N)
    xq = torch.empty(bx, dtype=torch.uint8, device=dev) if xq is None else _gpu(xq, "xq", dev, torch.uint8, bx)
    wq = torch.empty(bw, dtype=torch.uint8, device=dev) if wq is None else _gpu(wq, "wq", dev, torch.uint8, bw)
    ws = _ws(ws, dev)
    w_scales_in = _opt(w_scales_in, "w_scales_in", dev)
    w_tscale_in = _opt(w_tscale_in, "w_tscale_in", dev)
    if ws is None:
        ws = workspace(QAD_OP_W4A4_LINEAR, M, N, K, dev)
    if (w_scales_in is None) != (w_tscale_in is None):
        raise ValueError("frozen weight scales need both w_scales_in and w_tscale_in")
    if w_scales_in is not None and (w_scales_in.dtype != torch.uint8 or w_scales_in.numel() != N * (K // 16)
                                    or w_tscale_in.dtype != torch.float32 or w_tscale_in.numel() != 1):
        raise ValueError("w_scales_in must be uint8 [N, K/16] and w_tscale_in float32 [1]")
    with torch.cuda.device(dev):
        _check(lib().qad_w4a4_linear_fwd(_p(x), _p(w), _dt(x), M, N, K, _p(w_scales_in), _p(w_tscale_in), _p(y), _p(xq),
                                         _p(wq), _p(ws), 0 if ws is None else ws.numel(), _stream(dev)),
               "qad_w4a4_linear_fwd")
    return y, xq, wq


def qad_w4a4_linear_bwd(grad_y: torch.Tensor, xq: torch.Tensor, wq: torch.Tensor, K: int, grad_x=True, grad_w=True):
    """Straight-through backward from the forward's packed operands xq, wq
    (for x [M, K], w [N, K]): returns (grad_x [M, K] or None, grad_w [N, K]
    or None)."""
    _gpu(grad_y, "grad_y", dtype=torch.bfloat16)
    dev = grad_y.device
    if grad_y.dim() != 2:
        raise ValueError("grad_y [M, N]")
    M, N = grad_y.shape
    _gpu(xq, "xq", dev, torch.uint8, nvfp4_packed_bytes(M, K))
    _gpu(wq, "wq", dev, torch.uint8, nvfp4_packed_bytes(N, K))
    gx = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if grad_x is True else (
        _gpu(grad_x, "grad_x", dev, torch.bfloat16, M * K) if isinstance(grad_x, torch.Tensor) else None)
    gw = torch.empty((N, K), dtype=torch.bfloat16, device=dev) if grad_w is True else (
        _gpu(grad_w, "grad_w", dev, torch.bfloat16, N * K) if isinstance(grad_w, torch.Tensor) else None)
    with torch.cuda.device(dev):
        _check(lib().qad_w4a4_linear_bwd(_p(grad_y), _p(xq), _p(wq), M, N, K, _p(gx), _p(gw), None, 0, _stream(dev)),
               "qad_w4a4_linear_bwd")
    return gx, gw


def qad_kl_topk_fwd_bwd(teacher: torch.Tensor, student: torch.Tensor, k: int, temperature: float = 1.0,
                        grad_scale: float | None = None, grad_dtype=torch.bfloat16, row_loss=False,
                        loss_out: torch.Tensor | None = None, grad: torch.Tensor | None = None,
                        ws: torch.Tensor | None = None):
    """KL over the teacher's top-k entries of each row (ties with the k-th
    largest kept, both softmaxes renormalised over them).  Returns (loss
    f32[1], row_loss f32[tokens] or None, grad or None)."""
    tokens, vocab, dev = _logits(teacher, student)
    loss_out = _opt(loss_out, "loss_out", dev, torch.float32, 1)
    grad = _opt(grad, "grad", dev, _FLOAT, tokens * vocab)
    ws = _ws(ws, dev)
    if grad_scale is None:
        grad_scale = 1.0 / tokens if tokens else 0.0
    if loss_out is None:
        loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    rows = torch.empty(tokens, dtype=torch.float32, device=dev) if row_loss is True else (
        _gpu(row_loss, "row_loss", dev, torch.float32, tokens) if isinstance(row_loss, torch.Tensor) else None)
    if grad is None and grad_dtype is not None:
        grad = torch.empty((tokens, vocab), dtype=grad_dtype, device=dev)
    gt = _dt(grad) if grad is not None else QAD_BF16
    if ws is None:
        ws = workspace(QAD_OP_KL_TOPK, 1, tokens, vocab, dev)
    with torch.cuda.device(dev):
        _check(lib().qad_kl_topk_fwd_bwd(_p(teacher), _p(student), _dt(teacher), tokens, vocab, int(k), temperature,
                                         grad_scale, _p(loss_out), _p(rows), _p(grad), gt, _p(ws),
                                         0 if ws is None else ws.numel(), _stream(dev)), "qad_kl_topk_fwd_bwd")
    return loss_out, rows, grad


def qad_kl_topp_fwd_bwd(teacher: torch.Tensor, student: torch.Tensor, top_p: float, temperature: float = 1.0,
                        grad_scale: float | None = None, grad_dtype=torch.bfloat16, row_loss=False, tau=False,
                        loss_out: torch.Tensor | None = None, grad: torch.Tensor | None = None,
                        ws: torch.Tensor | None = None):
    """KL over the teacher's nucleus of each row: the entries at or above the
    largest teacher value at which the teacher mass reaches top_p (ties
    kept), both softmaxes renormalised over them.  Returns (loss f32[1],
    row_loss f32[tokens] or None, grad or None, tau f32[tokens] or None)."""
    tokens, vocab, dev = _logits(teacher, student)
    loss_out = _opt(loss_out, "loss_out", dev, torch.float32, 1)
    grad = _opt(grad, "grad", dev, _FLOAT, tokens * vocab)
    ws = _ws(ws, dev)
    if grad_scale is None:
        grad_scale = 1.0 / tokens if tokens else 0.0
    if loss_out is None:
        loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    rows = torch.empty(tokens, dtype=torch.float32, device=dev) if row_loss is True else (
        _gpu(row_loss, "row_loss", dev, torch.float32, tokens) if isinstance(row_loss, torch.Tensor) else None)
    taus = torch.empty(tokens, dtype=torch.float32, device=dev) if tau is True else (
        _gpu(tau, "tau", dev, torch.float32, tokens) if isinstance(tau, torch.Tensor) else None)
    if grad is None and grad_dtype is not None:
        grad = torch.empty((tokens, vocab), dtype=grad_dtype, device=dev)
    gt = _dt(grad) if grad is not None else QAD_BF16
    if ws is None:
        ws = workspace(QAD_OP_KL_TOPP, 1, tokens, vocab, dev)
    with torch.cuda.device(dev):
        _check(lib().qad_kl_topp_fwd_bwd(_p(teacher), _p(student), _dt(teacher), tokens, vocab, float(top_p),
                                         temperature, grad_scale, _p(loss_out), _p(rows), _p(grad), gt, _p(taus),
                                         _p(ws), 0 if ws is None else ws.numel(), _stream(dev)), "qad_kl_topp_fwd_bwd")
    return loss_out, rows, grad, taus


def qad_check_finite(values: torch.Tensor) -> bool:
    """True if every value is finite (synchronises the current stream)."""
    _gpu(values, "values", dtype=torch.float32)
    with torch.cuda.device(values.device):
        st = lib().qad_check_finite(_p(values), values.numel(), _stream(values.device))
    if st == 6:
        return False
    _check(st, "qad_check_finite")
    return True
