"""QAD hot path on MI355X: NVFP4 simulated quantization and the fused KL loss.

The computation lives in libqad.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/libqad.h); this package is its thin Python binding plus
the seeded synthetic input generators.  Build with
``python -m nvfp4_quantization_aware_amd.build``.
"""
from ._lib import (QAD_BF16, QAD_F32, QAD_OP_AMAX, QAD_OP_KL, QAD_OP_KL_TOPK, QAD_OP_KL_TOPP, QAD_OP_W4A4_LINEAR,  # noqa: F401
                   QAD_OP_MSE_CALIBRATE, QAD_OP_QUANTIZE, QadError, fp8_quantize, lib, nvfp4_amax, nvfp4_frozen_sgd_step,
                   nvfp4_mse_calibrate, nvfp4_packed_bytes, nvfp4_unpack,
                   nvfp4_qdq_bwd, nvfp4_qdq_bwd_clipped, nvfp4_qdq_fwd, nvfp4_quantize, nvfp4_quantize_noalloc,
                   qad_check_finite,
                   qad_kl_fwd_bwd, qad_kl_topk_fwd_bwd, qad_kl_topp_fwd_bwd, qad_w4a4_linear_bwd, qad_w4a4_linear_fwd,
                   qad_workspace_bytes, set_wait_limit_us, workspace)
