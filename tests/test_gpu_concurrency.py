"""Entry points running at the same time on two streams (default priority,
separate workspaces) give exactly what they give one after the other.

The one-pass kernels assume that the workgroups exchanging partial results
are resident together; a kernel on another stream can take part of the GPU,
and then a wait may reach its bound and the workgroup computes the missing
values itself.  Either way the outputs must not change.
"""
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import synth
from gpu_util import announce, gpu_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def same(a, b):
    return a.dtype == b.dtype and a.shape == b.shape and torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_two_streams_match_sequential(dev):
    w, _ = synth.moe_weights_bf16(experts=64, rows=512, cols=1024, seed=11, with_grad=False)
    t, s = synth.logits_bf16(tokens=512, vocab=65536, seed=12)
    w, t, s = w.to(dev), t.to(dev), s.to(dev)
    ws_q = q.workspace(q.QAD_OP_QUANTIZE, *w.shape, dev)
    ws_k = q.workspace(q.QAD_OP_KL_TOPK, 1, *t.shape, dev)
    announce("concurrency: sequential reference")
    ref_q = q.nvfp4_quantize(w, ws=ws_q)
    ref_k = q.qad_kl_topk_fwd_bwd(t, s, 1000, row_loss=True, ws=ws_k)
    ref_kl = q.qad_kl_fwd_bwd(t, s, row_loss=True)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    for rep in range(3):
        announce("concurrency: two streams, round %d" % rep)
        sa.wait_stream(torch.cuda.current_stream(dev))
        sb.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(sa):
            out_q = q.nvfp4_quantize(w, ws=ws_q)
            out_kl = q.qad_kl_fwd_bwd(t, s, row_loss=True)
        with torch.cuda.stream(sb):
            out_k = q.qad_kl_topk_fwd_bwd(t, s, 1000, row_loss=True, ws=ws_k)
        torch.cuda.synchronize()
        for a, b in zip(out_q, ref_q):
            assert same(a, b), ("quantize", rep)
        for a, b in zip(out_k, ref_k):
            assert same(a, b), ("top-k KL", rep)
        for a, b in zip(out_kl, ref_kl):
            assert same(a, b), ("KL", rep)
