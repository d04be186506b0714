"""The bounded waits of the one-pass kernels and what follows a wait that
gives up.

The dynamic quantizers exchange chunk maxima between the workgroups of a
tensor, and the KL segment kernels exchange per-segment row statistics; a
workgroup that waits longer than the bound (qad_set_wait_limit_us) computes
what it waited for from the inputs itself, with the same arithmetic.  With
the bound set to 0 every wait that does not find its data on the first look
gives up at once, so those paths run for most workgroups (forced from the
host; every kernel still ends normally).  Every output must equal the
normal path's bit for bit.
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


def run_all(w, t, s):
    out = []
    out += list(q.nvfp4_quantize(w))                    # one pass: 16 chunks per tensor
    out.append(q.nvfp4_qdq_fwd(w))
    out += list(q.fp8_quantize(w))
    for tt, ss in ((t, s), (t.float(), s.float())):      # 3 record segments per row
        out += list(q.qad_kl_fwd_bwd(tt, ss, row_loss=True))
        out += list(q.qad_kl_topk_fwd_bwd(tt, ss, 300, row_loss=True))
        out += list(q.qad_kl_topp_fwd_bwd(tt, ss, 0.9, row_loss=True, tau=True))
    return [o for o in out if o is not None]


def test_wait_fallbacks_bit_identical(dev):
    w, _ = synth.moe_weights_bf16(experts=8, rows=256, cols=1024, seed=7, with_grad=False)
    t, s = synth.logits_bf16(tokens=24, vocab=40000, seed=8)
    w, t, s = w.to(dev), t.to(dev), s.to(dev)
    announce("fallback: normal path")
    ref = run_all(w, t, s)
    torch.cuda.synchronize()
    prev = q.set_wait_limit_us(0)
    try:
        announce("fallback: every wait gives up at once")
        got = run_all(w, t, s)
        torch.cuda.synchronize()
    finally:
        q.set_wait_limit_us(prev)
    assert prev == 20000 and q.set_wait_limit_us(-1) == 20000
    assert len(got) == len(ref)
    for i, (a, b) in enumerate(zip(got, ref)):
        assert a.dtype == b.dtype and a.shape == b.shape, i
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (i, tuple(a.shape), a.dtype)


def test_wait_fallbacks_many_subgroups_and_segments(dev):
    # tensors of many 16-chunk sub-groups with a ragged last chunk (bf16 and
    # fp32), and logit rows of 9 segments with a ragged last one: the
    # cooperative fallbacks claim and scan sub-groups / segments from several
    # workgroups at once; results must not change
    w, _ = synth.moe_weights_bf16(experts=3, rows=1000, cols=4112, seed=9, with_grad=False)
    t, s = synth.logits_bf16(tokens=16, vocab=131072 + 8, seed=10)
    w, t, s = w.to(dev), t.to(dev), s.to(dev)

    def run():
        out = list(q.nvfp4_quantize(w)) + list(q.nvfp4_quantize(w.float()))
        out += list(q.fp8_quantize(w))
        out += list(q.qad_kl_fwd_bwd(t, s, row_loss=True))
        out += list(q.qad_kl_topk_fwd_bwd(t, s, 4096, row_loss=True))
        return [o for o in out if o is not None]

    announce("fallback many sub-groups: normal path")
    ref = run()
    torch.cuda.synchronize()
    prev = q.set_wait_limit_us(0)
    try:
        announce("fallback many sub-groups: every wait gives up at once")
        got = run()
        torch.cuda.synchronize()
    finally:
        q.set_wait_limit_us(prev)
    assert len(got) == len(ref)
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (i, tuple(a.shape), a.dtype)
