"""Every entry point captured in one HIP graph (torch.cuda.CUDAGraph) and
replayed: a training loop that captures its step replays the same launches
on the same buffers with new data in them.  The library launches only
kernels on the caller's stream (buffers are cleared by fill kernels, never by
memset nodes, and nothing synchronises or allocates inside a call), so each
replay must give exactly what an eager call gives on the same inputs.

Three replays, each after the inputs were refilled in place with new seeded
data and an eager pass on separate outputs and workspaces ran and was
synchronised; every output of every replay is compared with the eager one
bit for bit (the W4A4 linear's sums have a fixed order, so its products are
compared exactly as well).  Shapes take both
dynamic-scale paths (one pass with co-resident chunks; amax pass then coding
for a tensor too large for one pass), one-pass KL records over several
segments, and the top-k / top-p selection kernels together with their
redo kernels.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from gpu_util import announce, gpu_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


class Inputs:
    """Static input tensors, refilled in place from a seed."""

    def __init__(self, dev):
        bf = torch.bfloat16
        self.moe = torch.empty((3, 64, 1024), dtype=bf, device=dev)
        self.gmoe = torch.empty_like(self.moe)
        self.act = torch.empty((1, 16384, 4096), dtype=bf, device=dev)      # 128 MiB: amax pass, then coding
        self.w = torch.empty((2, 128, 512), dtype=bf, device=dev)
        self.f8 = torch.empty((2, 64, 520), dtype=torch.float32, device=dev)
        self.t = torch.empty((24, 40000), dtype=bf, device=dev)             # 3 record segments per row
        self.s = torch.empty_like(self.t)
        self.x = torch.empty((256, 512), dtype=bf, device=dev)
        self.wl = torch.empty((384, 512), dtype=bf, device=dev)
        self.gy = torch.empty((256, 384), dtype=bf, device=dev)

    def refill(self, seed):
        g = torch.Generator(device=self.moe.device)
        g.manual_seed(seed)
        for name, scale in (("moe", 0.02), ("gmoe", 1e-3), ("act", 1.0), ("w", 0.05), ("f8", 3.0), ("t", 3.0),
                            ("x", 1.0), ("wl", 0.05), ("gy", 1.0)):
            ten = getattr(self, name)
            ten.copy_(torch.randn(ten.shape, generator=g, device=ten.device) * scale)
        self.s.copy_(self.t.float() + 0.5 * torch.randn(self.t.shape, generator=g, device=self.t.device))
        self.t[5, :20000] = 1.5          # a plateau of 20000 tied teacher logits


KL_LOSS = 13   # index of the full-vocabulary KL loss in step()'s outputs


def step(inp: Inputs, ws):
    """Every entry point once; returns the list of output tensors."""
    out = []
    codes, scales, ts, y = q.nvfp4_quantize(inp.moe, ws=ws["moe"])
    out += [codes, scales, ts, y]
    out.append(q.nvfp4_qdq_bwd(inp.gmoe))
    out.append(q.nvfp4_qdq_bwd_clipped(inp.gmoe, inp.moe, scales, ts))
    out.append(q.nvfp4_qdq_fwd(inp.act, ws=ws["act"]))
    sc, tsw = q.nvfp4_mse_calibrate(inp.w, ws=ws["mse"])
    out += [sc, tsw, q.nvfp4_qdq_fwd(inp.w, sc, tsw)]
    out += list(q.fp8_quantize(inp.f8, ws=ws["fp8"]))
    out += list(q.qad_kl_fwd_bwd(inp.t, inp.s, row_loss=True, ws=ws["kl"]))
    out += list(q.qad_kl_topk_fwd_bwd(inp.t, inp.s, 300, grad_dtype=torch.float32, row_loss=True, ws=ws["topk"]))
    out += list(q.qad_kl_topp_fwd_bwd(inp.t, inp.s, 0.9, row_loss=True, tau=True, ws=ws["topp"]))
    y, xq, wq = q.qad_w4a4_linear_fwd(inp.x, inp.wl, ws=ws["lin"])
    out.append(y)
    # the packed operands' defined parts (their padding is never written)
    out += list(q.nvfp4_unpack(xq, *inp.x.shape)) + list(q.nvfp4_unpack(wq, *inp.wl.shape))
    out += list(q.qad_w4a4_linear_bwd(inp.gy, xq, wq, inp.x.shape[1]))
    return out


def workspaces(inp: Inputs, dev):
    return {
        "moe": q.workspace(q.QAD_OP_QUANTIZE, *inp.moe.shape, dev),
        "act": q.workspace(q.QAD_OP_QUANTIZE, *inp.act.shape, dev),
        "mse": q.workspace(q.QAD_OP_MSE_CALIBRATE, *inp.w.shape, dev),
        "fp8": q.workspace(q.QAD_OP_QUANTIZE, *inp.f8.shape, dev),
        "kl": q.workspace(q.QAD_OP_KL, 1, *inp.t.shape, dev),
        "topk": q.workspace(q.QAD_OP_KL_TOPK, 1, *inp.t.shape, dev),
        "topp": q.workspace(q.QAD_OP_KL_TOPP, 1, *inp.t.shape, dev),
        "lin": q.workspace(q.QAD_OP_W4A4_LINEAR, inp.x.shape[0], inp.wl.shape[0], inp.x.shape[1], dev),
    }


def test_graph_replays_match_eager(dev):
    announce("graph: inputs and an eager warm-up")
    inp = Inputs(dev)
    inp.refill(1)
    ws_graph, ws_eager = workspaces(inp, dev), workspaces(inp, dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step(inp, ws_graph)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    announce("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static = step(inp, ws_graph)
    torch.cuda.synchronize()
    losses = []
    for r, seed in enumerate((11, 12, 13)):
        announce("graph: replay %d (seed %d) against eager" % (r, seed))
        inp.refill(seed)
        eager = step(inp, ws_eager)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert len(eager) == len(static)
        for i, (a, b) in enumerate(zip(static, eager)):
            if a is None or b is None:
                assert a is None and b is None, i
                continue
            assert a.dtype == b.dtype and a.shape == b.shape, i
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (r, i, tuple(a.shape), a.dtype)
        losses.append(float(static[KL_LOSS].item()))
    # each replay computed on its own inputs, not on those of the capture
    assert len(set(losses)) == len(losses) and all(np.isfinite(losses)), losses
