#!/usr/bin/env python3
"""Benchmark of the QAD hot path on one MI355X.

One step runs every step of the hot path once over synthetic inputs resident
in HBM, in the launch configuration the parity tests check:
  moe   : dynamic NVFP4 QDQ forward of 128 expert matrices 2048 x 4096 bf16
          (N(0,0.02^2), 16 outlier input columns x20 per expert) + the
          straight-through backward of a bf16 N(0,(1e-3)^2) gradient;
  act   : W4A4 activation QDQ forward of 32768 x 4096 bf16 (Student-t nu=3,
          8 outlier channels x30; amax recomputed each call) + STE backward;
  mse   : MSE calibration of an 8192 x 8192 bf16 N(0,0.02^2) weight (64
          candidates amax*k/6, k in [0.5, 1]) + QDQ with the frozen scales;
  kl    : KL(teacher || student) loss (mean, fp32) + bf16 gradient over 8192
          tokens x 131072 vocabulary, teacher N(0,3^2), student = teacher +
          N(0,0.5^2), T = 1.
`value` is the step's algorithmic HBM bytes (every input read once, every
output written once) divided by the step time.  Per-part times come from HIP
events recorded on the stream the kernels run on.  The smallest configuration
(one fp32 256 x 1024 tensor) is timed on its own, in microseconds.  The CPU
baseline times the CPU oracle, single-threaded and on all host cores, on a
bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 QDQ GB/s and KL fwd+bwd tokens/s, % of HBM roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
GiB = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-fraction", type=float, default=0.25,
                    help="share of one step the CPU-oracle baseline runs (every part in proportion)")
    return ap.parse_args()


class phase:
    """Marks one part of the run as a named ROCTX range (torch.cuda.nvtx maps
    to ROCTX on ROCm), the device synchronised before the range closes, so
    that a kernel trace taken with rocprofv3 --marker-trace can assign every
    dispatch to the part that issued it."""

    def __init__(self, name):
        self.name = name

    def __enter__(self):
        import torch
        torch.cuda.synchronize()
        torch.cuda.nvtx.range_push(self.name)
        return self

    def __exit__(self, *exc):
        import torch
        torch.cuda.synchronize()
        torch.cuda.nvtx.range_pop()
        return False


def ensure_built():
    from nvfp4_quantization_aware_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from nvfp4_quantization_aware_amd import build
        build.build()


class Workload:
    """Inputs, outputs and workspaces of one step, allocated once."""

    def __init__(self, dev):
        import torch
        import nvfp4_quantization_aware_amd as q
        from nvfp4_quantization_aware_amd import synth
        self.q = q
        E, R2, C2 = 128, 2048, 4096
        T3, H3 = 32768, 4096
        R4 = C4 = 8192
        N5, V5 = 8192, 131072
        self.shapes = dict(moe=(E, R2, C2), act=(T3, H3), mse=(R4, C4), kl=(N5, V5))
        self.w2, self.g2 = synth.moe_weights_bf16(E, R2, C2, seed=2, device=dev)
        x3, self.g3 = synth.student_t_activations_bf16(T3, H3, seed=3, device=dev)
        self.x3 = x3.unsqueeze(0)
        self.w4 = synth.gaussian_weight_bf16(R4, C4, seed=4, device=dev).unsqueeze(0)
        self.t5, self.s5 = synth.logits_bf16(N5, V5, seed=5, device=dev)
        bf = torch.bfloat16
        self.y2 = torch.empty_like(self.w2)
        self.gx2 = torch.empty_like(self.g2)
        self.y3 = torch.empty_like(self.x3)
        self.gx3 = torch.empty_like(self.g3)
        self.sc4 = torch.empty((1, R4, C4 // 16), dtype=torch.uint8, device=dev)
        self.ts4 = torch.empty(1, dtype=torch.float32, device=dev)
        self.y4 = torch.empty_like(self.w4)
        self.l5 = torch.empty(1, dtype=torch.float32, device=dev)
        self.gr5 = torch.empty((N5, V5), dtype=bf, device=dev)
        self.ws2 = q.workspace(q.QAD_OP_QUANTIZE, E, R2, C2, dev)
        self.ws3 = q.workspace(q.QAD_OP_QUANTIZE, 1, T3, H3, dev)
        self.ws4 = q.workspace(q.QAD_OP_MSE_CALIBRATE, 1, R4, C4, dev)
        self.ws5 = q.workspace(q.QAD_OP_KL, 1, N5, V5, dev)
        n2, n3, n4, n5 = E * R2 * C2, T3 * H3, R4 * C4, N5 * V5
        # algorithmic bytes: each input read once, each output written once
        self.bytes = {
            "moe_qdq_fwd": 2 * n2 + 2 * n2,
            "moe_ste_bwd": 2 * n2 + 2 * n2,
            "act_qdq_fwd": 2 * n3 + 2 * n3,
            "act_ste_bwd": 2 * n3 + 2 * n3,
            "mse_calibrate": 2 * n4 + n4 // 16,
            "mse_frozen_qdq": 2 * n4 + n4 // 16 + 2 * n4,
            "kl_fwd_bwd": 2 * n5 + 2 * n5 + 2 * n5,
        }
        self.parts = list(self.bytes)

    def step(self, ev=None):
        q = self.q
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        q.nvfp4_qdq_fwd(self.w2, y=self.y2, ws=self.ws2)
        rec(1)
        q.nvfp4_qdq_bwd(self.g2, self.gx2)
        rec(2)
        q.nvfp4_qdq_fwd(self.x3, y=self.y3, ws=self.ws3)
        rec(3)
        q.nvfp4_qdq_bwd(self.g3, self.gx3)
        rec(4)
        q.nvfp4_mse_calibrate(self.w4, scales_out=self.sc4, tscale_out=self.ts4, ws=self.ws4)
        rec(5)
        q.nvfp4_qdq_fwd(self.w4, self.sc4, self.ts4, y=self.y4)
        rec(6)
        q.qad_kl_fwd_bwd(self.t5, self.s5, loss_out=self.l5, grad=self.gr5, ws=self.ws5)
        rec(7)


def kernel_source_digest() -> str:
    """sha256 of the KL kernels' sources as code: comments removed and
    whitespace collapsed, so that only a change to the code itself counts."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "nvfp4_quantization_aware_amd", "csrc")
    parts = []
    for n in ("kl_kernels.hip", "qad_device.h", "qad_internal.h"):
        t = open(os.path.join(csrc, n)).read()
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        parts.append(" ".join(t.split()).encode())
    return hashlib.sha256(b"".join(parts)).hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the kernel's code changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "kl_seg_bf16_kernel_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel") != kernel or rec.get("code_sha256") != kernel_source_digest():
        return None
    return rec["traffic_bytes"]


def _host_cpu():
    """CPU model and logical CPU count of the host the oracle ran on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def cpu_baseline(fraction: float):
    """The CPU oracle on `fraction` of one step (the same share of every part,
    so its GB/s compares directly with the GPU step): single-threaded, then
    the same oracle functions with OpenMP over tensors / rows on every host
    core (oracle/oracle_omp.c).  Also the KL in binary32 (the oracle's timing
    variant), one core and all cores, on a sample of the KL rows."""
    import numpy as np
    import oracle
    from nvfp4_quantization_aware_amd import synth
    oracle.build(force=False)
    bits = synth.bf16_bits
    experts = max(1, round(128 * fraction))
    rows3 = max(16, round(32768 * fraction))
    rows4 = max(16, round(8192 * fraction))
    rows5 = max(2, round(8192 * fraction))
    rows_f32 = max(2, rows5 // 8)
    one, omp = {}, {}

    def timed(store, name, fn, nbytes):
        t0 = time.perf_counter()
        r = fn()
        store[name] = (time.perf_counter() - t0, nbytes)
        return r

    w, g = synth.moe_weights_bf16(experts, 2048, 4096, seed=2)
    w, g = bits(w), bits(g)

    def moe_fwd():
        for e in range(experts):
            oracle.nvfp4_quantize(w[e])

    timed(one, "moe_qdq_fwd", moe_fwd, 4 * w.size)
    timed(one, "moe_ste_bwd", lambda: np.copy(g), 4 * g.size)   # the oracle's STE is the identity
    timed(omp, "moe_qdq_fwd", lambda: oracle.omp_quantize_batch(w), 4 * w.size)
    timed(omp, "moe_ste_bwd", lambda: np.copy(g), 4 * g.size)
    del w, g
    x, g3 = synth.student_t_activations_bf16(rows3, 4096, seed=3)
    x, g3 = bits(x), bits(g3)
    timed(one, "act_qdq_fwd", lambda: oracle.nvfp4_quantize(x), 4 * x.size)
    timed(one, "act_ste_bwd", lambda: np.copy(g3), 4 * g3.size)
    timed(omp, "act_qdq_fwd", lambda: oracle.omp_quantize_tensor(x), 4 * x.size)
    timed(omp, "act_ste_bwd", lambda: np.copy(g3), 4 * g3.size)
    del x, g3
    w4 = bits(synth.gaussian_weight_bf16(rows4, 8192, seed=4))
    b_cal, b_qdq = 2 * w4.size + w4.size // 16, 2 * w4.size + w4.size // 16 + 2 * w4.size
    sc, ts = timed(one, "mse_calibrate", lambda: oracle.mse_calibrate(w4), b_cal)
    timed(one, "mse_frozen_qdq", lambda: oracle.nvfp4_quantize(w4, sc, ts), b_qdq)
    sc, ts = timed(omp, "mse_calibrate", lambda: oracle.omp_mse_calibrate(w4), b_cal)
    timed(omp, "mse_frozen_qdq", lambda: oracle.omp_quantize_tensor(w4, sc, ts), b_qdq)
    del w4
    t5, s5 = synth.logits_bf16(rows5, 131072, seed=5)
    t5, s5 = bits(t5), bits(s5)
    timed(one, "kl_fwd_bwd", lambda: oracle.kl_fwd_bwd(t5, s5, grad_scale=1.0 / 8192), 6 * t5.size)
    timed(omp, "kl_fwd_bwd", lambda: oracle.omp_kl_fwd_bwd(t5, s5, grad_scale=1.0 / 8192), 6 * t5.size)
    kl32 = {}
    timed(kl32, "one", lambda: oracle.kl_fwd_bwd_f32(t5[:rows_f32], s5[:rows_f32], grad_scale=1.0 / 8192), 0)
    timed(kl32, "omp", lambda: oracle.omp_kl_fwd_bwd_f32(t5, s5, grad_scale=1.0 / 8192), 0)

    def rate(store):
        secs = sum(t for t, _ in store.values())
        return secs, sum(b for _, b in store.values()) / secs / 1e9

    secs1, gbs1 = rate(one)
    secs_n, gbs_n = rate(omp)
    cores = oracle.omp_threads()
    return {
        "value": round(gbs1, 4),
        "unit": "GB/s",
        "cores": 1,
        "host": _host_cpu(),
        "kind": "oracle",
        "seconds": round(secs1, 2),
        "part_seconds": {k: round(v[0], 3) for k, v in one.items()},
        "kl_tokens_per_s": round(rows5 / one["kl_fwd_bwd"][0], 2),
        "all_cores": {"value": round(gbs_n, 4), "unit": "GB/s", "cores": cores, "kind": "oracle (OpenMP)",
                      "seconds": round(secs_n, 2), "part_seconds": {k: round(v[0], 3) for k, v in omp.items()},
                      "kl_tokens_per_s": round(rows5 / omp["kl_fwd_bwd"][0], 2)},
        "kl_binary32": {"tokens_per_s_1_core": round(rows_f32 / kl32["one"][0], 2),
                        "tokens_per_s_all_cores": round(rows5 / kl32["omp"][0], 2), "cores": cores,
                        "rows": {"1_core": rows_f32, "all_cores": rows5}},
        "sample": ("1/%d of one step, every part in proportion: %d of 128 experts QDQ + STE copy, %d of "
                   "32768 activation rows QDQ + STE copy, %d of 8192 rows MSE calibration + frozen QDQ, "
                   "%d of 8192 KL rows fwd+bwd (binary64); same generators and seeds as the GPU workload; "
                   "binary32 KL on %d rows (1 core) and %d rows (all cores)"
                   % (round(1 / fraction), experts, rows3, rows4, rows5, rows_f32, rows5)),
    }


def time_c1(dev, iters=200):
    """The smallest configuration: dynamic NVFP4 quantization of one fp32
    256 x 1024 tensor (N(0,1), 0.1% outliers x50) emitting packed codes,
    block scales, the tensor scale and bf16 values.  1.7 MB of traffic takes
    about 0.2 us at peak bandwidth, so the call is bound by launch latency:
    reported in microseconds (median of single timed calls, the mean of
    back-to-back calls, and per call of a HIP graph of 20 calls replayed) and
    GB/s, outside the step's value."""
    import torch
    import nvfp4_quantization_aware_amd as q
    from nvfp4_quantization_aware_amd import synth
    x = synth.outlier_tensor_f32(256, 1024, seed=1, device=dev).unsqueeze(0)
    n = x.numel()
    codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(n // 16, dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    y = torch.empty(n, dtype=torch.bfloat16, device=dev)
    ws = q.workspace(q.QAD_OP_QUANTIZE, 1, 256, 1024, dev)
    f = lambda: q.nvfp4_quantize(x, codes=codes, scales_out=scales, tscale_out=ts, y=y, ws=ws)
    for _ in range(5):
        f()
    torch.cuda.synchronize()
    singles = []
    for _ in range(50):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        f()
        e1.record()
        torch.cuda.synchronize()
        singles.append(e0.elapsed_time(e1) * 1e3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        f()
    e1.record()
    torch.cuda.synchronize()
    mean_us = e0.elapsed_time(e1) * 1e3 / iters
    med_us = sorted(singles)[len(singles) // 2]
    # the same calls captured once into a HIP graph and replayed: the GPU-side
    # time per call without the host's launch overhead
    per_graph = 20
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        f()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            f()
    graph.replay()
    torch.cuda.synchronize()
    reps = 10
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
    nbytes = 4 * n + n // 2 + n // 16 + 4 + 2 * n
    return {"shape": [256, 1024], "dtype": "f32", "bytes": nbytes, "us_median_single": round(med_us, 2),
            "us_mean_back_to_back": round(mean_us, 2), "us_per_call_graph_replay": round(graph_us, 2),
            "GB/s": round(nbytes / (med_us * 1e-6) / 1e9, 1),
            "GB/s_graph_replay": round(nbytes / (graph_us * 1e-6) / 1e9, 1), "bound": "launch latency"}


def time_wait0(wl, iters=5):
    """The one-pass kernels with every device-side wait giving up at once
    (qad_set_wait_limit_us(0)): what the exact fallbacks cost when other work
    keeps workgroups from being resident together.  The MoE QDQ forward and
    the KL forward + backward of the step, next to their normal times."""
    import torch
    q = wl.q
    calls = {"moe_qdq_fwd": lambda: q.nvfp4_qdq_fwd(wl.w2, y=wl.y2, ws=wl.ws2),
             "kl_fwd_bwd": lambda: q.qad_kl_fwd_bwd(wl.t5, wl.s5, loss_out=wl.l5, grad=wl.gr5, ws=wl.ws5)}
    out = {}
    for name, f in calls.items():
        res = {}
        for label, limit in (("normal_ms", None), ("wait0_ms", 0)):
            prev = q.set_wait_limit_us(limit) if limit is not None else None
            try:
                f()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(iters):
                    f()
                e1.record()
                torch.cuda.synchronize()
            finally:
                if prev is not None:
                    q.set_wait_limit_us(prev)
            res[label] = round(e0.elapsed_time(e1) / iters, 4)
        res["ratio"] = round(res["wait0_ms"] / res["normal_ms"], 3)
        out[name] = res
    return out


def act_accountings(parts):
    """The activation path (forward QDQ + straight-through backward) under its
    two byte accountings: each tensor read or written once (1 GiB), and with
    the amax pass's second read of the 256 MiB input counted (1.25 GiB)."""
    ms = parts["act_qdq_fwd"]["ms"] + parts["act_ste_bwd"]["ms"]
    uniq = parts["act_qdq_fwd"]["bytes"] + parts["act_ste_bwd"]["bytes"]
    reread = uniq + parts["act_qdq_fwd"]["bytes"] // 2
    out = {"ms": round(ms, 4)}
    for name, b in (("unique_1GiB", uniq), ("with_amax_reread_1.25GiB", reread)):
        gbs = b / (ms * 1e-3) / 1e9
        out[name] = {"bytes": b, "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def time_topk(wl, dev, k=4096, iters=10):
    """Teacher-top-k KL (k = 4096, the pages' run) on the same 8192 x 131072
    logits, timed on its own after the step (not part of the step's value)."""
    import torch
    q = wl.q
    N5, V5 = wl.shapes["kl"]
    ws = q.workspace(q.QAD_OP_KL_TOPK, 1, N5, V5, dev)
    print("[bench] top-k KL", file=sys.stderr, flush=True)
    for _ in range(2):
        q.qad_kl_topk_fwd_bwd(wl.t5, wl.s5, k, loss_out=wl.l5, grad=wl.gr5, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        q.qad_kl_topk_fwd_bwd(wl.t5, wl.s5, k, loss_out=wl.l5, grad=wl.gr5, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = 6 * N5 * V5
    return {"k": k, "ms": round(ms, 4), "tokens_per_s": round(N5 / (ms * 1e-3), 1),
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes": nbytes, "iters": iters}


def time_fp8(wl, iters=10):
    """FP8 (E4M3) per-tensor QDQ forward with dynamic scales on the MoE weight
    batch (one pass, per-expert scales) and on the activation tensor (amax
    pass first), timed on their own after the step."""
    import torch
    q = wl.q
    res = {}
    for name, x, y, ws in (("fp8_qdq_fwd_moe", wl.w2, wl.y2, wl.ws2), ("fp8_qdq_fwd_act", wl.x3, wl.y3, wl.ws3)):
        B = x.shape[0] if x.dim() == 3 else 1
        ts = torch.empty(B, dtype=torch.float32, device=x.device)
        for _ in range(2):
            q.fp8_quantize(x, codes=None, y=y, tscale_out=ts, ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            q.fp8_quantize(x, codes=None, y=y, tscale_out=ts, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        nbytes = 4 * x.numel()
        res[name] = {"shape": list(x.shape), "ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": nbytes}
    return res


def time_topp(wl, dev, top_p=0.9, iters=10):
    """Teacher-top-p (nucleus) KL on the same 8192 x 131072 logits: thresholds
    (three streaming reads of the teacher) then the masked one-pass KL, timed
    on its own after the step."""
    import torch
    q = wl.q
    N5, V5 = wl.shapes["kl"]
    ws = q.workspace(q.QAD_OP_KL_TOPP, 1, N5, V5, dev)
    print("[bench] top-p KL", file=sys.stderr, flush=True)
    for _ in range(2):
        q.qad_kl_topp_fwd_bwd(wl.t5, wl.s5, top_p, loss_out=wl.l5, grad=wl.gr5, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        q.qad_kl_topp_fwd_bwd(wl.t5, wl.s5, top_p, loss_out=wl.l5, grad=wl.gr5, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = 6 * N5 * V5
    return {"top_p": top_p, "ms": round(ms, 4), "tokens_per_s": round(N5 / (ms * 1e-3), 1),
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes": nbytes, "iters": iters}


def time_clipped_ste(wl, iters=10):
    """Clipped straight-through backward on the MoE weight batch with the
    forward's dynamic scales (taken once before timing): reads grad_y and x
    (2 B each per element) and the block scales (1/16 B), writes grad_x
    (2 B), timed on its own after the step."""
    import torch
    q = wl.q
    w, g, gx = wl.w2, wl.g2, wl.gx2
    _, scales, ts, _ = q.nvfp4_quantize(w, codes=False, y=False, ws=wl.ws2)
    for _ in range(2):
        q.nvfp4_qdq_bwd_clipped(g, w, scales, ts, grad_x=gx)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        q.nvfp4_qdq_bwd_clipped(g, w, scales, ts, grad_x=gx)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = 6 * w.numel() + w.numel() // 16
    return {"shape": list(w.shape), "ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": nbytes}


def time_sgd_step(wl, iters=10):
    """Frozen-scale SGD step on the MoE weight batch, the clipped
    straight-through gradient fused in (scales: the forward's, taken once
    before timing): reads w and its gradient (2 B each per element) and the
    block scales (1/16 B), writes the stepped weights (2 B) out of place, so
    every timed call does the same work."""
    import torch
    q = wl.q
    w, g, wo = wl.w2, wl.g2, wl.gx2
    _, scales, ts, _ = q.nvfp4_quantize(w, codes=False, y=False, ws=wl.ws2)
    for _ in range(2):
        q.nvfp4_frozen_sgd_step(w, g, scales, ts, 5e-6, 1.0, w_out=wo)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        q.nvfp4_frozen_sgd_step(w, g, scales, ts, 5e-6, 1.0, w_out=wo)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = 6 * w.numel() + w.numel() // 16
    return {"shape": list(w.shape), "lr": 5e-6, "clip_coef": 1.0, "ms": round(ms, 4),
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": nbytes}


def time_linear(wl, dev, iters=10):
    """W4A4 fake-quant linear of one MoE expert's projection: 8192 tokens of the
    activation workload (x [8192, 4096]) times expert 0 of the MoE weights
    (w [2048, 4096]); forward (both QDQ passes + the bf16 MFMA product) and
    straight-through backward (two products), timed on their own."""
    import torch
    q = wl.q
    x = wl.x3[0, :8192]
    w = wl.w2[0]
    M, K = x.shape
    N = w.shape[0]
    ws = q.workspace(q.QAD_OP_W4A4_LINEAR, M, N, K, dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    xq = torch.empty(q.nvfp4_packed_bytes(M, K), dtype=torch.uint8, device=dev)
    wq = torch.empty(q.nvfp4_packed_bytes(N, K), dtype=torch.uint8, device=dev)
    gy = torch.empty((M, N), dtype=torch.bfloat16, device=dev).normal_(0, 1e-3)
    gx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    res = {"shape_MNK": [M, N, K], "peak_TFLOPs_bf16": 2500.0}
    for name, f, flops in (("fwd", lambda: q.qad_w4a4_linear_fwd(x, w, y=y, xq=xq, wq=wq, ws=ws), 2 * M * N * K),
                           ("bwd", lambda: q.qad_w4a4_linear_bwd(gy, xq, wq, K, grad_x=gx, grad_w=gw),
                            4 * M * N * K)):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        res[name] = {"ms": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
                     "frac_mfma_bf16": round(flops / (ms * 1e-3) / 1e12 / 2500.0, 4)}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: every part of this hot path runs on a single MI355X "
              "(per-expert tensors and token rows are independent; see the sharding notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    ensure_built()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    wl = Workload(dev)
    torch.cuda.synchronize()
    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    with phase("warmup"):
        for _ in range(args.warmup):
            wl.step()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(K)]
    print("[bench] timing %d steps" % K, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    with phase("timed_steps"):
        wall0 = time.perf_counter()
        t_start.record()
        for k in range(K):
            wl.step(evs[k])
        t_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / K
    part_ms = {}
    for i, name in enumerate(wl.parts):
        part_ms[name] = sum(evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(K)) / K
    total_bytes = sum(wl.bytes.values())
    parts = {}
    for name in wl.parts:
        gbs = wl.bytes[name] / (part_ms[name] * 1e-3) / 1e9
        parts[name] = {"ms": round(part_ms[name], 4), "bytes": wl.bytes[name], "GB/s": round(gbs, 1),
                       "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    dom = max(wl.parts, key=lambda n: part_ms[n])
    dom_gbs = wl.bytes[dom] / (part_ms[dom] * 1e-3) / 1e9
    kl_tokens_s = wl.shapes["kl"][0] / (part_ms["kl_fwd_bwd"] * 1e-3)
    qdq_bytes = sum(wl.bytes[n] for n in wl.parts if n != "kl_fwd_bwd")
    qdq_ms = sum(part_ms[n] for n in wl.parts if n != "kl_fwd_bwd")
    out = {
        "metric": METRIC,
        "value": round(total_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "qad_hot_path_step: moe 128x2048x4096 bf16 dynamic QDQ fwd + STE bwd; "
                        "act 32768x4096 bf16 dynamic QDQ fwd + STE bwd; mse 8192x8192 bf16 "
                        "64-candidate calibration + frozen QDQ; kl 8192x131072 bf16 fwd+bwd T=1",
            "storage": "bf16 in/out, e2m1+e4m3 scales, fp32 tensor scales",
            "bytes_per_step": total_bytes,
            "parallelism": "single GPU",
        },
        "frac_hbm_step": round(total_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        # the same ratio against what a plain copy reaches on this machine (the
        # straight-through copy of the 2 GiB MoE gradient in the same steps)
        "frac_of_measured_copy": round(total_bytes / (ms_step * 1e-3) / 1e9 / parts["moe_ste_bwd"]["GB/s"], 4),
        "nvfp4_qdq_GBps": round(qdq_bytes / (qdq_ms * 1e-3) / 1e9, 1),
        "kl_tokens_per_s": round(kl_tokens_s, 1),
        "parts": parts,
        "act_fwd_bwd": act_accountings(parts),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("kl_seg_bf16_kernel<1, false>") if dom == "kl_fwd_bwd" else None},
        "wall_s_timed": round(wall, 3),
    }
    ext = {}
    for name, fn in (("kl_topk_fwd_bwd", lambda: time_topk(wl, dev)), ("kl_topp_fwd_bwd", lambda: time_topp(wl, dev)),
                     ("fp8", lambda: time_fp8(wl)), ("w4a4_linear", lambda: time_linear(wl, dev)),
                     ("nvfp4_qdq_bwd_clipped_moe", lambda: time_clipped_ste(wl)),
                     ("nvfp4_frozen_sgd_step_moe", lambda: time_sgd_step(wl)),
                     ("c1_fp32_quantize_256x1024", lambda: time_c1(dev)), ("wait0_fallbacks", lambda: time_wait0(wl))):
        with phase(name):
            r = fn()
        if name == "fp8":
            ext.update(r)
        else:
            ext[name] = r
    out["extensions"] = ext
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args.cpu_fraction)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
