#!/usr/bin/env python3
"""Benchmark of one fused-chain workload on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the fused chain over one batch of synthetic input (one
kernel launch: GEMM0 + epilogue + on-chip hand-off + GEMM1 + epilogue, or
conv + bias + ReLU + pool).  The headline workload (default: conv3x3 + ReLU +
2x2 max pool on x[32,112,112,60->64], the largest configuration) gives
`value`; the other configurations -- the tiny and register-resident two-GEMM
chains, the LDS-resident two-GEMM shape under the LDS-resident kernel, the
streamed variant and the profiler's choice, and the conv3x3 -> conv1x1 chain --
are measured in the same run and reported under `configs`.  Inputs are
resident in HBM before the timed region; the step rotates over enough copies of the activations and outputs
(> 2x the 256 MiB Infinity Cache) that every step reads its inputs from HBM.
Timing: HIP events on the stream the kernels run on (torch's current stream).

Prints ONE JSON line: throughput in TFLOP/s (algorithmic FLOPs), the roofline
position of the fused kernel, the unfused two-kernel baseline, and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12   # 2516.6: 256 CUs x 4096 fp16 FLOP/clk x 2.4 GHz (dense)
PEAK_HBM_GBS = 8000.0                          # HBM3E, 8 TB/s
RIDGE = PEAK_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
METRIC = "fused-chain TFLOP/s & % of fp16 MFMA peak; HBM bytes vs unfused"
COLD_BYTES = 640 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_src_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "gemm_conv_chain_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + f.read())
    return h.hexdigest()[:16]


class Problem:
    """Device buffers, step functions and the byte/FLOP model of one workload."""

    def __init__(self, name, cold=True, variant=None):
        import numpy as np
        import torch

        import gemm_conv_chain_amd as fc
        from gemm_conv_chain_amd import inputs

        self.fc, self.torch, self.np = fc, torch, np
        self.name = name
        self.bn = False
        self.traffic_key = name   # entry of the measured-traffic table
        self.spec, d = inputs.workload(name)
        self.host = d
        dev = torch.device("cuda:0")
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        s = self.spec
        if s["kind"] == "gemm2":
            M, K0, N0, N1 = s["M"], s["K0"], s["N0"], s["N1"]
            self.act = s["act"]
            self.flops = 2 * M * (K0 * N0 + N0 * N1)
            self.flops_exec = self.flops
            wbytes = 2 * (K0 * N0 + N0 + N0 * N1 + N1)
            self.bytes_fused = 2 * (M * K0 + M * N1) + wbytes
            self.bytes_interm = 2 * M * N0
            self.W = [t(d["W0"]), t(d["b0"]), t(d["W1"]), t(d["b1"])]
            per_set = 2 * (M * K0 + M * N1)
            self.nsets = max(1, math.ceil(COLD_BYTES / per_set)) if cold else 1
            A = t(d["A"])
            self.X = [A] + [A.clone() for _ in range(self.nsets - 1)]
            self.Y = [torch.empty((M, N1), dtype=torch.float16, device=dev) for _ in range(self.nsets)]
            self.H = torch.empty((M, N0), dtype=torch.float16, device=dev)
            default = "rf" if name != "b2b_gemm_lds" else "lds"
            if variant is None:
                variant = default
            if variant != default:
                self.traffic_key = name + "@" + variant
            self.config = {"workload": name, "M": M, "K0": K0, "N0": N0, "N1": N1, "act": self.act,
                           "variant": variant,
                           "dist": s["dist"] + "(-1,1)/sqrt(K)" if s["dist"] == "uniform" else "normal(0,1)/sqrt(K)"}
            self.kernel = {"rf": "k_chain_rf", "lds": "k_gemm_lds", "stream": "k_chain_stream"}[variant]
        elif s["kind"] == "gemmN":
            M, wd = s["M"], s["widths"]
            self.acts = s["acts"]
            self.flops = 2 * M * sum(wd[i] * wd[i + 1] for i in range(len(wd) - 1))
            self.flops_exec = self.flops
            wbytes = 2 * sum(wd[i] * wd[i + 1] + wd[i + 1] for i in range(len(wd) - 1))
            self.bytes_fused = 2 * (M * wd[0] + M * wd[-1]) + wbytes
            self.bytes_interm = 2 * M * sum(wd[1:-1])
            self.W = [t(x) for x in d["Ws"]] + [t(x) for x in d["bs"]]
            per_set = 2 * (M * wd[0] + M * wd[-1])
            self.nsets = max(1, math.ceil(COLD_BYTES / per_set)) if cold else 1
            A = t(d["A"])
            self.X = [A] + [A.clone() for _ in range(self.nsets - 1)]
            self.Y = [torch.empty((M, wd[-1]), dtype=torch.float16, device=dev) for _ in range(self.nsets)]
            self.Hs = [torch.empty((M, x), dtype=torch.float16, device=dev) for x in wd[1:-1]]
            self.config = {"workload": name, "M": M, "widths": wd, "acts": self.acts, "variant": "rf",
                           "dist": "uniform(-1,1)/sqrt(K)"}
            self.kernel = "k_chain_rf"
        elif s["kind"] == "conv2":
            n, h, w, c, k0, k1 = s["n"], s["h"], s["w"], s["c"], s["k0"], s["k1"]
            npix = n * h * w
            self.flops = 2 * npix * (9 * c * k0 + k0 * k1)
            self.flops_exec = self.flops
            wbytes = 2 * (9 * c * k0 + k0 + k0 * k1 + k1)
            self.bytes_fused = 2 * (npix * c + npix * k1) + wbytes
            self.bytes_interm = 2 * npix * k0
            self.W = [t(d["w0"]), t(d["b0"]), t(d["w1"]), t(d["b1"])]
            per_set = 2 * (npix * c + npix * k1)
            self.nsets = max(1, math.ceil(COLD_BYTES / per_set)) if cold else 1
            x = t(d["x"])
            self.X = [x] + [x.clone() for _ in range(self.nsets - 1)]
            self.Y = [torch.empty((n, h, w, k1), dtype=torch.float16, device=dev) for _ in range(self.nsets)]
            self.H = torch.empty((n, h, w, k0), dtype=torch.float16, device=dev)
            self.config = {"workload": name, "x": [n, h, w, c], "conv0": "3x3 s1 p1 %d->%d +b ReLU" % (c, k0),
                           "conv1": "1x1 %d->%d +b" % (k0, k1)}
            default = self.fc.conv2_auto_config(n, h, w, c, k0, k1)["variant"]
            self.conv_variant = variant or default
            if self.conv_variant != default:
                self.traffic_key = name + "@" + self.conv_variant
            self.config["variant"] = self.conv_variant
            self.kernel = "k_conv2_pipe" if self.conv_variant == "pipe" else "k_chain_rf"
        elif s["kind"] == "convN":
            n, h, w, c, ks = s["n"], s["h"], s["w"], s["c"], s["ks"]
            self.acts = s["acts"]
            npix = n * h * w
            chans = [9 * c] + ks
            self.flops = 2 * npix * sum(chans[i] * chans[i + 1] for i in range(len(ks)))
            self.flops_exec = self.flops
            wbytes = 2 * sum(chans[i] * chans[i + 1] + chans[i + 1] for i in range(len(ks)))
            self.bytes_fused = 2 * (npix * c + npix * ks[-1]) + wbytes
            self.bytes_interm = 2 * npix * sum(ks[:-1])
            self.W = [t(x) for x in d["ws"]] + [t(x) for x in d["bs"]]
            per_set = 2 * (npix * c + npix * ks[-1])
            self.nsets = max(1, math.ceil(COLD_BYTES / per_set)) if cold else 1
            x = t(d["x"])
            self.X = [x] + [x.clone() for _ in range(self.nsets - 1)]
            self.Y = [torch.empty((n, h, w, ks[-1]), dtype=torch.float16, device=dev) for _ in range(self.nsets)]
            self.Hs = [torch.empty((n, h, w, k), dtype=torch.float16, device=dev) for k in ks[:-1]]
            self.config = {"workload": name, "x": [n, h, w, c], "conv0": "3x3 s1 p1 %d->%d +b %s" % (c, ks[0], self.acts[0]),
                           "conv1x1": ["%d->%d +b %s" % (ks[i - 1], ks[i], self.acts[i]) for i in range(1, len(ks))]}
            default = self.fc.convN_auto_variant(n, h, w, c, ks)
            self.conv_variant = variant or default
            if self.conv_variant != default:
                self.traffic_key = name + "@" + self.conv_variant
            self.config["variant"] = self.conv_variant
            self.kernel = "k_conv2_pipe" if self.conv_variant == "pipe" else "k_chain_rf"
        else:
            n, h, w, c, cp, k = s["n"], s["h"], s["w"], s["c"], s["cpad"], s["k"]
            npix = n * h * w
            self.flops = 2 * npix * k * 9 * c               # algorithmic: the 60 real channels
            self.flops_exec = 2 * npix * k * 9 * cp         # executed: padded to 64
            npool = n * (h // 2) * (w // 2)
            self.bn = bool(s.get("bn"))
            self.pool = s.get("pool", "max2x2")
            self.bytes_fused = 2 * (npix * cp + 9 * cp * k + k + npool * k) + (2 * k if self.bn else 0)
            self.bytes_interm = 2 * npix * k
            xp = fc.pad_channels(t(d["x"]), cp)             # input preparation, outside the timed chain
            wp = fc.pad_weight_channels(t(d["w"]), cp)
            self.W = [wp, t(d["scale"]), t(d["shift"])] if self.bn else [wp, t(d["b"])]
            per_set = 2 * (npix * cp + npool * k)
            self.nsets = max(1, math.ceil(COLD_BYTES / per_set)) if cold else 1
            self.X = [xp] + [xp.clone() for _ in range(self.nsets - 1)]
            self.Y = [torch.empty((n, h // 2, w // 2, k), dtype=torch.float16, device=dev) for _ in range(self.nsets)]
            self.H = torch.empty((n, h, w, k), dtype=torch.float16, device=dev)
            self.conv_variant = variant or "auto"
            if variant:
                self.traffic_key = name + "@" + variant
            if variant == "winograd":
                if self.bn:
                    raise ValueError("the Winograd chain takes a bias, not a batch-norm scale")
                # weight transform once per weight tensor, outside the timed step (like the padding)
                self.U = fc.winograd_weights(wp)
                tiles = n * (h // 2) * (w // 2)
                self.flops_exec = 2 * tiles * 16 * cp * k   # 16 products per tile, channel and output channel
                self.flops_note = ("value and roofline count the direct convolution's %.2f GFLOP per launch; the "
                                   "Winograd kernel executes %.2f GFLOP on the matrix cores"
                                   % (self.flops / 1e9, self.flops_exec / 1e9))
            self.config = {"workload": name, "x": [n, h, w, c], "channels_padded_to": cp, "variant": self.conv_variant,
                           "conv": "3x3 s1 p1 %d->%d %s ReLU" % (c, k, "x scale + shift" if self.bn else "+b"),
                           "pool": ("avg" if self.pool == "avg2x2" else "max") + " 2x2 s2"}
            self.kernel = {"lds_weights": "k_conv_w", "winograd": "k_conv_pool_wino"}.get(variant, "k_conv_pool_wr")
        torch.cuda.synchronize()

    def step(self, i):
        fc, j, s = self.fc, i % self.nsets, self.spec
        if s["kind"] == "gemm2":
            W0, b0, W1, b1 = self.W
            fc.chain_gemm2(self.X[j], W0, b0, W1, b1, act=self.act, out=self.Y[j], variant=self.config["variant"])
        elif s["kind"] == "gemmN":
            n = len(self.acts)
            fc.chain_gemmN(self.X[j], self.W[:n], self.W[n:], self.acts, out=self.Y[j])
        elif s["kind"] == "conv2":
            w0, b0, w1, b1 = self.W
            rf = self.conv_variant == "rf"   # the register form at the full workload's rule: 8 waves, 2 stages
            fc.chain_conv2(self.X[j], w0, b0, w1, b1, act="relu", out=self.Y[j], variant=self.conv_variant,
                           waves=8 if rf else 0, stages=2 if rf else 0)
        elif s["kind"] == "convN":
            n = len(self.acts)
            fc.chain_convN(self.X[j], self.W[:n], self.W[n:], self.acts, out=self.Y[j], variant=self.conv_variant)
        elif self.bn:
            w, sc, sh = self.W
            fc.chain_conv_bn_pool(self.X[j], w, sc, sh, act="relu", pool="max2x2", out=self.Y[j],
                                  variant=self.conv_variant)
        elif self.conv_variant == "winograd":
            fc.chain_conv_pool_winograd(self.X[j], self.U, self.W[1], act="relu", pool=self.pool, out=self.Y[j])
        else:
            w, b = self.W
            fc.chain_conv_pool(self.X[j], w, b, act="relu", pool=self.pool, out=self.Y[j], variant=self.conv_variant)

    def step_unfused(self, i):
        """The two-kernel baseline: the intermediate goes to HBM and back."""
        fc, j, s = self.fc, i % self.nsets, self.spec
        if s["kind"] == "gemm2":
            W0, b0, W1, b1 = self.W
            fc.gemm_bias_act(self.X[j], W0, b0, act=self.act, out=self.H)
            fc.gemm_bias_act(self.H, W1, b1, act="none", out=self.Y[j])
        elif s["kind"] == "gemmN":
            n = len(self.acts)
            src = self.X[j]
            for k in range(n):
                dst = self.Hs[k] if k < n - 1 else self.Y[j]
                fc.gemm_bias_act(src, self.W[k], self.W[n + k], act=self.acts[k], out=dst)
                src = dst
        elif s["kind"] == "conv2":
            w0, b0, w1, b1 = self.W
            fc.conv_bias_act(self.X[j], w0, b0, act="relu", out=self.H)
            k0 = self.H.shape[-1]
            fc.gemm_bias_act(self.H.view(-1, k0), w1, b1, act="none", out=self.Y[j].view(-1, self.Y[j].shape[-1]))
        elif s["kind"] == "convN":
            n = len(self.acts)
            fc.conv_bias_act(self.X[j], self.W[0], self.W[n], act=self.acts[0], out=self.Hs[0])
            for k in range(1, n):
                src = self.Hs[k - 1]
                dst = self.Hs[k] if k < n - 1 else self.Y[j]
                fc.gemm_bias_act(src.view(-1, src.shape[-1]), self.W[k], self.W[n + k], act=self.acts[k],
                                 out=dst.view(-1, dst.shape[-1]))
        elif self.bn:
            w, sc, sh = self.W
            fc.chain_conv_bn_pool(self.X[j], w, sc, sh, act="relu", pool="none", out=self.H)
            fc.maxpool2x2(self.H, out=self.Y[j])
        else:
            w, b = self.W
            fc.conv_bias_act(self.X[j], w, b, act="relu", out=self.H)
            if self.pool == "avg2x2":
                fc.avgpool2x2(self.H, out=self.Y[j])
            else:
                fc.maxpool2x2(self.H, out=self.Y[j])


WARMUP_SECONDS = 0.25


def time_steps(torch, fn, steps, warmup, warmup_seconds=None):
    """Time `steps` launches of fn (one fused step each) after `warmup` eager ones.

    The timed steps are captured once into a HIP graph and replayed on the
    stream the kernels run on, bracketed by synchronisation and two HIP events:
    the GPU then runs the steps back to back, so elapsed / steps is the mean
    duration of one step as the device executes it (what the kernel trace
    reports), with no host launch gaps in between.  Each step still reads its
    own rotating buffer set.  Before the timed replay the graph is replayed
    untimed for at least `warmup_seconds` (default WARMUP_SECONDS): an idle GPU
    starts at low clocks and takes a fraction of a second of work to reach the
    clocks it runs at under load (measured: the first 1.7 ms replay of the
    conv+pool chain ran ~18% slower than the following ones).  Returns (ms per
    step, mean ms per launch, wall ms per step, method)."""
    if warmup_seconds is None:
        warmup_seconds = WARMUP_SECONDS
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(warmup + i)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        g.replay()                      # untimed replays: graph upload, clocks up
        torch.cuda.synchronize()
        while time.perf_counter() - w0 < warmup_seconds:
            g.replay()
            torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w0) * 1e3 / steps
        ms = t0.elapsed_time(t1) / steps
        return ms, ms, wall, "hip-graph"
    except Exception as e:  # capture unsupported: eager launches, one event pair each
        log("graph capture failed (%s); timing eager launches" % e)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    w0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        ev[i][0].record()
        fn(warmup + i)
        ev[i][1].record()
    t1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - w0) * 1e3 / steps
    per = [a.elapsed_time(b) for a, b in ev]
    return t0.elapsed_time(t1) / steps, sum(per) / len(per), wall, "eager"


def cpu_baseline(prob, seconds):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    s, d = prob.spec, prob.host
    cores = oracle.num_threads()
    actk = {"relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH, "none": oracle.ACT_NONE,
            "hardswish": oracle.ACT_HARDSWISH}
    if s["kind"] in ("gemm2", "gemmN"):
        M = s["M"]
        per_row = prob.flops / M

        def run(rows):
            t = time.perf_counter()
            if s["kind"] == "gemm2":
                oracle.chain_gemm2(d["A"][:rows], d["W0"], d["b0"], actk[s["act"]], d["W1"], d["b1"])
            else:
                oracle.chain_gemmN(d["A"][:rows], d["Ws"], d["bs"], [actk[a] for a in s["acts"]])
            return time.perf_counter() - t

        probe = min(M, 2048)
        tp = run(probe)
        rows = int(min(M, max(probe, probe * seconds / max(tp, 1e-6))))
        t = run(rows) if rows != probe else tp
        passes = 1
        if rows == M:   # the whole workload is quick: repeat it for a stable time (up to ~2 s)
            while t < min(seconds, 2.0) and passes < 100:
                t += run(M)
                passes += 1
        sample = "first %d of %d rows" % (rows, M) if rows < M else "all %d rows x %d passes" % (M, passes)
        return {"value": per_row * rows * passes / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": sample + " (fp64, unfused, same seeded inputs)", "seconds": round(t, 3),
                "cpu_model": cpu_model()}
    n = s["n"]
    per_img = prob.flops / n

    def run(imgs):
        t = time.perf_counter()
        if s["kind"] == "conv2":
            oracle.chain_conv2(d["x"][:imgs], d["w0"], d["b0"], oracle.ACT_RELU, d["w1"], d["b1"])
        elif s["kind"] == "convN":
            oracle.chain_convN(d["x"][:imgs], d["ws"], d["bs"], [actk[a] for a in s["acts"]])
        elif s.get("bn"):
            oracle.chain_conv_bn_pool(d["x"][:imgs], d["w"], d["scale"], d["shift"], oracle.ACT_RELU)
        elif s.get("pool") == "avg2x2":
            oracle.chain_conv_avgpool(d["x"][:imgs], d["w"], d["b"], oracle.ACT_RELU)
        else:
            oracle.chain_conv_pool(d["x"][:imgs], d["w"], d["b"], oracle.ACT_RELU)
        return time.perf_counter() - t

    tp = run(1)
    imgs = int(min(n, max(1, seconds / max(tp, 1e-6))))
    t = run(imgs) if imgs != 1 else tp
    return {"value": per_img * imgs / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "first %d of %d images (fp64, unfused, same seeded inputs)" % (imgs, n),
            "seconds": round(t, 3), "cpu_model": cpu_model()}


def mfma_probe(torch, fc, waves_per_simd=2, iters=2048):
    """The matrix-core rate the GPU sustains on register operands (fc_probe_mfma:
    8 independent 32x32x16 fp16 MFMAs per round, every CU), event-timed on the
    current stream after one warm-up launch, and the shader clock derived from
    the kernel's own counters (s_memtime ticks over 100 MHz s_memrealtime ticks)."""
    n = torch.cuda.get_device_properties(0).multi_processor_count
    stamps = torch.zeros(4 * n, dtype=torch.int64, device="cuda")
    sink = torch.zeros(n, dtype=torch.float32, device="cuda")
    fc.probe_mfma(stamps, sink, waves_per_simd, iters)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    blocks = fc.probe_mfma(stamps, sink, waves_per_simd, iters)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    flops = blocks * 4 * waves_per_simd * iters * 8 * 32768
    st = stamps.view(-1, 4)[:blocks].cpu().tolist()
    clk = sorted((b[1] - b[0]) / ((b[3] - b[2]) / 100e6) / 1e9 for b in st if b[3] > b[2])
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4), "waves_per_simd": waves_per_simd,
            "pct_of_nominal": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 1),
            "sclk_ghz_median": round(clk[len(clk) // 2], 3) if clk else None}


def read_probe(torch, fc, nbytes, copies=5):
    """The rate at which the GPU streams nbytes from memory once (fc_probe_read,
    event-timed), on buffers evicted from the 256 MiB Infinity Cache by the
    other copies (copies x nbytes > 256 MiB): mean of one pass over the
    copies after a first, untimed pass."""
    n16 = nbytes // 16
    bufs = [torch.empty(n16 * 4, dtype=torch.int32, device="cuda").fill_(i + 1) for i in range(copies)]
    sink = torch.zeros(2 * torch.cuda.get_device_properties(0).multi_processor_count, dtype=torch.int32,
                       device="cuda")
    for b in bufs:
        fc.probe_read(b, sink)
    torch.cuda.synchronize()
    ms = []
    for b in bufs:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        fc.probe_read(b, sink)
        t1.record()
        torch.cuda.synchronize()
        ms.append(t0.elapsed_time(t1))
    m = sum(ms) / len(ms)
    del bufs
    return {"bytes": nbytes, "us": round(m * 1e3, 2), "tb_per_s": round(nbytes / (m * 1e-3) / 1e12, 3)}


def launch_floor(torch, fc, steps=50):
    """Per-launch time of an almost empty kernel (one block reading 16 bytes)
    replayed back to back from a captured HIP graph, like the chains' steps:
    the floor under the small-problem rows."""
    buf = torch.zeros(4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    ms, _, _, _ = time_steps(torch, lambda i: fc.probe_read(buf, sink), steps, 3)
    return round(ms, 5)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measured_traffic(name, kernel_hash):
    """HBM bytes per launch from the committed rocprofv3 PMC summary
    (profiles/traffic.json), if it was taken on the current kernel sources;
    else None.  These counters come from separate profiling runs, not from
    this process: the JSON marks them with traffic_source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        db = json.load(f)
    e = db.get("workloads", {}).get(name)
    if not e or e.get("src_hash") != kernel_hash:
        return None
    return e


def roofline(prob, ms_kernel, tr):
    """Roofline position of one launch of the fused kernel: algorithmic bytes
    (HBM side of the ridge) or FLOPs (MFMA side) over the event-timed mean
    launch duration, against MI355X's published peaks."""
    ai = prob.flops / prob.bytes_fused
    ksec = ms_kernel * 1e-3
    traffic = None
    if tr is not None:
        traffic = int(tr["fetch_kib"] * tr["fetch_scale"] * 1024 + tr["write_kib"] * tr["write_scale"] * 1024)
    if ai < RIDGE:
        achieved = prob.bytes_fused / ksec / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        achieved = prob.flops / ksec / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(PEAK_F16_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": traffic}
    if tr is not None:
        roof["traffic_source"] = "profiles/traffic.json[%s] (rocprofv3 FETCH_SIZE/WRITE_SIZE, src %s)" % (
            prob.traffic_key, tr.get("src_hash"))
        roof["traffic_over_algorithmic"] = round(traffic / prob.bytes_fused, 4)
        if "mfma_busy_frac" in tr:
            # rocprofv3 counters of the same kernel (profiled dispatches, which run a little slower)
            roof["mfma_busy_frac_pmc"] = tr["mfma_busy_frac"]
    roof.update({"kernel": prob.kernel, "kernel_ms": round(ms_kernel, 5), "flop_per_byte": round(ai, 1),
                 "algorithmic_bytes": prob.bytes_fused, "algorithmic_flops": prob.flops,
                 "executed_flops": prob.flops_exec})
    if getattr(prob, "flops_note", None):
        roof["flops_note"] = prob.flops_note
        roof["executed_frac"] = round(prob.flops_exec / ksec / 1e12 / PEAK_F16_TFLOPS, 4)
    return roof


_MODEL_VARIANT = {"k_chain_rf": "rf", "k_gemm_lds": "lds", "k_chain_stream": "stream", "k_conv_w": "lds_weights",
                  "k_conv_pool_wino": "winograd", "k_conv_pool_wr": "reg_weights", "k_conv2_pipe": "pipe"}


def traffic_model(prob, tr):
    """Predicted bytes of the kernel's tile schedule beside the measured FETCH
    (gemm_conv_chain_amd.traffic_model: algorithmic reads, Welder's per-tile
    MemTraffic, and an LRU model of each XCD's L2 = the predicted FETCH_SIZE),
    in MB per launch; None for workloads without a model."""
    from gemm_conv_chain_amd import traffic_model as tm
    m = tm.for_workload(prob.spec, _MODEL_VARIANT.get(prob.kernel))
    if m is None:
        return None
    mb = lambda v: round(v / 1e6, 3)
    rec = {"unit": "MB", "kernel": m["kernel"], "blocks": m["blocks"],
           "read_algorithmic": mb(m["read_algorithmic"]), "read_per_tile": mb(m["read_per_tile"]),
           "read_l2_model": mb(m["read_l2_model"]), "write": mb(m["write"]),
           "lds_bytes_per_block": m["lds_bytes_per_block"], "lds_fits": m["lds_fits"]}
    if tr is not None:
        fetch = tr["fetch_kib"] * tr["fetch_scale"] * 1024
        rec["measured_read"] = mb(fetch)
        rec["measured_read_over_l2_model"] = round(fetch / m["read_l2_model"], 4)
    return rec


def measure(torch, fc, prob, steps, warmup, unfused=True, warm=True):
    """Time the fused step (and the unfused two-kernel baseline); returns the
    record of one workload."""
    ms_step, ms_kernel, ms_wall, method = time_steps(torch, prob.step, steps, warmup)
    log("%s fused:   %.4f ms/step (%s, events), kernel %.4f ms, wall %.4f ms"
        % (prob.name, ms_step, method, ms_kernel, ms_wall))
    h = kernel_src_hash()
    tr = measured_traffic(prob.traffic_key, h)
    roof = roofline(prob, ms_kernel, tr)
    roof["timing"] = method
    model = traffic_model(prob, tr)
    if model is not None:
        roof["traffic_model"] = model
    if warm and prob.nsets > 1:
        # secondary: the same launch on one buffer set (inputs warm in the 256 MiB Infinity Cache / L2)
        warm_ms, _, _, _ = time_steps(torch, lambda i: prob.step(0), steps, 2)
        roof["warm_cache_kernel_ms"] = round(warm_ms, 5)
        log("%s fused, warm cache: %.4f ms/step" % (prob.name, warm_ms))
    un = None
    if unfused:
        u_step, _, _, _ = time_steps(torch, prob.step_unfused, max(5, steps // 2), 2)
        ub = prob.bytes_fused + 2 * prob.bytes_interm
        un = {"ms_per_step": round(u_step, 5), "algorithmic_bytes": ub,
              "fused_over_unfused_bytes": round(prob.bytes_fused / ub, 4),
              "speedup_fused": round(u_step / ms_step, 3)}
        if tr is not None and "unfused_bytes" in tr and roof["traffic"] is not None:
            un["profiled_bytes"] = tr["unfused_bytes"]
            un["profiled_fused_over_unfused"] = round(roof["traffic"] / tr["unfused_bytes"], 4)
        log("%s unfused: %.4f ms/step -> fused speedup %.2fx" % (prob.name, u_step, u_step / ms_step))
    tflops = prob.flops / (ms_step * 1e-3) / 1e12
    return {"ms_per_step": round(ms_step, 5), "tflops": round(tflops, 3),
            "pct_fp16_mfma_peak": round(100 * tflops / PEAK_F16_TFLOPS, 2), "roofline": roof, "unfused": un,
            "config": dict(prob.config, cache="cold (rotating %d buffer sets)" % prob.nsets
                           if prob.nsets > 1 else "warm")}


# The other configurations, measured in the same run beside the headline one
# (one record each; the two-GEMM LDS-resident shape under each kernel variant
# and under the profiler's choice, the three-stage GEMM and conv chains).
SIDE_CONFIGS = [("b2b_gemm_tiny", None), ("b2b_gemm_rf", None), ("b2b_gemm_lds", None), ("b2b_gemm_lds", "stream"),
                ("b2b_gemm_lds", "tuned"), ("gemm3_rf", None), ("conv3x3_conv1x1", None), ("conv3x3_conv1x1", "tuned"),
                ("conv3x3_conv1x1x2", None), ("conv3x3_relu_maxpool", "winograd")]
WORKLOADS = ["b2b_gemm_tiny", "b2b_gemm_rf", "b2b_gemm_lds", "gemm3_rf", "conv3x3_conv1x1", "conv3x3_conv1x1x2",
             "conv3x3_relu_maxpool", "conv3x3_bn_relu_maxpool", "conv3x3_relu_avgpool"]


def tune(fc, prob, name):
    """Profile every configuration of the workload's chain on its first buffer
    set (the library caches the fastest for the shape; the timed steps then run
    it under the 'auto' form)."""
    kind = prob.spec["kind"]
    if kind == "gemm2":
        W0, b0, W1, b1 = prob.W
        best, table, _ = fc.tune_chain_gemm2_table(prob.X[0], W0, b0, W1, b1, act=prob.act, out=prob.Y[0], reps=10)
        prob.config["variant"] = "auto"
        prob.kernel = {"rf": "k_chain_rf", "lds": "k_gemm_lds", "stream": "k_chain_stream"}[best["variant"]]
        default = "lds" if name == "b2b_gemm_lds" else "rf"
        prob.traffic_key = name if best["variant"] == default else name + "@" + best["variant"]
    elif kind == "conv_pool":
        if prob.bn:
            w, sc, sh = prob.W
            best, table, _ = fc.tune_conv_pool(prob.X[0], w, sh, scale=sc, pool="max2x2", out=prob.Y[0], reps=10)
        else:
            w, b = prob.W
            best, table, _ = fc.tune_conv_pool(prob.X[0], w, b, pool=prob.pool, out=prob.Y[0], reps=10)
        prob.conv_variant = "auto"
        prob.config["variant"] = "auto"
        prob.kernel = "k_conv_w" if best["variant"] == "lds_weights" else "k_conv_pool_wr"
        prob.traffic_key = name + "@" + best["variant"]
    elif kind == "conv2":
        w0, b0, w1, b1 = prob.W
        s = prob.spec
        default = fc.conv2_auto_config(s["n"], s["h"], s["w"], s["c"], s["k0"], s["k1"])["variant"]   # untuned rule
        best, table, _ = fc.tune_chain_conv2(prob.X[0], w0, b0, w1, b1, act="relu", out=prob.Y[0], reps=10)
        prob.conv_variant = "auto"
        prob.config["variant"] = "auto"
        prob.kernel = "k_conv2_pipe" if best["variant"] == "pipe" else "k_chain_rf"
        prob.traffic_key = name if best["variant"] == default else name + "@" + best["variant"]
    elif kind == "convN":
        n = len(prob.acts)
        default = prob.fc.convN_auto_variant(prob.spec["n"], prob.spec["h"], prob.spec["w"], prob.spec["c"],
                                             prob.spec["ks"])   # untuned rule
        best, table, _ = fc.tune_chain_convN(prob.X[0], prob.W[:n], prob.W[n:], prob.acts, out=prob.Y[0], reps=10)
        prob.conv_variant = "auto"
        prob.config["variant"] = "auto"
        prob.kernel = "k_conv2_pipe" if best["variant"] == "pipe" else "k_chain_rf"
        prob.traffic_key = name if best["variant"] == default else name + "@" + best["variant"]
    else:
        raise ValueError("--tune applies to the two-GEMM, the conv3x3 -> conv1x1 (-> conv1x1) and the pooled conv "
                         "workloads")
    log("%s tuned: %s waves %d stages %d (%s)" % (name, best["variant"], best["waves"], best["stages"], ", ".join(
        "%s/%d/%d %.2f us" % (r["variant"], r["waves"], r["stages"], r["us"]) for r in table)))
    prob.config.update(tuned={"best": {"variant": best["variant"], "waves": best["waves"], "stages": best["stages"]},
                              "table": [{"variant": r["variant"], "waves": r["waves"], "stages": r["stages"],
                                         "us": round(r["us"], 2)} for r in table]})


def main():
    global WARMUP_SECONDS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=WARMUP_SECONDS,
                    help="untimed replays of the captured steps before each timed replay (GPU clocks up)")
    ap.add_argument("--workload", default="conv3x3_relu_maxpool", choices=WORKLOADS,
                    help="the headline workload (default: the conv3x3 + ReLU + 2x2 max-pool chain on "
                         "x[32,112,112,60->64], the largest configuration)")
    ap.add_argument("--variant", choices=["rf", "lds", "stream", "pipe", "lds_weights", "reg_weights", "winograd"],
                    default=None,
                    help="kernel form: GEMM chains rf / lds / stream (default rf, or lds for b2b_gemm_lds); "
                         "conv3x3 -> conv1x1 chains pipe / rf (default: the library's choice); "
                         "conv + pool chains lds_weights / reg_weights (default: the library's choice) or "
                         "winograd (F(2x2,3x3), its own numerics)")
    ap.add_argument("--warm", action="store_true", help="reuse one buffer set (cache-warm timing)")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the headline workload (no per-configuration sub-records)")
    ap.add_argument("--tune", action="store_true",
                    help="two-GEMM, conv -> 1x1 and pooled conv workloads: profile every kernel configuration on the GPU "
                         "first (chain_gemm2_tune_ex / chain_conv_pool_tune / chain_conv2_tune / chain_convN_tune) and time "
                         "the fastest")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-probe", action="store_true", help="skip the matrix-core rate / clock probe")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 256 MiB device copy (known bytes, for PMC counter calibration)")
    args = ap.parse_args()
    WARMUP_SECONDS = max(0.0, args.warmup_seconds)

    if args.gpus != 1:
        print("bench.py: measures one GPU only (the fused chain needs no collectives; "
              "--gpus %d is not supported)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import gemm_conv_chain_amd as fc
    fc.lib()

    prob = Problem(args.workload, cold=not args.warm, variant=args.variant)
    log("workload %s: %d buffer set(s), %.1f MB fused algorithmic bytes, %.3f GFLOP"
        % (args.workload, prob.nsets, prob.bytes_fused / 1e6, prob.flops / 1e9))
    if args.tune:
        if prob.spec["kind"] not in ("gemm2", "conv2", "convN", "conv_pool") or args.variant == "winograd":
            print("bench.py: --tune applies to the two-GEMM, the conv3x3 -> conv1x1 (-> conv1x1) and the pooled "
                  "direct-conv workloads", file=sys.stderr)
            sys.exit(2)
        tune(fc, prob, args.workload)

    head = measure(torch, fc, prob, args.steps, args.warmup, unfused=not args.no_unfused)

    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    probe = None
    if not args.no_probe:
        probe = mfma_probe(torch, fc)
        log("mfma probe: %.1f TFLOP/s (%.1f%% of nominal), shader clock %s GHz"
            % (probe["tflops"], probe["pct_of_nominal"], probe["sclk_ghz_median"]))
        # the read rate of a stream the size of the 65536 x 576 fp16 row matrix
        # of the two-GEMM LDS-resident workload, and the graph launch floor
        probe["hbm_read"] = read_probe(torch, fc, 65536 * 576 * 2)
        probe["launch_floor_ms"] = launch_floor(torch, fc)
        log("read probe: %.2f TB/s streaming %.1f MB once; graph launch floor %.4f ms"
            % (probe["hbm_read"]["tb_per_s"], probe["hbm_read"]["bytes"] / 1e6, probe["launch_floor_ms"]))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(prob, args.cpu_seconds)
        log("oracle:  %.5f TFLOP/s on %d threads (%s)" % (cpu["value"], cpu["cores"], cpu["sample"]))
    host = prob.host

    side = None
    if not args.no_configs:
        del prob
        torch.cuda.empty_cache()
        side = {}
        for name, variant in SIDE_CONFIGS:
            if name == args.workload and variant in (None, args.variant) and not args.tune:
                continue
            key = name if variant is None else name + "@" + variant
            p = Problem(name, cold=not args.warm, variant=None if variant == "tuned" else variant)
            if variant == "tuned":
                tune(fc, p, name)
            rec = measure(torch, fc, p, args.steps, args.warmup, unfused=not args.no_unfused, warm=False)
            if probe:
                rec["pct_of_measured_mfma_peak"] = round(100 * rec["tflops"] / probe["tflops"], 2)
                if p.spec["kind"] == "gemm2" and p.spec["M"] <= 4096:
                    # launch-bound: the step against an almost empty graph-replayed launch
                    rec["launch_floor_ms"] = probe["launch_floor_ms"]
                    rec["over_launch_floor"] = round(rec["ms_per_step"] / probe["launch_floor_ms"], 2)
            side[key] = rec
            del p
            torch.cuda.empty_cache()
            if variant == "tuned":
                fc.tune_clear()

    tflops = head["tflops"]
    out = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_seconds": WARMUP_SECONDS, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "accumulate": "f32", "data": "synthetic",
        "config": head["config"],
        "pct_fp16_mfma_peak": head["pct_fp16_mfma_peak"],
        "pct_of_measured_mfma_peak": round(100 * tflops / probe["tflops"], 2) if probe else None,
        "mfma_probe": probe,
        "roofline": head["roofline"], "unfused": head["unfused"], "cpu_baseline": cpu,
        "configs": side, "kernel_src": kernel_src_hash(),
    }
    del host
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
