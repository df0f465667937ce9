"""Seeded synthetic inputs for the fused-chain workloads.

This module only draws random numbers and casts them to fp16; it holds none of
the method's arithmetic.  Both the GPU tests/bench and the CPU oracle take
their inputs from here.

Recipe (the pages give no workloads of their own: BOLT's microbenchmarks used
layers from BERT and ResNet-50 whose shapes are not printed, so these stand in):

* one ``numpy.random.default_rng(seed)`` (PCG64) per workload, seed 0 unless
  stated;
* tensors drawn in the order  activations, first weight, first bias, second
  weight, second bias;
* each drawn in fp64, multiplied by its scale, then cast with
  ``astype(float16)`` (round to nearest even);
* every tensor of a GEMM chain is scaled by 1/sqrt(K) where K is the reduction
  length of the contraction the tensor feeds (A, W0, b0: K0; W1, b1: N0);
  conv weights and biases by 1/sqrt(fan_in) with fan_in = R*S*C of the real
  (unpadded) channels.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["gemm2_inputs", "conv2_inputs", "conv_pool_inputs", "workload", "WORKLOADS",
           "pad_last_dim_np"]


def _draw(rng, dist, shape, scale):
    if dist == "uniform":
        a = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        a = rng.standard_normal(size=shape)
    else:
        raise ValueError(dist)
    if scale != 1.0:
        a *= scale
    return a.astype(np.float16)


def gemm2_inputs(M, K0, N0, N1, dist="uniform", seed=0, scaled=True):
    """A[M,K0], W0[K0,N0], b0[N0], W1[N0,N1], b1[N1] (fp16)."""
    rng = np.random.default_rng(seed)
    s0 = 1.0 / math.sqrt(K0) if scaled else 1.0
    s1 = 1.0 / math.sqrt(N0) if scaled else 1.0
    A = _draw(rng, dist, (M, K0), s0)
    W0 = _draw(rng, dist, (K0, N0), s0)
    b0 = _draw(rng, dist, (N0,), s0)
    W1 = _draw(rng, dist, (N0, N1), s1)
    b1 = _draw(rng, dist, (N1,), s1)
    return dict(A=A, W0=W0, b0=b0, W1=W1, b1=b1)


def gemmN_inputs(M, widths, dist="uniform", seed=0, scaled=True):
    """A[M,widths[0]], Ws[i] [widths[i], widths[i+1]], bs[i] [widths[i+1]] (fp16);
    A, W0, b0 scaled by 1/sqrt(widths[0]), W_i and b_i by 1/sqrt(widths[i])."""
    rng = np.random.default_rng(seed)
    s0 = 1.0 / math.sqrt(widths[0]) if scaled else 1.0
    A = _draw(rng, dist, (M, widths[0]), s0)
    Ws, bs = [], []
    for i in range(len(widths) - 1):
        si = 1.0 / math.sqrt(widths[i]) if scaled else 1.0
        Ws.append(_draw(rng, dist, (widths[i], widths[i + 1]), si))
        bs.append(_draw(rng, dist, (widths[i + 1],), si))
    return dict(A=A, Ws=Ws, bs=bs)


def conv2_inputs(n, h, w, c, k0, k1, r=3, s=3, seed=0):
    """x[n,h,w,c] ~ N(0,1); w0 HWIO [r,s,c,k0], b0 ~ N(0,1)/sqrt(r*s*c);
    w1 [c1=k0, k1], b1 ~ N(0,1)/sqrt(k0)."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, "normal", (n, h, w, c), 1.0)
    f0 = 1.0 / math.sqrt(r * s * c)
    w0 = _draw(rng, "normal", (r, s, c, k0), f0)
    b0 = _draw(rng, "normal", (k0,), f0)
    f1 = 1.0 / math.sqrt(k0)
    w1 = _draw(rng, "normal", (k0, k1), f1)
    b1 = _draw(rng, "normal", (k1,), f1)
    return dict(x=x, w0=w0, b0=b0, w1=w1, b1=b1)


def convN_inputs(n, h, w, c, ks, seed=0):
    """x[n,h,w,c] ~ N(0,1); ws[0] HWIO [3,3,c,ks[0]] and bs[0] ~ N(0,1)/sqrt(9c);
    ws[i] [ks[i-1], ks[i]] and bs[i] ~ N(0,1)/sqrt(ks[i-1]) (1x1 stages)."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, "normal", (n, h, w, c), 1.0)
    f0 = 1.0 / math.sqrt(9 * c)
    ws = [_draw(rng, "normal", (3, 3, c, ks[0]), f0)]
    bs = [_draw(rng, "normal", (ks[0],), f0)]
    for i in range(1, len(ks)):
        fi = 1.0 / math.sqrt(ks[i - 1])
        ws.append(_draw(rng, "normal", (ks[i - 1], ks[i]), fi))
        bs.append(_draw(rng, "normal", (ks[i],), fi))
    return dict(x=x, ws=ws, bs=bs)


def conv_pool_inputs(n, h, w, c, k, r=3, s=3, seed=0):
    """x[n,h,w,c] ~ U(-1,1); w HWIO [r,s,c,k] and b[k] ~ N(0,1)/sqrt(r*s*c)."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, "uniform", (n, h, w, c), 1.0)
    f = 1.0 / math.sqrt(r * s * c)
    wt = _draw(rng, "normal", (r, s, c, k), f)
    b = _draw(rng, "normal", (k,), f)
    return dict(x=x, w=wt, b=b)


def conv_bn_pool_inputs(n, h, w, c, k, seed=0):
    """conv_pool_inputs plus a batch-norm scale and shift per output channel:
    scale ~ U(0.5, 1.5) with every fourth channel negated (so both signs
    occur), shift ~ N(0,1)/sqrt(9c) (like the bias)."""
    d = conv_pool_inputs(n, h, w, c, k, seed=seed)
    rng = np.random.default_rng(seed + 1000003)
    sc = rng.uniform(0.5, 1.5, k)
    sc[::4] *= -1.0
    d["scale"] = sc.astype(np.float16)
    d["shift"] = d.pop("b")
    return d


def pad_last_dim_np(a, axis, to):
    """Zero-pad ``axis`` of an fp16 array up to ``to`` entries (a bit copy)."""
    pad = [(0, 0)] * a.ndim
    pad[axis] = (0, to - a.shape[axis])
    return np.pad(a, pad)


# The workloads: sizes, distributions and activations of each.
WORKLOADS = {
    "b2b_gemm_tiny": dict(kind="gemm2", M=512, K0=64, N0=64, N1=64, dist="uniform", act="relu",
                          desc="B2B GEMM A[512x64] W0[64x64] W1[64x64], ReLU"),
    "b2b_gemm_rf": dict(kind="gemm2", M=65536, K0=256, N0=64, N1=128, dist="uniform", act="relu",
                        desc="RF-resident B2B GEMM A[65536x256] W0[256x64] W1[64x128], ReLU"),
    "b2b_gemm_lds": dict(kind="gemm2", M=65536, K0=576, N0=256, N1=256, dist="normal", act="gelu_tanh",
                         desc="LDS-resident B2B GEMM A[65536x576] W0[576x256] W1[256x256], GELU(tanh)"),
    "gemm3_rf": dict(kind="gemmN", M=65536, widths=[256, 64, 64, 128], dist="uniform",
                     acts=["relu", "relu", "none"],
                     desc="three-GEMM register-resident chain A[65536x256] -> 64 (ReLU) -> 64 (ReLU) -> 128"),
    "conv3x3_conv1x1": dict(kind="conv2", n=32, h=56, w=56, c=64, k0=64, k1=256, act="relu",
                            desc="NHWC x[32,56,56,64] conv3x3 64->64 +b+ReLU -> conv1x1 64->256 +b"),
    "conv3x3_conv1x1x2": dict(kind="convN", n=32, h=56, w=56, c=64, ks=[64, 64, 256], acts=["relu", "relu", "none"],
                              desc="NHWC x[32,56,56,64] conv3x3 64->64 +b+ReLU -> conv1x1 64->64 +b+ReLU "
                                   "-> conv1x1 64->256 +b"),
    "conv3x3_bn_relu_maxpool": dict(kind="conv_pool", bn=True, n=32, h=112, w=112, c=60, cpad=64, k=128, act="relu",
                                    desc="NHWC x[32,112,112,60->64] conv3x3 60->128 x scale + shift (batch norm) "
                                         "+ReLU -> maxpool2x2"),
    "conv3x3_relu_avgpool": dict(kind="conv_pool", pool="avg2x2", n=32, h=112, w=112, c=60, cpad=64, k=128,
                                 act="relu", desc="NHWC x[32,112,112,60->64] conv3x3 60->128 +b+ReLU -> avgpool2x2"),
    "conv3x3_relu_maxpool": dict(kind="conv_pool", n=32, h=112, w=112, c=60, cpad=64, k=128, act="relu",
                                 desc="NHWC x[32,112,112,60->64] conv3x3 60->128 +b+ReLU -> maxpool2x2"),
}


def workload(name, seed=0, **override):
    """Inputs (fp16 numpy) for a named workload; ``override`` shrinks sizes."""
    spec = dict(WORKLOADS[name])
    spec.update(override)
    if spec["kind"] == "gemm2":
        return spec, gemm2_inputs(spec["M"], spec["K0"], spec["N0"], spec["N1"], spec["dist"], seed)
    if spec["kind"] == "gemmN":
        return spec, gemmN_inputs(spec["M"], spec["widths"], spec["dist"], seed)
    if spec["kind"] == "conv2":
        return spec, conv2_inputs(spec["n"], spec["h"], spec["w"], spec["c"], spec["k0"], spec["k1"], seed=seed)
    if spec["kind"] == "convN":
        return spec, convN_inputs(spec["n"], spec["h"], spec["w"], spec["c"], spec["ks"], seed=seed)
    if spec["kind"] == "conv_pool" and spec.get("bn"):
        return spec, conv_bn_pool_inputs(spec["n"], spec["h"], spec["w"], spec["c"], spec["k"], seed=seed)
    if spec["kind"] == "conv_pool":
        return spec, conv_pool_inputs(spec["n"], spec["h"], spec["w"], spec["c"], spec["k"], seed=seed)
    raise ValueError(spec["kind"])
