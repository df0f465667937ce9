"""GPU parity of the Winograd F(2x2,3x3) conv + pool against the oracle.

Two references, on the same seeded inputs:
* the oracle's F(2x2,3x3) under its fp16 model (U rounded once, V rounded
  after each transform stage, rows first) -- the arithmetic the kernel
  performs, so only fp32-vs-fp64 accumulation separates them (element-wise
  tolerance, argmax on every tie-free window);
* the oracle's direct convolution (the conv the chain stands for), at the
  same tolerance 1e-2 max|ref| + 1e-3 as the direct kernels: the precision
  lost to the transforms has to fit inside it.
The transformed weights are compared bit for bit with the oracle's fp16 U.
"""
import numpy as np
import pytest

import oracle
from oracle import winograd as owino
from gemm_conv_chain_amd import inputs
from parity import assert_close, check_full, diagnostics, pool_tie_mask, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ACTS = {"none": oracle.ACT_NONE, "relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH,
        "hardswish": oracle.ACT_HARDSWISH}


@pytest.fixture(scope="module")
def fc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_conv_chain_amd as m
    m.lib()
    return m


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def u_layout(U):
    """oracle U [4, 4, C, K] -> the library's [16, C/8, K, 8] operand layout."""
    _, _, C, K = U.shape
    return np.ascontiguousarray(U.reshape(16, C // 8, 8, K).transpose(0, 1, 3, 2))


@pytest.mark.parametrize("c,k", [(64, 128), (32, 64), (8, 8), (24, 40), (64, 16)])
def test_winograd_weights_bit_exact(fc, c, k):
    d = inputs.conv_pool_inputs(1, 2, 2, c, k, seed=c + k)
    print("case winograd_weights", c, k, flush=True)
    U = to_np(fc.winograd_weights(dev(d["w"])))
    ref = u_layout(owino.weight_transform(d["w"], "fp16").astype(np.float16))
    assert U.shape == ref.shape
    assert np.array_equal(U.view(np.uint16), ref.view(np.uint16))


def run_both(fc, d, act, pool="max2x2", argmax=True):
    U = fc.winograd_weights(dev(d["w"]))
    x, b = dev(d["x"]), dev(d["b"])
    if pool == "max2x2" and argmax:
        y, am = fc.chain_conv_pool_winograd(x, U, b, act=act, pool=pool, argmax=True)
        y2 = fc.chain_conv_pool_winograd(x, U, b, act=act, pool=pool)
        torch.cuda.synchronize()
        y, am, y2 = to_np(y), to_np(am), to_np(y2)
        # pool-first (monotone act, no argmax) and per-element pooling agree bit for bit
        assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "y with and without argmax differ"
        return y, am
    y = fc.chain_conv_pool_winograd(x, U, b, act=act, pool=pool)
    torch.cuda.synchronize()
    return to_np(y), None


def check_wino(y, am, d, act, pool, what, full=False):
    a = ACTS[act]
    ym, amm, _, c64m = owino.chain_conv_pool(d["x"], d["w"], d["b"], a, pool, model="fp16")
    # the kernel's own arithmetic
    if full:
        check_full(y, ym.astype(np.float64), what + " vs fp16 model", ref16=ym)
    else:
        assert_close(y, ym.astype(np.float64), what + " vs fp16 model")
    if am is not None:
        free = ~pool_tie_mask(c64m, c64m.shape[1], c64m.shape[2])
        assert np.array_equal(am[free], amm[free]), "%s: argmax differs on %d tie-free windows" % (
            what, int(np.sum(am[free] != amm[free])))
        assert np.all(am < 4)
    # the conv it stands for
    if pool == "max2x2":
        yd, _, _, _ = oracle.chain_conv_pool(d["x"], d["w"], d["b"], a)
    else:
        yd, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["b"], a)
    if full:
        check_full(y, yd.astype(np.float64), what + " vs direct conv", ref16=yd)
    else:
        assert_close(y, yd.astype(np.float64), what + " vs direct conv")
    return diagnostics(y, yd.astype(np.float64), yd), diagnostics(y, ym.astype(np.float64), ym)


# n, h, w, c, k: partial last batch (tiles % 16), odd sizes (floor), batches
# straddling rows and images (w/2 < 16), several batches per block
SHAPES = [(2, 8, 10, 64, 128), (1, 6, 6, 32, 64), (3, 9, 7, 64, 48), (2, 16, 34, 64, 128), (1, 2, 2, 64, 16),
          (4, 5, 5, 32, 32), (2, 30, 34, 64, 128), (1, 3, 66, 32, 128)]


@pytest.mark.parametrize("n,h,w,c,k", SHAPES)
def test_winograd_pool_small(fc, n, h, w, c, k):
    d = inputs.conv_pool_inputs(n, h, w, c, k, seed=n * h * w + c)
    print("case wino pool", n, h, w, c, k, flush=True)
    y, am = run_both(fc, d, "relu")
    check_wino(y, am, d, "relu", "max2x2", "wino %s" % ((n, h, w, c, k),))


@pytest.mark.parametrize("act", ["none", "gelu_tanh", "hardswish"])
@pytest.mark.parametrize("c", [64, 32])
def test_winograd_activations(fc, act, c):
    d = inputs.conv_pool_inputs(2, 10, 14, c, 96, seed=c + 7)
    print("case wino act", act, c, flush=True)
    y, am = run_both(fc, d, act)
    check_wino(y, am, d, act, "max2x2", "wino " + act)


@pytest.mark.parametrize("c", [64, 32])
def test_winograd_avgpool(fc, c):
    d = inputs.conv_pool_inputs(2, 12, 18, c, 128, seed=c + 11)
    print("case wino avg", c, flush=True)
    y, _ = run_both(fc, d, "relu", pool="avg2x2")
    check_wino(y, None, d, "relu", "avg2x2", "wino avg")


def test_winograd_no_bias_unscaled(fc):
    # sensitivity: unit-variance weights, no bias (a dropped (xi, nu) term or a
    # wrong transform sign would not hide under the bias)
    d = inputs.conv_pool_inputs(2, 12, 20, 64, 128, seed=3)
    d["w"] = (d["w"].astype(np.float32) * 24).astype(np.float16)
    d["b"] = None
    print("case wino unscaled", flush=True)
    U = fc.winograd_weights(dev(d["w"]))
    y, am = fc.chain_conv_pool_winograd(dev(d["x"]), U, None, act="none", argmax=True)
    torch.cuda.synchronize()
    check_wino(to_np(y), to_np(am), d, "none", "max2x2", "wino unscaled")


def test_winograd_empty_and_degenerate(fc):
    d = inputs.conv_pool_inputs(1, 1, 8, 64, 32, seed=1)
    U = fc.winograd_weights(dev(d["w"]))
    y = fc.chain_conv_pool_winograd(dev(d["x"]), U, dev(d["b"]))
    torch.cuda.synchronize()
    assert y.shape == (1, 0, 4, 32)


@pytest.mark.slow
def test_winograd_full_size(fc):
    """The 32 x 112 x 112 x 60 (padded to 64) -> 128 conv + ReLU + 2x2 max
    pool at full size, in the launch the bench times; prints the tolerance
    study (error against the direct conv and against the fp16 model)."""
    spec, d = inputs.workload("conv3x3_relu_maxpool")
    print("case full wino conv3x3_relu_maxpool", flush=True)
    x = fc.pad_channels(dev(d["x"]), 64)
    w = fc.pad_weight_channels(dev(d["w"]), 64)
    U = fc.winograd_weights(w)
    y, am = fc.chain_conv_pool_winograd(x, U, dev(d["b"]), act="relu", argmax=True)
    torch.cuda.synchronize()
    y, am = to_np(y), to_np(am)
    dd = dict(x=to_np(x), w=to_np(w), b=d["b"])   # the padded channels are zero: the same conv
    direct, model = check_wino(y, am, dd, "relu", "max2x2", "full wino", full=True)
    print("tolerance study vs direct conv:", direct)
    print("tolerance study vs fp16 model:", model)
