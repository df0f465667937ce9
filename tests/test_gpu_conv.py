"""GPU parity of the conv chains, the single conv, the max pool and the channel
padding against the fp64 oracle (same seeded inputs)."""
import numpy as np
import pytest

import oracle
from gemm_conv_chain_amd import inputs
from parity import assert_close, check_full, pool_tie_mask, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_conv_chain_amd as m
    m.lib()
    return m


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


ACTS = {"none": oracle.ACT_NONE, "relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH,
        "hardswish": oracle.ACT_HARDSWISH}


def check_pool(y, am, x_np, w_np, b_np, what, act="relu", full=False):
    """y, am from the GPU; oracle on the (unpadded) inputs.  full: record the
    whole-tensor diagnostics (y against the oracle's pooled fp16 values)."""
    yo, amo, v, c64 = oracle.chain_conv_pool(x_np, w_np, b_np, ACTS[act], want_conv64=True)
    if full:
        check_full(y, yo.astype(np.float64), what, ref16=yo)
    else:
        assert_close(y, yo.astype(np.float64), what)
    if am is not None:
        ties = pool_tie_mask(c64, c64.shape[1], c64.shape[2])
        free = ~ties
        assert np.array_equal(am[free], amo[free]), "%s: argmax differs on %d tie-free windows" % (
            what, int(np.sum(am[free] != amo[free])))
        assert np.all(am < 4)
        # on tie windows the GPU's choice must still be a maximal position (to
        # within the same 2-ulp band)
        n, PO, QO, K = am.shape
        win = c64[:, :2 * PO, :2 * QO].reshape(n, PO, 2, QO, 2, K).transpose(0, 1, 3, 5, 2, 4).reshape(n, PO, QO, K, 4)
        picked = np.take_along_axis(win, am[..., None].astype(np.int64), -1)[..., 0]
        top = win.max(-1)
        assert np.all(top - picked <= 2 * np.maximum(np.abs(top), 2.0 ** -14) * 2.0 ** -10 + 1e-30)
        return int(np.sum(free)), int(np.sum(ties))
    return 0, 0


def pool_both(fc, x, w, b, act="relu"):
    """The fused conv+pool with and without argmax: without argmax and with a
    non-decreasing activation the kernel pools the fp32 accumulators before
    bias/activation/rounding, which must give bit-identical y."""
    y, am = fc.chain_conv_pool(x, w, b, act=act, pool="max2x2", argmax=True)
    y2 = fc.chain_conv_pool(x, w, b, act=act, pool="max2x2")
    torch.cuda.synchronize()
    y, am, y2 = to_np(y), to_np(am), to_np(y2)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "y with and without argmax differ"
    return y, am


@pytest.mark.parametrize("n,h,w,c,k", [(2, 8, 10, 64, 128), (1, 5, 7, 32, 64), (2, 9, 6, 64, 72), (1, 4, 6, 96, 64),
                                       (1, 12, 12, 64, 8), (3, 3, 17, 32, 32),
                                       (1, 6, 10, 128, 64)])   # c = 128: the largest weights that fit in LDS with k = 64
def test_conv_pool_small(fc, n, h, w, c, k):
    d = inputs.conv_pool_inputs(n, h, w, c, k, seed=h * w)
    print("case conv_pool", n, h, w, c, k, flush=True)
    y, am = pool_both(fc, dev(d["x"]), dev(d["w"]), dev(d["b"]))
    free, ties = check_pool(y, am, d["x"], d["w"], d["b"], "conv_pool small")
    assert free > 0


@pytest.mark.parametrize("act", ["none", "gelu_tanh", "hardswish"])
@pytest.mark.parametrize("c", [64, 32])
def test_conv_pool_activations(fc, act, c):
    # the pool decides on the fp16 activation output; argmax ties are
    # checked as in check_pool (for "none" the post-activation values can be
    # negative, so ties at zero are rare)
    d = inputs.conv_pool_inputs(2, 10, 14, c, 96, seed=17)
    print("case conv_pool act", act, "c", c, flush=True)
    y, am = pool_both(fc, dev(d["x"]), dev(d["w"]), dev(d["b"]), act=act)
    free, _ = check_pool(y, am, d["x"], d["w"], d["b"], "conv_pool " + act, act=act)
    assert free > 0


def test_conv_pool_many_tiles_ragged(fc):
    # several tiles per block and per wave, and a partial last tile (765
    # windows = 47 full 16-window tiles + 13), C = 64 (compile-time chunk path)
    d = inputs.conv_pool_inputs(3, 30, 34, 64, 128, seed=23)
    print("case conv_pool 3x30x34x64->128", flush=True)
    y, am = pool_both(fc, dev(d["x"]), dev(d["w"]), dev(d["b"]))
    check_pool(y, am, d["x"], d["w"], d["b"], "conv_pool many tiles")


def test_conv_bias_act_many_tiles_ragged(fc):
    # the unfused conv: 2*33*35 = 2310 pixels = 36 full 64-row tiles + 6 rows
    d = inputs.conv_pool_inputs(2, 33, 35, 64, 128, seed=29)
    print("case conv_bias_act 2x33x35x64->128", flush=True)
    y = to_np(fc.conv_bias_act(dev(d["x"]), dev(d["w"]), dev(d["b"]), act="relu"))
    assert_close(y, oracle.conv_bias_act(d["x"], d["w"], d["b"], oracle.ACT_RELU), "conv_bias_act many tiles")


@pytest.mark.parametrize("act", ["gelu_tanh", "hardswish"])
def test_conv2_act(fc, act):
    d = inputs.conv2_inputs(2, 9, 11, 64, 64, 128, seed=31)
    print("case conv2", act, flush=True)
    y = to_np(fc.chain_conv2(dev(d["x"]), dev(d["w0"]), dev(d["b0"]), dev(d["w1"]), dev(d["b1"]), act=act))
    ref, _ = oracle.chain_conv2(d["x"], d["w0"], d["b0"], ACTS[act], d["w1"], d["b1"])
    assert_close(y, ref, "conv2 " + act)


def test_conv_pool_padded_channels(fc):
    # 60 real channels zero-padded to 64 on the GPU; the oracle uses the 60
    d = inputs.conv_pool_inputs(2, 12, 14, 60, 128, seed=5)
    x = fc.pad_channels(dev(d["x"]), 64)
    w = fc.pad_weight_channels(dev(d["w"]), 64)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(x)[..., :60].view(np.uint16), d["x"].view(np.uint16))
    assert not np.any(to_np(x)[..., 60:].astype(np.float64))
    assert np.array_equal(to_np(w)[:, :, :60].view(np.uint16), d["w"].view(np.uint16))
    assert not np.any(to_np(w)[:, :, 60:].astype(np.float64))
    y, am = fc.chain_conv_pool(x, w, dev(d["b"]), argmax=True)
    torch.cuda.synchronize()
    check_pool(to_np(y), to_np(am), d["x"], d["w"], d["b"], "conv_pool padded")


def test_conv_pool_degenerate(fc):
    # conv output of height 1: the pooled output is empty (floor)
    d = inputs.conv_pool_inputs(1, 1, 8, 32, 32, seed=1)
    y = fc.chain_conv_pool(dev(d["x"]), dev(d["w"]), dev(d["b"]))
    torch.cuda.synchronize()
    assert y.shape == (1, 0, 4, 32)


@pytest.mark.parametrize("n,h,w,c,k,act", [(2, 7, 9, 64, 64, "relu"), (1, 6, 6, 32, 128, "gelu_tanh"),
                                           (1, 5, 11, 64, 24, "none"), (2, 6, 10, 64, 128, "hardswish")])
def test_conv_bias_act(fc, n, h, w, c, k, act):
    d = inputs.conv_pool_inputs(n, h, w, c, k, seed=n * h)
    a = ACTS[act]
    print("case conv_bias_act", n, h, w, c, k, act, flush=True)
    y = to_np(fc.conv_bias_act(dev(d["x"]), dev(d["w"]), dev(d["b"]), act=act))
    assert_close(y, oracle.conv_bias_act(d["x"], d["w"], d["b"], a), "conv_bias_act")


@pytest.mark.parametrize("n,h,w,c,k0,k1", [(2, 7, 9, 64, 64, 256), (1, 5, 6, 32, 32, 40), (1, 8, 8, 32, 128, 64),
                                           (3, 4, 13, 96, 40, 8)])
def test_conv2_small(fc, n, h, w, c, k0, k1):
    d = inputs.conv2_inputs(n, h, w, c, k0, k1, seed=h + w)
    print("case conv2", n, h, w, c, k0, k1, flush=True)
    y = to_np(fc.chain_conv2(dev(d["x"]), dev(d["w0"]), dev(d["b0"]), dev(d["w1"]), dev(d["b1"]), act="relu"))
    ref, _ = oracle.chain_conv2(d["x"], d["w0"], d["b0"], oracle.ACT_RELU, d["w1"], d["b1"])
    assert_close(y, ref, "conv2 small")


def test_conv2_fused_equals_unfused(fc):
    d = inputs.conv2_inputs(2, 14, 14, 64, 64, 256, seed=2)
    x, w0, b0, w1, b1 = (dev(d[k]) for k in ("x", "w0", "b0", "w1", "b1"))
    fused = to_np(fc.chain_conv2(x, w0, b0, w1, b1))
    H = fc.conv_bias_act(x, w0, b0, act="relu")
    un = to_np(fc.gemm_bias_act(H.reshape(-1, 64), w1, b1, act="none")).reshape(fused.shape)
    assert_close(fused, un.astype(np.float64), "conv2 fused vs unfused")


def test_conv_pool_fused_equals_unfused(fc):
    d = inputs.conv_pool_inputs(2, 16, 16, 64, 128, seed=3)
    x, w, b = dev(d["x"]), dev(d["w"]), dev(d["b"])
    yf, af = fc.chain_conv_pool(x, w, b, argmax=True, variant="lds_weights")
    v = fc.conv_bias_act(x, w, b, act="relu")
    yu, au = fc.maxpool2x2(v, argmax=True)
    torch.cuda.synchronize()
    # the LDS-weights form and the unfused conv share the accumulation order: bit-identical
    assert np.array_equal(to_np(yf).view(np.uint16), to_np(yu).view(np.uint16))
    assert np.array_equal(to_np(af), to_np(au))
    # the register-weights form sums the two channel halves last: within the tolerance
    yr = fc.chain_conv_pool(x, w, b, variant="reg_weights")
    assert_close(to_np(yr), to_np(yu).astype(np.float64), "reg-weights fused vs unfused")


def test_maxpool2x2(fc):
    rng = np.random.default_rng(0)
    v = rng.standard_normal((2, 7, 9, 24)).astype(np.float16)
    v[0, 0, 0, :] = 0.0
    v[0, 1, 1, :] = 0.0
    v[0, 0, 1, :] = 0.0
    v[0, 1, 0, :] = 0.0          # an all-equal window: argmax must be 0
    y, am = fc.maxpool2x2(dev(v), argmax=True)
    yo, amo = oracle.maxpool2x2(v)
    assert np.array_equal(to_np(y).view(np.uint16), yo.view(np.uint16))
    assert np.array_equal(to_np(am), amo)


@pytest.mark.slow
def test_conv_pool_full_size(fc):
    """Conv+ReLU+MaxPool at full size, in the launch the bench times (no
    argmax, pool taken on the accumulators) and with argmax (bit-identical
    y): every pooled output against the oracle, argmax on every tie-free
    window."""
    spec, d = inputs.workload("conv3x3_relu_maxpool")
    print("case full conv3x3_relu_maxpool", flush=True)
    x = fc.pad_channels(dev(d["x"]), 64)
    w = fc.pad_weight_channels(dev(d["w"]), 64)
    y, am = pool_both(fc, x, w, dev(d["b"]))
    free, ties = check_pool(y, am, d["x"], d["w"], d["b"], "full conv3x3_relu_maxpool", full=True)
    print("argmax: %d tie-free windows equal, %d tie windows (y only)" % (free, ties), flush=True)
    assert free > 0.5 * am.size


@pytest.mark.slow
@pytest.mark.parametrize("variant", ["auto", "rf"])
def test_conv2_full_size(fc, variant):
    # "auto" is the pipelined two-group form at this shape (the bench's launch)
    spec, d = inputs.workload("conv3x3_conv1x1")
    print("case full conv3x3_conv1x1", variant, flush=True)
    args = [dev(d[k]) for k in ("x", "w0", "b0", "w1", "b1")]
    y = to_np(fc.chain_conv2(*args, variant=variant, waves=8 if variant == "rf" else 0))
    ref, _ = oracle.chain_conv2(d["x"], d["w0"], d["b0"], oracle.ACT_RELU, d["w1"], d["b1"])
    check_full(y, ref, "full conv3x3_conv1x1 " + variant)


@pytest.mark.parametrize("n,h,w,k1", [
    (1, 1, 1, 8),          # one pixel: one row tile, 31 of its 32 rows outside the image
    (1, 2, 17, 256),       # odd width: a second column block with one valid column
    (3, 5, 7, 40),         # odd height: the last row pair has one valid row
    (2, 33, 35, 256),      # several tiles per block, ragged in both directions
    (1, 16, 16, 200),      # k1 not a multiple of 64
    (4, 28, 28, 64),
    (40, 9, 10, 128),      # more row tiles than blocks: odd block ranges walk backward
])
def test_conv2_pipe(fc, n, h, w, k1):
    d = inputs.conv2_inputs(n, h, w, 64, 64, k1, seed=n + h + w + k1)
    print("case conv2 pipe", n, h, w, k1, flush=True)
    args = [dev(d[k]) for k in ("x", "w0", "b0", "w1", "b1")]
    y = to_np(fc.chain_conv2(*args, act="relu", variant="pipe"))
    ref, _ = oracle.chain_conv2(d["x"], d["w0"], d["b0"], oracle.ACT_RELU, d["w1"], d["b1"])
    check_full(y, ref, "conv2 pipe %s" % ((n, h, w, k1),))
    rf = to_np(fc.chain_conv2(*args, act="relu", variant="rf", waves=8))
    # the same fp16 intermediate; the two forms differ only in fp32 summation order
    assert np.abs(y.astype(np.float64) - rf).max() <= 2 * np.abs(ref).max() * 2.0 ** -10 + 1e-3


@pytest.mark.parametrize("act", ["none", "gelu_tanh", "hardswish"])
def test_conv2_pipe_acts(fc, act):
    d = inputs.conv2_inputs(2, 9, 20, 64, 64, 96, seed=41)
    print("case conv2 pipe", act, flush=True)
    y = to_np(fc.chain_conv2(*(dev(d[k]) for k in ("x", "w0", "b0", "w1", "b1")), act=act, variant="pipe"))
    ref, _ = oracle.chain_conv2(d["x"], d["w0"], d["b0"], ACTS[act], d["w1"], d["b1"])
    check_full(y, ref, "conv2 pipe " + act)


@pytest.mark.parametrize("n,h,w,c,ks,acts", [
    (2, 9, 11, 64, [64, 64, 128], ["relu", "relu", "none"]),            # compile-time chunks, ragged last tile
    (1, 7, 13, 32, [96, 40, 64], ["relu", "gelu_tanh", "none"]),        # runtime chunks, odd widths
    (2, 6, 10, 64, [32, 128, 64, 56], ["relu", "hardswish", "relu", "none"]),   # four stages
    (1, 1, 3, 64, [64, 64, 64], ["none", "relu", "none"]),              # three pixels: one partial tile
])
def test_chain_convN(fc, n, h, w, c, ks, acts):
    d = inputs.convN_inputs(n, h, w, c, ks, seed=n * h + w)
    print("case convN", n, h, w, c, ks, acts, flush=True)
    y = to_np(fc.chain_convN(dev(d["x"]), [dev(x) for x in d["ws"]], [dev(b) for b in d["bs"]], acts))
    ref = oracle.chain_convN(d["x"], d["ws"], d["bs"], [ACTS[a] for a in acts])
    assert_close(y, ref, "convN %s" % (ks,))


def test_chain_convN_unscaled_zero_bias(fc):
    # sensitivity: unit-variance weights, zero biases (a dropped k chunk or a
    # wrong stage would not hide under the bias), many tiles
    d = inputs.convN_inputs(2, 20, 22, 64, [64, 48, 96], seed=41)
    ws = [(x.astype(np.float32) * 4).astype(np.float16) for x in d["ws"]]
    bs = [np.zeros_like(b) for b in d["bs"]]
    acts = ["relu", "relu", "none"]
    print("case convN unscaled", flush=True)
    y = to_np(fc.chain_convN(dev(d["x"]), [dev(x) for x in ws], [dev(b) for b in bs], acts))
    ref = oracle.chain_convN(d["x"], ws, bs, [ACTS[a] for a in acts])
    assert_close(y, ref, "convN unscaled")


@pytest.mark.parametrize("n,h,w,k2", [(1, 1, 1, 8), (1, 2, 17, 256), (3, 5, 7, 40), (2, 33, 35, 256),
                                       (1, 16, 16, 200), (4, 28, 28, 64), (40, 9, 10, 128)])
def test_convN_pipe(fc, n, h, w, k2):
    # three stages in the pipelined form: 1x1 images, ragged tile tails,
    # block counts above and below the CU count, odd and wide last stages
    d = inputs.convN_inputs(n, h, w, 64, [64, 64, k2], seed=h * w + k2)
    acts = ["relu", "relu", "none"]
    print("case convN pipe", (n, h, w, k2), flush=True)
    args = (dev(d["x"]), [dev(x) for x in d["ws"]], [dev(b) for b in d["bs"]], acts)
    y = to_np(fc.chain_convN(*args, variant="pipe"))
    ref = oracle.chain_convN(d["x"], d["ws"], d["bs"], [ACTS[a] for a in acts])
    check_full(y, ref, "convN pipe %s" % ((n, h, w, k2),))
    if k2 <= 128:
        rf = to_np(fc.chain_convN(*args, variant="rf"))
        # the same fp16 intermediates; the two forms differ only in fp32 summation order
        assert np.abs(y.astype(np.float64) - rf).max() <= 4 * np.abs(ref).max() * 2.0 ** -10 + 1e-3


@pytest.mark.parametrize("acts", [["gelu_tanh", "hardswish", "none"], ["none", "none", "relu"],
                                  ["hardswish", "gelu_tanh", "gelu_tanh"]])
def test_convN_pipe_acts(fc, acts):
    d = inputs.convN_inputs(2, 9, 20, 64, [64, 64, 96], seed=43)
    print("case convN pipe", acts, flush=True)
    y = to_np(fc.chain_convN(dev(d["x"]), [dev(x) for x in d["ws"]], [dev(b) for b in d["bs"]], acts,
                             variant="pipe"))
    ref = oracle.chain_convN(d["x"], d["ws"], d["bs"], [ACTS[a] for a in acts])
    check_full(y, ref, "convN pipe %s" % (acts,))


def test_convN_pipe_unscaled_zero_bias(fc):
    # unit-variance weights and zero biases: a dropped k chunk or a swapped
    # middle stage does not hide under the bias
    d = inputs.convN_inputs(2, 20, 22, 64, [64, 64, 96], seed=47)
    ws = [(x.astype(np.float32) * 4).astype(np.float16) for x in d["ws"]]
    bs = [np.zeros_like(b) for b in d["bs"]]
    acts = ["relu", "relu", "none"]
    print("case convN pipe unscaled", flush=True)
    y = to_np(fc.chain_convN(dev(d["x"]), [dev(x) for x in ws], [dev(b) for b in bs], acts, variant="pipe"))
    ref = oracle.chain_convN(d["x"], ws, bs, [ACTS[a] for a in acts])
    assert_close(y, ref, "convN pipe unscaled")


def test_convN_pipe_identity_middle_is_conv2(fc):
    # an identity middle 1x1 stage (zero bias, no activation) passes the fp16
    # intermediate through exactly (one nonzero product per output), so the
    # three-stage pipelined kernel must equal the two-stage one bit for bit
    d = inputs.conv2_inputs(2, 17, 35, 64, 64, 192, seed=53)
    x, w0, b0, w1, b1 = (dev(d[k]) for k in ("x", "w0", "b0", "w1", "b1"))
    eye, zero = dev(np.eye(64, dtype=np.float16)), dev(np.zeros(64, dtype=np.float16))
    print("case convN pipe identity middle", flush=True)
    y2 = to_np(fc.chain_conv2(x, w0, b0, w1, b1, act="relu", variant="pipe"))
    y3 = to_np(fc.chain_convN(x, [w0, eye, w1], [b0, zero, b1], ["relu", "none", "none"], variant="pipe"))
    assert np.array_equal(y2.view(np.uint16), y3.view(np.uint16))


@pytest.mark.slow
def test_convN_full_size(fc):
    spec, d = inputs.workload("conv3x3_conv1x1x2")
    print("case full conv3x3_conv1x1x2", flush=True)
    y = to_np(fc.chain_convN(dev(d["x"]), [dev(x) for x in d["ws"]], [dev(b) for b in d["bs"]], spec["acts"]))
    ref = oracle.chain_convN(d["x"], d["ws"], d["bs"], [ACTS[a] for a in spec["acts"]])
    check_full(y, ref, "full conv3x3_conv1x1x2")


def check_bn_pool(y, am, d, act, what, full=False):
    yo, amo, _, c64 = oracle.chain_conv_bn_pool(d["x"], d["w"], d["scale"], d["shift"], ACTS[act], want_conv64=True)
    if full:
        check_full(y, yo.astype(np.float64), what, ref16=yo)
    else:
        assert_close(y, yo.astype(np.float64), what)
    ties = pool_tie_mask(c64, c64.shape[1], c64.shape[2])
    free = ~ties
    assert np.array_equal(am[free], amo[free]), "%s: argmax differs on %d tie-free windows" % (
        what, int(np.sum(am[free] != amo[free])))
    return int(np.sum(free))


@pytest.mark.parametrize("n,h,w,c,k,act", [(2, 8, 10, 64, 128, "relu"), (1, 9, 7, 32, 64, "relu"),
                                           (2, 6, 14, 64, 96, "none"), (1, 10, 6, 64, 128, "gelu_tanh")])
def test_conv_bn_pool(fc, n, h, w, c, k, act):
    # batch-norm epilogue with both signs of scale; without argmax (ReLU/none)
    # the kernel pools max or min of the accumulators by the sign of the scale
    d = inputs.conv_bn_pool_inputs(n, h, w, c, k, seed=n + h * w)
    x, wt, sc, sh = dev(d["x"]), dev(d["w"]), dev(d["scale"]), dev(d["shift"])
    print("case conv_bn_pool", n, h, w, c, k, act, flush=True)
    y, am = fc.chain_conv_bn_pool(x, wt, sc, sh, act=act, argmax=True)
    y2 = fc.chain_conv_bn_pool(x, wt, sc, sh, act=act)
    torch.cuda.synchronize()
    y, am, y2 = to_np(y), to_np(am), to_np(y2)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "y with and without argmax differ"
    assert check_bn_pool(y, am, d, act, "conv_bn_pool") > 0


def test_conv_bn_no_pool(fc):
    # pool = none: conv + batch norm + act stored (many tiles, ragged)
    d = inputs.conv_bn_pool_inputs(2, 17, 23, 64, 128, seed=5)
    print("case conv_bn no pool", flush=True)
    y = to_np(fc.chain_conv_bn_pool(dev(d["x"]), dev(d["w"]), dev(d["scale"]), dev(d["shift"]), act="relu",
                                    pool="none"))
    ref = oracle.conv_bn_act(d["x"], d["w"], d["scale"], d["shift"], oracle.ACT_RELU)
    assert_close(y, ref, "conv_bn no pool")


def test_conv_bn_unit_scale_equals_bias_path(fc):
    # scale 1: fma(acc, 1, b) = acc + b, so y and argmax equal chain_conv_pool's bit for bit
    d = inputs.conv_pool_inputs(2, 12, 16, 64, 128, seed=8)
    x, w, b = dev(d["x"]), dev(d["w"]), dev(d["b"])
    one = torch.ones(128, dtype=torch.float16, device="cuda")
    print("case conv_bn unit scale", flush=True)
    for argmax in (True, None):
        r1 = fc.chain_conv_bn_pool(x, w, one, b, argmax=argmax)
        r0 = fc.chain_conv_pool(x, w, b, argmax=argmax)
        torch.cuda.synchronize()
        r1 = r1 if isinstance(r1, tuple) else (r1,)
        r0 = r0 if isinstance(r0, tuple) else (r0,)
        for p, q in zip(r1, r0):
            assert np.array_equal(to_np(p).view(np.uint8), to_np(q).view(np.uint8))


@pytest.mark.slow
def test_conv_bn_pool_full_size(fc):
    spec, d = inputs.workload("conv3x3_bn_relu_maxpool")
    print("case full conv3x3_bn_relu_maxpool", flush=True)
    x = fc.pad_channels(dev(d["x"]), 64)
    w = fc.pad_weight_channels(dev(d["w"]), 64)
    sc, sh = dev(d["scale"]), dev(d["shift"])
    y = to_np(fc.chain_conv_bn_pool(x, w, sc, sh))   # the launch the bench times
    y2, am = fc.chain_conv_bn_pool(x, w, sc, sh, argmax=True)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(np.uint16), to_np(y2).view(np.uint16))
    free = check_bn_pool(y, to_np(am), d, "relu", "full conv3x3_bn_relu_maxpool", full=True)
    assert free > 0.5 * y.size


@pytest.mark.parametrize("n,h,w,c,k,act", [(2, 8, 10, 64, 128, "relu"), (1, 9, 7, 32, 64, "gelu_tanh"),
                                           (3, 30, 34, 64, 128, "none")])
def test_conv_avgpool(fc, n, h, w, c, k, act):
    # the 2x2 average of the rounded conv output (many tiles and a ragged last
    # tile in the third case, the runtime-chunk path in the second)
    d = inputs.conv_pool_inputs(n, h, w, c, k, seed=7 * n + h)
    print("case conv_avgpool", n, h, w, c, k, act, flush=True)
    y = to_np(fc.chain_conv_pool(dev(d["x"]), dev(d["w"]), dev(d["b"]), act=act, pool="avg2x2"))
    yo, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["b"], ACTS[act])
    assert_close(y, yo.astype(np.float64), "conv_avgpool")


def test_conv_bn_avgpool(fc):
    d = inputs.conv_bn_pool_inputs(2, 12, 14, 64, 96, seed=9)
    print("case conv_bn_avgpool", flush=True)
    y = to_np(fc.chain_conv_bn_pool(dev(d["x"]), dev(d["w"]), dev(d["scale"]), dev(d["shift"]), act="relu",
                                    pool="avg2x2"))
    yo, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["shift"], oracle.ACT_RELU, scale=d["scale"])
    assert_close(y, yo.astype(np.float64), "conv_bn_avgpool")


@pytest.mark.slow
def test_conv_avgpool_full_size(fc):
    spec, d = inputs.workload("conv3x3_relu_avgpool")
    print("case full conv3x3_relu_avgpool", flush=True)
    x = fc.pad_channels(dev(d["x"]), 64)
    w = fc.pad_weight_channels(dev(d["w"]), 64)
    y = to_np(fc.chain_conv_pool(x, w, dev(d["b"]), act="relu", pool="avg2x2"))   # the launch the bench times
    yo, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["b"], oracle.ACT_RELU)
    check_full(y, yo.astype(np.float64), "full conv3x3_relu_avgpool", ref16=yo)


def test_avgpool2x2(fc):
    # the unfused baseline's pool kernel (odd sizes floor)
    rng = np.random.default_rng(1)
    v = rng.standard_normal((2, 7, 9, 24)).astype(np.float16)
    print("case avgpool2x2", flush=True)
    y = to_np(fc.avgpool2x2(dev(v)))
    yo = oracle.avgpool2x2(v)
    assert y.shape == yo.shape
    assert_close(y, yo.astype(np.float64), "avgpool2x2")


# ---- channel counts that are multiples of 8 but not of 32: each 8-channel
# group of a tap is one MFMA k-group, so taps straddle the 64-wide k chunks
# (c = 8: eight taps per chunk; c = 24, 40: a tap split across two chunks)
NARROW_C = [8, 24, 40]


@pytest.mark.parametrize("c", NARROW_C)
def test_conv_pool_narrow_channels(fc, c):
    d = inputs.conv_pool_inputs(2, 10, 18, c, 96, seed=c)
    print("case conv_pool narrow c", c, flush=True)
    y, am = pool_both(fc, dev(d["x"]), dev(d["w"]), dev(d["b"]))
    free, _ = check_pool(y, am, d["x"], d["w"], d["b"], "conv_pool c=%d" % c, full=True)
    assert free > 0


@pytest.mark.parametrize("c", NARROW_C)
def test_conv_bias_act_narrow_channels(fc, c):
    d = inputs.conv_pool_inputs(2, 11, 13, c, 64, seed=c + 1)
    print("case conv_bias_act narrow c", c, flush=True)
    y = to_np(fc.conv_bias_act(dev(d["x"]), dev(d["w"]), dev(d["b"]), act="gelu_tanh"))
    check_full(y, oracle.conv_bias_act(d["x"], d["w"], d["b"], oracle.ACT_GELU_TANH), "conv_bias_act c=%d" % c)


@pytest.mark.parametrize("c", NARROW_C)
def test_conv2_narrow_channels(fc, c):
    d = inputs.conv2_inputs(1, 9, 14, c, 64, 40, seed=c + 2)
    print("case conv2 narrow c", c, flush=True)
    y = to_np(fc.chain_conv2(dev(d["x"]), dev(d["w0"]), dev(d["b0"]), dev(d["w1"]), dev(d["b1"]), act="relu"))
    ref, _ = oracle.chain_conv2(d["x"], d["w0"], d["b0"], oracle.ACT_RELU, d["w1"], d["b1"])
    check_full(y, ref, "conv2 c=%d" % c)


@pytest.mark.parametrize("c", NARROW_C)
def test_chain_convN_narrow_channels(fc, c):
    ks, acts = [64, 48, 32], ["relu", "relu", "none"]
    d = inputs.convN_inputs(2, 7, 12, c, ks, seed=c + 3)
    print("case convN narrow c", c, flush=True)
    y = to_np(fc.chain_convN(dev(d["x"]), [dev(x) for x in d["ws"]], [dev(b) for b in d["bs"]], acts))
    ref = oracle.chain_convN(d["x"], d["ws"], d["bs"], [ACTS[a] for a in acts])
    check_full(y, ref, "convN c=%d" % c)


@pytest.mark.parametrize("c", NARROW_C)
def test_conv_bn_pool_narrow_channels(fc, c):
    d = inputs.conv_bn_pool_inputs(2, 8, 14, c, 128, seed=c + 4)
    x, wt, sc, sh = dev(d["x"]), dev(d["w"]), dev(d["scale"]), dev(d["shift"])
    print("case conv_bn_pool narrow c", c, flush=True)
    y, am = fc.chain_conv_bn_pool(x, wt, sc, sh, act="relu", argmax=True)
    torch.cuda.synchronize()
    assert check_bn_pool(to_np(y), to_np(am), d, "relu", "conv_bn_pool c=%d" % c, full=True) > 0


@pytest.mark.parametrize("c", NARROW_C)
def test_conv_avgpool_narrow_channels(fc, c):
    d = inputs.conv_pool_inputs(1, 12, 10, c, 32, seed=c + 5)
    print("case conv_avgpool narrow c", c, flush=True)
    y = to_np(fc.chain_conv_pool(dev(d["x"]), dev(d["w"]), dev(d["b"]), act="relu", pool="avg2x2"))
    yo, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["b"], oracle.ACT_RELU)
    check_full(y, yo.astype(np.float64), "conv_avgpool c=%d" % c, ref16=yo)
