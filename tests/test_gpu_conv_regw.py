"""GPU parity of the two kernel forms of the conv + activation + 2x2 pool chain
(weights resident in LDS / weights resident in registers with the input halo
streamed into LDS) against the fp64 oracle, on shapes that exercise the
register-weights kernel's tiling: partial row tiles (pooled widths that are not
a multiple of 8), odd heights, single windows, blocks whose range ends in a
tile of 1..3 row tiles, and several tiles per block."""
import numpy as np
import pytest

import oracle
from gemm_conv_chain_amd import inputs
from parity import assert_close, check_full, to_np
from test_gpu_conv import ACTS, check_bn_pool, check_pool, dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
VARIANTS = ["lds_weights", "reg_weights"]


@pytest.fixture(scope="module")
def fc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_conv_chain_amd as m
    m.lib()
    return m


def both(fc, x, w, b, variant, act="relu"):
    """y and argmax, plus y without argmax (the accumulator-pooling path),
    which must be bit-identical."""
    y, am = fc.chain_conv_pool(x, w, b, act=act, argmax=True, variant=variant)
    y2 = fc.chain_conv_pool(x, w, b, act=act, variant=variant)
    torch.cuda.synchronize()
    y, am, y2 = to_np(y), to_np(am), to_np(y2)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "y with and without argmax differ"
    return y, am


SHAPES = [
    (2, 8, 10, 64, 128),     # one row tile per pooled row, 5 of 8 windows valid
    (2, 9, 6, 64, 72),       # odd height, 72 columns: the second column half holds 8
    (1, 4, 6, 64, 96),
    (1, 2, 2, 64, 128),      # a single window
    (1, 3, 17, 64, 80),      # odd width: 8 windows per pooled row, last conv row and column unused
    (2, 12, 50, 64, 128),    # 25 windows per pooled row: the fourth row tile holds 1
    (3, 30, 34, 64, 128),    # 135 row tiles: one per block
    (5, 66, 130, 64, 128),   # 1485 row tiles: several tiles per block, partial last tiles
]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n,h,w,c,k", SHAPES)
def test_conv_pool_variants(fc, n, h, w, c, k, variant):
    d = inputs.conv_pool_inputs(n, h, w, c, k, seed=3 * n + h + w)
    print("case conv_pool", variant, n, h, w, c, k, flush=True)
    y, am = both(fc, dev(d["x"]), dev(d["w"]), dev(d["b"]), variant)
    free, ties = check_pool(y, am, d["x"], d["w"], d["b"], "conv_pool " + variant)
    assert free > 0


@pytest.mark.parametrize("n,h,w", [(2, 12, 50), (5, 66, 130)])
def test_variants_agree(fc, n, h, w):
    # the two kernel forms sum in different orders (the register form adds two
    # channel halves at the end): equal to within the tolerance, and mostly bit-equal
    d = inputs.conv_pool_inputs(n, h, w, 64, 128, seed=n + w)
    x, wt, b = dev(d["x"]), dev(d["w"]), dev(d["b"])
    print("case variants agree", n, h, w, flush=True)
    ya = to_np(fc.chain_conv_pool(x, wt, b, variant="lds_weights"))
    yb = to_np(fc.chain_conv_pool(x, wt, b, variant="reg_weights"))
    assert_close(yb, ya.astype(np.float64), "reg vs lds weights")
    assert np.mean(ya.view(np.uint16) == yb.view(np.uint16)) > 0.99


@pytest.mark.parametrize("act", ["none", "gelu_tanh", "hardswish"])
def test_reg_weights_activations(fc, act):
    d = inputs.conv_pool_inputs(2, 10, 34, 64, 96, seed=19)
    print("case reg_weights act", act, flush=True)
    y, am = both(fc, dev(d["x"]), dev(d["w"]), dev(d["b"]), "reg_weights", act=act)
    free, _ = check_pool(y, am, d["x"], d["w"], d["b"], "reg_weights " + act, act=act)
    assert free > 0


@pytest.mark.parametrize("n,h,w,k,act", [(2, 8, 10, 128, "relu"), (2, 14, 50, 96, "none"), (1, 10, 6, 128, "gelu_tanh")])
def test_reg_weights_bn(fc, n, h, w, k, act):
    # batch-norm scale of both signs: the accumulator-pooling path takes the
    # max or the min by the sign of the scale
    d = inputs.conv_bn_pool_inputs(n, h, w, 64, k, seed=n + h * w)
    x, wt, sc, sh = dev(d["x"]), dev(d["w"]), dev(d["scale"]), dev(d["shift"])
    print("case reg_weights bn", n, h, w, k, act, flush=True)
    y, am = fc.chain_conv_bn_pool(x, wt, sc, sh, act=act, argmax=True, variant="reg_weights")
    y2 = fc.chain_conv_bn_pool(x, wt, sc, sh, act=act, variant="reg_weights")
    torch.cuda.synchronize()
    y, am, y2 = to_np(y), to_np(am), to_np(y2)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
    assert check_bn_pool(y, am, d, act, "reg_weights bn") > 0


@pytest.mark.parametrize("scaled", [False, True])
def test_reg_weights_avgpool(fc, scaled):
    d = (inputs.conv_bn_pool_inputs if scaled else inputs.conv_pool_inputs)(3, 30, 34, 64, 128, seed=7)
    print("case reg_weights avg", scaled, flush=True)
    if scaled:
        y = to_np(fc.chain_conv_bn_pool(dev(d["x"]), dev(d["w"]), dev(d["scale"]), dev(d["shift"]), pool="avg2x2",
                                        variant="reg_weights"))
        yo, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["shift"], oracle.ACT_RELU, scale=d["scale"])
    else:
        y = to_np(fc.chain_conv_pool(dev(d["x"]), dev(d["w"]), dev(d["b"]), pool="avg2x2", variant="reg_weights"))
        yo, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["b"], oracle.ACT_RELU)
    assert_close(y, yo.astype(np.float64), "reg_weights avg")


def test_reg_weights_unscaled_zero_bias(fc):
    # sensitivity: unit-variance weights and zero bias, so a dropped tap, a
    # dropped channel half or a wrong partial sum cannot hide under the bias
    d = inputs.conv_pool_inputs(2, 20, 36, 64, 128, seed=41)
    w = (d["w"].astype(np.float32) * 24).astype(np.float16)
    b = np.zeros_like(d["b"])
    print("case reg_weights unscaled", flush=True)
    y, am = both(fc, dev(d["x"]), dev(w), dev(b), "reg_weights")
    check_pool(y, am, d["x"], w, b, "reg_weights unscaled")


def test_reg_weights_refuses_other_shapes(fc):
    d = inputs.conv_pool_inputs(1, 4, 4, 32, 128, seed=1)
    with pytest.raises(fc.FusedChainError):
        fc.chain_conv_pool(dev(d["x"]), dev(d["w"]), dev(d["b"]), variant="reg_weights")
    d = inputs.conv_pool_inputs(1, 4, 4, 64, 64, seed=1)
    with pytest.raises(fc.FusedChainError):
        fc.chain_conv_pool(dev(d["x"]), dev(d["w"]), dev(d["b"]), variant="reg_weights")
    with pytest.raises(fc.FusedChainError):
        fc.chain_conv_pool(dev(d["x"]), dev(d["w"]), dev(d["b"]), pool="none", variant="reg_weights")


@pytest.mark.slow
@pytest.mark.parametrize("variant", VARIANTS)
def test_conv_pool_full_size_variants(fc, variant):
    """Conv+ReLU+MaxPool at full size under each kernel form: every pooled
    output against the oracle, argmax on every tie-free window."""
    spec, d = inputs.workload("conv3x3_relu_maxpool")
    print("case full conv3x3_relu_maxpool", variant, flush=True)
    x = fc.pad_channels(dev(d["x"]), 64)
    w = fc.pad_weight_channels(dev(d["w"]), 64)
    y, am = both(fc, x, w, dev(d["b"]), variant)
    free, ties = check_pool(y, am, d["x"], d["w"], d["b"], "full conv3x3_relu_maxpool " + variant, full=True)
    assert free > 0.5 * am.size
