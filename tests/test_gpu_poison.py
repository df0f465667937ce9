"""LDS race check: every fused kernel run from the poison debug build.

libfusedchain_poison.so is the same source built with -DFC_DEBUG_POISON: each
kernel fills its LDS with a poison pattern (fp16 65504) when it starts, and
the kernels that reuse LDS buffers (the DMA rings of the streamed GEMM chain
and of the register-weights and Winograd conv kernels, the double-buffered
weight chunks of the LDS-resident chain) poison a buffer again as soon as the
barrier that releases it has passed, before its next producer writes it.  A
read that is not ordered after its producer -- a missing barrier, a wait that
retires too few DMA requests -- then picks up poison instead of stale but
plausible data.  The poison steps add LDS writes and barriers but leave the
arithmetic alone, so each case checks:

* the debug build's output equals the product build's bit for bit;
* it is finite (a poisoned operand overflows fp16) and argmax indices are
  valid (poison bytes are no pool index);
* it matches the oracle to the usual tolerance.

Shapes give every block several tiles (ring buffers reused many times),
several weight chunks and GEMM1 passes, ragged last tiles and image borders.
"""
import numpy as np
import pytest

import oracle
from gemm_conv_chain_amd import inputs
from parity import assert_close, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
ACTS = {"none": oracle.ACT_NONE, "relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH}


@pytest.fixture(scope="module")
def fc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_conv_chain_amd as m
    m.lib()
    with m.poison_build():
        pass   # loads the debug build (raises if it was not built)
    return m


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def both(fc, run):
    """run() with the product build, then with the poison build; numpy results."""
    def go():
        r = run()
        torch.cuda.synchronize()
        return [to_np(t) for t in (r if isinstance(r, tuple) else (r,))]
    prod = go()
    with fc.poison_build():
        pois = go()
    return prod, pois


def same_bits(prod, pois, what):
    for a, b in zip(prod, pois):
        assert a.shape == b.shape
        if a.dtype == np.float16:
            assert np.all(np.isfinite(b.astype(np.float32))), "%s: non-finite output in the poison build" % what
            bad = a.view(np.uint16) != b.view(np.uint16)
        else:
            bad = a != b
        assert not bad.any(), "%s: poison build differs from the product build at %d of %d elements" % (
            what, int(bad.sum()), a.size)


@pytest.mark.parametrize("variant,M,K0,N0,N1,act", [
    ("lds", 805, 576, 256, 512, "none"),          # 9 W0 chunks, 2 GEMM1 passes, ragged last block
    ("lds", 300, 64, 128, 256, "gelu_tanh"),
    ("stream", 65536 + 2048 + 77, 576, 256, 256, "none"),   # blocks with two tiles: the ring wraps
    ("stream", 700, 256, 128, 384, "gelu_tanh"),
    ("rf", 1000, 256, 64, 128, "none"),
    ("rf", 4100, 320, 128, 128, "relu"),     # the largest register-resident weights
])
def test_poison_chain_gemm2(fc, variant, M, K0, N0, N1, act):
    d = inputs.gemm2_inputs(M, K0, N0, N1, "uniform", seed=M % 97)
    print("case poison chain_gemm2", variant, M, K0, N0, N1, act, flush=True)
    args = [dev(d[k]) for k in ("A", "W0", "b0", "W1", "b1")]
    prod, pois = both(fc, lambda: fc.chain_gemm2(*args, act=act, variant=variant))
    same_bits(prod, pois, "chain_gemm2 " + variant)
    ref, _ = oracle.chain_gemm2(d["A"], d["W0"], d["b0"], ACTS[act], d["W1"], d["b1"])
    assert_close(pois[0], ref, "poison chain_gemm2 " + variant)


def test_poison_gemm_bias_act(fc):
    d = inputs.gemm2_inputs(300, 576, 320, 64, "uniform", seed=5)   # two column blocks
    print("case poison gemm_bias_act", flush=True)
    A, W, b = dev(d["A"]), dev(d["W0"]), dev(d["b0"])
    prod, pois = both(fc, lambda: fc.gemm_bias_act(A, W, b, act="none"))
    same_bits(prod, pois, "gemm_bias_act")
    assert_close(pois[0], oracle.gemm_bias_act(d["A"], d["W0"], d["b0"], oracle.ACT_NONE), "poison gemm_bias_act")


# 8 x 64 x 130: 2304 pooled row tiles (4.5 per register-weights block), 1152
# Winograd batches (4.5 per block), odd tile columns at the right border
POOL_SHAPE = (8, 64, 130, 64, 128)


@pytest.mark.parametrize("variant", ["lds_weights", "reg_weights"])
def test_poison_conv_pool(fc, variant):
    n, h, w, c, k = POOL_SHAPE
    d = inputs.conv_pool_inputs(n, h, w, c, k, seed=11)
    x, wt, b = dev(d["x"]), dev(d["w"]), dev(d["b"])
    print("case poison conv_pool", variant, flush=True)
    # average pool of the un-activated conv: nothing can hide a poisoned value
    prod, pois = both(fc, lambda: fc.chain_conv_pool(x, wt, b, act="none", pool="avg2x2", variant=variant))
    same_bits(prod, pois, "conv avgpool " + variant)
    ya, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["b"], oracle.ACT_NONE)
    assert_close(pois[0], ya, "poison conv avgpool " + variant)
    # max pool with argmax (the argmax staging and stores)
    prod, pois = both(fc, lambda: fc.chain_conv_pool(x, wt, b, act="relu", argmax=True, variant=variant))
    same_bits(prod, pois, "conv maxpool+argmax " + variant)
    assert np.all(pois[1] < 4)
    ym, _, _, _ = oracle.chain_conv_pool(d["x"], d["w"], d["b"], oracle.ACT_RELU)
    assert_close(pois[0], ym, "poison conv maxpool " + variant)


def test_poison_winograd(fc):
    n, h, w, c, k = POOL_SHAPE
    d = inputs.conv_pool_inputs(n, h, w, c, k, seed=13)
    x, wt, b = dev(d["x"]), dev(d["w"]), dev(d["b"])
    print("case poison winograd", flush=True)
    prod, pois = both(fc, lambda: fc.chain_conv_pool_winograd(x, fc.winograd_weights(wt), b, act="none",
                                                              pool="avg2x2"))
    same_bits(prod, pois, "winograd avgpool")
    ya, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["b"], oracle.ACT_NONE)
    assert_close(pois[0], ya, "poison winograd avgpool")
    prod, pois = both(fc, lambda: fc.chain_conv_pool_winograd(x, fc.winograd_weights(wt), b, act="relu",
                                                              argmax=True))
    same_bits(prod, pois, "winograd maxpool+argmax")
    assert np.all(pois[1] < 4)


def test_poison_conv_bias_act_and_conv2(fc):
    d = inputs.conv2_inputs(2, 30, 34, 64, 64, 256, seed=17)
    x, w0, b0, w1, b1 = (dev(d[k]) for k in ("x", "w0", "b0", "w1", "b1"))
    print("case poison conv_bias_act / chain_conv2", flush=True)
    prod, pois = both(fc, lambda: fc.conv_bias_act(x, w0, b0, act="none"))
    same_bits(prod, pois, "conv_bias_act")
    assert_close(pois[0], oracle.conv_bias_act(d["x"], d["w0"], d["b0"], oracle.ACT_NONE), "poison conv_bias_act")
    ref, _ = oracle.chain_conv2(d["x"], d["w0"], d["b0"], oracle.ACT_NONE, d["w1"], d["b1"])
    for variant, waves in (("pipe", 0), ("rf", 8)):
        prod, pois = both(fc, lambda: fc.chain_conv2(x, w0, b0, w1, b1, act="none", variant=variant, waves=waves))
        same_bits(prod, pois, "chain_conv2 " + variant)
        assert_close(pois[0], ref, "poison chain_conv2 " + variant)


def test_poison_convN_pipe(fc):
    # the three-stage pipelined form: H and H2 double-buffered, the halo ring
    # reused every three tiles
    ks = [64, 64, 192]
    d = inputs.convN_inputs(2, 30, 34, 64, ks, seed=19)
    x, ws, bs = dev(d["x"]), [dev(w) for w in d["ws"]], [dev(b) for b in d["bs"]]
    acts = ["relu", "gelu_tanh", "none"]
    print("case poison chain_convN", flush=True)
    ref = oracle.chain_convN(d["x"], d["ws"], d["bs"], [ACTS[a] for a in acts])
    for variant in ("pipe", "rf"):
        prod, pois = both(fc, lambda: fc.chain_convN(x, ws, bs, acts, variant=variant))
        same_bits(prod, pois, "chain_convN " + variant)
        assert_close(pois[0], ref, "poison chain_convN " + variant)
