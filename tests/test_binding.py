"""Host-only checks of the Python binding's argument validation: the C ABI
receives bare pointers, so the binding must refuse any tensor whose shape,
dtype or layout disagrees with the sizes the inputs imply -- a short bias, a
wrongly shaped output or argmax would otherwise make a kernel read or write
past an allocation.  All of these raise before the library is called; host
(CPU) tensors with consistent shapes get past the shape checks and are then
refused as non-device tensors."""
import pytest

torch = pytest.importorskip("torch")
import gemm_conv_chain_amd as fc  # noqa: E402

pytestmark = pytest.mark.cpu
H = torch.float16


def z(*shape, dtype=H):
    return torch.zeros(*shape, dtype=dtype)


def gemm2(**kw):
    a = dict(A=z(8, 64), W0=z(64, 64), b0=z(64), W1=z(64, 32), b1=z(32))
    a.update(kw)
    return fc.chain_gemm2(a["A"], a["W0"], a["b0"], a["W1"], a["b1"], out=kw.get("out"))


def test_gemm2_consistent_shapes_reach_the_device_check():
    with pytest.raises(TypeError, match="device tensor"):
        gemm2()
    with pytest.raises(TypeError, match="device tensor"):
        gemm2(b0=None, b1=None)


@pytest.mark.parametrize("kw,msg", [
    (dict(b0=z(63)), "b0 must have shape"),
    (dict(b1=z(33)), "b1 must have shape"),
    (dict(out=z(8, 31)), "out must have shape"),
    (dict(out=z(7, 32)), "out must have shape"),
    (dict(out=z(32, 8).t()), "out must be contiguous"),
    (dict(W0=z(60, 64)), "shape mismatch"),
    (dict(W1=z(56, 32)), "shape mismatch"),
    (dict(A=z(8, 64, 1)), "dims"),
])
def test_gemm2_mismatch_raises(kw, msg):
    with pytest.raises(ValueError, match=msg):
        gemm2(**kw)


def test_gemm2_dtype_and_layout():
    with pytest.raises(TypeError, match="float16"):
        gemm2(out=z(8, 32, dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        gemm2(A=z(64, 8).t())
    with pytest.raises(TypeError, match="tensor"):
        gemm2(b0=[0.0] * 64)


def test_tune_and_gemm_bias_act_mismatch():
    with pytest.raises(ValueError, match="out must have shape"):
        fc.tune_chain_gemm2(z(8, 64), z(64, 64), z(64), z(64, 32), z(32), out=z(8, 16))
    with pytest.raises(ValueError, match="b must have shape"):
        fc.gemm_bias_act(z(8, 64), z(64, 32), z(16))
    with pytest.raises(ValueError, match="out must have shape"):
        fc.gemm_bias_act(z(8, 64), z(64, 32), z(32), out=z(8, 64))


def test_chain_gemmN_mismatch():
    Ws = [z(64, 64), z(64, 32), z(32, 16)]
    bs = [z(64), z(32), z(16)]
    with pytest.raises(TypeError, match="device tensor"):
        fc.chain_gemmN(z(8, 64), Ws, bs, ["relu", "relu", "none"])
    with pytest.raises(ValueError, match="b1 must have shape"):
        fc.chain_gemmN(z(8, 64), Ws, [z(64), z(16), z(16)], ["relu", "relu", "none"])
    with pytest.raises(ValueError, match="out must have shape"):
        fc.chain_gemmN(z(8, 64), Ws, bs, ["relu", "relu", "none"], out=z(8, 32))


X, W, B = (1, 8, 8, 64), (3, 3, 64, 128), (128,)


@pytest.mark.parametrize("kw,msg,exc", [
    (dict(), "device tensor", TypeError),
    (dict(b=z(127)), "b must have shape", ValueError),
    (dict(out=z(1, 8, 8, 128)), "out must have shape", ValueError),
    (dict(out=z(1, 4, 4, 64)), "out must have shape", ValueError),
    (dict(argmax=z(1, 4, 4, 127, dtype=torch.uint8)), "argmax must have shape", ValueError),
    (dict(argmax=z(1, 4, 4, 128, dtype=torch.int8)), "argmax must be torch.uint8", TypeError),
    (dict(argmax=z(1, 4, 128, 4, dtype=torch.uint8).transpose(2, 3)), "argmax must be contiguous", ValueError),
    (dict(w=z(3, 3, 60, 128)), "channels", ValueError),
])
def test_conv_pool_mismatch(kw, msg, exc):
    a = dict(x=z(*X), w=z(*W), b=z(*B), out=None, argmax=None)
    a.update(kw)
    with pytest.raises(exc, match=msg):
        fc.chain_conv_pool(a["x"], a["w"], a["b"], out=a["out"], argmax=a["argmax"])


def test_conv_other_entry_points_mismatch():
    with pytest.raises(ValueError, match="out must have shape"):
        fc.chain_conv_pool(z(*X), z(*W), z(*B), pool="none", out=z(1, 4, 4, 128))
    with pytest.raises(ValueError, match="scale must have shape"):
        fc.chain_conv_bn_pool(z(*X), z(*W), z(64), z(*B))
    with pytest.raises(ValueError, match="shift must have shape"):
        fc.chain_conv_bn_pool(z(*X), z(*W), z(*B), z(64))
    with pytest.raises(ValueError, match="out must have shape"):
        fc.conv_bias_act(z(*X), z(*W), z(*B), out=z(1, 8, 8, 64))
    w0, b0 = z(3, 3, 64, 64), z(64)
    with pytest.raises(ValueError, match="b1 must have shape"):
        fc.chain_conv2(z(*X), w0, b0, z(64, 256), z(128))
    with pytest.raises(ValueError, match="w1 must be"):
        fc.chain_conv2(z(*X), w0, b0, z(32, 256), z(256))
    with pytest.raises(ValueError, match="out must have shape"):
        fc.chain_conv2(z(*X), w0, b0, z(1, 1, 64, 256), z(256), out=z(1, 8, 8, 128))
    with pytest.raises(ValueError, match="b2 must have shape"):
        fc.chain_convN(z(*X), [w0, z(64, 64), z(64, 32)], [b0, z(64), z(64)], ["relu", "relu", "none"])
    with pytest.raises(ValueError, match="argmax must have shape"):
        fc.maxpool2x2(z(1, 8, 8, 64), argmax=z(1, 8, 8, 64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="out must have shape"):
        fc.avgpool2x2(z(1, 8, 8, 64), out=z(1, 4, 4, 32))
    with pytest.raises(TypeError, match="device tensor"):
        fc.maxpool2x2(z(1, 8, 8, 64), argmax=True)
