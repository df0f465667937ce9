"""The fused chains captured in a HIP graph (as bench.py times them): every
replay must give what the eager launch gives on the same inputs, including
after the inputs are rewritten in place between replays, with eager work and
synchronisations in between."""
import numpy as np
import pytest

from gemm_conv_chain_amd import inputs

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
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_replays(step, inp, fresh, out, eager):
    """Capture step(); replay 3 times, rewriting inp between replays."""
    step()   # warm-up (first-call set-up happens outside the capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        src = fresh(r)
        inp.copy_(src)
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref = eager(src)
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        assert torch.equal(out, ref), "replay %d differs from the eager launch" % r


@pytest.mark.parametrize("variant", ["rf", "lds", "stream"])
def test_chain_gemm2_graph(fc, variant):
    print("case graph chain_gemm2", variant, flush=True)
    N0 = 64 if variant == "rf" else 256
    d = inputs.gemm2_inputs(1000, 256, N0, 128, "uniform", seed=11)
    A, W0, b0, W1, b1 = (dev(d[k]) for k in ("A", "W0", "b0", "W1", "b1"))
    out = torch.empty((1000, 128), dtype=torch.float16, device="cuda")
    step = lambda: fc.chain_gemm2(A, W0, b0, W1, b1, act="relu", out=out, variant=variant)
    fresh = lambda r: dev(inputs.gemm2_inputs(1000, 256, N0, 128, "uniform", seed=100 + r)["A"])
    eager = lambda src: fc.chain_gemm2(src, W0, b0, W1, b1, act="relu", variant=variant)
    check_replays(step, A, fresh, out, eager)


def test_chain_conv_pool_graph(fc):
    print("case graph chain_conv_pool", flush=True)
    d = inputs.conv_pool_inputs(2, 18, 22, 64, 128, seed=12)
    x, w, b = dev(d["x"]), dev(d["w"]), dev(d["b"])
    out = torch.empty((2, 9, 11, 128), dtype=torch.float16, device="cuda")
    step = lambda: fc.chain_conv_pool(x, w, b, act="relu", pool="max2x2", out=out)
    fresh = lambda r: dev(inputs.conv_pool_inputs(2, 18, 22, 64, 128, seed=200 + r)["x"])
    eager = lambda src: fc.chain_conv_pool(src, w, b, act="relu", pool="max2x2")
    check_replays(step, x, fresh, out, eager)


def test_chain_conv2_graph(fc):
    print("case graph chain_conv2", flush=True)
    d = inputs.conv2_inputs(2, 10, 14, 64, 64, 256, seed=13)
    x, w0, b0, w1, b1 = (dev(d[k]) for k in ("x", "w0", "b0", "w1", "b1"))
    out = torch.empty((2, 10, 14, 256), dtype=torch.float16, device="cuda")
    step = lambda: fc.chain_conv2(x, w0, b0, w1, b1, act="relu", out=out)
    fresh = lambda r: dev(inputs.conv2_inputs(2, 10, 14, 64, 64, 256, seed=300 + r)["x"])
    eager = lambda src: fc.chain_conv2(src, w0, b0, w1, b1, act="relu")
    check_replays(step, x, fresh, out, eager)


def test_chain_gemmN_graph(fc):
    print("case graph chain_gemmN", flush=True)
    wd = [256, 64, 64, 128]
    acts = ["relu", "relu", "none"]
    d = inputs.gemmN_inputs(1000, wd, "uniform", seed=14)
    A = dev(d["A"])
    Ws, bs = [dev(w) for w in d["Ws"]], [dev(b) for b in d["bs"]]
    out = torch.empty((1000, 128), dtype=torch.float16, device="cuda")
    step = lambda: fc.chain_gemmN(A, Ws, bs, acts, out=out)
    fresh = lambda r: dev(inputs.gemmN_inputs(1000, wd, "uniform", seed=400 + r)["A"])
    eager = lambda src: fc.chain_gemmN(src, Ws, bs, acts)
    check_replays(step, A, fresh, out, eager)


def test_chain_convN_graph(fc):
    print("case graph chain_convN", flush=True)
    ks = [64, 64, 256]
    acts = ["relu", "relu", "none"]
    d = inputs.convN_inputs(2, 10, 14, 64, ks, seed=15)
    x = dev(d["x"])
    ws, bs = [dev(w) for w in d["ws"]], [dev(b) for b in d["bs"]]
    out = torch.empty((2, 10, 14, 256), dtype=torch.float16, device="cuda")
    step = lambda: fc.chain_convN(x, ws, bs, acts, out=out)
    fresh = lambda r: dev(inputs.convN_inputs(2, 10, 14, 64, ks, seed=500 + r)["x"])
    eager = lambda src: fc.chain_convN(src, ws, bs, acts)
    check_replays(step, x, fresh, out, eager)


def test_chain_conv_bn_pool_graph(fc):
    print("case graph chain_conv_bn_pool", flush=True)
    d = inputs.conv_bn_pool_inputs(2, 18, 22, 64, 128, seed=16)
    x, w, sc, sh = dev(d["x"]), dev(d["w"]), dev(d["scale"]), dev(d["shift"])
    out = torch.empty((2, 9, 11, 128), dtype=torch.float16, device="cuda")
    step = lambda: fc.chain_conv_bn_pool(x, w, sc, sh, act="relu", pool="max2x2", out=out)
    fresh = lambda r: dev(inputs.conv_bn_pool_inputs(2, 18, 22, 64, 128, seed=600 + r)["x"])
    eager = lambda src: fc.chain_conv_bn_pool(src, w, sc, sh, act="relu", pool="max2x2")
    check_replays(step, x, fresh, out, eager)
