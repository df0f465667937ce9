"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one part of the oracle to something independent: a
hand-worked example under tests/golden/ (each file cites its passage), a
closed form, exact rational arithmetic, numpy's own fp16 conversion, or an
invariant that the mathematics guarantees.  A dropped term, a wrong sign or
index, a transposed operand, a flipped kernel or a misplaced rounding in the
oracle fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from golden_io import read_fields, read_rounding_cases
from gemm_conv_chain_amd import inputs

pytestmark = pytest.mark.cpu

RNG = np.random.default_rng(1234)


def f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16)


# ------------------------------------------------------------------ fp16 codec
def test_codec_golden_boundaries(orc):
    for v, bits in read_rounding_cases():
        got = int(orc.f64_to_f16(np.array([v])).view(np.uint16)[0])
        assert got == bits, (v, hex(got), hex(bits))


def test_codec_decode_all_patterns(orc):
    """Decoding every one of the 65536 bit patterns agrees with numpy."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_to_f64(pats.view(np.float16))
    ref = pats.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[np.isinf(ref)], ref[np.isinf(ref)])


def test_codec_encode_matches_numpy_on_every_boundary(orc):
    """fp64 -> fp16 at every representable value, every midpoint between
    neighbours and one fp64 ulp either side of each midpoint (numpy rounds
    double -> half directly and correctly)."""
    pats = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16)
    vals = pats.view(np.float16).astype(np.float64)
    nxt = np.append(vals[1:], 65536.0)          # 65536 = where the next binade would start
    mids = (vals + nxt) / 2.0                    # exact in fp64
    cand = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    cand = np.concatenate([cand, -cand])
    ours = orc.f64_to_f16(cand).view(np.uint16)
    with np.errstate(over='ignore'):
        ref = cand.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_codec_encode_random(orc):
    e = RNG.uniform(-30, 17, size=200000)
    v = np.sign(RNG.standard_normal(200000)) * 2.0 ** e
    with np.errstate(over='ignore'):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.f64_to_f16(v).view(np.uint16), ref)


# ------------------------------------------------------------------ activations
def test_relu(orc):
    s = np.array([-3.5, -1e-300, -0.0, 0.0, 1e-300, 2.25])
    assert np.array_equal(orc.act(orc.ACT_RELU, s), np.array([0, 0, 0, 0, 1e-300, 2.25]))
    assert np.array_equal(orc.act(orc.ACT_NONE, s), s)


def test_gelu_tanh_closed_form(orc):
    # values of 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) evaluated
    # independently with Python's math module
    s = np.array([0.0, 1.0, -1.0, 3.0, 10.0, 0.5])
    exp = np.array([0.0, 0.8411919906082768, -0.15880800939172324, 2.996362607918227, 10.0,
                    0.34571400982514394])
    assert np.allclose(orc.act(orc.ACT_GELU_TANH, s), exp, rtol=1e-15, atol=1e-16)


def test_gelu_odd_identity(orc):
    # gelu(x) - gelu(-x) = x exactly in real arithmetic
    x = RNG.uniform(-8, 8, 10000)
    g = orc.act(orc.ACT_GELU_TANH, x) - orc.act(orc.ACT_GELU_TANH, -x)
    assert np.max(np.abs(g - x)) < 1e-14


def test_hardswish_values(orc):
    # x * relu6(x + 3) / 6 at hand-worked points: 0 for x <= -3, x for x >= 3
    s = np.array([-4.0, -3.0, -1.0, 0.0, 1.0, 2.0, 3.0, 4.0, -1.5])
    exp = np.array([0.0, 0.0, -1.0 / 3.0, 0.0, 2.0 / 3.0, 5.0 / 3.0, 3.0, 4.0, -0.375])
    assert np.allclose(orc.act(orc.ACT_HARDSWISH, s), exp, rtol=1e-15, atol=0)


def test_hardswish_identities(orc):
    # the same function through ReLU differences, and the odd identity
    # hs(x) - hs(-x) = x, which holds for every real x
    x = RNG.uniform(-8, 8, 10000)
    relu = lambda v: np.maximum(v, 0.0)
    hs = orc.act(orc.ACT_HARDSWISH, x)
    assert np.max(np.abs(hs - x * (relu(x + 3) - relu(x - 3)) / 6)) < 1e-14
    assert np.max(np.abs(hs - orc.act(orc.ACT_HARDSWISH, -x) - x)) < 1e-14


# ------------------------------------------------------------------ GEMM
def test_gemm_golden(orc):
    g = read_fields("matmul_2x2.txt")
    C = orc.gemm_bias_act(f16(g["A"]), f16(g["B"]), None, orc.ACT_NONE)
    assert np.array_equal(C, g["C"])


def _exact_dot_f16(x, w):
    """Exact sum of fp16 products with Python integers (fp16 = int * 2^-24)."""
    xi = [int(Fraction(float(t)) * (1 << 24)) for t in x]
    wi = [int(Fraction(float(t)) * (1 << 24)) for t in w]
    return Fraction(sum(a * b for a, b in zip(xi, wi)), 1 << 48)


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 5, 7), (4, 16, 3), (2, 33, 9)])
def test_gemm_exact_brute_force(orc, M, K, N):
    X = f16(RNG.uniform(-2, 2, (M, K)))
    W = f16(RNG.uniform(-2, 2, (K, N)))
    b = f16(RNG.uniform(-1, 1, N))
    Y = orc.gemm_bias_act(X, W, b, orc.ACT_NONE)
    for m in range(M):
        for n in range(N):
            exact = _exact_dot_f16(X[m], W[:, n]) + Fraction(float(b[n]))
            assert abs(Fraction(Y[m, n]) - exact) <= Fraction(1, 1 << 40) * (1 + abs(exact))


def test_gemm_vs_numpy_with_bias_and_act(orc):
    X = f16(RNG.standard_normal((37, 70)))
    W = f16(RNG.standard_normal((70, 19)) / 8)
    b = f16(RNG.standard_normal(19))
    ref = X.astype(np.float64) @ W.astype(np.float64) + b.astype(np.float64)[None, :]
    for a, fn in [(orc.ACT_NONE, lambda t: t), (orc.ACT_RELU, lambda t: np.maximum(t, 0)),
                  (orc.ACT_GELU_TANH,
                   lambda t: 0.5 * t * (1 + np.tanh(math.sqrt(2 / math.pi) * (t + 0.044715 * t ** 3))))]:
        Y = orc.gemm_bias_act(X, W, b, a)
        assert np.allclose(Y, fn(ref), rtol=1e-12, atol=1e-12)


def test_gemm_not_transposed(orc):
    # a non-square case where using W^T or X^T would not even be shape-correct
    # in the same places: check one element by hand
    X = f16([[1, 2, 3]])
    W = f16([[1, 0], [0, 1], [1, 1]])
    Y = orc.gemm_bias_act(X, W, f16([10, 20]), orc.ACT_NONE)
    assert np.array_equal(Y, np.array([[1 + 3 + 10, 2 + 3 + 20]], dtype=np.float64))


# ------------------------------------------------------------------ conv
def _conv2d_single(orc, xg, wg, pad=1, stride=1):
    x = f16(xg)[None, :, :, None]
    w = f16(wg)[:, :, None, None]
    return orc.conv_bias_act(x, w, None, orc.ACT_NONE, stride=stride, pad=pad)[0, :, :, 0]


def test_conv_golden_ones(orc):
    g = read_fields("conv_ones_3x3.txt")
    assert np.array_equal(_conv2d_single(orc, g["x"], g["w"]), g["y"])


def test_conv_golden_no_flip_zero_pad(orc):
    g = read_fields("conv_sobel_3x3.txt")
    assert np.array_equal(_conv2d_single(orc, g["x"], g["w"]), g["y"])


def test_conv_delta_kernel_identity(orc):
    x = f16(RNG.standard_normal((2, 5, 6, 3)))
    w = np.zeros((3, 3, 3, 3))
    for c in range(3):
        w[1, 1, c, c] = 1.0
    y = orc.conv_bias_act(x, f16(w), None, orc.ACT_NONE)
    assert np.array_equal(y, x.astype(np.float64))


def _im2col_conv(x, w, b, stride, pad):
    """Independent route: explicit im2col (interview page, Conv item 1) + matmul."""
    n, H, W, C = x.shape
    R, S, _, K = w.shape
    P = (H + 2 * pad - R) // stride + 1
    Q = (W + 2 * pad - S) // stride + 1
    xp = np.zeros((n, H + 2 * pad, W + 2 * pad, C))
    xp[:, pad:pad + H, pad:pad + W, :] = x
    cols = np.empty((n, P, Q, R, S, C))
    for r in range(R):
        for s in range(S):
            cols[:, :, :, r, s, :] = xp[:, r:r + stride * P:stride, s:s + stride * Q:stride, :]
    return cols.reshape(n * P * Q, R * S * C) @ w.reshape(R * S * C, K) + b[None, :]


@pytest.mark.parametrize("shape,stride,pad", [((2, 7, 9, 5, 4, 3, 3), 1, 1), ((1, 8, 8, 3, 6, 3, 3), 2, 1),
                                              ((1, 6, 5, 4, 2, 1, 1), 1, 0), ((1, 5, 5, 2, 3, 3, 3), 1, 0)])
def test_conv_vs_im2col(orc, shape, stride, pad):
    n, H, W, C, K, R, S = shape
    x = f16(RNG.standard_normal((n, H, W, C)))
    w = f16(RNG.standard_normal((R, S, C, K)))
    b = f16(RNG.standard_normal(K))
    y = orc.conv_bias_act(x, w, b, orc.ACT_NONE, stride=stride, pad=pad)
    ref = _im2col_conv(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64), stride, pad)
    assert y.shape[1:3] == ((H + 2 * pad - R) // stride + 1, (W + 2 * pad - S) // stride + 1)
    assert np.allclose(y.reshape(ref.shape), ref, rtol=1e-12, atol=1e-12)


def test_conv1x1_equals_gemm_bitwise(orc):
    # interview page, "Conv optimisation" item 5: a 1x1 conv is a GEMM
    x = f16(RNG.standard_normal((2, 4, 5, 24)))
    w = f16(RNG.standard_normal((1, 1, 24, 40)) / 5)
    b = f16(RNG.standard_normal(40))
    y = orc.conv_bias_act(x, w, b, orc.ACT_RELU, stride=1, pad=0)
    g = orc.gemm_bias_act(x.reshape(-1, 24), w.reshape(24, 40), b, orc.ACT_RELU)
    assert np.array_equal(y.reshape(-1, 40), g)


def test_conv_channel_zero_pad_bitwise(orc):
    # padding channels 60 -> 64 with zeros (BOLT notes, "Kernel padding")
    # leaves every sum unchanged
    x = f16(RNG.uniform(-1, 1, (1, 6, 7, 60)))
    w = f16(RNG.standard_normal((3, 3, 60, 16)) / 20)
    b = f16(RNG.standard_normal(16) / 20)
    xp = np.pad(x, [(0, 0), (0, 0), (0, 0), (0, 4)])
    wp = np.pad(w, [(0, 0), (0, 0), (0, 4), (0, 0)])
    assert np.array_equal(orc.conv_bias_act(x, w, b, orc.ACT_RELU), orc.conv_bias_act(xp, wp, b, orc.ACT_RELU))


# ------------------------------------------------------------------ pool
def test_pool_golden(orc):
    g = read_fields("maxpool_4x4.txt")
    y, am = orc.maxpool2x2(f16(g["v"])[None, :, :, None])
    assert np.array_equal(y[0, :, :, 0].astype(np.float64), g["y"])
    assert np.array_equal(am[0, :, :, 0], g["argmax"].astype(np.uint8))


def test_pool_brute_force_and_floor(orc):
    v = f16(RNG.standard_normal((2, 7, 5, 3)))
    y, am = orc.maxpool2x2(v)
    assert y.shape == (2, 3, 2, 3)
    vv = v.astype(np.float64)
    for n in range(2):
        for i in range(3):
            for j in range(2):
                for k in range(3):
                    win = [vv[n, 2 * i + dy, 2 * j + dx, k] for dy in (0, 1) for dx in (0, 1)]
                    assert float(y[n, i, j, k]) == max(win)
                    assert am[n, i, j, k] == win.index(max(win))


def test_pool_ties_take_first(orc):
    v = f16(np.array([[[[0.0], [0.0]], [[0.0], [0.0]]], [[[1.0], [2.0]], [[2.0], [2.0]]]]))
    y, am = orc.maxpool2x2(v)
    assert list(am.ravel()) == [0, 1]


def test_pool_commutes_with_relu(orc):
    v = f16(RNG.standard_normal((1, 8, 8, 4)))
    r = f16(np.maximum(v.astype(np.float64), 0))
    y1, _ = orc.maxpool2x2(r)
    y2, _ = orc.maxpool2x2(v)
    assert np.array_equal(y1.astype(np.float64), np.maximum(y2.astype(np.float64), 0))


# ------------------------------------------------------------------ chains
def test_chain_gemm2_is_unfused_composition(orc):
    X = f16(RNG.standard_normal((33, 40)) / 6)
    W0 = f16(RNG.standard_normal((40, 24)) / 6)
    b0 = f16(RNG.standard_normal(24) / 6)
    W1 = f16(RNG.standard_normal((24, 16)) / 5)
    b1 = f16(RNG.standard_normal(16) / 5)
    for a in (orc.ACT_RELU, orc.ACT_GELU_TANH):
        ref, H = orc.chain_gemm2(X, W0, b0, a, W1, b1)
        # the intermediate is the fp16 (numpy RNE) rounding of stage 1
        h64 = orc.gemm_bias_act(X, W0, b0, a)
        assert np.array_equal(H.view(np.uint16), h64.astype(np.float16).view(np.uint16))
        # stage 2 consumes the ROUNDED intermediate, no activation
        exp = H.astype(np.float64) @ W1.astype(np.float64) + b1.astype(np.float64)
        assert np.allclose(ref, exp, rtol=1e-12, atol=1e-13)
        # and differs measurably from consuming the unrounded one
        unr = h64 @ W1.astype(np.float64) + b1.astype(np.float64)
        assert not np.array_equal(ref, unr)


def test_chain_conv2_is_unfused_composition(orc):
    x = f16(RNG.standard_normal((1, 6, 5, 8)))
    w0 = f16(RNG.standard_normal((3, 3, 8, 16)) / 8)
    b0 = f16(RNG.standard_normal(16) / 8)
    w1 = f16(RNG.standard_normal((16, 24)) / 4)
    b1 = f16(RNG.standard_normal(24) / 4)
    ref, H = orc.chain_conv2(x, w0, b0, orc.ACT_RELU, w1, b1)
    h64 = orc.conv_bias_act(x, w0, b0, orc.ACT_RELU)
    assert np.array_equal(H.view(np.uint16), h64.astype(np.float16).view(np.uint16))
    assert np.allclose(ref.reshape(-1, 24),
                       H.reshape(-1, 16).astype(np.float64) @ w1.astype(np.float64) + b1.astype(np.float64),
                       rtol=1e-12, atol=1e-13)


def test_chain_conv_pool_tiled_equals_whole(orc):
    """Welder tile propagation (see tile_propagation.txt): a pooled output tile
    of t x t needs a 2t x 2t conv (reuse) tile, which needs a (2t+2) x (2t+2)
    input halo for a 3x3 / stride 1 / pad 1 conv.  Evaluating the chain tile by
    tile on halo slices must reproduce the whole-tensor result bit for bit."""
    g = read_fields("tile_propagation.txt")
    t = 2
    assert tuple(g["pool_out_1x1_needs_conv"][0]) == (2, 2)
    assert tuple(g["pool_out_1x1_needs_in"][0]) == (4, 4)
    assert tuple(g["pool_out_8x8_needs_in"][0]) == (2 * 8 + 2, 2 * 8 + 2)
    assert tuple(g["conv_only_out_1x1_needs_in"][0]) == (3, 3)
    x = f16(RNG.uniform(-1, 1, (1, 9, 10, 4)))
    w = f16(RNG.standard_normal((3, 3, 4, 6)) / 6)
    b = f16(RNG.standard_normal(6) / 6)
    y, am, v, _ = orc.chain_conv_pool(x, w, b, orc.ACT_RELU)
    n, H, W, C = x.shape
    xp = np.zeros((n, H + 2, W + 2, C), dtype=np.float16)
    xp[:, 1:H + 1, 1:W + 1] = x
    PO, QO = y.shape[1], y.shape[2]
    for i0 in range(0, PO, t):
        for j0 in range(0, QO, t):
            th, tw = min(t, PO - i0), min(t, QO - j0)
            halo = xp[:, 2 * i0:2 * i0 + 2 * th + 2, 2 * j0:2 * j0 + 2 * tw + 2]
            assert halo.shape[1:3] == (2 * th + 2, 2 * tw + 2)
            yt, amt, _, _ = orc.chain_conv_pool(np.ascontiguousarray(halo), w, b, orc.ACT_RELU, pad=0)
            assert np.array_equal(yt.view(np.uint16), y[:, i0:i0 + th, j0:j0 + tw].view(np.uint16))
            assert np.array_equal(amt, am[:, i0:i0 + th, j0:j0 + tw])


def test_threads_do_not_change_results(orc):
    X = f16(RNG.standard_normal((300, 64)) / 8)
    W = f16(RNG.standard_normal((64, 32)) / 8)
    n0 = orc.num_threads()
    try:
        orc.set_threads(1)
        a = orc.gemm_bias_act(X, W, None, orc.ACT_RELU)
        orc.set_threads(max(2, n0))
        b = orc.gemm_bias_act(X, W, None, orc.ACT_RELU)
    finally:
        orc.set_threads(n0)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ N-stage GEMM chains
def test_chain_gemmN_two_stages_is_chain_gemm2(orc):
    # the Python composition of single operators equals the C two-GEMM chain
    d = inputs.gemm2_inputs(37, 24, 40, 16, "uniform", seed=9)
    ref2, _ = orc.chain_gemm2(d["A"], d["W0"], d["b0"], orc.ACT_GELU_TANH, d["W1"], d["b1"])
    refn = orc.chain_gemmN(d["A"], [d["W0"], d["W1"]], [d["b0"], d["b1"]], [orc.ACT_GELU_TANH, orc.ACT_NONE])
    assert np.array_equal(ref2, refn)


def test_chain_gemmN_identity_stage(orc):
    # an identity middle GEMM (zero bias, no activation) reproduces its fp16
    # input exactly, so the three-stage chain equals the two-stage one
    d = inputs.gemm2_inputs(29, 16, 32, 24, "uniform", seed=10)
    eye = np.eye(32, dtype=np.float16)
    zero = np.zeros(32, dtype=np.float16)
    ref2, _ = orc.chain_gemm2(d["A"], d["W0"], d["b0"], orc.ACT_RELU, d["W1"], d["b1"])
    ref3 = orc.chain_gemmN(d["A"], [d["W0"], eye, d["W1"]], [d["b0"], zero, d["b1"]],
                           [orc.ACT_RELU, orc.ACT_NONE, orc.ACT_NONE])
    assert np.array_equal(ref2, ref3)


def test_chain_gemmN_intermediates_rounded(orc):
    # stage by stage by hand: each intermediate is the fp16 rounding of the
    # previous stage's fp64 result (checked against numpy's float16 cast)
    d = inputs.gemmN_inputs(11, [16, 24, 8, 32], "uniform", seed=12)
    X = d["A"].astype(np.float64)
    acts = [orc.ACT_RELU, orc.ACT_HARDSWISH, orc.ACT_NONE]
    for i in range(3):
        Y = X @ d["Ws"][i].astype(np.float64) + d["bs"][i].astype(np.float64)
        Y = orc.act(acts[i], Y)
        X = Y.astype(np.float16).astype(np.float64) if i < 2 else Y
    ref = orc.chain_gemmN(d["A"], d["Ws"], d["bs"], acts)
    assert np.max(np.abs(ref - X)) <= 1e-12 * max(1.0, np.max(np.abs(X)))


def test_chain_convN_two_stages_is_chain_conv2(orc):
    # the Python composition of single operators equals the C two-stage conv chain
    d = inputs.conv2_inputs(2, 5, 7, 8, 16, 24, seed=13)
    ref2, _ = orc.chain_conv2(d["x"], d["w0"], d["b0"], orc.ACT_RELU, d["w1"], d["b1"])
    refn = orc.chain_convN(d["x"], [d["w0"], d["w1"]], [d["b0"], d["b1"]], [orc.ACT_RELU, orc.ACT_NONE])
    assert np.array_equal(ref2, refn)


def test_chain_convN_identity_stage(orc):
    # an identity 1x1 stage (zero bias, no activation) reproduces its fp16 input
    d = inputs.convN_inputs(1, 6, 5, 8, [16, 16, 24], seed=14)
    eye = np.eye(16, dtype=np.float16)
    zero = np.zeros(16, dtype=np.float16)
    acts = [orc.ACT_RELU, orc.ACT_NONE, orc.ACT_NONE]
    ref3 = orc.chain_convN(d["x"], [d["ws"][0], eye, d["ws"][2].reshape(16, 24)], [d["bs"][0], zero, d["bs"][2]],
                           acts)
    ref2, _ = orc.chain_conv2(d["x"], d["ws"][0], d["bs"][0], orc.ACT_RELU, d["ws"][2].reshape(16, 24), d["bs"][2])
    assert np.array_equal(ref2, ref3)


def test_chain_convN_stages_by_hand(orc):
    # each 1x1 stage is a per-pixel matrix product of the fp16-rounded previous
    # stage (numpy fp64 matmul and numpy's float16 cast)
    d = inputs.convN_inputs(1, 4, 6, 8, [16, 8, 24], seed=15)
    acts = [orc.ACT_RELU, orc.ACT_HARDSWISH, orc.ACT_NONE]
    X = orc.conv_bias_act(d["x"], d["ws"][0], d["bs"][0], acts[0])
    for i in (1, 2):
        Xh = X.astype(np.float16).astype(np.float64)
        X = orc.act(acts[i], Xh @ d["ws"][i].astype(np.float64) + d["bs"][i].astype(np.float64))
    ref = orc.chain_convN(d["x"], d["ws"], d["bs"], acts)
    assert np.max(np.abs(ref - X)) <= 1e-12 * max(1.0, np.max(np.abs(X)))


# ------------------------------------------------------- batch-norm epilogue
def test_conv_bn_pool_golden(orc):
    # conv -> scale -1, shift 5 -> ReLU -> pool, worked by hand
    g = read_fields("conv_bn_relu_pool_sobel.txt")
    x = f16(g["x"])[None, :, :, None]
    w = f16(g["w"])[:, :, None, None]
    y, am, v, c64 = orc.chain_conv_bn_pool(x, w, f16(g["scale"][0]), f16(g["shift"][0]), orc.ACT_RELU,
                                           want_conv64=True)
    assert np.array_equal(c64[0, :, :, 0], g["v"])
    assert np.array_equal(v[0, :, :, 0].astype(np.float64), g["v"])
    assert y.shape == (1, 1, 1, 1) and float(y[0, 0, 0, 0]) == g["y"][0, 0]
    assert int(am[0, 0, 0, 0]) == int(g["argmax"][0, 0])


def test_conv_bn_is_weight_folding(orc):
    # with power-of-two scales, multiplying the weights of output channel k by
    # scale[k] is exact, so BN folded into the weights (a plain conv + bias)
    # gives the epilogue form to fp64 rounding
    x = f16(RNG.standard_normal((2, 5, 6, 8)))
    w = f16(RNG.standard_normal((3, 3, 8, 12)) / 8)
    scale = f16([0.5, -1, 2, -0.25, 1, -2, 0.125, 4, -0.5, 1, -1, 0.25])
    shift = f16(RNG.standard_normal(12) / 4)
    wf = f16(w.astype(np.float64) * scale.astype(np.float64))
    for act in (orc.ACT_NONE, orc.ACT_RELU, orc.ACT_HARDSWISH):
        bn = orc.conv_bn_act(x, w, scale, shift, act)
        folded = orc.conv_bias_act(x, wf, shift, act)
        assert np.max(np.abs(bn - folded)) <= 1e-12 * max(1.0, np.max(np.abs(folded)))
    # the shift is added after the scale (it is not scaled itself)
    bn0 = orc.conv_bn_act(x, w, scale, np.zeros(12, dtype=np.float16), orc.ACT_NONE)
    bn1 = orc.conv_bn_act(x, w, scale, shift, orc.ACT_NONE)
    assert np.max(np.abs(bn0 + shift.astype(np.float64) - bn1)) <= 1e-12 * max(1.0, np.max(np.abs(bn1)))


def test_conv_bn_unit_scale_is_conv_bias(orc):
    # scale 1 reduces the batch-norm chain to the plain Conv+ReLU+MaxPool chain
    d = inputs.conv_pool_inputs(1, 6, 8, 8, 16, seed=31)
    y1, a1, v1, _ = orc.chain_conv_bn_pool(d["x"], d["w"], np.ones(16, dtype=np.float16), d["b"], orc.ACT_RELU)
    y0, a0, v0, _ = orc.chain_conv_pool(d["x"], d["w"], d["b"], orc.ACT_RELU)
    assert np.array_equal(v1.view(np.uint16), v0.view(np.uint16))
    assert np.array_equal(y1.view(np.uint16), y0.view(np.uint16)) and np.array_equal(a1, a0)


# ----------------------------------------------------------- average pool
def test_avgpool_golden(orc):
    g = read_fields("avgpool_4x4.txt")
    v = f16(g["v"])[None, :, :, None]
    y = orc.avgpool2x2(v)
    assert np.array_equal(y[0, :, :, 0].astype(np.float64), g["y"])


def test_avgpool_rounds_the_mean_once(orc):
    # the mean is formed exactly and rounded once: {1, 1, 1, 1 + 2^-10} has mean
    # 1 + 2^-12 (a quarter ulp above 1 -> 1.0); three values of 1 + 2^-10 give
    # 1 + 0.75 * 2^-10 (-> 1 + 2^-10); rounding each partial sum would differ
    a, b = 1.0, 1.0 + 2.0 ** -10
    v = f16([[a, a], [a, b]])[None, :, :, None]
    assert float(orc.avgpool2x2(v)[0, 0, 0, 0]) == 1.0
    v = f16([[a, b], [b, b]])[None, :, :, None]
    assert float(orc.avgpool2x2(v)[0, 0, 0, 0]) == b


def test_avgpool_bounds_and_constant(orc):
    v = f16(RNG.standard_normal((2, 7, 9, 5)))
    y = orc.avgpool2x2(v).astype(np.float64)
    ymax, _ = orc.maxpool2x2(v)
    assert y.shape == (2, 3, 4, 5)                          # floor for odd sizes
    assert np.all(y <= ymax.astype(np.float64))
    ymin = -orc.maxpool2x2(f16(-v.astype(np.float64)))[0].astype(np.float64)
    assert np.all(y >= ymin)
    c = np.full((1, 4, 6, 3), 0.3, dtype=np.float16)
    assert np.array_equal(orc.avgpool2x2(c).view(np.uint16), np.full((1, 2, 3, 3), 0.3, np.float16).view(np.uint16))


def test_chain_conv_avgpool_composition(orc):
    # the chain pools the rounded fp16 conv output (the same v as the max chain)
    d = inputs.conv_pool_inputs(1, 6, 8, 8, 16, seed=32)
    y, v = orc.chain_conv_avgpool(d["x"], d["w"], d["b"], orc.ACT_RELU)
    _, _, vmax, _ = orc.chain_conv_pool(d["x"], d["w"], d["b"], orc.ACT_RELU)
    assert np.array_equal(v.view(np.uint16), vmax.view(np.uint16))
    assert np.array_equal(y.view(np.uint16), orc.avgpool2x2(v).view(np.uint16))


# ------------------------------------------------------- Winograd F(2x2, 3x3)
def _brute_conv(x, w):
    """Direct 3x3 / stride 1 / pad 1 cross-correlation by explicit loops over
    (r, s, c) with Fractions (exact), x [n,H,W,C], w [3,3,C,K] (small ints)."""
    n, H, W, C = x.shape
    K = w.shape[-1]
    y = np.zeros((n, H, W, K), dtype=object)
    for im in range(n):
        for p in range(H):
            for q in range(W):
                for k in range(K):
                    s = Fraction(0)
                    for r in range(3):
                        for t in range(3):
                            pp, qq = p + r - 1, q + t - 1
                            if 0 <= pp < H and 0 <= qq < W:
                                for c in range(C):
                                    s += Fraction(float(x[im, pp, qq, c])) * Fraction(float(w[r, t, c, k]))
                    y[im, p, q, k] = s
    return y


def test_winograd_1d_identity():
    """F(2,3): A^T [(G g) (.) (B^T d)] equals the two correlation outputs
    d0 g0 + d1 g1 + d2 g2 and d1 g0 + d2 g1 + d3 g2 (exact on integers)."""
    from oracle import winograd as W
    BT, G, AT = W.matrices()
    for _ in range(50):
        d = RNG.integers(-9, 10, 4).astype(np.float64)
        g = RNG.integers(-9, 10, 3).astype(np.float64)
        y = AT @ ((G @ g) * (BT @ d))
        assert np.array_equal(y, [d[0] * g[0] + d[1] * g[1] + d[2] * g[2], d[1] * g[0] + d[2] * g[1] + d[3] * g[2]])


def test_winograd_exact_on_small_integers():
    """Every step is exact on small integers, so the fp64 F(2x2,3x3) conv of
    whole tiles equals brute-force direct convolution exactly (odd H and W:
    the last row / column is outside every whole tile)."""
    from oracle import winograd as W
    x = f16(RNG.integers(-4, 5, (2, 7, 9, 3)))
    w = f16(RNG.integers(-3, 4, (3, 3, 3, 5)))
    b = f16(RNG.integers(-2, 3, 5))
    got = W.conv_tiles(x, w, b, "exact")
    ref = _brute_conv(x, w)[:, :6, :8, :] + np.array([Fraction(float(v)) for v in b], dtype=object)
    assert got.shape == ref.shape
    assert all(Fraction(float(g)) == r for g, r in zip(got.ravel(), ref.ravel()))


def test_winograd_sobel_golden():
    """The hand-worked Sobel fixture (3x3 image -> one whole 2x2 tile)."""
    from oracle import winograd as W
    g = read_fields("conv_sobel_3x3.txt")
    y = W.conv_tiles(f16(g["x"])[None, :, :, None], f16(g["w"])[:, :, None, None], None, "exact")
    assert np.array_equal(y[0, :, :, 0], g["y"][:2, :2])


def test_winograd_multiplication_count():
    """The interview page's count: (m + r - 1)^2 = 16 products instead of
    m^2 r^2 = 36 for a 2x2 tile of a 3x3 filter, 4/9 of the direct work."""
    from oracle import winograd as W
    wino, direct = W.multiplications_per_tile()
    assert (wino, direct) == (16, 36)
    assert Fraction(wino, direct) == Fraction(4, 9)


def test_winograd_input_rounding_golden():
    """fp16 model of the input transform: rows first, one rounding per stage
    (hand-worked patch; the exact transform keeps 2^-10 that it loses)."""
    from oracle import winograd as W
    g = read_fields("winograd_input_rounding.txt")
    d = g["d"][None, :, :, None]
    assert np.array_equal(W.input_transform(d, "exact")[0, :, :, 0], g["v_exact"])
    assert np.array_equal(W.input_transform(d, "fp16")[0, :, :, 0], g["v_fp16"])


def test_winograd_weight_transform_closed_form():
    """U = G g G^T entry by entry from its closed form (corners are the
    filter's corners, the centre is the sum of the nine taps over 4, ...)."""
    from oracle import winograd as W
    w = f16(RNG.standard_normal((3, 3, 2, 3)))
    U = W.weight_transform(w, "exact")
    g = w.astype(np.float64)
    assert np.array_equal(U[0, 0], g[0, 0])
    assert np.array_equal(U[3, 3], g[2, 2])
    assert np.array_equal(U[0, 3], g[0, 2])
    assert np.allclose(U[1, 1], g.sum(axis=(0, 1)) / 4, rtol=0, atol=1e-15)
    assert np.allclose(U[0, 1], (g[0, 0] + g[0, 1] + g[0, 2]) / 2, rtol=0, atol=1e-15)
    assert np.allclose(U[2, 1], ((g[0] - g[1] + g[2]).sum(axis=0)) / 4, rtol=0, atol=1e-15)
    U16 = W.weight_transform(w, "fp16")
    assert np.array_equal(U16, U.astype(np.float16).astype(np.float64))


def test_winograd_fp16_model_error_bound(orc):
    """The fp16 model stays within its rounding bound of the exact transform,
    and the direct convolution equals the exact model up to fp64 rounding.
    With m = max |d| over a patch channel, |t| <= 2m and |V| <= 4m; each
    rounding errs by at most 2^-11 of its result, so |V16 - V| <= 2 (2^-11 2m)
    + 2^-11 4m = 2^-8 m (relative to V itself the error is unbounded: the sums
    cancel)."""
    from oracle import winograd as W
    x = f16(RNG.uniform(-1, 1, (2, 6, 10, 8)))
    w = f16(RNG.standard_normal((3, 3, 8, 16)) / 8)
    d = W.patches(x, 3, 5)
    V, V16 = W.input_transform(d, "exact"), W.input_transform(d, "fp16")
    m = np.abs(d).max(axis=(-3, -2), keepdims=True)
    assert np.all(np.abs(V16 - V) <= 2.0 ** -8 * m)
    assert np.any(V16 != V)   # the model does round
    direct = orc.conv_bias_act(x, w, None, orc.ACT_NONE)
    assert np.allclose(W.conv_tiles(x, w, None, "exact"), direct[:, :6, :10], rtol=0, atol=1e-12)
