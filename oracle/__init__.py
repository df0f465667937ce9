"""CPU oracle for the fused operator chains -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``gemm_conv_chain_amd``) never imports it, and it imports nothing from the
product; the two share no code.  The arithmetic lives in ``oracle.c`` (plain C,
fp64); this module only loads it with ctypes and marshals numpy arrays.

Every function takes fp16 arrays (``numpy.float16``) exactly as the GPU path
receives them and returns fp64 references (unrounded) plus fp16 tensors where
the chain rounds.  Semantics, with the passages they follow:

* ``gemm_bias_act``  -- GEMM + broadcast bias + element-wise activation, the
  epilogue kinds listed in the BOLT reading notes ("Prerequisite: Epilogue
  fusion").
* ``chain_gemm2``    -- D1 = act(A W0 + b0) W1 + b1, the two-GEMM persistent
  fusion of the BOLT notes ("Persistent kernel (GEMM/Conv) fusion"); fusion
  does not change the mathematics, so this is the unfused composition with the
  intermediate rounded once to fp16.
* ``conv_bias_act``  -- direct NHWC convolution (cross-correlation, zero pad),
  the operator whose implicit-GEMM form the interview page describes
  ("Conv optimisation", items 1-2).
* ``maxpool2x2``     -- 2x2/2 max pool with first-max argmax, the MaxPool
  operator tile of the Welder notes ("Operator-tile and Tile-graph").
* ``chain_conv2``    -- conv3x3 + bias + act -> fp16 -> 1x1 conv (a GEMM,
  interview page item 5) + bias.
* ``chain_conv_pool``-- conv + bias + ReLU -> fp16 -> maxpool, the Welder
  Conv -> ReLU -> MaxPool tile graph (Figure 5 in the Welder notes).
* ``winograd``       -- (submodule, numpy fp64) the same conv by Winograd
  F(2x2, 3x3) (interview page, "Conv optimisation", item 3), exactly and under
  the fp16 rounding model of a half-precision implementation.

Parity status: every function is pinned by ``tests/test_oracle_pins.py``
(hand-worked examples under ``tests/golden/``, brute force on tiny inputs,
closed forms and invariants).  The whole fused chain has no printed numeric
example on the pages; it is pinned through its parts and the
fused == unfused-tiled invariant.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ACT_NONE, ACT_RELU, ACT_GELU_TANH, ACT_HARDSWISH = 0, 1, 2, 3

_lock = threading.Lock()
_lib = None

_p16 = ctypes.POINTER(ctypes.c_uint16)
_p64 = ctypes.POINTER(ctypes.c_double)
_pu8 = ctypes.POINTER(ctypes.c_uint8)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    """liboracle.so, or the build named by $FC_ORACLE_LIB (the address- and
    undefined-behaviour-sanitizer build the host sanitizer test runs the pins
    against)."""
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("FC_ORACLE_LIB") or _LIB
            if path == _LIB and not os.path.exists(_LIB):
                build(force=True)
            L = ctypes.CDLL(path)
            L.orc_f16_to_f64.restype = ctypes.c_double
            L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
            L.orc_f64_to_f16.restype = ctypes.c_uint16
            L.orc_f64_to_f16.argtypes = [ctypes.c_double]
            L.orc_f16_to_f64_array.argtypes = [_p16, _p64, _i64]
            L.orc_f64_to_f16_array.argtypes = [_p64, _p16, _i64]
            L.orc_act.restype = ctypes.c_double
            L.orc_act.argtypes = [ctypes.c_int, ctypes.c_double]
            L.orc_act_array.argtypes = [ctypes.c_int, _p64, _p64, _i64]
            L.orc_num_threads.restype = ctypes.c_int
            L.orc_set_num_threads.argtypes = [ctypes.c_int]
            L.orc_gemm_bias_act.argtypes = [_p16, _p16, _p16, ctypes.c_int, _i64, _i64, _i64, _p64]
            L.orc_conv_bias_act.argtypes = [_p16, _p16, _p16, ctypes.c_int] + [_i64] * 9 + [_p64]
            L.orc_maxpool2x2.argtypes = [_p16, _i64, _i64, _i64, _i64, _p16, _pu8]
            L.orc_chain_gemm2.argtypes = [_p16, _p16, _p16, ctypes.c_int, _p16, _p16,
                                          _i64, _i64, _i64, _i64, _p16, _p64]
            L.orc_chain_conv2.argtypes = [_p16, _p16, _p16, ctypes.c_int, _p16, _p16] + [_i64] * 10 + [_p16, _p64]
            L.orc_chain_conv_pool.argtypes = [_p16, _p16, _p16, ctypes.c_int] + [_i64] * 9 + [_p16, _p64, _p16, _pu8]
            _lib = L
    return _lib


# ---------------------------------------------------------------- helpers
def _h(a):
    """fp16 ndarray (or None) -> (keepalive, uint16 pointer)."""
    if a is None:
        return None, None
    a = np.ascontiguousarray(a)
    if a.dtype != np.float16:
        raise TypeError("oracle inputs are fp16 arrays, got %s" % a.dtype)
    u = a.view(np.uint16)
    return u, u.ctypes.data_as(_p16)


def _d(a):
    return a.ctypes.data_as(_p64)


def set_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ---------------------------------------------------------------- codec
def f64_to_f16(v) -> np.ndarray:
    """Round fp64 values to fp16 (RNE) with the oracle's own codec."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_f64_to_f16_array(_d(v), out.ctypes.data_as(_p16), v.size)
    return out.view(np.float16)


def f16_to_f64(h) -> np.ndarray:
    keep, p = _h(np.asarray(h, dtype=np.float16))
    out = np.empty(keep.shape, dtype=np.float64)
    lib().orc_f16_to_f64_array(p, _d(out), keep.size)
    return out


def act(kind: int, s) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float64)
    out = np.empty_like(s)
    lib().orc_act_array(int(kind), _d(s), _d(out), s.size)
    return out


# ---------------------------------------------------------------- operators
def gemm_bias_act(X, W, b, act_kind: int) -> np.ndarray:
    """fp64 [M,N] = act(X @ W + b), X [M,K], W [K,N], b [N] or None."""
    M, K = X.shape
    K2, N = W.shape
    assert K == K2
    kx, px = _h(X)
    kw, pw = _h(W)
    kb, pb = _h(b)
    out = np.empty((M, N), dtype=np.float64)
    lib().orc_gemm_bias_act(px, pw, pb, int(act_kind), M, K, N, _d(out))
    return out


def conv_bias_act(x, w, b, act_kind: int, stride: int = 1, pad: int = 1) -> np.ndarray:
    """fp64 NHWC [n,P,Q,K]; x [n,H,W,C], w HWIO [R,S,C,K], b [K] or None."""
    n, H, Wd, C = x.shape
    R, S, C2, K = w.shape
    assert C == C2
    P = (H + 2 * pad - R) // stride + 1
    Q = (Wd + 2 * pad - S) // stride + 1
    kx, px = _h(x)
    kw, pw = _h(w)
    kb, pb = _h(b)
    out = np.empty((n, max(P, 0), max(Q, 0), K), dtype=np.float64)
    lib().orc_conv_bias_act(px, pw, pb, int(act_kind), n, H, Wd, C, K, R, S, stride, pad, _d(out))
    return out


def maxpool2x2(v):
    """(y fp16 [n,P//2,Q//2,K], argmax uint8) of fp16 v [n,P,Q,K]."""
    n, P, Q, K = v.shape
    kv, pv = _h(v)
    y = np.empty((n, P // 2, Q // 2, K), dtype=np.uint16)
    am = np.empty((n, P // 2, Q // 2, K), dtype=np.uint8)
    lib().orc_maxpool2x2(pv, n, P, Q, K, y.ctypes.data_as(_p16), am.ctypes.data_as(_pu8))
    return y.view(np.float16), am


def avgpool2x2(v) -> np.ndarray:
    """fp16 [n, P//2, Q//2, K]: 2x2 stride-2 average pool of fp16 v [n,P,Q,K]
    (floor for odd sizes) -- each window's four values summed and halved twice,
    exact in fp64, then rounded once to fp16.  A partial reduction of the
    epilogue (BOLT notes, "Prerequisite: Epilogue fusion")."""
    v = np.asarray(v, dtype=np.float16)
    n, P, Q, K = v.shape
    P2, Q2 = P // 2, Q // 2
    w = v[:, :2 * P2, :2 * Q2, :].astype(np.float64).reshape(n, P2, 2, Q2, 2, K)
    s = w[:, :, 0, :, 0] + w[:, :, 0, :, 1] + w[:, :, 1, :, 0] + w[:, :, 1, :, 1]
    return f64_to_f16(s / 4.0)


def chain_gemm2(A, W0, b0, act_kind: int, W1, b1):
    """(ref fp64 [M,N1], H fp16 [M,N0]) for D1 = act(A W0 + b0) W1 + b1."""
    M, K0 = A.shape
    _, N0 = W0.shape
    _, N1 = W1.shape
    ka, pa = _h(A)
    k0, p0 = _h(W0)
    kb0, pb0 = _h(b0)
    k1, p1 = _h(W1)
    kb1, pb1 = _h(b1)
    H = np.empty((M, N0), dtype=np.uint16)
    ref = np.empty((M, N1), dtype=np.float64)
    lib().orc_chain_gemm2(pa, p0, pb0, int(act_kind), p1, pb1, M, K0, N0, N1,
                          H.ctypes.data_as(_p16), _d(ref))
    return ref, H.view(np.float16)


def chain_gemmN(A, Ws, bs, acts):
    """fp64 [M, widths[n]] of the N-stage chain X_{i+1} = act_i(X_i W_i + b_i)
    (BOLT notes, "Persistent kernel (GEMM/Conv) fusion", applied to more than
    two GEMMs): each intermediate is rounded once to fp16, as the fused GPU
    chain keeps it; the last result is returned unrounded.  Built from the
    single-operator gemm_bias_act and the fp16 codec (nothing else)."""
    X = np.asarray(A, dtype=np.float16)
    n = len(Ws)
    for i in range(n):
        Y = gemm_bias_act(X, Ws[i], bs[i], acts[i])
        if i == n - 1:
            return Y
        X = f64_to_f16(Y)


def chain_conv2(x, w0, b0, act_kind: int, w1, b1, stride: int = 1, pad: int = 1):
    """(ref fp64 [n,P,Q,K1], H fp16 [n,P,Q,K0]); w1 is [K0,K1] or [1,1,K0,K1]."""
    n, H_, Wd, C = x.shape
    R, S, C2, K0 = w0.shape
    w1 = np.asarray(w1).reshape(K0, -1)
    K1 = w1.shape[1]
    P = (H_ + 2 * pad - R) // stride + 1
    Q = (Wd + 2 * pad - S) // stride + 1
    kx, px = _h(x)
    kw0, pw0 = _h(w0)
    kb0, pb0 = _h(b0)
    kw1, pw1 = _h(w1)
    kb1, pb1 = _h(b1)
    Hb = np.empty((n, P, Q, K0), dtype=np.uint16)
    ref = np.empty((n, P, Q, K1), dtype=np.float64)
    lib().orc_chain_conv2(px, pw0, pb0, int(act_kind), pw1, pb1, n, H_, Wd, C, K0, R, S, stride, pad, K1,
                          Hb.ctypes.data_as(_p16), _d(ref))
    return ref, Hb.view(np.float16)


def chain_convN(x, ws, bs, acts, stride: int = 1, pad: int = 1):
    """fp64 [n,P,Q,K_last] of a conv3x3 followed by 1x1 convs, each stage
    act_i(stage_i(X_i) + b_i) with every intermediate rounded once to fp16
    (BOLT notes, "Persistent kernel (GEMM/Conv) fusion": several convs fused
    under the residence rule; interview page, Conv item 5: a 1x1 conv is a
    GEMM over the pixels).  ws[0] is HWIO [R,S,C,K0]; ws[i > 0] is [K_{i-1},
    K_i] or [1,1,K_{i-1},K_i].  Built from conv_bias_act, gemm_bias_act and
    the fp16 codec; the last stage is returned unrounded."""
    Y = conv_bias_act(x, ws[0], bs[0], acts[0], stride, pad)
    n, P, Q, K = Y.shape
    for i in range(1, len(ws)):
        X = f64_to_f16(Y).reshape(n * P * Q, K)
        w = np.asarray(ws[i]).reshape(K, -1)
        Y = gemm_bias_act(X, w, bs[i], acts[i])
        K = w.shape[1]
        Y = Y.reshape(n, P, Q, K)
    return Y


def conv_bn_act(x, w, scale, shift, act_kind: int, stride: int = 1, pad: int = 1) -> np.ndarray:
    """fp64 act(conv(x, w) * scale[k] + shift[k]): batch normalisation at
    inference written as a per-channel scale and shift (interview page, the
    inference simplification that replaces BN by a scale and a bias), applied
    to the bias-free convolution.  Built from conv_bias_act (zero bias, no
    activation) and act()."""
    K = w.shape[-1]
    s = conv_bias_act(x, w, np.zeros(K, dtype=np.float16), ACT_NONE, stride, pad)
    t = s * np.asarray(scale, dtype=np.float16).astype(np.float64) + np.asarray(shift, dtype=np.float16).astype(np.float64)
    return act(act_kind, t)


def chain_conv_bn_pool(x, w, scale, shift, act_kind: int = ACT_RELU, want_conv64=False):
    """(y fp16, argmax uint8, v fp16, conv64 fp64 or None) of
    maxpool2x2(fp16(conv_bn_act(...))) -- the Welder Conv+ReLU+MaxPool chain
    with a batch-norm epilogue; built from conv_bn_act, the fp16 codec and
    maxpool2x2."""
    c64 = conv_bn_act(x, w, scale, shift, act_kind)
    v = f64_to_f16(c64)
    y, am = maxpool2x2(v)
    return y, am, v, (c64 if want_conv64 else None)


def chain_conv_avgpool(x, w, b, act_kind: int = ACT_RELU, scale=None):
    """(y fp16, v fp16) of avgpool2x2(fp16(act(conv(x, w) [* scale] + b))):
    the Conv+act+pool chain with an average instead of a maximum; with a scale
    the conv output is batch-normalised as in conv_bn_act.  Built from
    conv_bias_act / conv_bn_act, the fp16 codec and avgpool2x2."""
    c = conv_bn_act(x, w, scale, b, act_kind) if scale is not None else conv_bias_act(x, w, b, act_kind)
    v = f64_to_f16(c)
    return avgpool2x2(v), v


def chain_conv_pool(x, w, b, act_kind: int = ACT_RELU, stride: int = 1, pad: int = 1, want_conv64=False):
    """(y fp16, argmax uint8, v fp16 conv output, conv64 fp64 or None)."""
    n, H_, Wd, C = x.shape
    R, S, C2, K = w.shape
    P = (H_ + 2 * pad - R) // stride + 1
    Q = (Wd + 2 * pad - S) // stride + 1
    kx, px = _h(x)
    kw, pw = _h(w)
    kb, pb = _h(b)
    v = np.empty((n, P, Q, K), dtype=np.uint16)
    c64 = np.empty((n, P, Q, K), dtype=np.float64) if want_conv64 else None
    y = np.empty((n, P // 2, Q // 2, K), dtype=np.uint16)
    am = np.empty((n, P // 2, Q // 2, K), dtype=np.uint8)
    lib().orc_chain_conv_pool(px, pw, pb, int(act_kind), n, H_, Wd, C, K, R, S, stride, pad,
                              v.ctypes.data_as(_p16), _d(c64) if c64 is not None else None,
                              y.ctypes.data_as(_p16), am.ctypes.data_as(_pu8))
    return y.view(np.float16), am, v.view(np.float16), c64
