"""Winograd F(2x2, 3x3) convolution for the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; the product library never imports it.

What it follows.  The interview page ("Conv optimisation", item 3, Winograd
transform) states the method's claim: F(m, r) replaces the m^2 r^2
multiplications of an m x m output tile of an r x r filter by (m + r - 1)^2,
i.e. 16 instead of 36 for m = 2, r = 3 (4/9 of the work), at the price of
extra transform arithmetic and a small loss of precision.  The page prints
neither the transform matrices nor their order of evaluation; the plainest
reading is the minimal filtering algorithm of Lavin and Gray ("Fast
Algorithms for Convolutional Neural Networks", CVPR 2016), written here from
its definition:

    U = G g G^T          (per input channel c and output channel k; g 3x3)
    V = B^T d B          (per 4x4 input patch d of a 2x2 output tile)
    M = sum_c U (.) V    (16 independent channel contractions)
    Y = A^T M A          (the 2x2 output tile)

with
    B^T = [[1, 0, -1, 0], [0, 1, 1, 0], [0, -1, 1, 0], [0, 1, 0, -1]]
    G   = [[1, 0, 0], [1/2, 1/2, 1/2], [1/2, -1/2, 1/2], [0, 0, 1]]
    A^T = [[1, 1, 1, 0], [0, 1, -1, -1]].

Output tile (i, j) holds conv outputs (2i + a, 2j + b), a, b in {0, 1}, of the
3x3, stride-1, pad-1 cross-correlation; its patch is input rows 2i - 1 ..
2i + 2 and columns 2j - 1 .. 2j + 2, zero outside the image.  Only whole
tiles are formed (floor(P/2) x floor(Q/2) of them): the 2x2 pool that follows
drops an odd last row or column the same way.

Two precision models:

* ``"exact"`` -- every step in fp64.  For fp16 inputs the transforms are exact
  (sums of a few dyadic numbers) and the result equals the direct convolution
  up to fp64 rounding of the contraction; on small-integer inputs it is exact.
* ``"fp16"`` -- where a half-precision implementation rounds: U rounded once to
  fp16 (from its exact value); V computed row stage first (t = B^T d, each
  entry one fp16 rounding of a two-term sum), then column stage (V = t B, again
  one rounding per entry); M and Y unrounded (fp64 here).  This is this
  build's reading of "extra transforms in half precision"; the rounding order
  is part of the model (column-first would round different values).

Parity status: pinned in tests/test_oracle_pins.py -- the 1-D F(2,3) identity,
exact agreement with brute-force direct convolution on small integers, the
hand-worked Sobel fixture, the 16-versus-36 multiplication count the page
gives, and a hand-worked patch (tests/golden/winograd_input_rounding.txt)
that separates the fp16 model from the exact one and from column-first order.
"""
from __future__ import annotations

import numpy as np

BT = np.array([[1, 0, -1, 0], [0, 1, 1, 0], [0, -1, 1, 0], [0, 1, 0, -1]], dtype=np.float64)
G = np.array([[1, 0, 0], [0.5, 0.5, 0.5], [0.5, -0.5, 0.5], [0, 0, 1]], dtype=np.float64)
AT = np.array([[1, 1, 1, 0], [0, 1, -1, -1]], dtype=np.float64)


def _codec():
    from . import f64_to_f16   # the oracle's own fp16 rounding (plain C, RNE)
    return f64_to_f16


def matrices():
    """(B^T, G, A^T) of F(2x2, 3x3) as fp64 arrays (copies)."""
    return BT.copy(), G.copy(), AT.copy()


def weight_transform(w, model: str = "exact") -> np.ndarray:
    """U[4, 4, C, K] = G g G^T for each (c, k), g = w[:, :, c, k] (w HWIO fp16
    [3, 3, C, K]).  model "fp16": U rounded once to fp16 (returned as fp64
    values of those fp16 numbers)."""
    w64 = np.asarray(w, dtype=np.float16).astype(np.float64)
    assert w64.shape[:2] == (3, 3)
    U = np.einsum("ar,rsck,bs->abck", G, w64, G)
    if model == "fp16":
        return _codec()(U).astype(np.float64)
    assert model == "exact"
    return U


def patches(x, TH: int, TW: int) -> np.ndarray:
    """d[n, TH, TW, 4, 4, C]: the zero-padded 4x4 input patch of every whole
    2x2 output tile (rows 2i-1 .. 2i+2, columns 2j-1 .. 2j+2)."""
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    n, H, W, C = x64.shape
    xp = np.zeros((n, 2 * TH + 2, 2 * TW + 2, C))
    hh, ww = min(H, 2 * TH + 1), min(W, 2 * TW + 1)
    xp[:, 1:1 + hh, 1:1 + ww, :] = x64[:, :hh, :ww, :]
    d = np.empty((n, TH, TW, 4, 4, C))
    for a in range(4):
        for b in range(4):
            d[:, :, :, a, b, :] = xp[:, a:a + 2 * TH:2, b:b + 2 * TW:2, :]
    return d


def input_transform(d, model: str = "exact") -> np.ndarray:
    """V[..., 4, 4, C] = B^T d B over the patch axes (-3, -2) of d."""
    if model == "exact":
        return np.einsum("xa,...abc,yb->...xyc", BT, d, BT)
    assert model == "fp16"
    rnd = _codec()
    t = rnd(np.einsum("xa,...abc->...xbc", BT, d)).astype(np.float64)    # rows first: one rounding per entry
    return rnd(np.einsum("...xbc,yb->...xyc", t, BT)).astype(np.float64)  # then columns: one rounding


def conv_tiles(x, w, b=None, model: str = "exact") -> np.ndarray:
    """fp64 conv output [n, 2*TH, 2*TW, K] (+ b) of the 3x3 / stride 1 / pad 1
    cross-correlation over whole 2x2 tiles, by F(2x2, 3x3), TH = H // 2,
    TW = W // 2.  Images are processed one at a time (bounded memory)."""
    n, H, W, C = np.asarray(x).shape
    K = np.asarray(w).shape[-1]
    TH, TW = H // 2, W // 2
    U = weight_transform(w, model)                       # [4, 4, C, K]
    out = np.empty((n, 2 * TH, 2 * TW, K))
    for im in range(n):
        V = input_transform(patches(np.asarray(x)[im:im + 1], TH, TW), model)[0]   # [TH, TW, 4, 4, C]
        Vf = V.reshape(TH * TW, 4, 4, C)
        M = np.empty((TH * TW, 4, 4, K))
        for xi in range(4):
            for nu in range(4):
                M[:, xi, nu, :] = Vf[:, xi, nu, :] @ U[xi, nu]   # the 16 channel contractions
        Y = np.einsum("ia,tabk,jb->tijk", AT, M, AT)             # [tiles, 2, 2, K]
        out[im] = Y.reshape(TH, TW, 2, 2, K).transpose(0, 2, 1, 3, 4).reshape(2 * TH, 2 * TW, K)
    if b is not None:
        out += np.asarray(b, dtype=np.float16).astype(np.float64)
    return out


def multiplications_per_tile() -> tuple[int, int]:
    """(element-wise products of F(2x2,3x3) per tile, channel and output
    channel; products of the direct 3x3 convolution for the same 2x2 outputs)."""
    U = weight_transform(np.zeros((3, 3, 1, 1), dtype=np.float16))
    return int(U.shape[0] * U.shape[1]), 2 * 2 * 3 * 3


def chain_conv_pool(x, w, b, act_kind: int, pool: str = "max2x2", model: str = "exact"):
    """(y fp16, argmax uint8 or None, v fp16, c64 fp64) of pool(fp16(act(conv + b)))
    with the convolution evaluated by F(2x2, 3x3) under ``model``; the pooled
    window is the Winograd output tile.  Built from conv_tiles, the oracle's
    activation, fp16 codec and pools."""
    from . import act, avgpool2x2, f64_to_f16, maxpool2x2
    c64 = act(act_kind, conv_tiles(x, w, b, model))
    v = f64_to_f16(c64)
    if pool == "max2x2":
        y, am = maxpool2x2(v)
        return y, am, v, c64
    assert pool == "avg2x2"
    return avgpool2x2(v), None, v, c64
