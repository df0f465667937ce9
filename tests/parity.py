"""Comparison helpers for GPU-vs-oracle parity (test infrastructure)."""
import numpy as np

# Tolerance of the fused chains against the fp64 oracle:
#   max |gpu - ref| <= REL * max |ref| + ABS   over the whole compared tensor.
REL = 1e-2
ABS = 1e-3


def to_np(t):
    return t.detach().cpu().numpy()


def assert_close(gpu, ref, what=""):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite GPU output" % what
    if r.size == 0:
        return 0.0
    err = float(np.max(np.abs(g - r)))
    tol = REL * float(np.max(np.abs(r))) + ABS
    assert err <= tol, "%s: max|err| %.3e > tol %.3e (max|ref| %.3e)" % (what, err, tol, np.max(np.abs(r)))
    return err


def ulp16(x):
    """Spacing of fp16 values at |x| (subnormal spacing 2^-24 below 2^-14)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def pool_tie_mask(conv64, P, Q):
    """Windows whose argmax is not robust: the fp64 post-activation maximum is
    <= 0 (all values tied at 0 after ReLU) or the top two values differ by at
    most 2 fp16 ulps of the maximum (fp32 vs fp64 accumulation can move each
    rounded value by one ulp).  conv64: [n, P, Q, K] fp64 -> bool [n, P/2, Q/2, K]."""
    n, _, _, K = conv64.shape
    PO, QO = P // 2, Q // 2
    w = conv64[:, :2 * PO, :2 * QO, :].reshape(n, PO, 2, QO, 2, K).transpose(0, 1, 3, 5, 2, 4).reshape(
        n, PO, QO, K, 4)
    s = np.sort(w, axis=-1)
    top, second = s[..., 3], s[..., 2]
    return (top <= 0) | (top - second <= 2 * ulp16(top))
