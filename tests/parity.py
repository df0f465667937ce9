"""Comparison helpers for GPU-vs-oracle parity (test infrastructure)."""
import json
import os

import numpy as np

# Tolerance of the fused chains against the fp64 oracle:
#   max |gpu - ref| <= REL * max |ref| + ABS   over the whole compared tensor.
REL = 1e-2
ABS = 1e-3

# Diagnostics of every whole-tensor comparison made in this process (what,
# elements, max|err|, tolerance, fraction bit-equal to fp16(ref), max fp16-ulp
# distance); written as JSON lines to $FC_PARITY_DIAG when that is set.
DIAG = []


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


def ordered16(h):
    """fp16 bit patterns -> integers in the order of the values (+0 and -0 both
    0), so that |ordered16(a) - ordered16(b)| counts the fp16 values between a
    and b: their distance in units in the last place."""
    u = np.asarray(h, dtype=np.float16).view(np.uint16).astype(np.int64)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)


def diagnostics(gpu16, ref64, ref16=None):
    """Fraction of GPU outputs bit-equal to the oracle's fp16 rounding of its
    fp64 result, and the largest distance between the two in fp16 ulps.
    ref16 (the oracle's own rounding) is computed with the oracle's codec when
    not given."""
    g = np.asarray(gpu16, dtype=np.float16)
    if ref16 is None:
        import oracle
        ref16 = oracle.f64_to_f16(np.asarray(ref64, dtype=np.float64))
    r = np.asarray(ref16, dtype=np.float16)
    if g.size == 0:
        return {"elements": 0, "bit_equal_frac": 1.0, "max_ulp": 0}
    d = np.abs(ordered16(g) - ordered16(r))
    return {"elements": int(g.size), "bit_equal_frac": float(np.mean(d == 0)), "max_ulp": int(d.max()),
            "frac_within_1ulp": float(np.mean(d <= 1))}


def check_full(gpu16, ref64, what, ref16=None):
    """Whole-tensor comparison: the tolerance over every element (max|ref|
    over the whole tensor), plus the bit-equality / ulp diagnostics, printed
    and recorded."""
    err = assert_close(gpu16, ref64, what)
    r = np.asarray(ref64, dtype=np.float64)
    rec = {"what": what, "max_err": err, "tol": REL * float(np.max(np.abs(r))) + ABS if r.size else ABS}
    rec.update(diagnostics(gpu16, ref64, ref16))
    DIAG.append(rec)
    print("parity %-40s n=%d max|err| %.3e tol %.3e bit-equal %.4f max %d ulp" % (
        what, rec["elements"], err, rec["tol"], rec["bit_equal_frac"], rec["max_ulp"]), flush=True)
    path = os.environ.get("FC_PARITY_DIAG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    return rec


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
