"""gemm_conv_chain_amd -- Python binding of libfusedchain (MI355X / gfx950).

Argument marshalling only: every computation runs in the HIP kernels of
``libfusedchain.so`` behind the C ABI in ``include/fusedchain.h``.  PyTorch is
used for device memory and the current stream; there is no CPU or PyTorch
fallback -- if the library is missing, every call raises.

The functions mirror the C entry points:

* ``chain_gemm2(A, W0, b0, W1, b1, act)``      D1 = act(A W0 + b0) W1 + b1
* ``chain_conv_pool(x, w, b, act, pool)``      maxpool2x2(act(conv3x3(x) + b))
* ``chain_conv2(x, w0, b0, w1, b1, act)``      conv1x1(act(conv3x3(x) + b0)) + b1
* ``gemm_bias_act``, ``conv_bias_act``, ``maxpool2x2``   single operators
* ``pad_channels`` / ``pad_weight_channels``   zero padding of channel counts
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re

__all__ = ["TuneEntry", "tune_chain_gemm2_table", "auto_config", "tune_conv_pool", "conv_auto_config", "CONV_VARIANT", "lib", "FusedChainError", "chain_gemm2", "tune_chain_gemm2", "auto_variant", "tune_clear", "chain_gemmN", "chain_conv_pool", "chain_conv_bn_pool", "chain_conv2", "chain_convN", "convN_auto_variant", "tune_chain_convN",
           "gemm_bias_act", "conv_bias_act", "maxpool2x2", "avgpool2x2", "pad_channels", "pad_weight_channels", "abi_version", "ACT", "VARIANT",
           "LIB_PATH", "POISON_LIB_PATH", "poison_build", "HEADER_PATH", "exported_names"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfusedchain.so")
POISON_LIB_PATH = os.path.join(_HERE, "libfusedchain_poison.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fusedchain.h")

ACT = {"none": 0, "relu": 1, "gelu_tanh": 2, "hardswish": 3}
POOL = {"none": 0, "max2x2": 1, "avg2x2": 2}
VARIANT = {"auto": 0, "rf": 1, "lds": 2, "stream": 3, "pipe": 4}
CONV_VARIANT = {"auto": 0, "lds_weights": 1, "reg_weights": 2}


class FusedChainError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (fn, _lib_status_str(status), detail))


class ConvShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n", "h", "w", "c", "k", "r", "s", "stride", "pad")]


class TuneEntry(ctypes.Structure):
    """One configuration timed by the profiler: kernel form, tile-owning waves
    per block (0 = the form's own block shape), pipeline stages of the
    register-resident row stream (0 = the default 4, or 2), microseconds per
    launch."""
    _fields_ = [("variant", ctypes.c_int32), ("waves", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("us", ctypes.c_float)]


_lib = None
_poison_lib = None
_override = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


def lib():
    """The library every call goes through: libfusedchain.so (built by
    ``gemm_conv_chain_amd.build``), or the poison debug build inside a
    ``poison_build()`` block."""
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def poison_build():
    """Route every call inside the with-block through libfusedchain_poison.so,
    the -DFC_DEBUG_POISON build: its kernels overwrite each LDS buffer with a
    poison pattern (fp16 65504) when the barrier that releases it has passed,
    so a read that races its producer changes the results.  Test use only."""
    global _override, _poison_lib
    if _poison_lib is None:
        _poison_lib = _load(POISON_LIB_PATH)
    prev, _override = _override, _poison_lib
    try:
        yield _poison_lib
    finally:
        _override = prev


def _load(path):
    if not os.path.exists(path):
        raise FusedChainError("load", -1, "%s not built: run python -m gemm_conv_chain_amd.build"
                              % os.path.basename(path))
    L = ctypes.CDLL(path)
    L.fc_abi_version.restype = _i32
    L.fc_status_str.restype = ctypes.c_char_p
    L.fc_status_str.argtypes = [ctypes.c_int]
    L.fc_last_error.restype = ctypes.c_char_p
    L.chain_gemm2.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp]
    L.chain_gemm2_variant.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                      ctypes.c_int, _vp]
    L.chain_gemmN.argtypes = [_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(ctypes.c_int),
                              ctypes.POINTER(_i32), _vp, _i64, _vp]
    L.chain_conv_pool.argtypes = [_vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp, ctypes.POINTER(ConvShape),
                                  _vp, _vp]
    L.chain_conv2.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _i32, _vp, ctypes.POINTER(ConvShape), _vp]
    L.gemm_bias_act.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _i64, _i32, _i32, _vp]
    L.conv_bias_act.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, ctypes.POINTER(ConvShape), _vp]
    L.maxpool2x2.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
    L.avgpool2x2.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp]
    L.pad_channels.argtypes = [_vp, _vp, _i64, _i32, _i32, _i32, _vp]
    L.chain_gemm2_tune.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                   ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float), _vp]
    L.chain_gemm2_auto_variant.argtypes = [_i64, _i32, _i32, _i32, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.chain_convN.argtypes = [_vp, ctypes.POINTER(ConvShape), _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                              ctypes.POINTER(ctypes.c_int), ctypes.POINTER(_i32), _vp, _vp]
    L.chain_convN_variant.argtypes = [_vp, ctypes.POINTER(ConvShape), _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                      ctypes.POINTER(ctypes.c_int), ctypes.POINTER(_i32), _vp, ctypes.c_int, _vp]
    L.chain_convN_auto_variant.argtypes = [ctypes.POINTER(ConvShape), _i32, ctypes.POINTER(_i32),
                                           ctypes.POINTER(ctypes.c_int)]
    L.chain_convN_tune.argtypes = [_vp, ctypes.POINTER(ConvShape), _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                   ctypes.POINTER(ctypes.c_int), ctypes.POINTER(_i32), _vp, _i32,
                                   ctypes.POINTER(TuneEntry), _i32, ctypes.POINTER(_i32), ctypes.POINTER(TuneEntry), _vp]
    L.chain_conv_bn_pool.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp,
                                     ctypes.POINTER(ConvShape), _vp, _vp]
    L.chain_conv_pool_ex.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp,
                                     ctypes.POINTER(ConvShape), _vp, ctypes.c_int, _i32, _vp]
    L.chain_gemm2_ex.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                 ctypes.c_int, _i32, _i32, _vp]
    L.fc_probe_mfma.argtypes = [_i32, _i32, _vp, _vp, _i32, ctypes.POINTER(_i32), _vp]
    L.fc_probe_read.argtypes = [_vp, _i64, _vp, _i32, ctypes.POINTER(_i32), _vp]
    L.chain_gemm2_tune_ex.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                      ctypes.POINTER(TuneEntry), _i32, ctypes.POINTER(_i32),
                                      ctypes.POINTER(TuneEntry), _vp]
    L.chain_gemm2_auto_config.argtypes = [_i64, _i32, _i32, _i32, ctypes.c_int, ctypes.POINTER(TuneEntry)]
    L.chain_conv_pool_tune.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp,
                                       ctypes.POINTER(ConvShape), _vp, _i32, ctypes.POINTER(TuneEntry), _i32,
                                       ctypes.POINTER(_i32), ctypes.POINTER(TuneEntry), _vp]
    L.chain_conv_pool_auto_config.argtypes = [ctypes.POINTER(ConvShape), ctypes.c_int, ctypes.c_int, _i32,
                                              ctypes.POINTER(TuneEntry)]
    L.chain_conv2_ex.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _i32, _vp, ctypes.POINTER(ConvShape),
                                 _i32, _i32, _vp]
    L.chain_conv2_variant.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _i32, _vp, ctypes.POINTER(ConvShape),
                                      ctypes.c_int, _i32, _i32, _vp]
    L.chain_conv2_tune.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _i32, _vp, ctypes.POINTER(ConvShape),
                                   _i32, ctypes.POINTER(TuneEntry), _i32, ctypes.POINTER(_i32),
                                   ctypes.POINTER(TuneEntry), _vp]
    L.chain_conv2_auto_config.argtypes = [ctypes.POINTER(ConvShape), _i32, ctypes.c_int, ctypes.POINTER(TuneEntry)]
    L.winograd_weights.argtypes = [_vp, _vp, _i32, _i32, _vp]
    L.chain_conv_pool_winograd.argtypes = [_vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp,
                                           ctypes.POINTER(ConvShape), _vp, _vp]
    L.fc_tune_clear.restype = None
    L.fc_tune_clear.argtypes = []
    for name in ("chain_conv2_auto_config", "chain_conv2_ex", "chain_conv2_variant", "chain_conv2_tune", "winograd_weights", "chain_conv_pool_winograd", "chain_gemm2_ex", "chain_gemm2_tune_ex", "chain_gemm2_auto_config", "chain_conv_pool_tune",
                 "chain_conv_pool_auto_config", "chain_conv_pool_ex", "avgpool2x2", "fc_probe_mfma", "fc_probe_read", "chain_conv_bn_pool", "chain_convN", "chain_convN_variant", "chain_convN_auto_variant", "chain_convN_tune", "chain_gemm2_tune", "chain_gemm2_auto_variant", "chain_gemm2", "chain_gemm2_variant", "chain_gemmN", "chain_conv_pool", "chain_conv2", "gemm_bias_act",
                 "conv_bias_act", "maxpool2x2", "pad_channels"):
        getattr(L, name).restype = ctypes.c_int
    return L


def _lib_status_str(s):
    try:
        return lib().fc_status_str(int(s)).decode()
    except Exception:
        return str(s)


def abi_version() -> int:
    return int(lib().fc_abi_version())


def exported_names():
    """Function names declared in include/fusedchain.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([A-Za-z_0-9]+)\s*\(", text, re.M)))


def _check(fn, status):
    if status != 0:
        raise FusedChainError(fn, status, lib().fc_last_error().decode())


# ------------------------------------------------------------ tensor helpers
# The C ABI sees pointers only, so every size the kernels rely on is checked
# here, against the sizes the inputs imply, before the library is called:
# shapes, dtypes and contiguity first (ValueError / TypeError, testable with
# host tensors), then that every tensor is a device tensor on one device.
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ndim(t, name, ndim):
    """t (may be None) is a tensor with ndim dimensions; returns its shape."""
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor, got %s" % (name, type(t).__name__))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    return tuple(t.shape)


def _validate(items):
    """items: (tensor or None, name, shape, dtype) with shape a tuple of ints
    or None (any shape) and dtype None for float16.  Checks every shape,
    dtype and contiguity, then that all tensors sit on one CUDA device."""
    torch = _torch()
    live = []
    for t, name, shape, dtype in items:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor, got %s" % (name, type(t).__name__))
        want = torch.float16 if dtype is None else dtype
        if t.dtype != want:
            raise TypeError("%s must be %s, got %s" % (name, want, t.dtype))
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        live.append((t, name))
    dev = None
    for t, name in live:
        if not t.is_cuda:
            raise TypeError("%s must be a device tensor" % name)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, the other tensors on %s" % (name, t.device, dev))


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _act(a):
    return ACT[a] if isinstance(a, str) else int(a)


def _empty(shape, like, dtype=None):
    torch = _torch()
    return torch.empty(shape, dtype=like.dtype if dtype is None else dtype, device=like.device)


def _gemm2_shapes(A, W0, b0, W1, b1, out):
    M, K0 = _ndim(A, "A", 2)
    K0w, N0 = _ndim(W0, "W0", 2)
    N0w, N1 = _ndim(W1, "W1", 2)
    if K0w != K0 or N0w != N0:
        raise ValueError("shape mismatch A%s W0%s W1%s" % (tuple(A.shape), tuple(W0.shape), tuple(W1.shape)))
    if out is None:
        _validate([(A, "A", None, None), (W0, "W0", None, None), (b0, "b0", (N0,), None), (W1, "W1", None, None),
                   (b1, "b1", (N1,), None)])
        out = _empty((M, N1), A)
    _validate([(A, "A", None, None), (W0, "W0", None, None), (b0, "b0", (N0,), None), (W1, "W1", None, None),
               (b1, "b1", (N1,), None), (out, "out", (M, N1), None)])
    return M, K0, N0, N1, out


# ------------------------------------------------------------ entry points
def chain_gemm2(A, W0, b0, W1, b1, act="relu", out=None, variant="auto", waves=None, stages=0):
    """D1 [M, N1] = act(A [M,K0] @ W0 [K0,N0] + b0) @ W1 [N0,N1] + b1 (fp16).
    ``waves`` / ``stages`` (explicit variant only, chain_gemm2_ex): tile-owning
    waves per block and row-stream pipeline stages (4 or 2; 0 = 4) of the
    register-resident form."""
    M, K0, N0, N1, out = _gemm2_shapes(A, W0, b0, W1, b1, out)
    v = VARIANT[variant] if isinstance(variant, str) else int(variant)
    if waves is None and not stages:
        _check("chain_gemm2", lib().chain_gemm2_variant(_ptr(A), _ptr(W0), _ptr(b0), _act(act), _ptr(W1), _ptr(b1),
                                                        _ptr(out), M, K0, N0, N1, v, _stream(A)))
    else:
        _check("chain_gemm2_ex", lib().chain_gemm2_ex(_ptr(A), _ptr(W0), _ptr(b0), _act(act), _ptr(W1), _ptr(b1),
                                                      _ptr(out), M, K0, N0, N1, v, int(waves or 0), int(stages),
                                                      _stream(A)))
    return out


_VARIANT_NAME = {v: k for k, v in VARIANT.items()}


def tune_chain_gemm2(A, W0, b0, W1, b1, act="relu", out=None, reps=20):
    """Time every applicable variant of chain_gemm2 on these tensors (blocking),
    cache the fastest for this shape (later variant='auto' calls use it).
    Returns (best variant name, {variant name: us per launch}, out)."""
    M, K0, N0, N1, out = _gemm2_shapes(A, W0, b0, W1, b1, out)
    best = ctypes.c_int(-1)
    us = (ctypes.c_float * 4)()
    _check("chain_gemm2_tune", lib().chain_gemm2_tune(_ptr(A), _ptr(W0), _ptr(b0), _act(act), _ptr(W1), _ptr(b1),
                                                      _ptr(out), M, K0, N0, N1, int(reps), ctypes.byref(best), us,
                                                      _stream(A)))
    times = {_VARIANT_NAME[v]: float(us[v]) for v in (1, 2, 3) if us[v] >= 0}
    return _VARIANT_NAME[best.value], times, out


def tune_chain_gemm2_table(A, W0, b0, W1, b1, act="relu", out=None, reps=20):
    """Time every configuration of chain_gemm2 for these tensors (blocking) and
    cache the fastest.  Returns (best, table, out) where best and the table rows
    are dicts {variant, waves, us}."""
    M, K0, N0, N1, out = _gemm2_shapes(A, W0, b0, W1, b1, out)
    table = (TuneEntry * 16)()
    best = TuneEntry()
    n = _i32(0)
    _check("chain_gemm2_tune_ex", lib().chain_gemm2_tune_ex(_ptr(A), _ptr(W0), _ptr(b0), _act(act), _ptr(W1), _ptr(b1),
                                                            _ptr(out), M, K0, N0, N1, int(reps), table, 16,
                                                            ctypes.byref(n), ctypes.byref(best), _stream(A)))
    return _entry(best, _VARIANT_NAME), [_entry(table[i], _VARIANT_NAME) for i in range(min(n.value, 16))], out


def _entry(e, names):
    return {"variant": names[e.variant], "waves": int(e.waves), "stages": int(e.stages), "us": float(e.us)}


def auto_config(M, K0, N0, N1, act="relu"):
    """{variant, waves, stages} that chain_gemm2(variant='auto') runs for this shape."""
    e = TuneEntry()
    _check("chain_gemm2_auto_config", lib().chain_gemm2_auto_config(int(M), int(K0), int(N0), int(N1), _act(act),
                                                                    ctypes.byref(e)))
    d = _entry(e, _VARIANT_NAME)
    d.pop("us")
    return d


_CONV_VARIANT_NAME = {v: k for k, v in CONV_VARIANT.items()}


def tune_conv_pool(x, w, b, act="relu", pool="max2x2", scale=None, out=None, argmax=None, reps=20):
    """Time every configuration of the pooled conv chain for these tensors
    (blocking) and cache the fastest (chain_conv_pool_tune).  b is the bias,
    or the shift when scale is given.  Returns (best, table, out) with
    dict rows {variant, waves, us}."""
    sh = _conv_shape(x, w)
    P, Q = _conv_out_hw(sh)
    p = POOL[pool] if isinstance(pool, str) else int(pool)
    oshape = (sh.n, P // 2, Q // 2, sh.k)
    am = _argmax_tensor(argmax, oshape, x) if argmax is not True else None
    items = [(x, "x", None, None), (w, "w", None, None), (b, "b" if scale is None else "shift", (sh.k,), None),
             (scale, "scale", (sh.k,), None), (am, "argmax", oshape, _torch().uint8)]
    if out is None:
        _validate(items)
        out = _empty(oshape, x)
    _validate(items + [(out, "out", oshape, None)])
    if argmax is True:
        am = _argmax_tensor(True, oshape, x)
    table = (TuneEntry * 16)()
    best = TuneEntry()
    n = _i32(0)
    _check("chain_conv_pool_tune", lib().chain_conv_pool_tune(_ptr(x), _ptr(w), _ptr(scale), _ptr(b), _act(act), p,
                                                              _ptr(out), ctypes.byref(sh), _ptr(am), int(reps), table,
                                                              16, ctypes.byref(n), ctypes.byref(best), _stream(x)))
    return (_entry(best, _CONV_VARIANT_NAME), [_entry(table[i], _CONV_VARIANT_NAME) for i in range(min(n.value, 16))],
            out)


def conv_auto_config(n, h, w, c, k, act="relu", pool="max2x2", argmax=False):
    """{variant, waves, stages} that the pooled conv chain runs under variant='auto' (stages 0)."""
    e = TuneEntry()
    sh = ConvShape(n, h, w, c, k, 3, 3, 1, 1)
    p = POOL[pool] if isinstance(pool, str) else int(pool)
    _check("chain_conv_pool_auto_config", lib().chain_conv_pool_auto_config(ctypes.byref(sh), _act(act), p,
                                                                            1 if argmax else 0, ctypes.byref(e)))
    d = _entry(e, _CONV_VARIANT_NAME)
    d.pop("us")
    return d


def auto_variant(M, K0, N0, N1, act="relu"):
    """Name of the variant chain_gemm2(variant='auto') runs for this shape."""
    v = ctypes.c_int(-1)
    _check("chain_gemm2_auto_variant", lib().chain_gemm2_auto_variant(int(M), int(K0), int(N0), int(N1), _act(act),
                                                                      ctypes.byref(v)))
    return _VARIANT_NAME[v.value]


def probe_mfma(stamps, sink, waves_per_simd=2, iters=2048):
    """Enqueue the matrix-core rate probe (fc_probe_mfma) on the current
    stream; stamps: int64 [4 * n], sink: float32 [n] with n >= the CU count
    (checked by the library before launching).  Returns the grid
    size (blocks); FLOPs per launch = blocks * 4 * waves_per_simd * iters * 8 * 32768."""
    torch = _torch()
    _validate([(stamps, "stamps", None, torch.int64), (sink, "sink", None, torch.float32)])
    blocks = _i32(0)
    capacity = min(stamps.numel() // 4, sink.numel())
    _check("fc_probe_mfma", lib().fc_probe_mfma(int(waves_per_simd), int(iters), _ptr(stamps), _ptr(sink),
                                                int(capacity), ctypes.byref(blocks), _stream(stamps)))
    return blocks.value


def probe_read(buf, sink):
    """Enqueue the memory read-rate probe (fc_probe_read) over the bytes of the
    contiguous device tensor buf on the current stream; sink: int32 [n] with n
    >= the grid (2 x the CU count for large buffers).  Returns the grid size."""
    torch = _torch()
    _validate([(buf, "buf", None, getattr(buf, "dtype", None)), (sink, "sink", None, torch.int32)])
    blocks = _i32(0)
    _check("fc_probe_read", lib().fc_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                int(sink.numel()), ctypes.byref(blocks), _stream(buf)))
    return blocks.value


def tune_clear():
    """Forget every tuned variant choice."""
    lib().fc_tune_clear()


def chain_gemmN(A, Ws, bs, acts, out=None):
    """D = act[n-1](... act[0](A @ Ws[0] + bs[0]) ... @ Ws[n-1] + bs[n-1]) (fp16; n = 3 or 4),
    every intermediate rounded once to fp16 and kept on chip."""
    n = len(Ws)
    if len(bs) != n or len(acts) != n:
        raise ValueError("Ws, bs and acts must have the same length")
    M, K = _ndim(A, "A", 2)
    widths = [K]
    for i, W in enumerate(Ws):
        r, c = _ndim(W, "W%d" % i, 2)
        if r != widths[i]:
            raise ValueError("W%d has %d rows, the previous width is %d" % (i, r, widths[i]))
        widths.append(c)
    items = [(A, "A", None, None)]
    for i in range(n):
        items += [(Ws[i], "W%d" % i, None, None), (bs[i], "b%d" % i, (widths[i + 1],), None)]
    if out is None:
        _validate(items)
        out = _empty((M, widths[-1]), A)
    _validate(items + [(out, "out", (M, widths[-1]), None)])
    Wp = (_vp * n)(*[W.data_ptr() for W in Ws])
    bp = (_vp * n)(*[None if b is None else b.data_ptr() for b in bs])
    ap = (ctypes.c_int * n)(*[_act(a) for a in acts])
    wp = (_i32 * (n + 1))(*widths)
    _check("chain_gemmN", lib().chain_gemmN(_ptr(A), n, Wp, bp, ap, wp, _ptr(out), M, _stream(A)))
    return out


def gemm_bias_act(A, W, b, act="none", out=None):
    """C [M, N] = act(A [M,K] @ W [K,N] + b) (fp16)."""
    M, K = _ndim(A, "A", 2)
    Kw, N = _ndim(W, "W", 2)
    if Kw != K:
        raise ValueError("shape mismatch A%s W%s" % (tuple(A.shape), tuple(W.shape)))
    items = [(A, "A", None, None), (W, "W", None, None), (b, "b", (N,), None)]
    if out is None:
        _validate(items)
        out = _empty((M, N), A)
    _validate(items + [(out, "out", (M, N), None)])
    _check("gemm_bias_act", lib().gemm_bias_act(_ptr(A), _ptr(W), _ptr(b), _act(act), _ptr(out), M, K, N,
                                                _stream(A)))
    return out


def _conv_shape(x, w, stride=1, pad=1):
    n, h, wd, c = _ndim(x, "x", 4)
    r, s, c2, k = _ndim(w, "w", 4)
    if c2 != c:
        raise ValueError("x has %d channels, w expects %d" % (c, c2))
    return ConvShape(n, h, wd, c, k, r, s, stride, pad)


def _conv_out_hw(sh):
    P = (sh.h + 2 * sh.pad - sh.r) // sh.stride + 1
    Q = (sh.w + 2 * sh.pad - sh.s) // sh.stride + 1
    return max(P, 0), max(Q, 0)


def _argmax_tensor(argmax, oshape, like):
    """None/False: no argmax; True: allocate one; else the caller's uint8 tensor."""
    if argmax is True:
        return _empty(oshape, like, _torch().uint8)
    if argmax is None or argmax is False:
        return None
    return argmax


def chain_conv_pool(x, w, b, act="relu", pool="max2x2", out=None, argmax=None, variant="auto", waves=0):
    """y = maxpool2x2(act(conv3x3(x, w) + b)) (or act(conv+b) with pool='none').
    ``argmax``: None, True (allocate) or a uint8 tensor; returns y or (y, argmax).
    ``variant``: kernel form ("auto", "lds_weights", "reg_weights"); ``waves``:
    tile-owning waves per block of the pooled "lds_weights" form (0 = 8)."""
    return _conv_pool("chain_conv_pool", x, w, None, b, act, pool, out, argmax, variant, waves)


def chain_conv_bn_pool(x, w, scale, shift, act="relu", pool="max2x2", out=None, argmax=None, variant="auto",
                       waves=0):
    """y = maxpool2x2(act(conv3x3(x, w) * scale + shift)) per output channel (batch
    norm at inference as a scale and a shift); pool='none' stores act(...)."""
    if scale is None:
        raise ValueError("scale is required")
    return _conv_pool("chain_conv_bn_pool", x, w, scale, shift, act, pool, out, argmax, variant, waves)


def _conv_pool(fn, x, w, scale, b, act, pool, out, argmax, variant="auto", waves=0):
    sh = _conv_shape(x, w)
    P, Q = _conv_out_hw(sh)
    p = POOL[pool] if isinstance(pool, str) else int(pool)
    v = CONV_VARIANT[variant] if isinstance(variant, str) else int(variant)
    oshape = (sh.n, P // 2, Q // 2, sh.k) if p else (sh.n, P, Q, sh.k)
    am = _argmax_tensor(argmax, oshape, x) if argmax is not True else None   # the caller's, checked below
    items = [(x, "x", None, None), (w, "w", None, None), (b, "b" if scale is None else "shift", (sh.k,), None),
             (scale, "scale", (sh.k,), None), (am, "argmax", oshape, _torch().uint8)]
    if out is None:
        _validate(items)
        out = _empty(oshape, x)
    _validate(items + [(out, "out", oshape, None)])
    if argmax is True:
        am = _argmax_tensor(True, oshape, x)
    st = lib().chain_conv_pool_ex(_ptr(x), _ptr(w), _ptr(scale), _ptr(b), _act(act), p, _ptr(out), ctypes.byref(sh),
                                  _ptr(am), v, int(waves), _stream(x))
    _check(fn, st)
    return (out, am) if am is not None else out


def winograd_weights(w, out=None):
    """U = G g G^T of a 3x3 HWIO weight w [3, 3, c, k] for chain_conv_pool_winograd,
    in the library's operand layout, returned as a [16, c/8, k, 8] fp16 tensor."""
    r, s, c, k = _ndim(w, "w", 4)
    if (r, s) != (3, 3):
        raise ValueError("w must be [3, 3, c, k], got %s" % ((r, s, c, k),))
    if c % 8 or k % 8:
        raise ValueError("c=%d and k=%d must be multiples of 8" % (c, k))
    oshape = (16, c // 8, k, 8)
    if out is None:
        _validate([(w, "w", None, None)])
        out = _empty(oshape, w)
    _validate([(w, "w", None, None), (out, "out", oshape, None)])
    _check("winograd_weights", lib().winograd_weights(_ptr(w), _ptr(out), c, k, _stream(w)))
    return out


def chain_conv_pool_winograd(x, U, b, act="relu", pool="max2x2", out=None, argmax=None):
    """y = pool2x2(act(conv3x3(x, w) + b)) with the conv by Winograd F(2x2, 3x3)
    from U = winograd_weights(w).  ``argmax`` as for chain_conv_pool (max pool)."""
    n, h, wd, c = _ndim(x, "x", 4)
    ushape = _ndim(U, "U", 4)
    if ushape[0] != 16 or ushape[1] != c // 8 or ushape[3] != 8 or c % 8:
        raise ValueError("U must be [16, %d, k, 8] (winograd_weights of a [3, 3, %d, k] weight), got %s"
                         % (c // 8, c, ushape))
    k = ushape[2]
    sh = ConvShape(n, h, wd, c, k, 3, 3, 1, 1)
    p = POOL[pool] if isinstance(pool, str) else int(pool)
    oshape = (n, h // 2, wd // 2, k)
    am = _argmax_tensor(argmax, oshape, x) if argmax is not True else None
    items = [(x, "x", None, None), (U, "U", None, None), (b, "b", (k,), None),
             (am, "argmax", oshape, _torch().uint8)]
    if out is None:
        _validate(items)
        out = _empty(oshape, x)
    _validate(items + [(out, "out", oshape, None)])
    if argmax is True:
        am = _argmax_tensor(True, oshape, x)
    st = lib().chain_conv_pool_winograd(_ptr(x), _ptr(U), _ptr(b), _act(act), p, _ptr(out), ctypes.byref(sh),
                                        _ptr(am), _stream(x))
    _check("chain_conv_pool_winograd", st)
    return (out, am) if am is not None else out


def conv_bias_act(x, w, b, act="relu", out=None):
    """y NHWC = act(conv3x3(x, w) + b)."""
    sh = _conv_shape(x, w)
    P, Q = _conv_out_hw(sh)
    items = [(x, "x", None, None), (w, "w", None, None), (b, "b", (sh.k,), None)]
    if out is None:
        _validate(items)
        out = _empty((sh.n, P, Q, sh.k), x)
    _validate(items + [(out, "out", (sh.n, P, Q, sh.k), None)])
    _check("conv_bias_act", lib().conv_bias_act(_ptr(x), _ptr(w), _ptr(b), _act(act), _ptr(out), ctypes.byref(sh),
                                                _stream(x)))
    return out


def _w1x1(t, name, kin):
    """A 1x1 conv weight: [kin, kout] or [1, 1, kin, kout]; returns kout."""
    shp = _ndim(t, name, None)
    if len(shp) == 2 and shp[0] == kin:
        return shp[1]
    if len(shp) == 4 and shp[:3] == (1, 1, kin):
        return shp[3]
    raise ValueError("%s must be [%d, k] or [1, 1, %d, k], got %s" % (name, kin, kin, shp))


def _conv2_prep(x, w0, b0, w1, b1, out):
    sh = _conv_shape(x, w0)
    P, Q = _conv_out_hw(sh)
    k1 = _w1x1(w1, "w1", sh.k)
    items = [(x, "x", None, None), (w0, "w0", None, None), (b0, "b0", (sh.k,), None), (w1, "w1", None, None),
             (b1, "b1", (k1,), None)]
    if out is None:
        _validate(items)
        out = _empty((sh.n, P, Q, k1), x)
    _validate(items + [(out, "out", (sh.n, P, Q, k1), None)])
    return sh, k1, out


def chain_conv2(x, w0, b0, w1, b1, act="relu", out=None, waves=0, stages=0, variant="auto"):
    """y = conv1x1(act(conv3x3(x, w0) + b0), w1) + b1; w1 is [k0, k1] or [1,1,k0,k1].
    ``variant``: kernel form ("auto", "rf" or "pipe"); for "rf", ``waves``:
    tile-owning waves per block (1..8) and ``stages``: row-stream pipeline
    stages (4 or 2; 0 = 4).  waves > 0 with variant "auto" means "rf"."""
    sh, k1, out = _conv2_prep(x, w0, b0, w1, b1, out)
    v = VARIANT[variant] if isinstance(variant, str) else int(variant)
    if v == 0 and waves:
        v = VARIANT["rf"]
    _check("chain_conv2", lib().chain_conv2_variant(_ptr(x), _ptr(w0), _ptr(b0), _act(act), _ptr(w1), _ptr(b1), k1,
                                                    _ptr(out), ctypes.byref(sh), v, int(waves), int(stages),
                                                    _stream(x)))
    return out


def tune_chain_conv2(x, w0, b0, w1, b1, act="relu", out=None, reps=20):
    """Time every block shape of the conv3x3 -> conv1x1 chain for these tensors
    (blocking) and cache the fastest (chain_conv2_tune).  Returns (best, table,
    out) with dict rows {variant, waves, us}."""
    sh, k1, out = _conv2_prep(x, w0, b0, w1, b1, out)
    table = (TuneEntry * 16)()
    best = TuneEntry()
    n = _i32(0)
    _check("chain_conv2_tune", lib().chain_conv2_tune(_ptr(x), _ptr(w0), _ptr(b0), _act(act), _ptr(w1), _ptr(b1), k1,
                                                      _ptr(out), ctypes.byref(sh), int(reps), table, 16,
                                                      ctypes.byref(n), ctypes.byref(best), _stream(x)))
    return _entry(best, _VARIANT_NAME), [_entry(table[i], _VARIANT_NAME) for i in range(min(n.value, 16))], out


def conv2_auto_config(n, h, w, c, k0, k1, act="relu"):
    """{variant, waves, stages} that chain_conv2 runs for this shape (waves=0)."""
    e = TuneEntry()
    sh = ConvShape(n, h, w, c, k0, 3, 3, 1, 1)
    _check("chain_conv2_auto_config", lib().chain_conv2_auto_config(ctypes.byref(sh), int(k1), _act(act),
                                                                    ctypes.byref(e)))
    d = _entry(e, _VARIANT_NAME)
    d.pop("us")
    return d


def convN_auto_variant(n, h, w, c, ks):
    """The kernel form ("pipe" or "rf") chain_convN runs for x [n,h,w,c] and
    stage widths ks (host only)."""
    sh = ConvShape(n, h, w, c, ks[0], 3, 3, 1, 1)
    kp = (_i32 * len(ks))(*ks)
    v = ctypes.c_int(-1)
    _check("chain_convN_auto_variant", lib().chain_convN_auto_variant(ctypes.byref(sh), len(ks), kp, ctypes.byref(v)))
    return _VARIANT_NAME[v.value]


def _convN_prep(x, ws, bs, acts, out):
    n = len(ws)
    if len(bs) != n or len(acts) != n:
        raise ValueError("ws, bs and acts must have the same length")
    sh = _conv_shape(x, ws[0])
    P, Q = _conv_out_hw(sh)
    ks = [sh.k]
    for i in range(1, n):
        ks.append(_w1x1(ws[i], "w%d" % i, ks[-1]))
    items = [(x, "x", None, None)]
    for i in range(n):
        items += [(ws[i], "w%d" % i, None, None), (bs[i], "b%d" % i, (ks[i],), None)]
    if out is None:
        _validate(items)
        out = _empty((sh.n, P, Q, ks[-1]), x)
    _validate(items + [(out, "out", (sh.n, P, Q, ks[-1]), None)])
    wp = (_vp * n)(*[w.data_ptr() for w in ws])
    bp = (_vp * n)(*[None if b is None else b.data_ptr() for b in bs])
    ap = (ctypes.c_int * n)(*[_act(a) for a in acts])
    kp = (_i32 * n)(*ks)
    return sh, n, wp, bp, ap, kp, out


def chain_convN(x, ws, bs, acts, out=None, variant="auto"):
    """y = stage_{n-1}(... stage_0(x)): stage 0 = act[0](conv3x3(x, ws[0]) + bs[0]),
    stage i > 0 = act[i](1x1 conv with ws[i] [k_{i-1}, k_i] (or [1,1,k_{i-1},k_i]) + bs[i]);
    n = 3 or 4, every intermediate rounded once to fp16 and kept on chip.
    ``variant``: kernel form ("auto", "rf" or "pipe")."""
    sh, n, wp, bp, ap, kp, out = _convN_prep(x, ws, bs, acts, out)
    v = VARIANT[variant] if isinstance(variant, str) else int(variant)
    _check("chain_convN", lib().chain_convN_variant(_ptr(x), ctypes.byref(sh), n, wp, bp, ap, kp, _ptr(out), v,
                                                    _stream(x)))
    return out


def tune_chain_convN(x, ws, bs, acts, out=None, reps=20):
    """Time each kernel form of the N-stage conv chain for these tensors
    (blocking) and cache the fastest (chain_convN_tune).  Returns (best,
    table, out) with dict rows {variant, waves, stages, us}."""
    sh, n, wp, bp, ap, kp, out = _convN_prep(x, ws, bs, acts, out)
    table = (TuneEntry * 4)()
    best = TuneEntry()
    cnt = _i32(0)
    _check("chain_convN_tune", lib().chain_convN_tune(_ptr(x), ctypes.byref(sh), n, wp, bp, ap, kp, _ptr(out),
                                                      int(reps), table, 4, ctypes.byref(cnt), ctypes.byref(best),
                                                      _stream(x)))
    return _entry(best, _VARIANT_NAME), [_entry(table[i], _VARIANT_NAME) for i in range(min(cnt.value, 4))], out


def avgpool2x2(x, out=None):
    """y [n, h/2, w/2, c] = 2x2/2 average pool of NHWC x (fp16 mean of each window)."""
    n, h, w, c = _ndim(x, "x", 4)
    oshape = (n, h // 2, w // 2, c)
    if out is None:
        _validate([(x, "x", None, None)])
        out = _empty(oshape, x)
    _validate([(x, "x", None, None), (out, "out", oshape, None)])
    _check("avgpool2x2", lib().avgpool2x2(_ptr(x), _ptr(out), n, h, w, c, _stream(x)))
    return out


def maxpool2x2(x, out=None, argmax=None):
    """y [n, h/2, w/2, c] = 2x2/2 max pool of NHWC x (+ optional argmax)."""
    n, h, w, c = _ndim(x, "x", 4)
    oshape = (n, h // 2, w // 2, c)
    am = _argmax_tensor(argmax, oshape, x) if argmax is not True else None   # the caller's, checked below
    items = [(x, "x", None, None), (am, "argmax", oshape, _torch().uint8)]
    if out is None:
        _validate(items)
        out = _empty(oshape, x)
    _validate(items + [(out, "out", oshape, None)])
    if argmax is True:
        am = _argmax_tensor(True, oshape, x)
    _check("maxpool2x2", lib().maxpool2x2(_ptr(x), _ptr(out), _ptr(am), n, h, w, c, _stream(x)))
    return (out, am) if am is not None else out


def pad_channels(x, c_out):
    """Zero-pad the channels (last dim) of NHWC x to c_out."""
    _ndim(x, "x", None)
    _validate([(x, "x", None, None)])
    c_in = x.shape[-1]
    out = _torch().empty(tuple(x.shape[:-1]) + (c_out,), dtype=x.dtype, device=x.device)
    _check("pad_channels", lib().pad_channels(_ptr(x), _ptr(out), x.numel() // max(c_in, 1), c_in, c_out, 1,
                                              _stream(x)))
    return out


def pad_weight_channels(w, c_out):
    """Zero-pad the input channels of HWIO w [r,s,c,k] to c_out."""
    _ndim(w, "w", 4)
    _validate([(w, "w", None, None)])
    r, s, c_in, k = w.shape
    out = _torch().empty((r, s, c_out, k), dtype=w.dtype, device=w.device)
    _check("pad_channels", lib().pad_channels(_ptr(w), _ptr(out), r * s, c_in, c_out, k, _stream(w)))
    return out
