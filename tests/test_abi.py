"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments synchronously (validation runs
before any HIP call, so these need no GPU and launch nothing)."""
import ctypes

import pytest

import gemm_conv_chain_amd as fc

pytestmark = pytest.mark.cpu

OK, E_NULL, E_SHAPE, E_ALIGN, E_UNSUP, E_HIP, E_ARG = range(7)
P = ctypes.c_void_p(0x10000)       # fake, 16-byte aligned device pointers:
P2 = ctypes.c_void_p(0x20000)      # validation never dereferences them
BAD = ctypes.c_void_p(0x10002)     # misaligned
NUL = None


@pytest.fixture(scope="module")
def L():
    return fc.lib()


def test_exports_every_declared_symbol(L):
    names = fc.exported_names()
    for n in ("chain_gemm2", "chain_gemm2_variant", "chain_gemmN", "chain_conv_pool", "chain_conv2", "gemm_bias_act",
              "conv_bias_act", "maxpool2x2", "pad_channels", "fc_abi_version", "fc_status_str", "fc_last_error",
              "chain_gemm2_tune", "chain_gemm2_auto_variant", "fc_tune_clear", "chain_convN", "chain_conv_bn_pool", "fc_probe_mfma", "chain_conv_pool_ex", "chain_gemm2_ex",
              "chain_gemm2_tune_ex", "chain_gemm2_auto_config", "chain_conv_pool_tune", "chain_conv_pool_auto_config",
              "chain_conv2_variant", "chain_convN_variant", "chain_convN_auto_variant", "chain_convN_tune", "chain_conv2_ex", "chain_conv2_tune", "chain_conv2_auto_config"):
        assert n in names
    for n in names:
        assert hasattr(L, n), n


def test_poison_build_exports_the_same_abi(L):
    # the LDS-poison debug build is the same library with extra LDS writes
    with fc.poison_build() as D:
        assert fc.lib() is D and D is not L
        for n in fc.exported_names():
            assert hasattr(D, n), n
        assert D.fc_abi_version() == L.fc_abi_version()
        # validation is unchanged: a null operand is refused before any HIP call
        assert D.chain_gemm2(NUL, P, P, 1, P, P, P, 64, 64, 64, 64, NUL) == E_NULL
    assert fc.lib() is L


def test_version_and_status_strings(L):
    assert fc.abi_version() == 4
    for code, name in enumerate(["FC_OK", "FC_E_NULL", "FC_E_SHAPE", "FC_E_ALIGN", "FC_E_UNSUPPORTED", "FC_E_HIP",
                                 "FC_E_ARG"]):
        assert L.fc_status_str(code).decode() == name


def g2(L, A=P, W0=P, b0=NUL, act=1, W1=P, b1=NUL, D1=P2, M=512, K0=64, N0=64, N1=64, variant=0):
    return L.chain_gemm2_variant(A, W0, b0, act, W1, b1, D1, M, K0, N0, N1, variant, None)


def test_chain_gemm2_validation(L):
    assert g2(L, A=NUL) == E_NULL
    assert g2(L, D1=NUL) == E_NULL
    assert g2(L, M=-1) == E_SHAPE
    assert g2(L, K0=0) == E_SHAPE
    assert g2(L, K0=60) == E_SHAPE          # not a multiple of 8 (128-bit vectors)
    assert g2(L, N1=20) == E_SHAPE
    assert g2(L, A=BAD) == E_ALIGN
    assert g2(L, b0=BAD) == E_ALIGN
    assert g2(L, act=7) == E_ARG
    assert g2(L, act=4) == E_ARG
    assert g2(L, variant=5) == E_ARG
    assert g2(L, variant=4) == E_ARG
    assert g2(L, N0=256, N1=16136, variant=3) == E_UNSUP   # streamed: biases must fit beside the weight buffers
    assert g2(L, N0=264) == E_UNSUP          # residence: one block owns all N0 <= 256
    assert g2(L, N0=256, variant=1) == E_UNSUP   # register-resident needs N0 <= 128
    assert b"N0" in L.fc_last_error()


def gn(L, n=3, widths=(64, 64, 64, 64, 64), W=None, b=None, acts=None, A=P, D=P2, M=512):
    Wp = (ctypes.c_void_p * 4)(*([P.value] * 4 if W is None else W))
    bp = None if b is None else (ctypes.c_void_p * 4)(*b)
    ap = (ctypes.c_int * 4)(*(acts or [1, 1, 1, 0]))
    wp = (ctypes.c_int32 * 5)(*widths)
    return L.chain_gemmN(A, n, Wp, bp, ap, wp, D, M, None)


def test_chain_gemmN_validation(L):
    assert gn(L, n=2) == E_UNSUP                    # two GEMMs: chain_gemm2
    assert gn(L, n=5) == E_UNSUP
    assert gn(L, widths=(64, 60, 64, 64, 64)) == E_SHAPE
    assert gn(L, widths=(64, 64, 0, 64, 64)) == E_SHAPE
    assert gn(L, A=NUL) == E_NULL
    assert gn(L, W=[P.value, None, P.value, P.value]) == E_NULL
    assert gn(L, W=[P.value, BAD.value, P.value, P.value]) == E_ALIGN
    assert gn(L, acts=[1, 9, 1, 0]) == E_ARG
    assert gn(L, widths=(64, 136, 64, 64, 64)) == E_UNSUP   # an intermediate wider than 128
    assert b"128" in L.fc_last_error()
    assert gn(L, M=0) == OK                          # nothing to launch


def test_gemm_bias_act_validation(L):
    assert L.gemm_bias_act(NUL, P, NUL, 0, P2, 8, 8, 8, None) == E_NULL
    assert L.gemm_bias_act(P, P, NUL, 0, P2, 8, 12, 8, None) == E_SHAPE
    assert L.gemm_bias_act(P, P, BAD, 0, P2, 8, 8, 8, None) == E_ALIGN
    assert L.gemm_bias_act(P, P, NUL, 4, P2, 8, 8, 8, None) == E_ARG


def shape(n=1, h=8, w=8, c=64, k=128, r=3, s=3, stride=1, pad=1):
    return fc.ConvShape(n, h, w, c, k, r, s, stride, pad)


def test_conv_validation(L):
    sh = shape()
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, None, NUL, None) == E_NULL
    assert L.chain_conv_pool(NUL, P, NUL, 1, 1, P2, ctypes.byref(sh), NUL, None) == E_NULL
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, ctypes.byref(shape(c=60)), NUL, None) == E_SHAPE
    # any c % 8 == 0 is implemented (n = 0: validated, nothing to launch)
    for c in (8, 24, 40, 56):
        assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, ctypes.byref(shape(n=0, c=c)), NUL, None) == OK
        assert L.conv_bias_act(P, P, NUL, 1, P2, ctypes.byref(shape(n=0, c=c)), None) == OK
        assert L.chain_conv2(P, P, NUL, 1, P, NUL, 64, P2, ctypes.byref(shape(n=0, c=c, k=64)), None) == OK
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, ctypes.byref(shape(k=136)), NUL, None) == E_UNSUP
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, ctypes.byref(shape(r=5, s=5)), NUL, None) == E_UNSUP
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, ctypes.byref(shape(stride=2)), NUL, None) == E_UNSUP
    assert L.chain_conv_pool(P, P, NUL, 1, 3, P2, ctypes.byref(sh), NUL, None) == E_ARG   # pool kinds are 0..2
    assert L.chain_conv_pool(P, P, NUL, 1, 0, P2, ctypes.byref(sh), P, None) == E_ARG  # argmax needs a pool
    assert L.chain_conv_pool(BAD, P, NUL, 1, 1, P2, ctypes.byref(sh), NUL, None) == E_ALIGN
    assert L.conv_bias_act(P, P, NUL, 1, P2, ctypes.byref(shape(h=-1)), None) == E_SHAPE
    assert L.chain_conv2(P, P, NUL, 1, P, NUL, 20, P2, ctypes.byref(shape(k=64)), None) == E_SHAPE
    assert L.chain_conv2(P, P, NUL, 1, P, NUL, 256, P2, ctypes.byref(shape(k=256)), None) == E_UNSUP
    assert L.chain_conv2(P, P, NUL, 1, NUL, NUL, 256, P2, ctypes.byref(shape(k=64)), None) == E_NULL
    # weights-resident kernels: the HWIO weights must fit in LDS
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, ctypes.byref(shape(c=96, k=96)), NUL, None) == E_UNSUP
    assert L.chain_conv2(P, P, NUL, 1, P, NUL, 64, P2, ctypes.byref(shape(c=64, k=128)), None) == E_UNSUP
    # pixel indices are decoded in 32 bits: n*h*w must stay below 2^31
    big = shape(n=32768, h=256, w=256)
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, ctypes.byref(big), NUL, None) == E_UNSUP
    assert L.chain_conv2(P, P, NUL, 1, P, NUL, 64, P2, ctypes.byref(shape(n=32768, h=256, w=256, k=64)),
                         None) == E_UNSUP
    assert b"2^31" in L.fc_last_error()
    # 3x3 tap offsets are 32-bit: (w + 2) * c must stay below 2^30 (a very wide row)
    wide = shape(n=1, h=1, w=(1 << 24), c=64)
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, ctypes.byref(wide), NUL, None) == E_UNSUP
    assert b"32 bits" in L.fc_last_error()
    assert L.conv_bias_act(P, P, NUL, 1, P2, ctypes.byref(wide), None) == E_UNSUP
    assert L.chain_conv2(P, P, NUL, 1, P, NUL, 64, P2, ctypes.byref(shape(n=1, h=1, w=(1 << 24), k=64)), None) == E_UNSUP
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, ctypes.byref(shape(n=1, h=1, w=(1 << 24) - 3)), NUL, None) == OK


def test_conv_variant_validation(L):
    sh = shape(c=64, k=128)
    ex = L.chain_conv_pool_ex
    assert ex(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(sh), NUL, 3, 0, None) == E_ARG
    assert ex(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(sh), NUL, -1, 0, None) == E_ARG
    # register-weights form: c == 64, 64 < k <= 128 and a pool
    assert ex(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(shape(c=32, k=128)), NUL, 2, 0, None) == E_UNSUP
    assert ex(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(shape(c=64, k=64)), NUL, 2, 0, None) == E_UNSUP
    assert ex(P, P, NUL, NUL, 1, 0, P2, ctypes.byref(sh), NUL, 2, 0, None) == E_UNSUP
    assert ex(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(shape(c=128, k=128)), NUL, 1, 0, None) == E_UNSUP   # LDS form: weights exceed LDS
    assert ex(P, P, NUL, NUL, 1, 2, P2, ctypes.byref(shape(h=1)), NUL, 2, 0, None) == OK                 # empty pooled output
    # tile-owning waves: 0..8 for the pooled LDS-weights form only
    assert ex(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(sh), NUL, 1, 9, None) == E_ARG
    assert ex(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(sh), NUL, 2, 4, None) == E_ARG
    assert ex(P, P, NUL, NUL, 1, 0, P2, ctypes.byref(sh), NUL, 1, 4, None) == E_ARG
    assert ex(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(shape(h=1)), NUL, 1, 4, None) == OK


def test_tuner_validation(L):
    E = fc.TuneEntry
    t = (E * 4)()
    n = ctypes.c_int32(0)
    b = E()
    tx = L.chain_gemm2_tune_ex
    assert tx(P, P, NUL, 1, P, NUL, P2, 512, 64, 64, 64, 0, t, 4, ctypes.byref(n), ctypes.byref(b), None) == E_SHAPE
    assert tx(P, P, NUL, 1, P, NUL, P2, 512, 64, 64, 64, 1001, t, 4, ctypes.byref(n), ctypes.byref(b), None) == E_SHAPE
    assert tx(P, P, NUL, 1, P, NUL, P2, 0, 64, 64, 64, 5, t, 4, ctypes.byref(n), ctypes.byref(b), None) == E_SHAPE
    assert tx(P, P, NUL, 1, P, NUL, P2, 512, 64, 64, 64, 5, None, 4, ctypes.byref(n), ctypes.byref(b), None) == E_NULL
    assert tx(P, P, NUL, 1, P, NUL, P2, 512, 64, 64, 60, 5, t, 4, ctypes.byref(n), ctypes.byref(b), None) == E_SHAPE
    ct = L.chain_conv_pool_tune
    sh = shape(c=64, k=128)
    assert ct(P, P, NUL, NUL, 1, 0, P2, ctypes.byref(sh), NUL, 5, t, 4, ctypes.byref(n), ctypes.byref(b), None) == E_ARG
    assert ct(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(sh), NUL, 0, t, 4, ctypes.byref(n), ctypes.byref(b), None) == E_SHAPE
    assert ct(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(shape(h=1)), NUL, 5, t, 4, ctypes.byref(n), ctypes.byref(b), None) == E_SHAPE
    assert ct(P, P, NUL, NUL, 1, 1, P2, ctypes.byref(sh), NUL, 5, None, 4, ctypes.byref(n), ctypes.byref(b), None) == E_NULL
    # explicit configurations
    gx = L.chain_gemm2_ex
    assert gx(P, P, NUL, 1, P, NUL, P2, 512, 64, 64, 64, 1, 9, 0, None) == E_ARG
    assert gx(P, P, NUL, 1, P, NUL, P2, 512, 64, 64, 64, 0, 0, 0, None) == E_ARG   # AUTO is not a configuration
    assert gx(P, P, NUL, 1, P, NUL, P2, 512, 64, 64, 64, 2, 4, 0, None) == E_ARG   # LDS form takes waves == 0
    assert gx(P, P, NUL, 1, P, NUL, P2, 0, 64, 64, 64, 1, 2, 0, None) == OK
    # pipeline stages of the register-resident form: 4 (= 0) or 2, 2 built for 4 or 9 chunks of K0
    assert gx(P, P, NUL, 1, P, NUL, P2, 0, 256, 64, 64, 1, 2, 2, None) == OK
    assert gx(P, P, NUL, 1, P, NUL, P2, 0, 576, 64, 64, 1, 2, 4, None) == OK
    assert gx(P, P, NUL, 1, P, NUL, P2, 512, 64, 64, 64, 1, 2, 2, None) == E_UNSUP
    assert gx(P, P, NUL, 1, P, NUL, P2, 512, 256, 64, 64, 1, 2, 3, None) == E_ARG
    assert gx(P, P, NUL, 1, P, NUL, P2, 512, 256, 64, 64, 2, 0, 2, None) == E_ARG   # LDS form takes stages == 0
    # the untuned rule, queried without a GPU
    fc.tune_clear()
    assert fc.auto_config(65536, 256, 64, 128) == {"variant": "rf", "waves": 8, "stages": 2}   # two-stage ring at 8 waves
    assert fc.auto_config(512, 64, 64, 64) == {"variant": "rf", "waves": 1, "stages": 0}   # 16 one-wave blocks
    assert fc.auto_config(20000, 256, 64, 128) == {"variant": "rf", "waves": 4, "stages": 0}
    assert fc.auto_config(65536, 576, 256, 256, "gelu_tanh") == {"variant": "stream", "waves": 0, "stages": 0}
    assert fc.conv_auto_config(32, 112, 112, 64, 128) == {"variant": "reg_weights", "waves": 0, "stages": 0}
    assert fc.conv_auto_config(2, 8, 8, 32, 64) == {"variant": "lds_weights", "waves": 8, "stages": 0}
    # conv3x3 -> conv1x1: the pipelined two-group form where it applies, else the register-resident one
    assert fc.conv2_auto_config(32, 56, 56, 64, 64, 256) == {"variant": "pipe", "waves": 0, "stages": 0}
    assert fc.conv2_auto_config(1, 7, 9, 64, 64, 40) == {"variant": "pipe", "waves": 0, "stages": 0}
    assert fc.conv2_auto_config(32, 56, 56, 64, 64, 264)["variant"] == "rf"    # k1 > 256
    assert fc.conv2_auto_config(32, 56, 56, 32, 64, 256)["variant"] == "rf"    # c != 64
    assert fc.conv2_auto_config(32, 56, 56, 64, 96, 256)["variant"] == "rf"    # k0 != 64


def test_empty_tensors_may_be_null(L):
    # nothing to compute: NULL data pointers of empty tensors are accepted
    assert g2(L, A=NUL, D1=NUL, M=0) == OK
    assert L.chain_conv_pool(P, P, NUL, 1, 1, NUL, ctypes.byref(shape(h=1)), NUL, None) == OK
    assert L.chain_conv_pool(NUL, P, NUL, 1, 1, NUL, ctypes.byref(shape(h=1)), NUL, None) == E_NULL
    assert L.chain_conv2(NUL, P, NUL, 1, P, NUL, 64, NUL, ctypes.byref(shape(n=0, k=64)), None) == OK
    assert L.maxpool2x2(NUL, NUL, NUL, 2, 1, 9, 8, None) == OK
    assert g2(L, W0=NUL, M=0) == E_NULL


def test_pool_and_pad_validation(L):
    assert L.maxpool2x2(NUL, P2, NUL, 1, 4, 4, 8, None) == E_NULL
    assert L.maxpool2x2(P, P2, NUL, 1, 4, 4, 12, None) == E_SHAPE
    assert L.maxpool2x2(P, P2, ctypes.c_void_p(0x30004), 1, 4, 4, 8, None) == E_ALIGN
    assert L.pad_channels(P, P2, 10, 60, 56, 1, None) == E_SHAPE
    assert L.pad_channels(NUL, P2, 10, 60, 64, 1, None) == E_NULL


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    A = torch.zeros(4, 8, dtype=torch.float16)
    with pytest.raises(TypeError):
        fc.chain_gemm2(A, A.T.contiguous(), None, A, None)


def test_tune_validation(L):
    import ctypes as C
    best, us = C.c_int(-1), (C.c_float * 4)()

    def tune(A=P, W0=P, D1=P2, M=512, K0=64, N0=64, N1=64, act=1, reps=5):
        return L.chain_gemm2_tune(A, W0, NUL, act, P, NUL, D1, M, K0, N0, N1, reps, C.byref(best), us, None)
    assert tune(A=NUL) == E_NULL
    assert tune(D1=BAD) == E_ALIGN
    assert tune(K0=60) == E_SHAPE
    assert tune(M=0) == E_SHAPE            # nothing to time
    assert tune(reps=0) == E_SHAPE
    assert tune(reps=1001) == E_SHAPE
    assert tune(act=9) == E_ARG
    assert tune(N0=264) == E_UNSUP
    assert best.value == -1                # nothing written on failure


def test_auto_variant_rule(L):
    # without tuning, 'auto' follows the static rule: register-resident when
    # W0 and W1 fit in LDS with N0 <= 128, else streamed weights, else LDS
    fc.tune_clear()
    assert fc.auto_variant(65536, 256, 64, 128, "relu") == "rf"
    assert fc.auto_variant(65536, 576, 256, 256, "gelu_tanh") == "stream"
    assert fc.auto_variant(4096, 64, 256, 16136, "relu") == "lds"
    v = ctypes.c_int(-1)
    assert L.chain_gemm2_auto_variant(-1, 64, 64, 64, 1, ctypes.byref(v)) == E_SHAPE
    assert L.chain_gemm2_auto_variant(64, 64, 64, 64, 1, None) == E_NULL
    assert L.chain_gemm2_auto_variant(64, 64, 264, 64, 1, ctypes.byref(v)) == E_UNSUP


def test_chain_convN_validation(L):
    import ctypes as C
    sh = fc.ConvShape(1, 8, 8, 64, 64, 3, 3, 1, 1)

    def cn(n=3, k=(64, 64, 128), w=(P, P, P, P), acts=(1, 1, 0, 0), x=P, y=P2, shape=sh):
        kp = (C.c_int32 * 4)(*(list(k) + [0] * (4 - len(k))))
        wp = (C.c_void_p * 4)(*w)
        ap = (C.c_int * 4)(*acts)
        return L.chain_convN(x, C.byref(shape) if shape is not None else None, n, wp, None, ap, kp, y, None)
    assert cn(n=2) == E_UNSUP                 # two stages: chain_conv2
    assert cn(n=5) == E_UNSUP
    assert cn(shape=None) == E_NULL
    assert cn(k=(72, 64, 128)) == E_SHAPE     # k[0] must equal shape0.k
    assert cn(k=(64, 60, 128)) == E_SHAPE     # not a multiple of 8
    assert cn(w=(P, NUL, P, P)) == E_NULL
    assert cn(x=NUL) == E_NULL
    assert cn(y=BAD) == E_ALIGN
    assert cn(acts=(1, 9, 0, 0)) == E_ARG
    assert cn(k=(64, 136, 128)) == E_UNSUP    # intermediate wider than 128: not register-resident
    assert cn(shape=fc.ConvShape(0, 8, 8, 48, 64, 3, 3, 1, 1)) == OK        # c % 8 == 0 is enough
    assert cn(shape=fc.ConvShape(0, 8, 8, 44, 64, 3, 3, 1, 1)) == E_SHAPE
    # three stages at c = 64, k = {64, 64, <= 256} run the pipelined form,
    # which is not bound by the register-residence LDS rule
    assert cn(k=(64, 64, 256), shape=fc.ConvShape(0, 8, 8, 64, 64, 3, 3, 1, 1)) == OK

    def cv(v, n=3, k=(64, 64, 128), shape=fc.ConvShape(0, 8, 8, 64, 64, 3, 3, 1, 1)):
        kp = (C.c_int32 * 4)(*(list(k) + [0] * (4 - len(k))))
        wp = (C.c_void_p * 4)(P, P, P, P)
        ap = (C.c_int * 4)(1, 1, 0, 0)
        return L.chain_convN_variant(P, C.byref(shape), n, wp, None, ap, kp, P2, v, None)
    AUTO, RF, PIPE = 0, fc.VARIANT["rf"], fc.VARIANT["pipe"]
    assert cv(AUTO) == OK and cv(RF) == OK and cv(PIPE) == OK
    for v in (fc.VARIANT["lds"], fc.VARIANT["stream"], 5, -1):
        assert cv(v) == E_ARG
    assert cv(PIPE, k=(64, 64, 264)) == E_UNSUP                 # k[2] > 256
    assert cv(PIPE, k=(64, 64, 256)) == OK
    assert cv(RF, k=(64, 64, 256)) == OK
    assert cv(RF, k=(64, 136, 128)) == E_UNSUP                  # intermediate wider than 128
    assert cv(PIPE, k=(64, 32, 128)) == E_UNSUP                 # the middle stage must be 64 wide
    assert cv(PIPE, n=4, k=(64, 64, 64, 64)) == E_UNSUP
    assert cv(RF, n=4, k=(64, 64, 64, 64)) == OK
    assert cv(PIPE, k=(96, 64, 128), shape=fc.ConvShape(0, 8, 8, 64, 96, 3, 3, 1, 1)) == E_UNSUP
    assert cv(PIPE, shape=fc.ConvShape(0, 8, 8, 32, 64, 3, 3, 1, 1)) == E_UNSUP


def test_chain_convN_auto_variant(L):
    import ctypes as C
    RF, PIPE = fc.VARIANT["rf"], fc.VARIANT["pipe"]

    def av(shape, ks):
        kp = (C.c_int32 * len(ks))(*ks)
        v = C.c_int(-1)
        r = L.chain_convN_auto_variant(C.byref(shape), len(ks), kp, C.byref(v))
        return r, v.value
    sh = lambda c, k: fc.ConvShape(2, 8, 8, c, k, 3, 3, 1, 1)
    assert av(sh(64, 64), [64, 64, 256]) == (OK, PIPE)
    assert av(sh(64, 64), [64, 64, 8]) == (OK, PIPE)
    assert av(sh(64, 64), [64, 32, 128]) == (OK, RF)        # middle stage not 64 wide
    assert av(sh(64, 64), [64, 64, 64, 64]) == (OK, RF)     # four stages
    assert av(sh(32, 64), [64, 64, 128]) == (OK, RF)        # c != 64
    assert av(sh(64, 32), [32, 64, 128]) == (OK, RF)        # k[0] != 64
    assert av(sh(64, 64), [64, 136, 128])[0] == E_UNSUP     # neither form takes it
    assert av(sh(64, 64), [72, 64, 128])[0] == E_SHAPE      # k[0] != shape.k
    assert av(sh(64, 64), [64, 64])[0] == E_UNSUP           # two stages: chain_conv2
    kp = (C.c_int32 * 3)(64, 64, 64)
    v = C.c_int(0)
    assert L.chain_convN_auto_variant(None, 3, kp, C.byref(v)) == E_NULL
    assert L.chain_convN_auto_variant(C.byref(sh(64, 64)), 3, None, C.byref(v)) == E_NULL
    assert L.chain_convN_auto_variant(C.byref(sh(64, 64)), 3, kp, None) == E_NULL
    # the tuner's argument checks (all decided before any HIP call)
    tab = (fc.TuneEntry * 4)()
    cnt, best = C.c_int32(0), fc.TuneEntry()
    wp = (C.c_void_p * 3)(P, P, P)
    ap = (C.c_int * 3)(1, 1, 0)

    def tn(shape, ks=(64, 64, 128), reps=5, table=tab, capacity=4, n=3):
        kp = (C.c_int32 * 3)(*ks)
        return L.chain_convN_tune(P, C.byref(shape), n, wp, None, ap, kp, P2, reps, table, capacity, C.byref(cnt),
                                  C.byref(best), None)
    assert tn(sh(64, 64), reps=0) == E_SHAPE
    assert tn(sh(64, 64), reps=1001) == E_SHAPE
    assert tn(fc.ConvShape(0, 8, 8, 64, 64, 3, 3, 1, 1)) == E_SHAPE     # empty: nothing to time
    assert tn(sh(64, 64), table=None) == E_NULL
    assert tn(sh(64, 64), ks=(64, 136, 128)) == E_UNSUP
    assert tn(sh(64, 64), n=2) == E_UNSUP
    # the binding's helper
    assert fc.convN_auto_variant(32, 56, 56, 64, [64, 64, 256]) == "pipe"
    assert fc.convN_auto_variant(32, 56, 56, 64, [64, 48, 96]) == "rf"


def test_chain_conv_bn_pool_validation(L):
    import ctypes as C
    sh = fc.ConvShape(1, 8, 8, 64, 64, 3, 3, 1, 1)

    def bn(x=P, w=P, scale=P, shift=NUL, act=1, pool=1, y=P2, am=NUL, shape=sh):
        return L.chain_conv_bn_pool(x, w, scale, shift, act, pool, y, C.byref(shape), am, None)
    assert bn(scale=NUL) == E_NULL            # the scale is what this entry adds
    assert bn(scale=BAD) == E_ALIGN
    assert bn(shift=BAD) == E_ALIGN
    assert bn(w=NUL) == E_NULL
    assert bn(act=5) == E_ARG
    assert bn(pool=3) == E_ARG
    assert bn(pool=0, am=P) == E_ARG           # argmax needs a pool
    assert bn(shape=fc.ConvShape(1, 8, 8, 64, 136, 3, 3, 1, 1)) == E_UNSUP


def test_empty_inputs_launch_nothing(L):
    # an empty batch or a pooled output of zero size is a no-op: FC_OK with
    # NULL data pointers, decided before any HIP call (so it runs without a GPU)
    import ctypes as C
    empty = fc.ConvShape(0, 8, 8, 64, 64, 3, 3, 1, 1)
    one_row = fc.ConvShape(1, 1, 8, 64, 64, 3, 3, 1, 1)    # 1x8 image: the 2x2 pool has no output
    assert L.chain_conv_pool(NUL, P, NUL, 1, 1, NUL, C.byref(empty), NUL, None) == OK
    assert L.chain_conv_pool(P, P, NUL, 1, 1, NUL, C.byref(one_row), NUL, None) == OK
    assert L.chain_conv_bn_pool(NUL, P, P, NUL, 1, 1, NUL, C.byref(empty), NUL, None) == OK
    assert L.chain_conv_bn_pool(P, P, P, NUL, 1, 1, NUL, C.byref(one_row), NUL, None) == OK
    kp = (C.c_int32 * 3)(64, 64, 128)
    wp = (C.c_void_p * 3)(P, P, P)
    ap = (C.c_int * 3)(1, 1, 0)
    assert L.chain_convN(NUL, C.byref(empty), 3, wp, None, ap, kp, NUL, None) == OK
    assert L.chain_gemm2_variant(NUL, P, NUL, 1, P, NUL, NUL, 0, 64, 64, 64, 3, None) == OK
    wd = (C.c_int32 * 4)(64, 64, 64, 64)
    assert L.chain_gemmN(NUL, 3, wp, None, ap, wd, NUL, 0, None) == OK


def test_probe_validation(L):
    import ctypes as C
    b = C.c_int32(0)
    assert L.fc_probe_mfma(2, 16, NUL, P, 256, C.byref(b), None) == E_NULL
    assert L.fc_probe_mfma(3, 16, P, P2, 256, C.byref(b), None) == E_SHAPE     # 1 or 2 waves per SIMD
    assert L.fc_probe_mfma(2, 0, P, P2, 256, C.byref(b), None) == E_SHAPE
    assert L.fc_probe_mfma(2, 16, C.c_void_p(0x10004), P2, 256, C.byref(b), None) == E_ALIGN


def test_avg_pool_validation(L):
    import ctypes as C
    sh = fc.ConvShape(1, 8, 8, 64, 64, 3, 3, 1, 1)
    assert L.chain_conv_pool(P, P, NUL, 1, 2, P2, C.byref(sh), P, None) == E_ARG    # argmax only with the max pool
    assert L.chain_conv_pool(P, P, NUL, 1, 3, P2, C.byref(sh), NUL, None) == E_ARG
    assert L.chain_conv_bn_pool(P, P, P, NUL, 1, 2, P2, C.byref(sh), P, None) == E_ARG


def test_residence_limits(L):
    # the register-resident chain holds W0 and W1 in LDS: K0 = 320 fits with
    # N0 = N1 = 128, K0 = 384 does not (auto then streams the weights); the conv
    # holds all 3x3 weights: c = 128 fits with k = 64, not with k = 72
    fc.tune_clear()
    assert fc.auto_variant(300, 320, 128, 128) == "rf"
    assert fc.auto_variant(300, 384, 128, 128) == "stream"
    assert g2(L, M=300, K0=384, N0=128, N1=128, variant=1) == E_UNSUP
    import ctypes as C
    assert L.chain_conv_pool(P, P, NUL, 1, 1, P2, C.byref(fc.ConvShape(1, 6, 10, 128, 72, 3, 3, 1, 1)), NUL,
                             None) == E_UNSUP


def test_winograd_validation(L):
    import ctypes as C
    ww = L.winograd_weights
    assert ww(P, P2, 12, 128, None) == E_SHAPE
    assert ww(P, P2, 64, 0, None) == E_SHAPE
    assert ww(NUL, P2, 64, 128, None) == E_NULL
    assert ww(P, BAD, 64, 128, None) == E_ALIGN
    assert ww(P, P2, 65536, 4096, None) == E_UNSUP   # 16 c k >= 2^31

    cw = L.chain_conv_pool_winograd

    def call(sh, pool=1, act=1, am=NUL, x=P, U=P, y=P2, b=NUL):
        return cw(x, U, b, act, pool, y, C.byref(sh), am, None)
    empty = shape(n=0)
    assert call(empty) == OK                            # validated, nothing to launch
    assert call(shape(n=0, c=32, k=64)) == OK
    assert call(shape(n=0, k=48)) == OK
    assert call(shape(n=0, c=8, k=64)) == E_UNSUP       # c must be 32 or 64
    assert call(shape(n=0, c=96, k=64)) == E_UNSUP
    assert call(shape(n=0, k=40)) == E_UNSUP            # k % 16
    assert call(shape(n=0, k=136)) == E_UNSUP
    assert call(shape(n=0, c=60)) == E_SHAPE
    assert call(shape(n=0, r=5, s=5)) == E_UNSUP
    assert call(empty, pool=0) == E_UNSUP               # the chain pools every output tile
    assert call(empty, pool=3) == E_ARG
    assert call(empty, pool=2, am=P) == E_ARG           # argmax needs the max pool
    assert call(empty, act=7) == E_ARG
    assert call(empty, U=NUL) == E_NULL
    assert call(shape(n=1), x=NUL) == E_NULL
    assert call(empty, am=BAD) == E_ALIGN
    assert call(empty, b=BAD) == E_ALIGN
    assert call(shape(n=1, h=1, w=8)) == OK             # pooled output empty (floor)
    big = shape(n=1, h=8192, w=2048, c=64, k=64)        # one image of 2 GiB: offsets exceed 31 bits
    assert call(big) == E_UNSUP
    assert b"2^31" in L.fc_last_error()


def test_conv2_waves_and_tuner_validation(L):
    import ctypes as C
    sh0 = shape(k=64)
    ex = L.chain_conv2_ex
    assert ex(P, P, NUL, 1, P, NUL, 64, P2, C.byref(shape(n=0, k=64)), 0, 0, None) == OK
    assert ex(P, P, NUL, 1, P, NUL, 64, P2, C.byref(shape(n=0, k=64)), 4, 0, None) == OK
    assert ex(P, P, NUL, 1, P, NUL, 64, P2, C.byref(shape(n=0, k=64)), 4, 2, None) == OK      # 9 chunks of 64
    assert ex(P, P, NUL, 1, P, NUL, 64, P2, C.byref(sh0), 9, 0, None) == E_ARG
    assert ex(P, P, NUL, 1, P, NUL, 64, P2, C.byref(sh0), -1, 0, None) == E_ARG
    assert ex(P, P, NUL, 1, P, NUL, 64, P2, C.byref(sh0), 4, 3, None) == E_ARG
    assert ex(P, P, NUL, 1, P, NUL, 64, P2, C.byref(sh0), 0, 2, None) == E_ARG               # stages need waves
    assert ex(P, P, NUL, 1, P, NUL, 64, P2, C.byref(shape(c=32, k=64)), 4, 2, None) == E_UNSUP  # 9c = 288
    assert ex(P, P, NUL, 1, P, NUL, 60, P2, C.byref(sh0), 0, 0, None) == E_SHAPE
    va = L.chain_conv2_variant
    RF, PIPE = fc.VARIANT["rf"], fc.VARIANT["pipe"]
    e0 = C.byref(shape(n=0, k=64))
    assert va(P, P, NUL, 1, P, NUL, 256, P2, e0, 0, 0, 0, None) == OK
    assert va(P, P, NUL, 1, P, NUL, 256, P2, e0, PIPE, 0, 0, None) == OK
    assert va(P, P, NUL, 1, P, NUL, 256, P2, e0, RF, 8, 2, None) == OK
    assert va(P, P, NUL, 1, P, NUL, 256, P2, e0, RF, 0, 0, None) == E_ARG       # RF needs waves
    assert va(P, P, NUL, 1, P, NUL, 256, P2, e0, PIPE, 8, 0, None) == E_ARG     # PIPE takes no waves
    assert va(P, P, NUL, 1, P, NUL, 256, P2, e0, PIPE, 0, 2, None) == E_ARG
    assert va(P, P, NUL, 1, P, NUL, 256, P2, e0, 0, 4, 0, None) == E_ARG        # AUTO takes no waves
    for v in (fc.VARIANT["lds"], fc.VARIANT["stream"], 5, -1):
        assert va(P, P, NUL, 1, P, NUL, 256, P2, e0, v, 0, 0, None) == E_ARG
    assert va(P, P, NUL, 1, P, NUL, 256, P2, C.byref(shape(n=0, c=32, k=64)), PIPE, 0, 0, None) == E_UNSUP
    assert va(P, P, NUL, 1, P, NUL, 256, P2, C.byref(shape(n=0, c=64, k=96)), PIPE, 0, 0, None) == E_UNSUP
    assert va(P, P, NUL, 1, P, NUL, 264, P2, e0, PIPE, 0, 0, None) == E_UNSUP
    assert va(NUL, P, NUL, 1, P, NUL, 256, P2, C.byref(shape(c=64, k=64)), PIPE, 0, 0, None) == E_NULL
    assert va(P, P, NUL, 1, P, NUL, 60, P2, e0, PIPE, 0, 0, None) == E_SHAPE
    tab = (fc.TuneEntry * 4)()
    n = C.c_int32(0)
    best = fc.TuneEntry()
    tn = L.chain_conv2_tune
    assert tn(P, P, NUL, 1, P, NUL, 64, P2, C.byref(sh0), 0, tab, 4, C.byref(n), C.byref(best), None) == E_SHAPE
    assert tn(P, P, NUL, 1, P, NUL, 64, P2, C.byref(sh0), 1001, tab, 4, C.byref(n), C.byref(best), None) == E_SHAPE
    assert tn(P, P, NUL, 1, P, NUL, 64, P2, C.byref(shape(n=0, k=64)), 5, tab, 4, C.byref(n), C.byref(best),
              None) == E_SHAPE
    assert tn(P, P, NUL, 1, P, NUL, 64, P2, C.byref(sh0), 5, None, 4, C.byref(n), C.byref(best), None) == E_NULL
    assert tn(P, P, NUL, 1, P, NUL, 64, P2, C.byref(shape(c=64, k=128)), 5, tab, 4, C.byref(n), C.byref(best),
              None) == E_UNSUP


def test_probe_read_validation(L):
    import ctypes as C
    blocks = C.c_int32(0)
    assert L.fc_probe_read(NUL, 64, P2, 8, C.byref(blocks), None) == E_NULL
    assert L.fc_probe_read(P, 8, P2, 8, C.byref(blocks), None) == E_SHAPE
    assert L.fc_probe_read(P, 72, P2, 8, C.byref(blocks), None) == E_SHAPE    # not a multiple of 16
    assert L.fc_probe_read(BAD, 64, P2, 8, C.byref(blocks), None) == E_ALIGN
