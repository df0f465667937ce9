"""The configuration profiler (BOLT notes, "Light-weight performance
profiler"; Welder notes, "Tile-graph Scheduling": candidate configurations
are measured on the GPU and the fastest is kept): every configuration it can
choose computes the chain correctly, every candidate is timed, the fastest is
cached per shape and then runs under 'auto'."""
import numpy as np
import pytest

import oracle
from gemm_conv_chain_amd import inputs
from parity import assert_close, to_np
from test_gpu_conv import check_pool, dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
ACTS = {"none": oracle.ACT_NONE, "relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH}


@pytest.fixture(scope="module")
def fc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_conv_chain_amd as m
    m.lib()
    return m


def gemm_ref(d, act):
    ref, _ = oracle.chain_gemm2(d["A"], d["W0"], d["b0"], ACTS[act], d["W1"], d["b1"])
    return ref


@pytest.mark.parametrize("waves", [1, 2, 4, 8])
@pytest.mark.parametrize("M,K0,N0,N1", [(512, 64, 64, 64), (1000, 256, 64, 128), (70001, 256, 64, 128),
                                        (333, 200, 96, 136)])
def test_gemm2_rf_waves(fc, M, K0, N0, N1, waves):
    # the register-resident form with 1..8 tile-owning waves per block (a block
    # covers 32 * waves rows per round); ragged last tiles, a runtime chunk count
    d = inputs.gemm2_inputs(M, K0, N0, N1, "uniform", seed=M + waves)
    A, W0, b0, W1, b1 = (dev(d[k]) for k in ("A", "W0", "b0", "W1", "b1"))
    print("case rf waves", M, K0, N0, N1, waves, flush=True)
    out = to_np(fc.chain_gemm2(A, W0, b0, W1, b1, act="relu", variant="rf", waves=waves))
    assert_close(out, gemm_ref(d, "relu"), "rf waves=%d" % waves)


@pytest.mark.parametrize("waves", [1, 3, 4, 8])
@pytest.mark.parametrize("n,h,w,c,k", [(3, 30, 34, 64, 128), (2, 9, 6, 32, 64)])
def test_conv_lds_weights_waves(fc, n, h, w, c, k, waves):
    d = inputs.conv_pool_inputs(n, h, w, c, k, seed=n * h + waves)
    print("case conv lds waves", n, h, w, c, k, waves, flush=True)
    y, am = fc.chain_conv_pool(dev(d["x"]), dev(d["w"]), dev(d["b"]), argmax=True, variant="lds_weights", waves=waves)
    y2 = fc.chain_conv_pool(dev(d["x"]), dev(d["w"]), dev(d["b"]), variant="lds_weights", waves=waves)
    torch.cuda.synchronize()
    y, am, y2 = to_np(y), to_np(am), to_np(y2)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
    check_pool(y, am, d["x"], d["w"], d["b"], "conv lds waves=%d" % waves)


@pytest.mark.parametrize("M,K0,N0,N1,act", [(512, 64, 64, 64, "relu"), (20000, 256, 64, 128, "relu"),
                                            (4000, 576, 256, 256, "gelu_tanh")])
def test_tune_gemm2_table(fc, M, K0, N0, N1, act):
    d = inputs.gemm2_inputs(M, K0, N0, N1, "uniform", seed=17)
    A, W0, b0, W1, b1 = (dev(d[k]) for k in ("A", "W0", "b0", "W1", "b1"))
    print("case tune table", M, K0, N0, N1, act, flush=True)
    fc.tune_clear()
    best, table, out = fc.tune_chain_gemm2_table(A, W0, b0, W1, b1, act=act, reps=3)
    torch.cuda.synchronize()
    print(best, table, flush=True)
    ref = gemm_ref(d, act)
    assert_close(to_np(out), ref, "tuned output")
    cfgs = {(r["variant"], r["waves"], r["stages"]) for r in table}
    assert all(r["us"] > 0 for r in table)
    if N0 <= 128:
        # M_t / waves per block: four values of the register-resident form,
        # and for 4 or 9 chunks of K0 two pipeline depths of each
        assert {("rf", w, 0) for w in (1, 2, 4, 8)} <= cfgs
        if (K0 + 63) // 64 in (4, 9):
            assert {("rf", w, 2) for w in (1, 2, 4, 8)} <= cfgs
    assert ("lds", 0, 0) in cfgs and ("stream", 0, 0) in cfgs     # the residence forms
    fastest = min(table, key=lambda r: r["us"])
    key = lambda r: (r["variant"], r["waves"], r["stages"])
    assert key(best) == key(fastest)
    assert fc.auto_config(M, K0, N0, N1, act) == {"variant": best["variant"], "waves": best["waves"],
                                                  "stages": best["stages"]}
    assert_close(to_np(fc.chain_gemm2(A, W0, b0, W1, b1, act=act)), ref, "auto after tuning")
    fc.tune_clear()
    assert fc.auto_config(M, K0, N0, N1, act)["variant"] == ("rf" if N0 <= 128 else "stream")
    if N0 <= 128:   # untuned: the smallest power-of-two wave count covering the row tiles, one block per CU
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        w = 1
        while w < 8 and w * cus < (M + 31) // 32:
            w *= 2
        assert fc.auto_config(M, K0, N0, N1, act)["waves"] == w


@pytest.mark.parametrize("pool", ["max2x2", "avg2x2"])
def test_tune_conv_pool(fc, pool):
    d = inputs.conv_pool_inputs(3, 30, 34, 64, 128, seed=23)
    x, w, b = dev(d["x"]), dev(d["w"]), dev(d["b"])
    print("case tune conv", pool, flush=True)
    fc.tune_clear()
    best, table, out = fc.tune_conv_pool(x, w, b, pool=pool, reps=3)
    torch.cuda.synchronize()
    print(best, table, flush=True)
    cfgs = {(r["variant"], r["waves"]) for r in table}
    assert cfgs == {("reg_weights", 0), ("lds_weights", 8), ("lds_weights", 4)}
    assert all(r["us"] > 0 for r in table)
    fastest = min(table, key=lambda r: r["us"])
    assert (best["variant"], best["waves"]) == (fastest["variant"], fastest["waves"])
    assert fc.conv_auto_config(3, 30, 34, 64, 128, pool=pool) == {"variant": best["variant"], "waves": best["waves"],
                                                                  "stages": 0}
    if pool == "max2x2":
        yo, _, _, _ = oracle.chain_conv_pool(d["x"], d["w"], d["b"], oracle.ACT_RELU)
    else:
        yo, _ = oracle.chain_conv_avgpool(d["x"], d["w"], d["b"], oracle.ACT_RELU)
    assert_close(to_np(out), yo.astype(np.float64), "tuned conv output")
    assert_close(to_np(fc.chain_conv_pool(x, w, b, pool=pool)), yo.astype(np.float64), "auto after tuning")
    # an argmax output selects another kernel: untuned, it keeps the rule
    assert fc.conv_auto_config(3, 30, 34, 64, 128, pool=pool, argmax=True)["variant"] == "reg_weights"
    fc.tune_clear()
    assert fc.conv_auto_config(3, 30, 34, 64, 128, pool=pool) == {"variant": "reg_weights", "waves": 0, "stages": 0}


@pytest.mark.parametrize("waves", [1, 2, 4, 8])
@pytest.mark.parametrize("n,h,w,c,k0,k1", [(2, 33, 35, 64, 64, 256), (1, 7, 9, 32, 96, 40)])
def test_conv2_waves(fc, n, h, w, c, k0, k1, waves):
    # every block shape and pipeline depth the profiler may choose computes the
    # chain (several rounds per block and a ragged last tile in the first shape)
    d = inputs.conv2_inputs(n, h, w, c, k0, k1, seed=h + waves)
    ref, _ = oracle.chain_conv2(d["x"], d["w0"], d["b0"], oracle.ACT_RELU, d["w1"], d["b1"])
    for stages in ((4, 2) if c == 64 else (4,)):
        print("case conv2 waves", waves, "stages", stages, n, h, w, c, k0, k1, flush=True)
        y = to_np(fc.chain_conv2(dev(d["x"]), dev(d["w0"]), dev(d["b0"]), dev(d["w1"]), dev(d["b1"]), act="relu",
                                 waves=waves, stages=stages))
        assert_close(y, ref, "conv2 waves=%d stages=%d" % (waves, stages))


@pytest.mark.parametrize("waves", [1, 8])
@pytest.mark.parametrize("M,K0,N0,N1", [(1000, 256, 64, 128), (70001, 256, 64, 128), (3000, 576, 64, 64)])
def test_gemm2_rf_two_stages(fc, M, K0, N0, N1, waves):
    # the two-stage row ring (one chunk in flight) of the register-resident form;
    # the same k order as the four-stage ring, so the two agree bit for bit
    d = inputs.gemm2_inputs(M, K0, N0, N1, "uniform", seed=M + 3 * waves)
    A, W0, b0, W1, b1 = (dev(d[k]) for k in ("A", "W0", "b0", "W1", "b1"))
    print("case rf two stages", M, K0, N0, N1, waves, flush=True)
    y2 = to_np(fc.chain_gemm2(A, W0, b0, W1, b1, act="relu", variant="rf", waves=waves, stages=2))
    y4 = to_np(fc.chain_gemm2(A, W0, b0, W1, b1, act="relu", variant="rf", waves=waves, stages=4))
    assert np.array_equal(y2.view(np.uint16), y4.view(np.uint16))
    assert_close(y2, gemm_ref(d, "relu"), "rf stages=2 waves=%d" % waves)


def test_tune_conv2(fc):
    d = inputs.conv2_inputs(4, 28, 28, 64, 64, 256, seed=5)
    args = [dev(d[k]) for k in ("x", "w0", "b0", "w1", "b1")]
    print("case tune conv2", flush=True)
    fc.tune_clear()
    rule = fc.conv2_auto_config(4, 28, 28, 64, 64, 256)
    assert rule == {"variant": "pipe", "waves": 0, "stages": 0}
    best, table, out = fc.tune_chain_conv2(*args, reps=3)
    torch.cuda.synchronize()
    print(best, table, flush=True)
    # the pipelined form, then block shapes (8, 4, 2, 1 waves) x pipeline stages (4, 2)
    assert table[0]["variant"] == "pipe"
    assert sorted((r["waves"], r["stages"]) for r in table[1:]) == [(w, s) for w in (1, 2, 4, 8) for s in (0, 2)]
    assert all(r["variant"] == "rf" for r in table[1:]) and all(r["us"] > 0 for r in table)
    fastest = min(table, key=lambda r: r["us"])
    assert (best["variant"], best["waves"], best["stages"]) == (fastest["variant"], fastest["waves"], fastest["stages"])
    assert fc.conv2_auto_config(4, 28, 28, 64, 64, 256) == {"variant": best["variant"], "waves": best["waves"],
                                                             "stages": best["stages"]}
    ref, _ = oracle.chain_conv2(d["x"], d["w0"], d["b0"], oracle.ACT_RELU, d["w1"], d["b1"])
    assert_close(to_np(out), ref, "tuned conv2 output")
    assert_close(to_np(fc.chain_conv2(*args)), ref, "conv2 auto after tuning")
    fc.tune_clear()
    assert fc.conv2_auto_config(4, 28, 28, 64, 64, 256) == rule


@pytest.mark.parametrize("ks,forms", [([64, 64, 128], ["pipe", "rf"]), ([64, 48, 96], ["rf"])])
def test_tune_convN(fc, ks, forms):
    d = inputs.convN_inputs(3, 20, 24, 64, ks, seed=7)
    ws, bs = [dev(w) for w in d["ws"]], [dev(b) for b in d["bs"]]
    x = dev(d["x"])
    acts = ["relu", "relu", "none"]
    print("case tune convN", ks, flush=True)
    fc.tune_clear()
    rule = fc.convN_auto_variant(3, 20, 24, 64, ks)
    assert rule == forms[0]
    best, table, out = fc.tune_chain_convN(x, ws, bs, acts, reps=3)
    torch.cuda.synchronize()
    print(best, table, flush=True)
    assert [r["variant"] for r in table] == forms and all(r["us"] > 0 for r in table)
    fastest = min(table, key=lambda r: r["us"])
    assert best["variant"] == fastest["variant"]
    assert fc.convN_auto_variant(3, 20, 24, 64, ks) == best["variant"]
    ref = oracle.chain_convN(d["x"], d["ws"], d["bs"], [oracle.ACT_RELU, oracle.ACT_RELU, oracle.ACT_NONE])
    assert_close(to_np(out), ref, "tuned convN output")
    assert_close(to_np(fc.chain_convN(x, ws, bs, acts)), ref, "convN auto after tuning")
    fc.tune_clear()
    assert fc.convN_auto_variant(3, 20, 24, 64, ks) == rule
