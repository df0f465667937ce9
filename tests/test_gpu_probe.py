"""The matrix-core rate probe bench.py reports beside the chains: it runs,
stays inside its buffers, and gives physically plausible numbers."""
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_conv_chain_amd as m
    m.lib()
    return m


def test_probe_mfma(fc):
    import bench
    print("case mfma probe", flush=True)
    r = bench.mfma_probe(torch, fc, waves_per_simd=2, iters=256)
    print(r, flush=True)
    # fp16 dense peak is ~2.5 PFLOP/s at 2.4 GHz: a register-only MFMA loop
    # must land well inside (0, 1.05 x peak], the clock inside (0.5, 3) GHz
    assert 100.0 < r["tflops"] <= 1.05 * bench.PEAK_F16_TFLOPS
    assert r["sclk_ghz_median"] is not None and 0.5 < r["sclk_ghz_median"] < 3.0


def test_probe_refuses_small_buffers(fc):
    stamps = torch.zeros(4 * 8, dtype=torch.int64, device="cuda")   # 8 blocks: smaller than the grid
    sink = torch.zeros(8, dtype=torch.float32, device="cuda")
    with pytest.raises(fc.FusedChainError):
        fc.probe_mfma(stamps, sink, 2, 16)
    torch.cuda.synchronize()
    assert int(stamps.abs().sum()) == 0        # nothing was launched
