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


def test_probe_read_reads_everything(fc):
    # the per-block XORs combine to the XOR of every 32-bit word of the buffer
    # (a ragged size: not a multiple of the grid's stride)
    import numpy as np
    n = 4 * 100003
    host = np.random.default_rng(3).integers(0, 2**31 - 1, n, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    sink = torch.zeros(2 * 1024, dtype=torch.int32, device="cuda")
    print("case read probe", flush=True)
    blocks = fc.probe_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink[:blocks].cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host.view(np.uint32))


def test_probe_read_rate_plausible(fc):
    import bench
    r = bench.read_probe(torch, fc, 64 << 20, copies=5)
    print(r, flush=True)
    assert 0.3 < r["tb_per_s"] < 1.2 * bench.PEAK_HBM_GBS / 1000.0
    assert 0 < bench.launch_floor(torch, fc, steps=10) < 0.1
