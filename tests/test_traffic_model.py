"""The per-tile traffic model (gemm_conv_chain_amd.traffic_model): hand-counted
halo tiles, the LRU cache, the ordering of its three read figures, and its
L2 prediction against the FETCH_SIZE counters committed under profiles/."""
import json
import os

import numpy as np
import pytest

from gemm_conv_chain_amd import inputs
from gemm_conv_chain_amd import traffic_model as tm

pytestmark = pytest.mark.cpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_lru_by_hand():
    seq = [np.array(x) for x in ([1, 2], [1, 3], [2], [1, 3])]
    # capacity 2: 1 2 | 1(hit) 3(evicts 2) | 2(miss, evicts 1) | 1(miss, evicts 3) 3(miss)
    assert tm.lru_misses([seq], capacity_lines=2) == 6
    assert tm.lru_misses([seq], capacity_lines=3) == 3
    # two XCDs are two caches
    assert tm.lru_misses([seq, seq], capacity_lines=3) == 6


def test_xcd_block_order():
    assert tm.xcd_blocks(16)[1] == [2, 3]            # renumbered: contiguous logical ranges
    assert tm.xcd_blocks(12)[1] == [1, 9]            # not a multiple of 8: hardware round robin
    assert sorted(sum(tm.xcd_blocks(64), [])) == list(range(64))


def test_register_weights_halo_by_hand():
    # 1 x 4 x 32 image, 64 channels (one 128-byte line per pixel), k = 128:
    # pooled 2 x 16 = 2 pooled rows x 2 row tiles of 8 windows; each row tile's
    # halo is 4 x 18 pixels clipped to 3 rows x 17 columns inside the image
    r = tm.conv_pool_wr(1, 4, 32, 64, 128)
    w = 9 * 64 * 128 * 2
    assert r["tiles"] == 4 and r["blocks"] == 4
    assert r["read_per_tile"] == 4 * 3 * 17 * 128 + 4 * w
    assert r["read_algorithmic"] == 4 * 32 * 128 + w
    # everything fits one L2: the blocks of each XCD fetch their halo lines and the weights once
    per_xcd = [set() for _ in range(8)]
    for x, blocks in enumerate(tm.xcd_blocks(4)):
        for b in blocks:
            q, jb = divmod(b, 2)
            for row in range(max(0, 2 * q - 1), min(4, 2 * q + 3)):
                for col in range(max(0, 16 * jb - 1), min(32, 16 * jb + 17)):
                    per_xcd[x].add(row * 32 + col)
    expect = sum(len(s) for s in per_xcd) * 128 + sum(1 for s in per_xcd if s) * w
    assert r["read_l2_model"] == expect


def test_winograd_halo_by_hand():
    # 1 x 8 x 16 image: 4 x 8 output tiles = 2 batches of 2 x 8 tiles, halo 6 x 18 clipped
    r = tm.conv_pool_wino(1, 8, 16, 64, 32)
    u = 16 * 64 * 32 * 2
    assert r["tiles"] == 2 and r["blocks"] == 2
    # batch 0: rows -1..4 -> 0..4 (5), batch 1: rows 3..8 -> 3..7 (5); columns -1..16 -> 0..15 (16)
    assert r["read_per_tile"] == 2 * 5 * 16 * 128 + 2 * u


def test_one_block_reads_each_line_once():
    # a single block whose whole working set fits the L2 reads every input line once
    r = tm.conv3x3_rows(1, 6, 10, 64, 0, 0, 0, "k_chain_rf", 32, False, waves=8, cus=1)
    assert r["blocks"] == 1
    assert r["read_l2_model"] == 6 * 10 * 128
    assert r["read_per_tile"] > r["read_l2_model"]


@pytest.mark.parametrize("name,variant", [("conv3x3_conv1x1", None), ("b2b_gemm_lds", "lds"),
                                          ("b2b_gemm_rf", None), ("gemm3_rf", None), ("conv3x3_conv1x1x2", None),
                                          ("conv3x3_conv1x1x2", "rf")])
def test_reads_ordered(name, variant):
    spec, _ = inputs.workload(name)
    r = tm.for_workload(spec, variant)
    assert r["read_algorithmic"] <= r["read_l2_model"] <= r["read_per_tile"]
    assert r["lds_fits"]


def _measured():
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        pytest.skip("no committed traffic counters")
    with open(p) as f:
        return json.load(f)["workloads"]


@pytest.mark.parametrize("key,variant", [("conv3x3_relu_maxpool", "reg_weights"),
                                         ("conv3x3_relu_maxpool@lds_weights", "lds_weights"),
                                         ("conv3x3_relu_maxpool@winograd", "winograd"),
                                         ("conv3x3_conv1x1", None), ("b2b_gemm_lds", "lds"),
                                         ("b2b_gemm_lds@stream", "stream"), ("b2b_gemm_rf", "rf"),
                                         ("conv3x3_conv1x1x2", None), ("conv3x3_conv1x1x2@rf", "rf")])
def test_l2_model_predicts_fetch(key, variant):
    """The model's L2 misses against the calibrated FETCH_SIZE of the same
    kernel at full size (profiles/traffic.json): within 10%, and closer than
    either bound (algorithmic or per-tile) wherever those differ from it."""
    import bench
    db = _measured()
    if key not in db:
        pytest.skip("no counters for " + key)
    e = db[key]
    if e.get("src_hash") != bench.kernel_src_hash():
        pytest.skip("the committed counters of %s were taken on other kernel sources" % key)
    fetch = e["fetch_kib"] * e["fetch_scale"] * 1024
    spec, _ = inputs.workload(key.split("@")[0])
    r = tm.for_workload(spec, variant)
    assert abs(fetch / r["read_l2_model"] - 1) < 0.10, (key, fetch, r)
    assert abs(fetch - r["read_l2_model"]) <= abs(fetch - r["read_per_tile"])
