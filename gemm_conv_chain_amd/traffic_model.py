"""Predicted memory traffic of the fused kernels' tile schedules.

The Welder notes ("Operator-tile and Tile-graph") price a tile configuration
by its memory traffic -- the sum, over the tiles, of the input tiles each one
loads and the output tiles it stores -- and check its footprint (what one tile
keeps on chip) against the memory it lives in.  This module computes, for the
launch each fused kernel actually makes (grid, block ranges, the XCD-aware
block order, tiles per step), three read figures beside the bytes written:

* ``read_algorithmic``: every input byte once (perfect reuse);
* ``read_per_tile``: Welder's MemTraffic -- each tile loads its whole input
  tile (conv halos included) and each block its resident weights, with no
  reuse between tiles;
* ``read_l2_model``: the same accesses replayed through one LRU cache per XCD
  (4 MiB L2, 128-byte lines; the blocks of an XCD advance one tile per step
  in lockstep): the misses are the reads the L2 sends to memory, i.e. the
  prediction for rocprofv3's FETCH_SIZE (which counts L2 misses, whether the
  Infinity Cache or HBM then serves them).

and the LDS footprint of one block against the 160 KiB of a compute unit.
Host-side model only: nothing here runs on or depends on the GPU.
"""
from __future__ import annotations

import math

import numpy as np

LINE = 128                      # bytes per L2 line
L2_BYTES = 4 << 20              # per XCD
N_XCD = 8
LDS_BYTES = 160 << 10           # per compute unit


def xcd_blocks(nblocks: int):
    """Logical block ids run by each XCD: hardware block b goes to XCD b % 8;
    the kernels renumber it (when nblocks % 8 == 0) so that XCD x owns the
    contiguous logical range [x n/8, (x+1) n/8)."""
    if nblocks % N_XCD:
        return [list(range(x, nblocks, N_XCD)) for x in range(N_XCD)]
    per = nblocks // N_XCD
    return [list(range(x * per, (x + 1) * per)) for x in range(N_XCD)]


def lru_misses(seq_per_xcd, capacity_lines: int = L2_BYTES // LINE) -> int:
    """Misses of one LRU cache per XCD over its sequence of line-id arrays."""
    total = 0
    for seq in seq_per_xcd:
        cache = {}
        miss = 0
        for lines in seq:
            for ln in lines.tolist():
                if ln in cache:
                    del cache[ln]
                else:
                    miss += 1
                    if len(cache) >= capacity_lines:
                        del cache[next(iter(cache))]
                cache[ln] = None
        total += miss
    return total


def _lines_of_pixels(pix, c):
    """Line ids of NHWC pixels (flat pixel ids, -1 = outside) of c fp16 channels."""
    pix = np.asarray(pix).ravel()
    pix = np.unique(pix[pix >= 0])
    bpp = 2 * c
    if bpp % LINE == 0:
        lpp = bpp // LINE
        return (pix[:, None] * lpp + np.arange(lpp)).ravel()
    first = (pix * bpp) // LINE
    last = (pix * bpp + bpp - 1) // LINE
    return np.unique(np.concatenate([np.arange(a, b + 1) for a, b in zip(first, last)]))


def _halo_pixels(nimg, r0, c0, nr, nc, H, W):
    """Flat pixel ids of the window rows r0..r0+nr-1, columns c0..c0+nc-1 of
    image nimg (-1 outside the image)."""
    rr = r0 + np.arange(nr)[:, None]
    cc = c0 + np.arange(nc)[None, :]
    ok = (rr >= 0) & (rr < H) & (cc >= 0) & (cc < W)
    return np.where(ok, (nimg * H + rr) * W + cc, -1)


def _weights_lines(nbytes, base):
    return base + np.arange(math.ceil(nbytes / LINE))


def _run(blocks_tiles, nblocks, weight_bytes, c, tile_pixels, out_bytes, lds_bytes):
    """blocks_tiles[lb] = list of steps, each a list of tile ids the block
    works on in that step; tile_pixels(t) = pixel ids the tile loads."""
    base = 1 << 40   # line ids of the weights, apart from the input's
    wl = _weights_lines(weight_bytes, base) if weight_bytes else np.zeros(0, dtype=np.int64)
    cache_lines = {}

    def lines(t):
        v = cache_lines.get(t)
        if v is None:
            v = _lines_of_pixels(tile_pixels(t), c)
            cache_lines[t] = v
        return v

    per_tile = 0
    seqs = []
    for xb in xcd_blocks(nblocks):
        seq = [wl for b in xb if blocks_tiles[b]]
        nsteps = max((len(blocks_tiles[b]) for b in xb), default=0)
        for s in range(nsteps):
            for b in xb:
                if s < len(blocks_tiles[b]):
                    for t in blocks_tiles[b][s]:
                        seq.append(lines(t))
        seqs.append(seq)
    for xb in xcd_blocks(nblocks):
        for b in xb:
            if blocks_tiles[b]:
                per_tile += len(wl) * LINE
                per_tile += sum(len(lines(t)) * LINE for st in blocks_tiles[b] for t in st)
    return {"read_per_tile": int(per_tile), "read_l2_model": int(lru_misses(seqs) * LINE),
            "write": int(out_bytes), "lds_bytes_per_block": int(lds_bytes),
            "lds_fits": bool(lds_bytes <= LDS_BYTES)}


def _ranges(ntiles, nblocks):
    return [(lb * ntiles // nblocks, (lb + 1) * ntiles // nblocks) for lb in range(nblocks)]


def conv_pool_wr(n, h, w, c, k, cus=256, argmax=False):
    """Register-weights conv + 2x2 pool (k_conv_pool_wr): row tile = one pooled
    row of 8 windows (halo 4 x 18 pixels), tiles of 2 row tiles taken in order
    (alternately by the block's two wave groups; odd blocks walk their range
    backward), one block per CU, weights
    read once per block; LDS: a ring of four 20 KiB halo buffers, four 4 KiB
    output staging areas and the bias/scale."""
    P2, Q2 = h // 2, w // 2
    JB = -(-Q2 // 8)
    nrt = n * P2 * JB
    nb = min(cus, nrt)
    bt = []
    for lb, (a, b) in enumerate(_ranges(nrt, nb)):
        if lb % 2 == 0:
            bt.append([list(range(s, min(s + 2, b))) for s in range(a, b, 2)])
        else:   # odd blocks walk their range backward
            bt.append([list(range(max(a, e - 2), e)) for e in range(b, a, -2)])

    def pix(rt):
        q, jb = divmod(rt, JB)
        img, i = divmod(q, P2)
        return _halo_pixels(img, 2 * i - 1, 16 * jb - 1, 4, 18, h, w)
    out = 2 * n * P2 * Q2 * k + (n * P2 * Q2 * k if argmax else 0)
    r = _run(bt, nb, 2 * 9 * c * k, c, pix, out, 4 * 20480 + 4 * 4096 + 1024)
    r.update(read_algorithmic=2 * (n * h * w * c + 9 * c * k), kernel="k_conv_pool_wr", tiles=nrt, blocks=nb)
    return r


def conv_pool_wino(n, h, w, c, k, cus=256, argmax=False):
    """Winograd conv + pool (k_conv_pool_wino): batch = 2 x 8 output tiles
    (halo 6 x 18 pixels), one batch per step, one block per CU, transformed
    weights (16 c k) read once per block."""
    TH, TW = h // 2, w // 2
    bh, bw = -(-TH // 2), -(-TW // 8)
    nbatch = n * bh * bw
    nb = min(nbatch, cus)
    bt = [[[t] for t in (range(a, b) if lb % 2 == 0 else range(b - 1, a - 1, -1))]
          for lb, (a, b) in enumerate(_ranges(nbatch, nb))]   # odd blocks walk backward

    def pix(bi):
        img, r = divmod(bi, bh * bw)
        ib, jb = divmod(r, bw)
        return _halo_pixels(img, 4 * ib - 1, 16 * jb - 1, 6, 18, h, w)
    out = 2 * n * TH * TW * k + (n * TH * TW * k if argmax else 0)
    ndma = -(-108 * (c // 8) // 64)
    lds = 2 * 16 * 16 * c * 2 + 2 * ndma * 1024 + 2 * 16 * k * 2 + 2 * 16 * k + 4 * k
    r = _run(bt, nb, 2 * 16 * c * k, c, pix, out, lds)
    r.update(read_algorithmic=2 * (n * h * w * c + 16 * c * k), kernel="k_conv_pool_wino", tiles=nbatch, blocks=nb)
    return r


def _rf_grid(ntiles, per_block, cus):
    grid = cus
    if grid * per_block > ntiles:
        grid = -(-ntiles // per_block)
    grid = max(grid, 1)
    tpb = -(-ntiles // grid)
    return -(-ntiles // tpb), tpb


def conv3x3_rows(n, h, w, c, weight_bytes, out_bytes, lds, kernel, rows_per_tile, pool, waves=8, cus=256):
    """Implicit-GEMM conv kernels whose waves each own a tile of GEMM rows
    (k_conv_w: 64 rows, k_chain_rf with the conv loader: 32 rows): a block's
    contiguous tile range, its waves on consecutive tiles, weights resident
    per block.  Rows are pixels (row-major) or, pooled, the four pixels of
    each 2x2 window in turn."""
    npix = n * h * w
    if pool:
        P2, Q2 = h // 2, w // 2
        nrows = 4 * n * P2 * Q2
    else:
        nrows = npix
    ntiles = -(-nrows // rows_per_tile)
    nb, tpb = _rf_grid(ntiles, waves, cus)
    bt = []
    for lb in range(nb):
        a, b = lb * tpb, min((lb + 1) * tpb, ntiles)
        bt.append([list(range(s, min(s + waves, b))) for s in range(a, b, waves)])
    dr, ds = np.meshgrid(np.arange(-1, 2), np.arange(-1, 2), indexing="ij")

    def pix(t):
        g = np.arange(t * rows_per_tile, min((t + 1) * rows_per_tile, nrows))
        if pool:
            win, e = g // 4, g % 4
            img, rem = win // (P2 * Q2), win % (P2 * Q2)
            p = 2 * (rem // Q2) + e // 2
            q = 2 * (rem % Q2) + e % 2
        else:
            img, rem = g // (h * w), g % (h * w)
            p, q = rem // w, rem % w
        pp = p[:, None] + dr.ravel()[None, :]
        qq = q[:, None] + ds.ravel()[None, :]
        ok = (pp >= 0) & (pp < h) & (qq >= 0) & (qq < w)
        return np.where(ok, (img[:, None] * h + pp) * w + qq, -1)
    r = _run(bt, nb, weight_bytes, c, pix, out_bytes, lds)
    r.update(kernel=kernel, tiles=ntiles, blocks=nb)
    return r


def conv_pool_w(n, h, w, c, k, cus=256, argmax=False):
    """LDS-weights conv + pool (k_conv_w, pooled rows, 64-row tiles)."""
    out = 2 * n * (h // 2) * (w // 2) * k + (n * (h // 2) * (w // 2) * k if argmax else 0)
    lds = 9 * c * k * 2 + k * 8 + 16 + 8 * 1024
    r = conv3x3_rows(n, h, w, c, 2 * 9 * c * k, out, lds, "k_conv_w", 64, True, cus=cus)
    r["read_algorithmic"] = 2 * (n * h * w * c + 9 * c * k)
    return r


def conv2_rf(n, h, w, c, k0, k1, cus=256, k_more=()):
    """conv3x3 -> conv1x1 (-> further conv1x1 widths k_more) in the
    register-resident chain (k_chain_rf with the 3x3 row loader, 32-row
    tiles), every weight matrix resident per block."""
    ks = [k0, k1] + list(k_more)
    wb = 2 * (9 * c * k0 + sum(ks[i] * ks[i + 1] for i in range(len(ks) - 1)))
    out = 2 * n * h * w * ks[-1]
    lds = wb + 4 * sum(ks) + 8 * 32 * 72 * 2
    r = conv3x3_rows(n, h, w, c, wb, out, lds, "k_chain_rf", 32, False, cus=cus)
    r["read_algorithmic"] = 2 * n * h * w * c + wb
    return r


def conv2_pipe(n, h, w, c, k0, k1, cus=256, mid=0):
    """conv3x3 -> conv1x1 in two pipelined wave groups (k_conv2_pipe): row
    tile = 2 image rows x 16 columns (halo 4 x 18 pixels), tiles of 2 row
    tiles taken in order (odd blocks walk their range backward), one block per
    CU, both weight matrices read once per block; LDS: three 20 KiB halo
    buffers, two 8 KiB intermediate tiles, four 8 KiB output staging tiles and
    the biases.  mid > 0: a middle 1x1 conv k0 -> mid (its weights resident
    too, two more 8 KiB intermediate tiles)."""
    P2, JB = -(-h // 2), -(-w // 16)
    nrt = n * P2 * JB
    nb = min(cus, nrt)
    bt = []
    for lb, (a, b) in enumerate(_ranges(nrt, nb)):
        if lb % 2 == 0:
            bt.append([list(range(s, min(s + 2, b))) for s in range(a, b, 2)])
        else:
            bt.append([list(range(max(a, e - 2), e)) for e in range(b, a, -2)])

    def pix(rt):
        q, jb = divmod(rt, JB)
        img, i = divmod(q, P2)
        return _halo_pixels(img, 2 * i - 1, 16 * jb - 1, 4, 18, h, w)
    wb = 2 * (9 * c * k0 + (k0 * mid + mid * k1 if mid else k0 * k1))
    out = 2 * n * h * w * k1
    r = _run(bt, nb, wb, c, pix, out, 3 * 20480 + (4 if mid else 2) * 8192 + 4 * 8192 + 4 * (128 + 256))
    r.update(read_algorithmic=2 * n * h * w * c + wb, kernel="k_conv2_pipe", tiles=nrt, blocks=nb)
    return r


def gemm_chain(M, K0, N0, N1, variant, cus=256):
    """Two-GEMM chain: the rows of A are read once by the tile that owns them
    (no halo), each block reads the weights once; the weights of all blocks
    of an XCD fit its L2, so an XCD fetches them once."""
    wb = 2 * (K0 * N0 + N0 * N1)
    if variant == "rf":
        ntiles = -(-M // 32)
        nb, _ = _rf_grid(ntiles, 8, cus)
        lds = 2 * (-(-K0 // 64) * 64 * N0 + N0 * N1) + 4 * (N0 + N1) + 8 * 32 * 72 * 2
    elif variant == "lds":
        nb = -(-M // 128)
        lds = 2 * 64 * (max(N0, 256) + 32) * 2 + 128 * (N0 + 8) * 2 + 4 * (N0 + 256)
    else:   # stream
        nb = min(cus, -(-M // 256))
        lds = 3 * 64 * 256 * 2 + 4 * (N0 + N1)
    a_bytes = 2 * M * K0
    return {"kernel": {"rf": "k_chain_rf", "lds": "k_gemm_lds", "stream": "k_chain_stream"}[variant],
            "blocks": nb, "read_algorithmic": a_bytes + wb, "read_per_tile": a_bytes + nb * wb,
            "read_l2_model": a_bytes + min(nb, N_XCD) * wb, "write": 2 * M * N1,
            "lds_bytes_per_block": lds, "lds_fits": lds <= LDS_BYTES}


def gemm_chain_n(M, widths, cus=256):
    """N-stage GEMM chain in the register-resident kernel: rows once, every
    weight matrix resident per block (fetched once per XCD)."""
    wb = 2 * sum(widths[i] * widths[i + 1] for i in range(len(widths) - 1))
    nb, _ = _rf_grid(-(-M // 32), 8, cus)
    a_bytes = 2 * M * widths[0]
    lds = wb + 4 * sum(widths[1:]) + 8 * 32 * 72 * 2
    return {"kernel": "k_chain_rf", "blocks": nb, "read_algorithmic": a_bytes + wb, "read_per_tile": a_bytes + nb * wb,
            "read_l2_model": a_bytes + min(nb, N_XCD) * wb, "write": 2 * M * widths[-1],
            "lds_bytes_per_block": lds, "lds_fits": lds <= LDS_BYTES}


def for_workload(spec: dict, variant: str | None = None, cus: int = 256, argmax: bool = False) -> dict | None:
    """The model for one of the bench's workloads (inputs.workload spec) in
    the kernel form the bench runs; None where no model is given."""
    kind = spec["kind"]
    if kind == "gemm2":
        v = variant or ("lds" if spec["N0"] > 128 else "rf")
        return gemm_chain(spec["M"], spec["K0"], spec["N0"], spec["N1"], v, cus)
    if kind == "gemmN":
        return gemm_chain_n(spec["M"], spec["widths"], cus)
    if kind == "conv2":
        if variant != "rf" and spec["c"] == 64 and spec["k0"] == 64 and spec["k1"] <= 256:
            return conv2_pipe(spec["n"], spec["h"], spec["w"], spec["c"], spec["k0"], spec["k1"], cus)
        return conv2_rf(spec["n"], spec["h"], spec["w"], spec["c"], spec["k0"], spec["k1"], cus)
    if kind == "convN":
        ks = spec["ks"]
        if (variant != "rf" and len(ks) == 3 and spec["c"] == 64 and ks[0] == 64 and ks[1] == 64
                and ks[2] <= 256):
            r = conv2_pipe(spec["n"], spec["h"], spec["w"], spec["c"], ks[0], ks[2], cus, mid=ks[1])
            return r
        return conv2_rf(spec["n"], spec["h"], spec["w"], spec["c"], ks[0], ks[1], cus, ks[2:])
    if kind == "conv_pool":
        n, h, w, c, k = spec["n"], spec["h"], spec["w"], spec["cpad"], spec["k"]
        if variant == "winograd":
            return conv_pool_wino(n, h, w, c, k, cus, argmax)
        if variant == "lds_weights":
            return conv_pool_w(n, h, w, c, k, cus, argmax)
        return conv_pool_wr(n, h, w, c, k, cus, argmax)
    return None
