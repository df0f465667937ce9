// conv2_pipe.hip -- conv3x3 (64 -> 64) + bias + activation -> conv1x1
// (64 -> k1 <= 256) + bias, in two pipelined wave groups with the input halo
// streamed into LDS; optionally (MID) with a middle conv1x1 (64 -> 64) + bias
// + activation between them.
//
// BOLT's persistent kernel fusion for a 3x3 -> 1x1 conv pair (BOLT notes,
// "Persistent kernel (GEMM/Conv) fusion": the 1x1 conv is a GEMM over the
// channels of the 3x3 conv's output, which stays on chip); both convs are
// implicit GEMMs (interview page, Conv items 2 and 5): rows are output pixels,
// k = (r*3 + s)*64 + c for the 3x3 conv and k = c for the 1x1 conv.
//
// Mapping to CDNA4 (gfx950), one block of 8 waves per CU:
//   * Rows: a "row tile" is 32 pixels, 2 image rows x 16 columns (MFMA row m
//     -> image row 2i + (m / 2) % 2, column 16 jb + 2 (m / 4) + m % 2), so its
//     3x3 input halo is 4 rows x 18 columns; a tile is 2 consecutive row tiles.
//   * Group 0 (waves 0..3) runs the 3x3 conv.  Wave q owns output channels
//     [32 (q % 2), + 32) of row tile q / 2 over the whole reduction (576 k):
//     its 576 x 32 slice of the HWIO weights sits in 144 registers as ready
//     MFMA fragments.  The tile's halo arrives by LDS-DMA (wave q
//     fetches row tile q / 2, channel half q % 2) two tiles ahead, pixels
//     outside the image masked to an offset outside the buffer resource (the
//     zero padding); operand A is read from the halo with ds_read_b128 in
//     MFMA layout, with the XOR slot swizzle that keeps every 16-lane group on
//     16 different bank groups.  Both convs are computed transposed (weights
//     as operand A, pixels as operand B), so a lane's accumulators are four
//     consecutive channels of one pixel: the epilogue (bias, activation, fp16)
//     writes the tile's [64 pixels][64 channels] intermediate H to LDS in
//     8-byte pieces.
//   * Group 1 (waves 4..7) runs the 1x1 conv of the previous tile: wave q owns
//     output channels [64 (q - 4), + 64); its 64 x 64 slice of W1 is 32
//     registers of fragments, H the pixel operand (ds_read_b128, 16-byte
//     chunks XOR-swizzled by row so the reads are conflict-free).  Bias,
//     fp16, a per-wave LDS staging tile, and 16-byte stores of whole 128-byte
//     runs of the output rows.
//   * MID: group 0 also runs the middle conv1x1 of the tile it convolved one
//     phase earlier (H -> H2, its 64 x 32 slice of the middle weights in 16
//     more registers), and group 1 reads H2 one phase later still.
//   * One barrier per phase: in phase k group 0 computes tile k (and requests
//     the halo of tile k + 2), group 1 tile k - 1 (k - 2 with MID).  Each SIMD holds one wave of
//     each group, so the 3x3 conv's matrix work overlaps the 1x1 conv and the
//     output stores (51 MB at the 32 x 56 x 56 x 256 workload: the stores set
//     this chain's floor).
#include "fc_dma.h"
#include "fc_launch.h"

namespace fc {

namespace {

constexpr int CP_THREADS = 512;
constexpr int CP_C = 64;                            // input channels
constexpr int CP_K0 = 64;                           // 3x3 conv output channels
constexpr int CP_K1P = 256;                         // 1x1 conv output channels (padded)
constexpr int CP_NBUF = 3;                          // halo ring depth (tiles)
constexpr int CP_HROW = 20;                         // halo row stride (pixels): 18 used + 2 padding
constexpr int CP_SLOTS = 4 * 4 * CP_HROW;           // 16-byte slots per row-tile halo (32 channels)
constexpr int CP_PART_BYTES = 16 * CP_SLOTS;        // 5 KiB: one row tile, one channel half
constexpr int CP_DMA_PER_PART = CP_SLOTS / 64;      // 1 KiB DMA instructions per part
constexpr int CP_BUF_BYTES = 4 * CP_PART_BYTES;     // one tile's halo (2 row tiles x 2 halves)
constexpr int CP_H_BYTES = 64 * CP_K0 * 2;          // one tile's intermediate [64][64] fp16
constexpr int CP_OST_BYTES = 64 * 64 * 2;           // per group-1 wave output staging [64][64] fp16
// LDS: the halo ring, H (and H2, the middle 1x1 conv's output, with MID)
// double-buffered, the output staging, the biases b0 | bm | b1
constexpr int CP_H_OFF = CP_NBUF * CP_BUF_BYTES;
constexpr int cp_ost_off(int mid) { return CP_H_OFF + 2 * CP_H_BYTES * (1 + mid); }
constexpr int cp_bias_off(int mid) { return cp_ost_off(mid) + 4 * CP_OST_BYTES; }
constexpr int cp_lds(int mid) { return cp_bias_off(mid) + (2 * CP_K0 + CP_K1P) * 4; }   // 110 / 126 KiB
constexpr int CP_W0_BYTES = 9 * CP_C * CP_K0 * 2;            // 72 KiB, staged once at the start
constexpr int CP_W1_BYTES = CP_K0 * CP_K1P * 2;              // 32 KiB
constexpr int CP_WM_BYTES = CP_K0 * CP_K0 * 2;               // 8 KiB (MID)
constexpr int CP_APD = 2;                                    // A-operand prefetch distance (k-steps)
static_assert(CP_SLOTS % 64 == 0, "whole DMA instructions per part");
static_assert(cp_lds(1) <= 160 * 1024 && CP_W0_BYTES + CP_W1_BYTES <= cp_bias_off(0) &&
                  CP_W0_BYTES + CP_W1_BYTES + CP_WM_BYTES <= cp_bias_off(1),
              "LDS budget");

// slot swizzle of halo pixel (hr, hc): 16 lanes of a 16-byte read land on 16
// different bank groups (rows r and r + 1 and columns with each hc % 4)
__device__ __forceinline__ int cp_swz(int hr, int hc) { return (hr & 1) | (((hc >> 2) & 1) << 1); }
// H / output staging: 16-byte chunk c of row r sits at chunk c ^ (r & 7)
__device__ __forceinline__ int cp_hoff(int r, int c8) { return r * 64 + ((c8 ^ (r & 7)) << 3); }

struct PipeArgs {
    const half_t* x;    // [NB, H, W, 64]
    const half_t* w0;   // HWIO [3, 3, 64, 64]
    const half_t* b0;   // [64] or null
    const half_t* w1;   // [64, K1]
    const half_t* b1;   // [K1] or null
    const half_t* wm;   // middle 1x1 conv [64, 64] (MID)
    const half_t* bm;   // [64] or null (MID)
    int act1, act2;     // activations after the middle (MID) and the last 1x1 conv
    half_t* y;          // [NB, H, W, K1]
    int NB, H, W, K1;
    int P2, JB;         // row pairs ceil(H / 2), column blocks ceil(W / 16)
    long nrt;           // row tiles in total = NB * P2 * JB
    int nblocks;
    FastDiv fjb, fp2;   // by JB, by P2
};

}  // namespace

// MID = 1: a middle 1x1 conv 64 -> 64 between the two, run by group 0 one
// phase after its 3x3 conv of the same tile (H -> H2 in LDS); group 1 then
// reads H2, one phase later still.
template <int ACT, int MID>
__global__ __launch_bounds__(CP_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_conv2_pipe(PipeArgs a)
{
    constexpr int CP_OST_OFF = cp_ost_off(MID), CP_BIAS_OFF = cp_bias_off(MID), CP_LDS = cp_lds(MID);
    constexpr int NST = 9 * CP_C / 16;   // k-steps of the 3x3 conv
    extern __shared__ __align__(16) char smem[];
    typedef FC_LDS char lds_char;
    typedef FC_LDS half8 lds_half8;
    typedef FC_LDS float lds_float;
    typedef Act<ACT> act;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, hh = lane >> 5;
    const int wq = wave & 3, wg = wave >> 2;
    lds_char* const lds = (lds_char*)smem;

    // ---- this block's row tiles (XCD-contiguous ranges; odd blocks walk
    // backward so neighbours reach the input rows they share at the same time)
    const long lb = xcd_block(blockIdx.x, gridDim.x);
    const long rt_begin = lb * a.nrt / a.nblocks;
    const long rt_end = (lb + 1) * a.nrt / a.nblocks;
    const int ntiles = (int)((rt_end - rt_begin + 1) / 2);
    const bool backward = lb & 1;
    auto tile_first = [&](int j) -> long { return backward ? max(rt_begin, rt_end - 2L * (j + 1)) : rt_begin + 2L * j; };
    auto tile_nrt = [&](int j) -> int {
        return (int)(backward ? rt_end - 2L * j - tile_first(j) : min(2L, rt_end - rt_begin - 2L * j));
    };
    struct RT {
        int n, i, jb;
    };
    auto decode = [&](long rt) -> RT {
        RT r;
        const unsigned q = a.fjb.div((unsigned)rt);
        r.jb = (int)((unsigned)rt - q * a.fjb.d);
        const unsigned n = a.fp2.div(q);
        r.i = (int)(q - n * a.fp2.d);
        r.n = (int)n;
        return r;
    };

    // ---- weights and biases: W0 [576][64] and W1 [64][K1P] natural in LDS,
    // then each wave takes its fragments into registers
    WTile W0n, W1n;
    W0n.p = (lds_half*)smem;
    W0n.ld = wtile_ld(CP_K0);
    W0n.swz = wtile_swz(CP_K0);
    W1n.p = (lds_half*)(lds + CP_W0_BYTES);
    W1n.ld = wtile_ld(CP_K1P);
    W1n.swz = wtile_swz(CP_K1P);
    if constexpr (kPoison) {
        lds_poison(smem, CP_LDS, tid, CP_THREADS);
        __syncthreads();
    }
    stage_natural<8>(a.w0, 9 * CP_C, CP_K0, CP_K0, 9 * CP_C, CP_K0, W0n, tid, CP_THREADS);
    stage_natural<8>(a.w1, CP_K0, a.K1, a.K1, CP_K0, CP_K1P, W1n, tid, CP_THREADS);
    WTile Wmn;
    Wmn.p = (lds_half*)(lds + CP_W0_BYTES + CP_W1_BYTES);
    Wmn.ld = wtile_ld(CP_K0);
    Wmn.swz = wtile_swz(CP_K0);
    if constexpr (MID > 0) stage_natural<8>(a.wm, CP_K0, CP_K0, CP_K0, CP_K0, CP_K0, Wmn, tid, CP_THREADS);
    __syncthreads();
    lds_float* const bsl = (lds_float*)(lds + CP_BIAS_OFF);   // b0 [64], bm [64], b1 [K1P] (past the weights)
    for (int i = tid; i < 2 * CP_K0 + CP_K1P; i += CP_THREADS) {
        float v = 0.0f;
        if (i < CP_K0) {
            if (a.b0) v = (float)a.b0[i];
        } else if (i < 2 * CP_K0) {
            if (MID > 0 && a.bm) v = (float)a.bm[i - CP_K0];
        } else if (a.b1 && i - 2 * CP_K0 < a.K1) {
            v = (float)a.b1[i - 2 * CP_K0];
        }
        bsl[i] = v;
    }
    __syncthreads();
    // after each group has its fragments in registers, LDS is reused for the
    // halos, H and the staging (one barrier in each branch below)
    auto release_weights = [&]() {
        __syncthreads();
        if constexpr (kPoison) {
            lds_poison(smem, CP_BIAS_OFF, tid, CP_THREADS);
            __syncthreads();
        }
    };
    auto buf_of = [&](int j) -> lds_char* { return lds + (j % CP_NBUF) * CP_BUF_BYTES; };
    auto h_of = [&](int j) -> lds_half* { return (lds_half*)(lds + CP_H_OFF + (j & 1) * CP_H_BYTES); };
    auto h2_of = [&](int j) -> lds_half* { return (lds_half*)(lds + CP_H_OFF + (2 + (j & 1)) * CP_H_BYTES); };

    // phase k: group 0 on tile k (and, MID, on tile k - 1's middle conv),
    // group 1 on tile k - 1 - MID
    const int nph = ntiles + 1 + MID;
    if (wg == 0) {
        // ---- group 0: halo DMA, the 3x3 conv, H to LDS
        half8 wf[NST];   // W0 rows 16 st + 8 hh + [0, 8), column 32 (wq % 2) + lr
#pragma unroll
        for (int st = 0; st < NST; ++st)
            wf[st] = frag_tr_at(W0n.p + frag_lane_off(W0n, 32 * (wq & 1), lane) + (16 * st + 8 * hh) * W0n.ld,
                                4 * W0n.ld);
        half8 wmf[MID > 0 ? 4 : 1];   // Wm rows 16 s + 8 hh + [0, 8), column 32 (wq % 2) + lr
        if constexpr (MID > 0) {
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                wmf[s2] = frag_tr_at(Wmn.p + frag_lane_off(Wmn, 32 * (wq & 1), lane) + (16 * s2 + 8 * hh) * Wmn.ld,
                                     4 * Wmn.ld);
        }
        release_weights();
        const int W = a.W;
        unsigned dma_off[CP_DMA_PER_PART];   // per-lane offsets from the halo origin
#pragma unroll
        for (int i = 0; i < CP_DMA_PER_PART; ++i) {
            const int slot = 64 * i + lane;
            const int p = slot >> 2, part = slot & 3;
            const int hr = p / CP_HROW, hcl = p - hr * CP_HROW;
            const int g = part ^ cp_swz(hr, hcl);
            dma_off[i] = hcl < 18 ? (unsigned)(hr * W + hcl) * (unsigned)(2 * CP_C) + (unsigned)(64 * (wq & 1) + 16 * g)
                                  : CS_OUTSIDE;
        }
        const long total_pix = (long)a.NB * a.H * W;
        // wave q fetches row tile q / 2, channel half q % 2 of tile j
        auto dma_tile = [&](int j) -> bool {
            const int u = wq >> 1;
            if (j >= ntiles || u >= tile_nrt(j)) return false;
            lds_char* const dst = buf_of(j) + wq * CP_PART_BYTES;
            if constexpr (kPoison) {   // released by the barrier of the tile before
                lds_poison(dst, CP_PART_BYTES, lane, 64);
                wave_lds_sync();
            }
            const RT t = decode(tile_first(j) + u);
            const int ih0 = 2 * t.i - 1, iw0 = 16 * t.jb - 1;
            const long base_pix = ((long)t.n * a.H + ih0) * W + iw0;
            const i32x4 rs =
                buf_rsrc((const void*)((long)a.x + base_pix * (2 * CP_C)), (total_pix - base_pix) * (long)(2 * CP_C));
            const int rlo = ih0 < 0 ? -ih0 : 0, rhi = min(4, a.H - ih0);
            const int clo = iw0 < 0 ? -iw0 : 0, chi = min(18, W - iw0);
            const unsigned long long cm = ((1ull << chi) - 1) & ~((1ull << clo) - 1);
            unsigned long long m_lo = 0;
            unsigned m_hi = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (r >= rlo && r < rhi) {
                    m_lo |= cm << (20 * r);
                    if (r == 3) m_hi = (unsigned)(cm >> 4);
                }
            const int quad = lane_id_here() >> 2;
#pragma unroll
            for (int i = 0; i < CP_DMA_PER_PART; ++i) {
                const unsigned win = i < 4 ? (unsigned)(m_lo >> (16 * i)) & 0xffffu : m_hi;
                dma16(rs, (win >> quad) & 1u ? dma_off[i] : CS_OUTSIDE, (const lds_half*)(dst + i * 1024));
            }
            return true;
        };
        const int u = wq >> 1, ct = wq & 1;
        dma_tile(0);
        if (dma_tile(1)) vm_wait<CP_DMA_PER_PART>();   // tile 0's part has landed
        else vm_wait<0>();
        __syncthreads();   // tile 0's halo visible
        for (int k = 0; k < nph; ++k) {
            if (k < ntiles && u < tile_nrt(k)) {
                // 36 k-steps: operand A of row tile u read from the halo (the
                // lane's address depends on the tap only through r % 2 and s)
                const lds_char* const buf = buf_of(k) + 2 * u * CP_PART_BYTES;
                const int ln = lane_id_here();
                const int m = ln & 31, hi = ln >> 5;
                const int dy = (m >> 1) & 1, dx = m & 1, w4 = m >> 2;
                const lds_char* const lb0 = buf + (dy * CP_HROW + 2 * w4 + dx) * 64;
                const lds_char* ap[2][3][2];
#pragma unroll
                for (int rp = 0; rp < 2; ++rp)
#pragma unroll
                    for (int sc = 0; sc < 3; ++sc)
#pragma unroll
                        for (int qo = 0; qo < 2; ++qo)
                            ap[rp][sc][qo] = lb0 + (((hi | 2 * qo) ^ cp_swz(dy + rp, 2 * w4 + dx + sc)) << 4);
                auto load_a = [&](int st) -> half8 {
                    const int tap = st >> 2, q = st & 3, r = tap / 3, sc = tap % 3;
                    return *reinterpret_cast<const lds_half8*>(ap[r & 1][sc][q & 1] + (q >> 1) * CP_PART_BYTES +
                                                               (r * CP_HROW + sc) * 64);
                };
                constexpr int R = CP_APD + 1;
                half8 af[R];
#pragma unroll
                for (int st = 0; st < CP_APD; ++st) af[st] = load_a(st);
                floatx16 acc = zero16();
#pragma unroll
                for (int st = 0; st < NST; ++st) {
                    if (st + CP_APD < NST) af[(st + CP_APD) % R] = load_a(st + CP_APD);
                    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch issued here
                    acc = mfma32x32x16(wf[st], af[st % R], acc);   // transposed: rows = channels
                }
                // epilogue: lane (pixel 32 u + lr) holds channels 32 ct + 8 g + 4 hh + [0, 4):
                // + b0, activation, fp16, 8 bytes to H [pixel][channel]
                lds_half* const hs = h_of(k);
                typedef FC_LDS half4 lds_half4;
                typedef FC_LDS floatx4 lds_floatx4;
                const int r = 32 * u + lr;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c0 = 32 * ct + 8 * g + 4 * hh;
                    const floatx4 bk = *reinterpret_cast<const lds_floatx4*>(bsl + c0);
                    half4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (half_t)act::f(acc[4 * g + e] + bk[e]);
                    *reinterpret_cast<lds_half4*>(hs + cp_hoff(r, c0 >> 3) + (c0 & 7)) = o;
                }
            }
            if constexpr (MID > 0) {
                // the middle 1x1 conv of tile k - 1 (its H published by the last
                // barrier): channels 32 ct.. of row tile u, + bm, act1, fp16 -> H2
                if (k >= 1 && k - 1 < ntiles && u < tile_nrt(k - 1)) {
                    const lds_half* const hs = h_of(k - 1);
                    floatx16 am = zero16();
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        const half8 hp = *reinterpret_cast<const lds_half8*>(hs + cp_hoff(32 * u + lr, 2 * s2 + hh));
                        am = mfma32x32x16(wmf[s2], hp, am);
                    }
                    lds_half* const h2 = h2_of(k - 1);
                    typedef FC_LDS half4 lds_half4;
                    typedef FC_LDS floatx4 lds_floatx4;
                    act_dispatch(a.act1, [&](auto act1) {
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int c0 = 32 * ct + 8 * g + 4 * hh;
                            const floatx4 bk = *reinterpret_cast<const lds_floatx4*>(bsl + CP_K0 + c0);
                            half4 o;
#pragma unroll
                            for (int e = 0; e < 4; ++e) o[e] = (half_t)act1.f(am[4 * g + e] + bk[e]);
                            *reinterpret_cast<lds_half4*>(h2 + cp_hoff(32 * u + lr, c0 >> 3) + (c0 & 7)) = o;
                        }
                    });
                }
            }
            if (dma_tile(k + 2)) vm_wait<CP_DMA_PER_PART>();   // tile k + 1's part has landed
            else vm_wait<0>();
            __syncthreads();
        }
    } else {
        // ---- group 1: the 1x1 conv of the previous tile, bias, stores
        half8 w1f[4][2];   // W1 rows 16 s + 8 hh + [0, 8), column 64 wq + 32 t + lr
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                w1f[s][t] = frag_tr_at(W1n.p + frag_lane_off(W1n, 64 * wq + 32 * t, lane) + (16 * s + 8 * hh) * W1n.ld,
                                       4 * W1n.ld);
        release_weights();
        lds_half* const ost = (lds_half*)(lds + CP_OST_OFF + wq * CP_OST_BYTES);
        const int K1 = a.K1;
        __syncthreads();   // (group 0's first barrier: tile 0's halo visible)
        for (int k = 0; k < nph; ++k) {
            const int j = k - 1 - MID;
            if (j >= 0) {
                const int nrt = tile_nrt(j);
                const lds_half* const hs = MID > 0 ? h2_of(j) : h_of(j);
                floatx16 acc[2][2];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    half8 hf[2];
#pragma unroll
                    for (int uu = 0; uu < 2; ++uu)
                        hf[uu] = *reinterpret_cast<const lds_half8*>(hs + cp_hoff(32 * uu + lr, 2 * s + hh));
#pragma unroll
                    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
                        for (int t = 0; t < 2; ++t)
                            acc[uu][t] = mfma32x32x16(w1f[s][t], hf[uu], s == 0 ? zero16() : acc[uu][t]);
                }
                // transposed result: lane (pixel 32 uu + lr) holds channels 64 wq + 32 t +
                // 8 g + 4 hh + [0, 4): + b1, fp16, 8 bytes to staging [pixel][64 channels]
                typedef FC_LDS half4 lds_half4;
                typedef FC_LDS floatx4 lds_floatx4;
                act_dispatch(a.act2, [&](auto act2) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int cl = 32 * t + 8 * g + 4 * hh;
                            const floatx4 bk = *reinterpret_cast<const lds_floatx4*>(bsl + 2 * CP_K0 + 64 * wq + cl);
#pragma unroll
                            for (int uu = 0; uu < 2; ++uu) {
                                half4 o;
#pragma unroll
                                for (int e = 0; e < 4; ++e) o[e] = (half_t)act2.f(acc[uu][t][4 * g + e] + bk[e]);
                                *reinterpret_cast<lds_half4*>(ost + cp_hoff(32 * uu + lr, cl >> 3) + (cl & 7)) = o;
                            }
                        }
                });
                wave_lds_sync();
                // stores: lane L takes 16 bytes (channels 64 wq + 8 (L % 8) + [0, 8))
                // of rows L / 8 + 8 i; row r -> pixel of row tile r / 32
                const int c8 = lane & 7, col = 64 * wq + 8 * c8;
#pragma unroll
                for (int uu = 0; uu < 2; ++uu) {
                    if (uu < nrt) {
                        const RT t = decode(tile_first(j) + uu);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int m = (lane >> 3) + 8 * i;   // row within the row tile
                            const int py = 2 * t.i + ((m >> 1) & 1), px = 16 * t.jb + 2 * (m >> 2) + (m & 1);
                            const half8 v = *reinterpret_cast<const lds_half8*>(ost + cp_hoff(32 * uu + m, c8));
                            if (py < a.H && px < a.W && col < K1)
                                st_out(reinterpret_cast<half8*>(a.y + (((long)t.n * a.H + py) * a.W + px) * K1 + col), v);
                        }
                    }
                }
                wave_lds_sync();   // the next tile overwrites the staging tile
            }
            __syncthreads();
        }
    }
}

template <int ACT, int MID>
static hipError_t launch_pipe(PipeArgs a, hipStream_t st)
{
    static std::atomic<unsigned long long> lds_set{0};
    hipError_t e = allow_full_lds((const void*)k_conv2_pipe<ACT, MID>, &lds_set);
    if (e != hipSuccess) return e;
    long nb = device_cu_count();   // one block per CU
    if (nb > a.nrt) nb = a.nrt;
    a.nblocks = (int)nb;
    hipLaunchKernelGGL((k_conv2_pipe<ACT, MID>), dim3((unsigned)nb), dim3(CP_THREADS), (size_t)cp_lds(MID), st, a);
    return hipGetLastError();
}

template <int MID>
static hipError_t launch_pipe_act(int act, const PipeArgs& a, hipStream_t st)
{
    switch (act) {
    case ACT_RELU: return launch_pipe<ACT_RELU, MID>(a, st);
    case ACT_GELU_TANH: return launch_pipe<ACT_GELU_TANH, MID>(a, st);
    case ACT_HARDSWISH: return launch_pipe<ACT_HARDSWISH, MID>(a, st);
    default: return launch_pipe<ACT_NONE, MID>(a, st);
    }
}

// The conv3x3 -> conv1x1 shapes this kernel takes (3x3/s1/p1 checked by the
// caller): 64 input channels, 64 intermediate channels, up to 256 outputs,
// and halo offsets within a 4-row window that fit 32 bits.
bool conv2_pipe_fits(int W, int C, int K0, int K1)
{
    return C == CP_C && K0 == CP_K0 && K1 > 0 && K1 <= CP_K1P && K1 % 8 == 0 && (long)W * C < (1L << 27);
}

static PipeArgs pipe_args(const half_t* x, const half_t* w0, const half_t* b0, const half_t* w1, const half_t* b1,
                          half_t* y, int NB, int H, int W, int K1)
{
    PipeArgs a{};
    a.x = x; a.w0 = w0; a.b0 = b0; a.w1 = w1; a.b1 = b1; a.y = y;
    a.NB = NB; a.H = H; a.W = W; a.K1 = K1;
    a.act1 = ACT_NONE; a.act2 = ACT_NONE;
    a.P2 = (H + 1) / 2;
    a.JB = (W + 15) / 16;
    a.nrt = (long)NB * a.P2 * a.JB;
    a.nblocks = 1;
    if (a.nrt > 0) {
        a.fjb = FastDiv::make((unsigned)a.JB);
        a.fp2 = FastDiv::make((unsigned)a.P2);
    }
    return a;
}

hipError_t run_chain_conv2_pipe(const half_t* x, const half_t* w0, const half_t* b0, int act, const half_t* w1,
                                const half_t* b1, half_t* y, int NB, int H, int W, int K1, hipStream_t st)
{
    const PipeArgs a = pipe_args(x, w0, b0, w1, b1, y, NB, H, W, K1);
    if (a.nrt == 0) return hipSuccess;
    return launch_pipe_act<0>(act, a, st);
}

// conv3x3 (64 -> 64, act0) -> conv1x1 (64 -> 64, act1) -> conv1x1 (64 -> K2, act2)
hipError_t run_chain_conv3_pipe(const half_t* x, const half_t* const* w, const half_t* const* b, const int* act,
                                half_t* y, int NB, int H, int W, int K2, hipStream_t st)
{
    PipeArgs a = pipe_args(x, w[0], b[0], w[2], b[2], y, NB, H, W, K2);
    if (a.nrt == 0) return hipSuccess;
    a.wm = w[1]; a.bm = b[1];
    a.act1 = act[1]; a.act2 = act[2];
    return launch_pipe_act<1>(act[0], a, st);
}

}  // namespace fc
