// conv_pool_wr.hip -- conv3x3 + bias/scale + activation + 2x2/2 pool with the
// weights held in registers as ready MFMA operands and the input halo
// streamed into LDS.
//
// Welder's Conv -> ReLU -> MaxPool tile graph (Welder notes, "Operator-tile
// and Tile-graph" / "Tile-graph Scheduling", Figure 5): one output tile of the
// pool needs a 2x2-larger tile of the conv, which needs a halo of the input
// one pixel wider on every side; the conv tile never leaves the chip.  The
// conv is an implicit GEMM (interview page, Conv item 2): GEMM rows are conv
// output pixels, k = (r*3 + s)*C + c, columns = output channels.
//
// Mapping to CDNA4 (gfx950), for C = 64 input channels and 65..128 output
// channels (the x[32,112,112,60->64] -> 128 workload):
//   * Block = 8 waves (512 threads), one block per CU: two groups of four
//     waves, one wave of each group per SIMD.  Wave q of a group computes
//     output columns [32 q, 32 q + 32) over the whole reduction (9 taps x 64
//     channels): it holds its 576 x 32 slice of the HWIO weights ONCE, as
//     ready MFMA operand-B fragments, in 144 registers (36 k-steps x 4); the
//     main loop reads no weights and the waves never exchange partial sums.
//     The weights arrive through LDS in 128-row pieces (natural layout, read
//     with the transposing LDS load).
//   * GEMM rows are ordered window-major: a 32-row MFMA tile ("row tile") is
//     8 consecutive 2x2 pool windows of one pooled row (window 2g + h of the
//     tile lands in lane half h, accumulator registers 4g..4g+3), so the pool
//     is three max (or a sum) per output in registers.  A row tile needs a
//     4-row x 18-column input halo (stored with a row stride of 20 pixels).
//   * A tile is 2 consecutive row tiles (64 pixels); the block's tiles
//     alternate between the two groups.  The groups run in ping-pong: in each
//     phase one group runs a tile's 72 MFMAs per wave and nothing else, while
//     the other group (the second wave of every SIMD) stores, runs its
//     previous tile's epilogue and requests a later tile's halo; one barrier
//     per phase.  Each SIMD's matrix pipe is then fed by one wave at a time
//     while the other wave's non-matrix work hides under it (two waves that
//     both run all phases tend to reach their non-matrix phases together).
//   * A tile's input halo goes straight from global memory into LDS by the
//     LDS-DMA load (buffer_load_dwordx4 ... lds), into a ring of four
//     buffers, three phases ahead of its MFMAs.  Pixels outside the image,
//     and the two padding columns, read zero from outside the buffer resource
//     -- the conv's zero padding needs no branch.
//   * Operand A is read from the halo with ds_read_b128 in MFMA layout.  A
//     pixel's channel half (32 channels) is four 16-byte slots; slot s of the
//     pixel in halo row hr, column hc is stored at s ^ wr_swz(hr, hc) with
//     wr_swz = (hr & 1) | ((hc >> 2) & 1) << 1.  The LDS (64 banks) serves 16
//     lanes of a 16-byte read per clock: such a group reads pixels of two
//     halo rows and four columns spaced 2 apart, i.e. four pixels with each
//     value of hc % 4 (the 64-byte piece, with the 20-pixel row stride); the
//     swizzle gives those four distinct slots, so the 16 lanes touch 16
//     different 16-byte bank groups for every tap.  The DMA picks, for every
//     LDS slot, the global 16 bytes that belong there (quads of lanes still
//     read one 64-byte segment: the fast address path).
//   * Per k-step a wave issues 2 ds_read_b128 and 2 MFMAs (32x32x16 f16,
//     fp32 accumulate), with no address arithmetic; the operands are read two
//     k-steps ahead.
//   * Work split: the row tiles of the whole problem are divided into equal
//     contiguous ranges, one per block (49 row tiles each at the workload
//     above); a range's last tile may hold 1 row tile (those MFMAs are
//     skipped, not masked).
//   * Epilogue per row tile: pool (or average), scale/bias, activation, fp16,
//     into the group's LDS staging area [2 row tiles][8 windows][128
//     columns] (two per group, alternate tiles); two phases later every
//     thread of the group stores one 16-byte piece, so every pooled pixel
//     leaves as whole 128-byte lines.
#include "fc_dma.h"
#include "fc_launch.h"

namespace fc {

namespace {

constexpr int WR_THREADS = 512;                     // two groups of 4 waves
constexpr int WR_NRT = 2;                           // row tiles per tile
constexpr int WR_NBUF = 4;                          // halo ring depth (tiles)
constexpr int WR_HROW = 20;                         // halo row stride (pixels): 18 used + 2 padding
constexpr int WR_HPIX = 4 * WR_HROW;                // pixels per row-tile halo
constexpr int WR_SLOTS = 4 * WR_HPIX;               // 16-byte slots per row-tile halo (32 channels)
constexpr int WR_PART_BYTES = 16 * WR_SLOTS;        // 5 KiB: one row tile, one channel half
constexpr int WR_DMA_PER_PART = WR_SLOTS / 64;      // 1 KiB DMA instructions per part (one part per wave)
constexpr int WR_BUF_BYTES = 2 * WR_NRT * WR_PART_BYTES;   // one tile's halo (2 row tiles x 2 halves)
constexpr int WR_STAGE_BYTES = WR_NRT * 8 * 128 * 2;       // one tile's pooled outputs [row tile][window][128]
constexpr int WR_STAGE_OFF = WR_NBUF * WR_BUF_BYTES;
constexpr int WR_BIAS_OFF = WR_STAGE_OFF + 4 * WR_STAGE_BYTES;   // two staging areas per group
constexpr int WR_LDS = WR_BIAS_OFF + 2 * 128 * 4;    // 97 KiB: one block per CU
constexpr int WR_WPIECE = 128;                      // weight rows staged through LDS at a time
constexpr int WR_APD = 2;                           // A-operand prefetch distance (k-steps)
static_assert(WR_SLOTS % 64 == 0, "whole DMA instructions per part");
static_assert(4 * WR_NRT == WR_THREADS / 64, "one halo part per wave of a group");
static_assert(2 * WR_STAGE_BYTES == 16 * WR_THREADS, "one 16-byte output piece per thread of a group");
static_assert(WR_LDS <= 160 * 1024, "one block per CU");

enum { WR_MAX = 0, WR_AVG = 1 };

// slot swizzle of halo pixel (hr, hc) (see the header comment)
__device__ __forceinline__ int wr_swz(int hr, int hc) { return (hr & 1) | (((hc >> 2) & 1) << 1); }

struct WrArgs {
    const half_t* x;   // [NB, H, W, 64]
    const half_t* w;   // HWIO [3, 3, 64, K]
    const half_t* b;   // [K] or null
    const half_t* s;   // [K] per-channel scale (batch norm at inference) or null = 1
    half_t* y;         // [NB, H/2, W/2, K]
    uint8_t* argmax;   // max pool only, nullable: [NB, H/2, W/2, K]
    int NB, H, W, K;
    int P2, Q2;        // pooled output size
    int JB;            // row tiles per pooled row = ceil(Q2 / 8)
    int act;
    long nrt;          // row tiles in total = NB * P2 * JB
    int nblocks;
    FastDiv fjb, fp2;  // by JB, by P2
};

}  // namespace

template <int EPI, int ACT, bool AM>
__global__ __launch_bounds__(WR_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_conv_pool_wr(WrArgs a)
{
    constexpr int C = 64;
    constexpr int KPB = 128;                 // block columns (padded)
    constexpr int NST = 9 * C / 16;          // k-steps of 16
    extern __shared__ __align__(16) char smem[];
    typedef FC_LDS char lds_char;
    typedef FC_LDS half8 lds_half8;
    typedef Act<ACT> act;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, hh = lane >> 5;
    const int wq = wave & 3, wg = wave >> 2;   // column quarter, group (owner of the tiles j with j % 2 == wg)

    // ---- this block's row tiles (block indices renumbered so that each XCD
    // works on one contiguous stretch: neighbouring ranges share halo rows,
    // which then meet in that XCD's L2)
    const long lb = xcd_block(blockIdx.x, gridDim.x);
    const long rt_begin = lb * a.nrt / a.nblocks;
    const long rt_end = (lb + 1) * a.nrt / a.nblocks;

    // ---- weights -> operand-B fragments in registers, through LDS in pieces.
    // wf[st]: HWIO rows k = 16 st + 8 hh + [0, 8), column 32 wq + lr.
    half8 wf[NST];
    {
        WTile Wn;
        Wn.p = (lds_half*)smem;
        Wn.ld = wtile_ld(KPB);
        Wn.swz = wtile_swz(KPB);
        static_assert(WR_WPIECE * KPB * 2 <= WR_LDS, "a weight piece fits the LDS of the block");
        static_assert(WR_WPIECE % 16 == 0, "whole k-steps per piece");
#pragma unroll
        for (int pc = 0; pc < (9 * C + WR_WPIECE - 1) / WR_WPIECE; ++pc) {
            const int r0 = pc * WR_WPIECE;
            if (pc > 0) __syncthreads();   // the previous piece's fragments are read
            if constexpr (kPoison) {
                lds_poison(smem, WR_WPIECE * Wn.ld * 2, tid, WR_THREADS);
                __syncthreads();
            }
            stage_natural<8>(a.w + (long)r0 * a.K, 9 * C - r0, a.K, a.K, WR_WPIECE, KPB, Wn, tid, WR_THREADS);
            __syncthreads();
#pragma unroll
            for (int st = r0 / 16; st < NST && st < (r0 + WR_WPIECE) / 16; ++st)
                wf[st] = frag_tr_at(Wn.p + frag_lane_off(Wn, 32 * wq, lane) + (16 * st - r0 + 8 * hh) * Wn.ld,
                                    4 * Wn.ld);
        }
        __syncthreads();   // LDS is reused for the halos
    }
    if constexpr (kPoison) {
        lds_poison(smem, WR_LDS, tid, WR_THREADS);
        __syncthreads();
    }
    lds_char* const lds = (lds_char*)smem;
    lds_half* const stage = (lds_half*)(lds + WR_STAGE_OFF);
    // bias and scale per column (fp32) in LDS, read by the epilogue (held in
    // registers they would push the main loop past 256 registers)
    typedef FC_LDS float lds_float;
    lds_float* const bsl = (lds_float*)(lds + WR_BIAS_OFF);
    for (int i = tid; i < KPB; i += WR_THREADS) {
        bsl[i] = (a.b && i < a.K) ? (float)a.b[i] : 0.0f;
        bsl[KPB + i] = (a.s && i < a.K) ? (float)a.s[i] : 1.0f;
    }

    // ---- row tile -> (n, pooled row i, column block jb)
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
    // tiles of this block: tile j covers row tiles [tile_first(j), + tile_nrt(j)).
    // Even blocks walk their range forward, odd blocks backward: neighbouring
    // ranges (which meet in the same XCD's L2) then reach the two input rows
    // their halos share at the same time -- both at the start or both at the
    // end -- and the second fetch of those rows hits in L2.
    const int ntiles = (int)((rt_end - rt_begin + WR_NRT - 1) / WR_NRT);
    const bool backward = lb & 1;
    auto tile_first = [&](int j) -> long {
        return backward ? max(rt_begin, rt_end - (long)WR_NRT * (j + 1)) : rt_begin + (long)WR_NRT * j;
    };
    auto tile_nrt = [&](int j) -> int {
        return (int)(backward ? rt_end - (long)WR_NRT * j - tile_first(j)
                              : min((long)WR_NRT, rt_end - rt_begin - (long)WR_NRT * j));
    };

    // ---- halo DMA.  Wave w fetches part w of a tile: row tile u = w / 2,
    // channel half c = w % 2 (5 instructions).  Lane L of instruction j fills
    // slot 64 j + L of the part: pixel p = slot / 4 of the halo (row p / 20,
    // column p % 20), global 16-byte chunk (slot % 4) ^ wr_swz of channels
    // [32 c, 32 c + 32).  The offsets from the halo origin are the same for
    // every tile; pixels outside the image (the conv's zero padding) are
    // masked to an offset outside the buffer resource, which reads zero.
    // Returns whether this wave issued the requests (a tile of one row tile
    // has no part for waves 2 and 3).
    const int W = a.W;
    // per-lane offsets from the halo origin (OUTSIDE for the two padding
    // columns), formed once: lane L of instruction i fills slot 64 i + L
    unsigned dma_off[WR_DMA_PER_PART];
#pragma unroll
    for (int i = 0; i < WR_DMA_PER_PART; ++i) {
        const int slot = 64 * i + lane;
        const int p = slot >> 2, part = slot & 3;
        const int hr = p / WR_HROW, hcl = p - hr * WR_HROW;
        const int g = part ^ wr_swz(hr, hcl);
        dma_off[i] = hcl < 18 ? (unsigned)(hr * W + hcl) * (unsigned)(2 * C) + (unsigned)(64 * (wq & 1) + 16 * g)
                              : CS_OUTSIDE;
    }
    const long total_pix = (long)a.NB * a.H * W;
    auto dma_tile = [&](int j) -> bool {
        const int u = wq >> 1;
        if (j >= ntiles || u >= tile_nrt(j)) return false;
        lds_char* const dst = lds + (j % WR_NBUF) * WR_BUF_BYTES + wq * WR_PART_BYTES;
        if constexpr (kPoison) {   // released by the barrier of the tile before
            lds_poison(dst, WR_PART_BYTES, lane, 64);
            wave_lds_sync();
        }
        const RT t = decode(tile_first(j) + u);
        const int ih0 = 2 * t.i - 1, iw0 = 16 * t.jb - 1;   // halo origin in the image
        // the origin's pixel index (one row / column before the image at its
        // top / left border: those pixels are masked below and never read)
        const long base_pix = ((long)t.n * a.H + ih0) * W + iw0;
        const i32x4 rs = buf_rsrc((const void*)((long)a.x + base_pix * (2 * C)), (total_pix - base_pix) * (long)(2 * C));
        // pixels of the halo inside the image, as a bit mask over the 80
        // halo pixels (bit 20 hr + hc; scalar work): rows [rlo, rhi), columns
        // [clo, chi)
        const int rlo = ih0 < 0 ? -ih0 : 0, rhi = min(4, a.H - ih0);
        const int clo = iw0 < 0 ? -iw0 : 0, chi = min(18, W - iw0);
        const unsigned long long cm = ((1ull << chi) - 1) & ~((1ull << clo) - 1);
        unsigned long long m_lo = 0;   // pixels 0..63
        unsigned m_hi = 0;             // pixels 64..79
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (r >= rlo && r < rhi) {
                m_lo |= cm << (20 * r);
                if (r == 3) m_hi = (unsigned)(cm >> 4);
            }
        const int quad = lane_id_here() >> 2;   // pixel of the lane within the instruction's 16
#pragma unroll
        for (int i = 0; i < WR_DMA_PER_PART; ++i) {
            const unsigned win = i < 4 ? (unsigned)(m_lo >> (16 * i)) & 0xffffu : m_hi;   // pixels 16 i .. 16 i + 15
            const unsigned off = (win >> quad) & 1u ? dma_off[i] : CS_OUTSIDE;
            dma16(rs, off, (const lds_half*)(dst + i * 1024));
        }
        return true;
    };

    floatx16 acc[2];

    // One tile: 36 k-steps over all 576 k, NRT row tiles (the first k-step
    // starts the accumulators from zero); the operands of k-step st + WR_APD
    // are read before the MFMAs of st.  Operand A: lane l
    // reads, for MFMA row m = l % 32 (window w = m / 4, dy = (m / 2) % 2,
    // dx = m % 2) and k-group l / 32, tap (r, s), k-step q of the tap
    // (channels 16 q + 8 (l / 32) + [0, 8)), slot 2 (q % 2) + l / 32 of halo
    // pixel (row dy + r, column 2w + dx + s) in the part of channel half
    // q / 2.  The lane's address depends on the tap only through r % 2 and s
    // (the swizzle) plus a constant, so the 12 lane addresses are formed once
    // per tile and each read takes its constant as the instruction's offset.
    auto compute = [&](auto nrt_c, const lds_char* buf) {
        constexpr int NRT = decltype(nrt_c)::value;
        constexpr int R = WR_APD + 1;
        const int ln = lane_id_here();
        const int m = ln & 31, hi = ln >> 5;
        const int dy = (m >> 1) & 1, dx = m & 1, w4 = m >> 2;
        const lds_char* const lb = buf + (dy * WR_HROW + 2 * w4 + dx) * 64;
        const lds_char* ap[2][3][2];
#pragma unroll
        for (int rp = 0; rp < 2; ++rp)
#pragma unroll
            for (int sc = 0; sc < 3; ++sc)
#pragma unroll
                for (int qo = 0; qo < 2; ++qo)
                    ap[rp][sc][qo] = lb + (((hi | 2 * qo) ^ wr_swz(dy + rp, 2 * w4 + dx + sc)) << 4);
        half8 af[R][NRT];
        auto load_a = [&](int st, half8 (&dst)[NRT]) {
            const int tap = st >> 2, q = st & 3, r = tap / 3, sc = tap % 3;
            const lds_char* const p = ap[r & 1][sc][q & 1] + (q >> 1) * WR_PART_BYTES + (r * WR_HROW + sc) * 64;
#pragma unroll
            for (int u = 0; u < NRT; ++u) dst[u] = *reinterpret_cast<const lds_half8*>(p + 2 * u * WR_PART_BYTES);
        };
#pragma unroll
        for (int st = 0; st < WR_APD; ++st) load_a(st, af[st]);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            if (st + WR_APD < NST) load_a(st + WR_APD, af[(st + WR_APD) % R]);
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch issued here
#pragma unroll
            for (int u = 0; u < NRT; ++u) acc[u] = mfma32x32x16(af[st % R][u], wf[st], st == 0 ? zero16() : acc[u]);
        }
    };

    // ---- epilogue of tile j, window by window: registers 4g..4g+3 of row
    // tile u hold window 2g + hh of column 32 wave + lr; pool, scale/bias,
    // act, fp16 into the staging area [u][window][128] of this tile's parity
    auto epilogue_sc = [&](auto scaled_c, int j, int nloc) {
        constexpr bool scaled = decltype(scaled_c)::value;   // false: every scale is 1
        const int col = 32 * wq + lr;
        const float bk = bsl[col], sk = bsl[KPB + col];
        lds_half* const sg = stage + (2 * wg + ((j >> 1) & 1)) * (WR_STAGE_BYTES / 2);
        if constexpr (kPoison) {   // this wave's columns of the area, released two barriers ago
#pragma unroll
            for (int i = 0; i < WR_NRT * 8; ++i) sg[i * 128 + col] = (half_t)65504.0f;
        }
        // with a non-decreasing activation and no argmax, pool the accumulators first
        constexpr bool fast = EPI == WR_MAX && act::monotone && !AM;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (u >= nloc) break;
            const int ut = u;
            long win0 = 0;
            int nw = 0;
            if constexpr (AM) {
                const RT t = decode(tile_first(j) + ut);
                win0 = ((long)t.n * a.P2 + t.i) * a.Q2 + 8 * t.jb;
                nw = min(8, a.Q2 - 8 * t.jb);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                floatx4 c;
#pragma unroll
                for (int e = 0; e < 4; ++e) c[e] = acc[u][4 * g + e];
                half_t best;
                if (fast) {
                    // fp16(act(fma(acc, s, b))) is monotone in acc (non-decreasing
                    // for s >= 0, non-increasing for s < 0): pool the accumulators
                    // first, then one scale/bias/act/convert per window
                    float pick = __builtin_fmaxf(__builtin_fmaxf(c[0], c[1]), __builtin_fmaxf(c[2], c[3]));
                    if (scaled) {
                        const float lo = __builtin_fminf(__builtin_fminf(c[0], c[1]), __builtin_fminf(c[2], c[3]));
                        pick = sk >= 0.0f ? pick : lo;
                    }
                    best = (half_t)act::f(__builtin_fmaf(pick, sk, bk));
                } else if (EPI == WR_AVG) {
                    // mean of the four rounded values (fp32 sum, exact quarter), one rounding
                    float sum = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum += (float)(half_t)act::f(__builtin_fmaf(c[e], sk, bk));
                    best = (half_t)(sum * 0.25f);
                } else {
                    // first maximum of the rounded values in window order
                    best = (half_t)act::f(__builtin_fmaf(c[0], sk, bk));
                    int bi = 0;
#pragma unroll
                    for (int e = 1; e < 4; ++e) {
                        const half_t v = (half_t)act::f(__builtin_fmaf(c[e], sk, bk));
                        const bool gt = v > best;
                        best = gt ? v : best;
                        bi = gt ? e : bi;
                    }
                    const int wi = 2 * g + hh;
                    if (AM && wi < nw && col < a.K) a.argmax[(win0 + wi) * a.K + col] = (uint8_t)bi;
                }
                sg[(8 * ut + 2 * g + hh) * 128 + col] = best;
            }
        }
    };
    auto epilogue = [&](int j, int nloc) {
        if (a.s) epilogue_sc(IntC<1>{}, j, nloc);
        else epilogue_sc(IntC<0>{}, j, nloc);
    };
    // ---- stores of tile j's staged outputs: thread t takes 16 bytes
    // (columns 8 (t % 16) + [0, 8)) of pooled pixel t / 16 of the tile: row
    // tile u = wave / 2 (wave-uniform: its decode is scalar work), window
    // 4 (wave % 2) + lane / 16.  The lane's part of the address is formed once.
    const int st_wi = 4 * (wq & 1) + (lane >> 4), st_c8 = 8 * (lane & 15);
    const int st_off = st_wi * a.K + st_c8;
    auto store_tile = [&](int j) {
        const int u = wq >> 1;
        if (u >= tile_nrt(j)) return;
        const RT t = decode(tile_first(j) + u);
        const half_t* const yrow = a.y + (((long)t.n * a.P2 + t.i) * a.Q2 + 8 * t.jb) * a.K;
        const lds_half* const sg = stage + (2 * wg + ((j >> 1) & 1)) * (WR_STAGE_BYTES / 2);
        const half8 v = *reinterpret_cast<const lds_half8*>(sg + (4 * wq + (lane >> 4)) * 128 + st_c8);
        if (st_c8 < a.K && st_wi < a.Q2 - 8 * t.jb) st_out(reinterpret_cast<half8*>(const_cast<half_t*>(yrow) + st_off), v);
    };

    // ---- phase loop (ping-pong).  Tile j belongs to group j % 2.  In phase
    // k, group k % 2 runs tile k's MFMAs and nothing else, while the other
    // group, one wave per SIMD beside it, stores its tile k - 3 (staged two
    // phases ago), runs the epilogue of its tile k - 1, requests the halo of
    // its tile k + 3 and waits for the halo of its tile k + 1; one barrier
    // ends every phase.  So the matrix cores of a SIMD always have one wave
    // feeding them, and each wave's non-matrix work hides under the other's
    // MFMAs.  The ring holds four halos: tile k + 3 reuses tile k - 1's
    // buffer, freed by the barrier that ended phase k - 1; each group stages
    // its outputs in two areas used by alternate tiles.  Memory-counter waits
    // count this wave's halo requests only: the vector-memory counter retires
    // loads in issue order, but a store can complete before an older load, so
    // a wait that counted stores could pass with the halo still in flight;
    // stores issued after the awaited requests only make the wait stricter.
    if (wg == 0) {
        dma_tile(0);
        if (dma_tile(2)) vm_wait<WR_DMA_PER_PART>();   // tile 0's part has landed
        else vm_wait<0>();
    } else {
        dma_tile(1);
    }
    __syncthreads();   // tile 0's halo visible
    for (int k = 0; k <= ntiles + 2; ++k) {
        if (wg == (k & 1)) {
            const lds_char* const buf = lds + (k % WR_NBUF) * WR_BUF_BYTES;
            if (k < ntiles) {
                if (tile_nrt(k) == WR_NRT) compute(IntC<WR_NRT>{}, buf);
                else compute(IntC<1>{}, buf);
            }
        } else {
            if (k >= 3) store_tile(k - 3);
            if (k >= 1 && k - 1 < ntiles) epilogue(k - 1, tile_nrt(k - 1));
            if (dma_tile(k + 3)) vm_wait<WR_DMA_PER_PART>();   // tile k + 1's part has landed
            else vm_wait<0>();
        }
        __syncthreads();
    }
}

template <int EPI, int ACT, bool AM>
static hipError_t launch_wr(WrArgs a, hipStream_t st)
{
    static std::atomic<unsigned long long> lds_set{0};
    hipError_t e = allow_full_lds((const void*)k_conv_pool_wr<EPI, ACT, AM>, &lds_set);
    if (e != hipSuccess) return e;
    long nb = device_cu_count();   // one block per CU
    if (nb > a.nrt) nb = a.nrt;
    a.nblocks = (int)nb;
    hipLaunchKernelGGL((k_conv_pool_wr<EPI, ACT, AM>), dim3((unsigned)nb), dim3(WR_THREADS), (size_t)WR_LDS, st, a);
    return hipGetLastError();
}

template <int EPI, bool AM>
static hipError_t launch_wr_act(const WrArgs& a, hipStream_t st)
{
    switch (a.act) {
    case ACT_RELU: return launch_wr<EPI, ACT_RELU, AM>(a, st);
    case ACT_GELU_TANH: return launch_wr<EPI, ACT_GELU_TANH, AM>(a, st);
    case ACT_HARDSWISH: return launch_wr<EPI, ACT_HARDSWISH, AM>(a, st);
    default: return launch_wr<EPI, ACT_NONE, AM>(a, st);
    }
}

// The conv+pool shapes this kernel takes (3x3/s1/p1 checked by the caller):
// C = 64 input channels, 65..128 output channels, and halo offsets within a
// 4-row window of the input that fit 32 bits.
bool conv_pool_wr_fits(int W, int C, int K) { return C == 64 && K > 64 && K <= 128 && (long)W * C < (1L << 27); }

hipError_t run_conv_pool_wr(const half_t* x, const half_t* w, const half_t* scale, const half_t* b, int act, bool avg,
                            half_t* y, uint8_t* argmax, int NB, int H, int W, int K, hipStream_t st)
{
    WrArgs a;
    a.x = x; a.w = w; a.s = scale; a.b = b; a.y = y; a.argmax = avg ? nullptr : argmax;
    a.NB = NB; a.H = H; a.W = W; a.K = K; a.act = act;
    a.P2 = H / 2; a.Q2 = W / 2;
    a.JB = (a.Q2 + 7) / 8;
    a.nrt = (long)NB * a.P2 * a.JB;
    if (a.nrt == 0) return hipSuccess;
    a.nblocks = 1;
    a.fjb = FastDiv::make((unsigned)a.JB);
    a.fp2 = FastDiv::make((unsigned)a.P2);
    if (avg) return launch_wr_act<WR_AVG, false>(a, st);
    return a.argmax ? launch_wr_act<WR_MAX, true>(a, st) : launch_wr_act<WR_MAX, false>(a, st);
}

}  // namespace fc
