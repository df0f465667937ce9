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
//   * Block = 4 waves (256 threads), one block per CU, one wave per SIMD.
//     Wave (kh, wc) computes output columns [64 wc, 64 wc + 64) over input
//     channels [32 kh, 32 kh + 32) of every tap: the reduction is split in two
//     (split-K), so that each wave holds its share of the HWIO weights ONCE,
//     as ready MFMA operand-B fragments, in 144 registers (9 taps x 2 k-steps
//     x 2 column tiles x 4); the main loop reads no weights.  The weights
//     arrive through LDS in 128-row pieces (natural layout, read with the
//     transposing LDS load).
//   * GEMM rows are ordered window-major: a 32-row MFMA tile ("row tile") is
//     8 consecutive 2x2 pool windows of one pooled row (window 2g + h of the
//     tile lands in lane half h, accumulator registers 4g..4g+3), so the pool
//     is three max (or a sum) per output in registers.  A row tile needs a
//     4-row x 18-column input halo (stored with a row stride of 20 pixels).
//   * A block tile is up to 4 consecutive row tiles (128 pixels).  Its input
//     halo goes straight from global memory into LDS by the LDS-DMA load
//     (buffer_load_dwordx4 ... lds), into two buffers: the next tile's halo is
//     requested while the current tile's 18 k-steps run on the matrix cores.
//     Pixels outside the image, and the two padding columns, read zero from
//     outside the buffer resource -- the conv's zero padding needs no branch.
//   * Operand A is read from the halo with ds_read_b128 in MFMA layout.  A
//     pixel's 32 channels of one half are four 16-byte slots; slot s of the
//     pixel in halo row hr, column hc is stored at s ^ wr_swz(hr, hc) with
//     wr_swz = (hr & 1) | ((hc >> 2) & 1) << 1.  The LDS (64 banks) serves 16
//     lanes of a 16-byte read per clock: such a group reads pixels of two
//     halo rows and four columns spaced 2 apart, i.e. four pixels with each
//     value of hc % 4 (the 64-byte piece, with the 20-pixel row stride); the
//     swizzle gives those four distinct slots, so the 16 lanes touch 16
//     different 16-byte bank groups for every tap.  The DMA picks, for every
//     LDS slot, the global 16 bytes that belong there (quads of lanes still
//     read one 64-byte segment: the fast address path).
//   * Per k-step a wave issues NRT ds_read_b128 and 2 NRT MFMAs (32x32x16
//     f16, fp32 accumulate); the next k-step's operands are read while the
//     current MFMAs run.
//   * After a tile, the two waves of a column half exchange partial sums
//     through LDS: wave kh finishes row tiles 2kh and 2kh + 1 (adds the
//     partner's partial of those rows) and hands the other two over.
//   * Work split: the row tiles of the whole problem are divided into equal
//     contiguous ranges, one per block (49 row tiles each at the workload
//     above), processed four at a time; a range's last tile may hold 1..3
//     row tiles (those MFMAs are skipped, not masked).
//   * Epilogue per row tile: pool (or average), scale/bias, activation, fp16;
//     the pooled values go through a 1 KiB per-wave LDS staging area and leave
//     as 16-byte stores of whole 128-byte channel runs.
#include "fc_dma.h"
#include "fc_launch.h"

namespace fc {

namespace {

constexpr int WR_THREADS = 256;
constexpr int WR_NRT = 2;                           // row tiles per block tile
constexpr int WR_HROW = 20;                         // halo row stride (pixels): 18 used + 2 padding
constexpr int WR_HPIX = 4 * WR_HROW;                // pixels per row-tile halo
constexpr int WR_SLOTS = 4 * WR_HPIX;               // 16-byte slots per row-tile halo (32 channels)
constexpr int WR_PART_BYTES = 16 * WR_SLOTS;        // 5 KiB: one row tile, one channel half
constexpr int WR_DMA_PER_PART = WR_SLOTS / 64;      // 1 KiB DMA instructions per part
constexpr int WR_BUF_BYTES = 2 * WR_NRT * WR_PART_BYTES;   // one tile's halo (2 row tiles x 2 halves)
constexpr int WR_RED_BYTES = 8192;                  // per-wave partial sums handed over (1 row tile x 2 column tiles)
constexpr int WR_STAGE = 1024;                      // per-wave output staging
constexpr int WR_RED_OFF = 2 * WR_BUF_BYTES;
constexpr int WR_STAGE_OFF = WR_RED_OFF + 4 * WR_RED_BYTES;
constexpr int WR_BIAS_OFF = WR_STAGE_OFF + 4 * WR_STAGE;
constexpr int WR_LDS = WR_BIAS_OFF + 2 * 128 * 4;    // 77 KiB: two blocks per CU
constexpr int WR_WPIECE = 128;                      // weight rows staged through LDS at a time
static_assert(WR_SLOTS % 64 == 0, "whole DMA instructions per part");
static_assert(2 * WR_LDS <= 160 * 1024, "two blocks per CU");

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
    extern __shared__ __align__(16) char smem[];
    typedef FC_LDS char lds_char;
    typedef FC_LDS half8 lds_half8;
    typedef FC_LDS floatx4 lds_floatx4;
    typedef Act<ACT> act;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wc = wave & 1, kh = wave >> 1;
    const int lr = lane & 31, hh = lane >> 5;

    // ---- this block's row tiles (block indices renumbered so that each XCD
    // works on one contiguous stretch: neighbouring ranges share halo rows,
    // which then meet in that XCD's L2)
    const long lb = xcd_block(blockIdx.x, gridDim.x);
    const long rt_begin = lb * a.nrt / a.nblocks;
    const long rt_end = (lb + 1) * a.nrt / a.nblocks;

    // ---- weights -> operand-B fragments in registers, through LDS in pieces.
    // wf[st][ct], st = 2 tap + q: HWIO rows k = 64 tap + 32 kh + 16 q + 8 hh +
    // [0, 8), column 64 wc + 32 ct + lr.
    half8 wf[18][2];
    {
        WTile Wn;
        Wn.p = (lds_half*)smem;
        Wn.ld = wtile_ld(KPB);
        Wn.swz = wtile_swz(KPB);
        static_assert(WR_WPIECE * KPB * 2 <= WR_LDS, "a weight piece fits the LDS of the block");
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
            for (int st = 0; st < 18; ++st) {
                const int krow0 = 64 * (st >> 1) + 16 * (st & 1);   // + 32 kh (runtime, wave-uniform)
                if (krow0 + 32 < r0 || krow0 >= r0 + WR_WPIECE) continue;
                const int kr = krow0 + 32 * kh - r0;
                if (kr < 0 || kr >= WR_WPIECE) continue;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    wf[st][ct] = frag_tr_at(Wn.p + frag_lane_off(Wn, 64 * wc + 32 * ct, lane) + (kr + 8 * hh) * Wn.ld,
                                            4 * Wn.ld);
            }
        }
        __syncthreads();   // LDS is reused for the halos
    }
    if constexpr (kPoison) {
        lds_poison(smem, WR_LDS, tid, WR_THREADS);
        __syncthreads();
    }
    lds_char* const lds = (lds_char*)smem;
    lds_half* const ost = (lds_half*)(lds + WR_STAGE_OFF + wave * WR_STAGE);
    // bias and scale per column (fp32) in LDS, read by the epilogue (held in
    // registers they would push the main loop past 256 registers)
    typedef FC_LDS float lds_float;
    lds_float* const bsl = (lds_float*)(lds + WR_BIAS_OFF);
    for (int i = tid; i < KPB; i += WR_THREADS) {
        bsl[i] = (a.b && i < a.K) ? (float)a.b[i] : 0.0f;
        bsl[KPB + i] = (a.s && i < a.K) ? (float)a.s[i] : 1.0f;
    }
    __syncthreads();

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

    // ---- halo DMA.  Wave w fetches part w of a tile: row tile u = w / 2,
    // channel half c = w % 2 (5 instructions).  Lane L of instruction j fills
    // slot 64 j + L of the part: pixel p = slot / 4 of the halo (row p / 20,
    // column p % 20), global 16-byte chunk (slot % 4) ^ ((p >> 1) & 3) of
    // channels [32 c, 32 c + 32).  Halos inside the image use the precomputed
    // per-lane offsets rel[j] (OUTSIDE for the two padding columns); halos
    // that cross the border take per-lane checks.
    const int W = a.W;
    auto dma_tile = [&](long rt, int nrt, lds_char* buf) {
        const int u = kh;   // row tile of this wave's part; channel half wc
        if (u >= nrt) return;
        const RT t = decode(rt + u);
        const int ih0 = 2 * t.i - 1, iw0 = 16 * t.jb - 1;   // halo origin in the image
        const bool inside = ih0 >= 0 && ih0 + 4 <= a.H && iw0 >= 0 && iw0 + 18 <= W;
        const int ib = inside ? ih0 : (ih0 < 0 ? 0 : ih0);
        const long base_pix = ((long)t.n * a.H + ib) * W + (inside ? iw0 : 0);
        const long total_pix = (long)a.NB * a.H * W;
        const i32x4 rs = buf_rsrc(a.x + base_pix * C, (total_pix - base_pix) * (long)(2 * C));
        lds_char* const dst = buf + wave * WR_PART_BYTES;
        // lane-derived values come from a lane id computed here: derived from
        // `lane` they are hoisted out of the tile loop and held across it
        const int ln = lane_id_here();
        if (inside) {
#pragma unroll
            for (int j = 0; j < WR_DMA_PER_PART; ++j) {
                const int slot = 64 * j + ln;
                const int p = slot >> 2, part = slot & 3;
                const int hr = p / WR_HROW, hcl = p - hr * WR_HROW;
                const int g = part ^ wr_swz(hr, hcl);
                const unsigned off =
                    hcl < 18 ? (unsigned)(hr * W + hcl) * (unsigned)(2 * C) + (unsigned)(64 * wc + 16 * g) : CS_OUTSIDE;
                dma16(rs, off, (const lds_half*)(dst + j * 1024));
            }
        } else {
#pragma unroll
            for (int j = 0; j < WR_DMA_PER_PART; ++j) {
                const int slot = 64 * j + ln;
                const int p = slot >> 2, part = slot & 3;
                const int hr = p / WR_HROW, hcl = p - hr * WR_HROW;
                const int ih = ih0 + hr, iw = iw0 + hcl;
                const bool ok = hcl < 18 && ih >= 0 && ih < a.H && iw >= 0 && iw < W;
                const int g = part ^ wr_swz(hr, hcl);
                const unsigned off =
                    ok ? (unsigned)((ih - ib) * W + iw) * (unsigned)(2 * C) + (unsigned)(64 * wc + 16 * g) : CS_OUTSIDE;
                dma16(rs, off, (const lds_half*)(dst + j * 1024));
            }
        }
    };

    // ---- A-operand offset in a part: lane l reads, for MFMA row m = l % 32
    // (window w = m / 4, dy = (m / 2) % 2, dx = m % 2) and k-group l / 32, tap
    // (r, s), k-step half q, slot 2q + l / 32 of halo pixel (row dy + r,
    // column 2w + dx + s).
    auto a_off = [&](int tap, int q) -> int {
        const int ln = lane_id_here();   // recomputed per k-step, not held across the loop
        const int m = ln & 31;
        const int r = tap / 3, s = tap % 3;
        const int hr = ((m >> 1) & 1) + r, hc = 2 * (m >> 2) + (m & 1) + s;
        return (hr * WR_HROW + hc) * 64 + (((2 * q + (ln >> 5)) ^ wr_swz(hr, hc)) << 4);
    };

    floatx16 acc[WR_NRT][2];
#pragma unroll
    for (int u = 0; u < WR_NRT; ++u)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[u][ct] = zero16();

    // One tile: 9 taps x 2 k-steps over this wave's channel half, NRT row
    // tiles; the operands of k-step st + 1 are read before the MFMAs of st.
    auto compute = [&](auto nrt_c, const lds_char* buf) {
        constexpr int NRT = decltype(nrt_c)::value;
        const lds_char* hb = buf + kh * WR_PART_BYTES;
        half8 af[2][NRT];
        auto load_a = [&](int st, half8 (&dst)[NRT]) {
            const int off = a_off(st >> 1, st & 1);
#pragma unroll
            for (int u = 0; u < NRT; ++u)
                dst[u] = *reinterpret_cast<const lds_half8*>(hb + 2 * u * WR_PART_BYTES + off);
        };
        load_a(0, af[0]);
#pragma unroll
        for (int st = 0; st < 18; ++st) {   // st = 2 tap + q
            if (st + 1 < 18) load_a(st + 1, af[(st + 1) & 1]);
#pragma unroll
            for (int u = 0; u < NRT; ++u)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) acc[u][ct] = mfma32x32x16(af[st & 1][u], wf[st][ct], acc[u][ct]);
        }
    };

    // ---- partial sums: wave (kh, wc) hands row tile 1 - kh to wave
    // (1 - kh, wc) through its area [ct][r / 4][lane] (float4).  (Row tiles
    // are named at compile time: a runtime index would move the accumulator
    // array to scratch memory.)
    lds_floatx4* const red_out = (lds_floatx4*)(lds + WR_RED_OFF + wave * WR_RED_BYTES);
    const lds_floatx4* const red_in = (const lds_floatx4*)(lds + WR_RED_OFF + (wave ^ 2) * WR_RED_BYTES);
    auto hand_over = [&](const floatx16 (&ac)[2]) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                floatx4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = ac[ct][4 * r4 + e];
                red_out[(ct * 4 + r4) * 64 + lane] = v;
            }
    };

    // ---- epilogue of one row tile, window by window: registers 4g..4g+3 of
    // column tile ct hold window 2g + hh; the partner's four values of that
    // window are added just before the window is pooled; then scale/bias,
    // act, fp16, staged and stored
    auto epilogue = [&](long rt, const floatx16 (&ac)[2]) {
        const RT t = decode(rt);
        const int K = a.K;
        const long win0 = ((long)t.n * a.P2 + t.i) * a.Q2 + 8 * t.jb;   // y index of the tile's first window
        const int nw = min(8, a.Q2 - 8 * t.jb);                          // valid windows
        // with a non-decreasing activation and no argmax, pool the accumulators first
        constexpr bool fast = EPI == WR_MAX && act::monotone && !AM;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int col = 64 * wc + 32 * ct + lr;
            const float bk = bsl[col], sk = bsl[KPB + col];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                floatx4 c = red_in[(ct * 4 + g) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) c[e] += ac[ct][4 * g + e];
                half_t best;
                if (fast) {
                    // fp16(act(fma(acc, s, b))) is monotone in acc (non-decreasing
                    // for s >= 0, non-increasing for s < 0): pool the accumulators
                    // first, then one scale/bias/act/convert per window
                    const float hi = __builtin_fmaxf(__builtin_fmaxf(c[0], c[1]), __builtin_fmaxf(c[2], c[3]));
                    const float lo = __builtin_fminf(__builtin_fminf(c[0], c[1]), __builtin_fminf(c[2], c[3]));
                    best = (half_t)act::f(__builtin_fmaf(sk >= 0.0f ? hi : lo, sk, bk));
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
                    if (AM && wi < nw && col < K) a.argmax[(win0 + wi) * K + col] = (uint8_t)bi;
                }
                // staged as [8 windows][64 columns]
                ost[(2 * g + hh) * 64 + 32 * ct + lr] = best;
            }
        }
        wave_lds_sync();
        // 16 bytes per lane: window lane / 8, columns 64 wc + 8 (lane % 8) + [0, 8)
        const int sw = lane >> 3, sc = lane & 7;
        const half8 v = *reinterpret_cast<const lds_half8*>(ost + sw * 64 + 8 * sc);
        const int col = 64 * wc + 8 * sc;
        if (sw < nw && col < K) st_out(reinterpret_cast<half8*>(a.y + (win0 + sw) * K + col), v);
        wave_lds_sync();   // the next row tile overwrites the staging area
    };
    // the partial-sum exchange and the epilogue of one tile (wave kh finishes
    // row tile kh)
    auto finish = [&](long rt, int nrt) {
        __syncthreads();   // every wave has read the previous tile's partial sums
        if (kh == 0) {
            if (nrt > 1) hand_over(acc[1]);
        } else {
            hand_over(acc[0]);
        }
        vm_wait<0>();      // the next tile's halo has landed (and this wave's stores are done)
        __syncthreads();   // ... for all waves; the partial sums are visible
        if (kh == 0) epilogue(rt, acc[0]);
        else if (nrt > 1) epilogue(rt + 1, acc[1]);
#pragma unroll
        for (int u = 0; u < WR_NRT; ++u)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc[u][ct] = zero16();
    };

    // ---- main loop over this block's full tiles (2 row tiles); the halo
    // buffers alternate between tiles, and each tile requests the next
    // tile's halo before its MFMAs.  A last tile of 1 row tile follows.
    long rt = rt_begin;
    int sb = 0;   // buffer of the current tile
    if (rt < rt_end) dma_tile(rt, (int)min((long)WR_NRT, rt_end - rt), lds);
    vm_wait<0>();
    __syncthreads();
    while (rt + WR_NRT <= rt_end) {
        const long rtn = rt + WR_NRT;
        if constexpr (kPoison) {   // the previous tile's halo buffer, released by its barriers
            lds_poison(lds + (sb ^ 1) * WR_BUF_BYTES, WR_BUF_BYTES, tid, WR_THREADS);
            __syncthreads();
        }
        if (rtn < rt_end) dma_tile(rtn, (int)min((long)WR_NRT, rt_end - rtn), lds + (sb ^ 1) * WR_BUF_BYTES);
        compute(IntC<WR_NRT>{}, lds + sb * WR_BUF_BYTES);
        finish(rt, WR_NRT);
        sb ^= 1;
        rt = rtn;
    }
    if (rt < rt_end) {
        compute(IntC<1>{}, lds + sb * WR_BUF_BYTES);
        finish(rt, 1);
    }
}

template <int EPI, int ACT, bool AM>
static hipError_t launch_wr(WrArgs a, hipStream_t st)
{
    static std::atomic<unsigned long long> lds_set{0};
    hipError_t e = allow_full_lds((const void*)k_conv_pool_wr<EPI, ACT, AM>, &lds_set);
    if (e != hipSuccess) return e;
    long nb = 2L * device_cu_count();   // two blocks per CU
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
