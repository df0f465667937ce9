// conv_chain.hip -- implicit-GEMM NHWC convolution chains.
//
//   conv3x3 -> bias -> act -> (fp16, registers) -> conv1x1 -> bias :
//       the register-resident chain kernel (chain_rf.h) with an implicit-GEMM
//       row loader (Conv3x3Rows).
//   conv3x3 -> bias -> ReLU -> 2x2/2 max pool (Welder's Conv+ReLU+MaxPool
//   tile graph):  k_conv_w<NTK, EPI_POOL>; the conv output tile never leaves
//   the VGPRs: the pool is a partial reduction of 4 accumulator registers.
//   the same with a 2x2/2 average instead of the maximum: k_conv_w<NTK, EPI_AVG>.
//   conv3x3 -> bias -> act, stored (unfused baseline): k_conv_w<NTK, EPI_STORE>.
//   2x2/2 max or average pool of a stored tensor (unfused baselines): k_pool2x2.
//   channel zero-padding (input preparation): k_pad_mid.
//
// Implicit GEMM (interview page, "Conv optimisation" item 2): the GEMM view is
// M = N*P*Q output pixels, K = R*S*C with index k = (r*S + s)*C + c (c
// fastest, matching HWIO weights read as a row-major [(R*S*C) x K] matrix),
// N = output channels; the unfolded input row of a pixel is never built, each
// 16-byte operand load computes its input address (and zero padding) on the
// fly.  One block owns all output channels (the residence rule of BOLT's
// persistent conv fusion: ThreadBlock_N = conv output channels).
#include "chain_rf.h"
#include "fc_launch.h"

namespace fc {

// ------------------------------------------------------------- row loader
// 3x3, stride 1, pad 1 NHWC conv pixels as GEMM rows (P = H, Q = W).  A lane
// reads 8 consecutive k at a time (one MFMA k-group): 8 consecutive channels
// of one (r, s) position, since C % 8 == 0 (the pages' alignment of 8 fp16 =
// 128 bits).
struct Conv3x3Rows {
    static constexpr bool kRaw = false;   // loads land in operand layout
    const half_t* x;
    int H, W, C;
    long M;   // N*H*W (< 2^31)
    FastDiv fhw, fw, fc8;    // by H*W, by W, by C/8
    // A GEMM row = one output pixel: its centre in x and a 9-bit mask whose
    // bit 3r+s says that tap (r, s) lies inside the image (0 for a row past M).
    struct Row {
        const half_t* pix;
        unsigned mask;
    };
    void set_divisors()
    {
        fhw = FastDiv::make((unsigned)H * (unsigned)W);
        fw = FastDiv::make((unsigned)W);
        fc8 = FastDiv::make((unsigned)C / 8);
    }
    __device__ __forceinline__ Row make(int n, int p, int q, bool ok) const
    {
        Row r;
        r.pix = x + (((long)n * H + p) * W + q) * C;
        // rows r with 0 <= p + r - 1 < H, columns s likewise
        const unsigned rm = 2u | (p > 0 ? 1u : 0u) | (p < H - 1 ? 4u : 0u);
        const unsigned sm = 2u | (q > 0 ? 1u : 0u) | (q < W - 1 ? 4u : 0u);
        const unsigned m = ((rm & 1u) ? sm : 0u) | ((rm & 2u) ? sm << 3 : 0u) | ((rm & 4u) ? sm << 6 : 0u);
        r.mask = ok ? m : 0u;
        return r;
    }
    __device__ __forceinline__ Row row(long m) const
    {
        const bool ok = m < M;
        const unsigned mm = ok ? (unsigned)m : 0u;
        const unsigned n = fhw.div(mm);
        const unsigned rem = mm - n * fhw.d;
        const unsigned p = fw.div(rem);
        return make((int)n, (int)p, (int)(rem - p * fw.d), ok);
    }
    // Chunk c, lane half hh, vector q: k = 64c + 16q + 8hh + [0, 8), the
    // MFMA's own k order, so that the two lanes holding one pixel's k-step
    // read contiguous bytes when their k-groups share a tap.  k-group
    // kg = k / 8 lies in tap rs = kg / (C/8) at channel 8 (kg % (C/8)); taps
    // past the ninth (k in the zero padding of the last chunk) read zero (bit
    // rs of the 9-bit tap mask is 0).  KCH = 9 chunks (9C rounded up to 64)
    // means C = 64, known at compile time: then rs = c and the channel is
    // 16q + 8hh.
    template <int KCH>
    __device__ __forceinline__ void load(const Row& r, int c, int hh, half8 out[4]) const
    {
        // An opaque copy of W keeps the compiler from hoisting every chunk's
        // tap offset out of the tile loop (nine values held across the whole
        // loop would spill); recomputing one is a couple of scalar operations.
        int w = W;
        asm volatile("" : "+s"(w));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            unsigned rs;
            int coff, cc;
            if (KCH == 9) {
                rs = (unsigned)c;
                coff = 16 * q + 8 * hh;
                cc = 64;
            } else {
                const unsigned kg = 8u * c + 2u * q + (unsigned)hh;   // k / 8
                rs = fc8.div(kg);
                coff = (int)(kg - rs * fc8.d) * 8;
                cc = C;
            }
            const int rr = (int)((rs * 11u) >> 5);       // rs / 3 for rs < 32
            const int ss = (int)rs - 3 * rr;
            const bool ok = (r.mask >> rs) & 1u;
            const int delta = ((rr - 1) * w + (ss - 1)) * cc + coff;   // |delta| < (W + 2) C < 2^31
            out[q] = ld16_if(r.pix + (ok ? delta : 0), ok);
        }
    }
};

// ------------------------------------------- weights-resident conv kernel
enum { EPI_STORE = 0, EPI_POOL = 1, EPI_AVG = 2 };
// the pooling epilogues enumerate GEMM rows window-major
__host__ __device__ constexpr bool epi_pools(int e) { return e != EPI_STORE; }

// With the chunk count known at compile time: CONVW_WPS waves per SIMD
// (4 * CONVW_WPS per block, 512 / CONVW_WPS registers each) and a register
// ring CONVW_RING pixel chunks deep.  Otherwise two waves per SIMD and a
// two-deep ring.
#ifndef CONVW_WPS
#define CONVW_WPS 2
#endif
#ifndef CONVW_RING
#define CONVW_RING 2
#endif
#ifndef CONVW_WPIPE   // W fragments read one k-step ahead (1) or just in time (0)
#define CONVW_WPIPE 0
#endif
__host__ __device__ constexpr int convw_wps(int KCH) { return KCH > 0 ? CONVW_WPS : 2; }
__host__ __device__ constexpr int convw_threads(int KCH) { return 256 * convw_wps(KCH); }
__host__ __device__ constexpr int convw_ring(int KCH) { return KCH > 0 ? CONVW_RING : 2; }

struct ConvWArgs {
    const half_t* x;   // [NB, H, W, C]
    const half_t* w;   // HWIO [3, 3, C, K]
    const half_t* b;   // [K] or null
    const half_t* s;   // [K] per-channel scale applied before b (batch-norm at inference), or null = 1
    half_t* y;         // STORE: [NB, H, W, K];  POOL: [NB, H/2, W/2, K]
    uint8_t* argmax;   // POOL only, nullable: [NB, H/2, W/2, K]
    int NB, H, W, C, K;
    int Kr;            // 9*C
    int Kp;            // 9*C rounded up to 64
    int act;
    long ntiles;       // 64-row tiles
    long tiles_per_block;
    int wpb;           // waves per block that own tiles (1..NWAVES; 0 = all); the others only stage weights
    // row decoding: STORE: pixel = (n, p, q) with fa = P*Q, fb = Q;
    // POOL: window = (n, i, j) with fa = (P/2)*(Q/2), fb = Q/2; fc8 = C/8
    FastDiv fa, fb, fc8;
};

// LDS: weights [Kp][KP] (natural, swizzled or padded), biases, scales, the
// tile counter, then a 1 KiB output staging area per wave.
constexpr int CW_OSTAGE = 1024;
__host__ __device__ inline size_t convw_lds_bytes(int KP, int Kp)
{
    return (size_t)Kp * wtile_ld(KP) * 2 + (size_t)KP * 8 + 16 + (size_t)8 * CW_OSTAGE;
}

// One wave = 64 GEMM rows (two 32-row MFMA tiles) x all K output channels.
// Rows: STORE enumerates pixels (n, p, q) linearly; POOL enumerates 2x2
// windows (n, i, j) and, inside a window, (dy, dx) in the order
// (0,0),(0,1),(1,0),(1,1): GEMM row 4*w + 2*dy + dx.  The MFMA result puts
// rows 4g'..4g'+3 of a 32x32 tile into one lane's registers 4g..4g+3, i.e. a
// whole window, so the pool is three max operations in registers.
// Non-transposed MFMA: operand A = pixel rows (16-byte loads from x), operand
// B = W fragments read from the natural (HWIO = [(r,s,c)][k]) LDS copy of the
// weights with the transposing LDS load.
// KCH: compile-time number of 64-wide k chunks (0 = runtime loop), see the
// register-resident chain kernel.
template <int NTK, int EPI, int KCH>
__global__ __launch_bounds__(convw_threads(KCH)) __attribute__((amdgpu_waves_per_eu(1, convw_wps(KCH))))
void k_conv_w(ConvWArgs a)
{
    constexpr int KP = 32 * NTK;
    constexpr int NTHR = convw_threads(KCH);
    constexpr int NWAVES = NTHR / 64;
    extern __shared__ __align__(16) char smem[];
    typedef FC_LDS float lds_float;
    WTile Wn;   // natural layout [Kp][KP] (rows = (r, s, c))
    Wn.p = (lds_half*)smem;
    Wn.ld = wtile_ld(KP);
    Wn.swz = wtile_swz(KP);
    lds_float* bs = (lds_float*)(Wn.p + a.Kp * Wn.ld);
    lds_float* ss = bs + KP;
    FC_LDS int* next_tile = (FC_LDS int*)(ss + KP);
    static_assert(convw_threads(KCH) <= 512, "eight staging areas");

    const int tid = threadIdx.x;
    // wave index in a scalar register (it is wave-uniform; derived per lane it
    // would hold a vector register, and the staging-area address built from it
    // across the whole kernel)
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, hh = lane >> 5;
    const long t_begin = (long)xcd_block(blockIdx.x, gridDim.x) * a.tiles_per_block;
    const long t_end = min(t_begin + a.tiles_per_block, a.ntiles);
    const int nch = KCH ? KCH : a.Kp >> 6;
    const long nrows = epi_pools(EPI) ? (long)a.NB * (a.H >> 1) * (a.W >> 1) * 4 : (long)a.NB * a.H * a.W;

    Conv3x3Rows ld;
    ld.x = a.x; ld.H = a.H; ld.W = a.W; ld.C = a.C; ld.M = (long)a.NB * a.H * a.W;
    ld.fc8 = a.fc8;

    // GEMM row -> conv output pixel
    auto make_row = [&](long gr) -> Conv3x3Rows::Row {
        const bool ok = gr < nrows;
        const unsigned g = ok ? (unsigned)gr : 0u;
        unsigned n, p, q;
        if (epi_pools(EPI)) {
            const unsigned win = g >> 2, e = g & 3u;
            n = a.fa.div(win);
            const unsigned rem = win - n * a.fa.d;
            const unsigned i = a.fb.div(rem);
            p = 2 * i + (e >> 1);
            q = 2 * (rem - i * a.fb.d) + (e & 1u);
        } else {
            n = a.fa.div(g);
            const unsigned rem = g - n * a.fa.d;
            p = a.fb.div(rem);
            q = rem - p * a.fb.d;
        }
        return ld.make((int)n, (int)p, (int)q, ok);
    };
    auto claim = [&]() -> long {
        int nt = 0;
        if (lane == 0) nt = __hip_atomic_fetch_add(next_tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return __builtin_amdgcn_readfirstlane(nt);
    };

    // Ring depth: chunk g of a wave's chunk sequence lives in register set
    // g % R, named at compile time (the chunk loops are fully unrolled, and a
    // copy of a loaded register would force a wait on the loads in flight).
    constexpr int R = convw_ring(KCH);
    constexpr int PD = R - 1;   // chunks in flight ahead of the one in use
    static_assert(KCH == 0 || KCH == 9, "the compile-time path is the C = 64 one");
    static_assert(KCH == 0 || (2 * KCH) % R == 0, "two tiles of chunks must fill whole ring turns");
    half8 ring[R][2][4];

    // ---- quad-coalesced rows (compile-time path, C = 64) ----
    // Lane 4i + m loads, for tile row 4i + j (j = 0..3), the 16-byte segment
    // m of each 64-byte half h of the pixel's 128 bytes in chunk c (tap c):
    // ring[.][h][j]; every quad of lanes reads 64 contiguous bytes.  The
    // in-quad transpose and the half swap turn these into the MFMA operands
    // of row tiles u = 0, 1 (tile rows 32u + lane%32), the same layout the
    // runtime-chunk path loads directly.  POOL: tile row 4i + j is element
    // j = 2dy + dx of the tile's window i; STORE: pixel tile*64 + 4i + j.
    const int qm = lane & 3;
    // A lane's four tile rows: the pixel of row j is base + off(j) with
    // off(j) = (dy W + dx) C (POOL, the window's 2x2 pixels) or j C (STORE,
    // consecutive pixels are C apart); bits 6j..6j+5 hold the tap masks of
    // row j: rows r (bits 6j + r) and columns s (bits 6j + 3 + s) of the 3x3
    // window that lie inside the image (all 0 for a row past the end).
    struct QRows {
        const half_t* base;
        unsigned bits;
    };
    auto tap_bits = [&](int p, int q, bool ok) -> unsigned {
        const unsigned rm = 2u | (p > 0 ? 1u : 0u) | (p < a.H - 1 ? 4u : 0u);
        const unsigned sm = 2u | (q > 0 ? 1u : 0u) | (q < a.W - 1 ? 4u : 0u);
        return ok ? rm | (sm << 3) : 0u;
    };
    auto make_qrows = [&](long tl) -> QRows {
        QRows r;
        r.bits = 0;
        const int qi = lane_id_here() >> 2;   // recomputed per tile, not held across the main loop
        if (epi_pools(EPI)) {
            const long wi = tl * 16 + qi;
            const bool ok = wi < (nrows >> 2);
            const unsigned g = ok ? (unsigned)wi : 0u;
            const unsigned n = a.fa.div(g);
            const unsigned rem = g - n * a.fa.d;
            const unsigned i = a.fb.div(rem);
            const unsigned j = rem - i * a.fb.d;
            r.base = a.x + (((long)n * a.H + 2 * i) * a.W + 2 * j) * 64;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                r.bits |= tap_bits((int)(2 * i) + (jj >> 1), (int)(2 * j) + (jj & 1), ok) << (6 * jj);
        } else {
            const long g0 = tl * 64 + 4 * qi;
            r.base = a.x + min(g0, nrows - 1) * 64;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const long gr = g0 + jj;
                const bool ok = gr < nrows;
                const unsigned g = ok ? (unsigned)gr : 0u;
                const unsigned n = a.fa.div(g);
                const unsigned rem = g - n * a.fa.d;
                const unsigned p = a.fb.div(rem);
                r.bits |= tap_bits((int)p, (int)(rem - p * a.fb.d), ok) << (6 * jj);
            }
        }
        return r;
    };
    auto load_q = [&](const QRows& r, int c, half8 (&A)[2][4]) {
        // An opaque copy of W keeps every chunk's tap offset from being
        // hoisted out of the tile loop (held across the loop, they spill).
        int w = a.W;
        asm volatile("" : "+s"(w));
        const int rr = c / 3, ss = c % 3;
        const int delta = ((rr - 1) * w + (ss - 1)) * 64 + 8 * qm;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const bool ok = (r.bits >> (6 * jj + rr)) & (r.bits >> (6 * jj + 3 + ss)) & 1u;
            const int off = epi_pools(EPI) ? ((jj >> 1) * w + (jj & 1)) * 64 : jj * 64;
            const half_t* p = r.base + (delta + off);
#pragma unroll
            for (int h = 0; h < 2; ++h) A[h][jj] = ld16_if(p + 32 * h, ok);
        }
    };

    const int wpb = a.wpb > 0 ? a.wpb : NWAVES;
    long tile = wave < wpb ? t_begin + wave : t_end;
    Conv3x3Rows::Row rows[2];
    QRows qrows;
    if (tile < t_end) {
        if constexpr (KCH > 0) {
            qrows = make_qrows(tile);
#pragma unroll
            for (int p = 0; p < PD; ++p) load_q(qrows, p, ring[p]);
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                rows[u] = make_row(tile * 64 + 32 * u + lr);
                ld.template load<KCH>(rows[u], 0, hh, ring[0][u]);
            }
        }
    }

    if constexpr (kPoison) {
        lds_poison(smem, (int)convw_lds_bytes(KP, a.Kp), tid, NTHR);
        __syncthreads();
    }
    stage_natural<8>(a.w, a.Kr, a.K, a.K, a.Kp, KP, Wn, tid, NTHR);
    for (int i = tid; i < KP; i += NTHR) {
        bs[i] = (a.b && i < a.K) ? (float)a.b[i] : 0.0f;
        ss[i] = (a.s && i < a.K) ? (float)a.s[i] : 1.0f;
    }
    if (tid == 0) *next_tile = (int)(t_begin + wpb);
    __syncthreads();

    // Per-lane parts of the W fragment addresses: column k_out = 32t + lane%32,
    // rows 64c + 16q + 8hh + [0,8) (the k the lane's operand holds at step q).
    const lds_half* wlane[NTK];
#pragma unroll
    for (int t = 0; t < NTK; ++t) wlane[t] = Wn.p + frag_lane_off(Wn, 32 * t, lane) + 8 * hh * Wn.ld;

    // Epilogue.  Lane holds output channel k = 32t + lr; register r = 4g + e
    // of tile (u, t) is tile row 32u + 8g + 4hh + e, so registers 4g..4g+3
    // hold the four elements of pool window 8u + 2g + hh.  Results go through
    // this wave's 1 KiB LDS staging area as [16 rows][32 channels] fp16 and
    // leave as 16-byte stores, four lanes per 64 contiguous bytes (2-byte
    // stores from every lane would cost the address unit a clock per lane).
    lds_half* const ost = (lds_half*)((FC_LDS char*)(next_tile + 4) + wave * CW_OSTAGE);
    typedef FC_LDS half8 lds_half8;
    auto epilogue = [&](long tl, const floatx16 (&acc)[2][NTK]) {
        const long row0 = tl * 64;
        int K = a.K;
        asm volatile("" : "+s"(K));   // keeps per-store offsets from being hoisted out of the tile loop
        // Every per-lane value of the epilogue derives from a lane id computed
        // here: derived from `lane`, the compiler hoists them out of the tile
        // loop, holds them across the main loop (where all registers are
        // taken) and spills them, and each tile's reload then waits for every
        // prefetch in flight.
        const int ln = lane_id_here();
        const int lr = ln & 31, hh = ln >> 5;
        const int rr = ln >> 2, grp = ln & 3;   // read-back: staged row, 8-channel group
        // per-lane bases; every (u, g, e, t) adds a constant (LDS instruction offsets)
        lds_half* const ow = ost + hh * 32 + lr;
        const lds_float* const bsl = bs + lr;
        const lds_float* const ssl = ss + lr;
        const lds_half8* const orb = reinterpret_cast<const lds_half8*>(ost + rr * 32 + 8 * grp);
        act_dispatch(a.act, [&](auto act) {
            if (epi_pools(EPI)) {
                // windows are enumerated like y's pixels
                const long win0 = row0 >> 2;
                half_t* yb = a.y + win0 * K;
                uint8_t* ab = a.argmax ? a.argmax + win0 * K : nullptr;
                const int nw = (int)min(16L, (nrows >> 2) - win0);
                // Pooled values go to the staging area as they are computed,
                // pass by pass, so each accumulator register dies once its
                // window is staged (no array of pooled values is held).
                // Whole output rows: four passes of four windows, each staged as
                // [4 windows][KP channels] fp16 (1 KiB for KP = 128) and stored
                // by KP/8 lanes per window row, 16 bytes each, so every store
                // instruction writes whole 256-byte rows of y.  Pass p holds
                // windows 4p..4p+3 = 8u + 2g + hh with u = p/2, g = 2(p%2) + gg.
                static_assert(4 * KP * 2 <= CW_OSTAGE, "four staged rows fit the staging area");
                constexpr int LPR = KP / 8;   // lanes per staged row
                const int sr = ln / LPR, sg = ln % LPR;
                const lds_half8* const srd = reinterpret_cast<const lds_half8*>(ost + sr * KP + 8 * sg);
                // argmax (first maximum of the rounded values) is only needed
                // with an argmax output or an activation that is not monotone
                const bool fast = EPI == EPI_POOL && decltype(act)::monotone && !ab;
                const int olane = hh * K + lr;
                int nwl = nw - hh;   // window 8u + 2g + hh is valid iff 8u + 2g < nwl
                asm volatile("" : "+v"(nwl));   // (opaque: compared against constants, not folded back)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int u = p >> 1;
#pragma unroll
                    for (int gg = 0; gg < 2; ++gg) {
                        const int g = 2 * (p & 1) + gg;
#pragma unroll
                        for (int t = 0; t < NTK; ++t) {
                            const float bk = bsl[32 * t];
                            const float sk = ssl[32 * t];
                            const floatx16& c = acc[u][t];
                            half_t best;
                            if (fast) {
                                // v = fp16(act(fma(acc, s, b))): the fused multiply-add
                                // (one rounding), a non-decreasing activation and the
                                // fp16 rounding are monotone in acc -- non-decreasing
                                // for s >= 0, non-increasing for s < 0 -- so the max
                                // of the four rounded values is v of the largest
                                // (s >= 0) or smallest (s < 0) accumulator: pool
                                // first, then one scale/bias/act/convert per window.
                                // (No scale: s = 1, and fma(acc, 1, b) = acc + b.)
                                const float hi = __builtin_fmaxf(__builtin_fmaxf(c[4 * g], c[4 * g + 1]),
                                                                 __builtin_fmaxf(c[4 * g + 2], c[4 * g + 3]));
                                const float lo = __builtin_fminf(__builtin_fminf(c[4 * g], c[4 * g + 1]),
                                                                 __builtin_fminf(c[4 * g + 2], c[4 * g + 3]));
                                best = (half_t)act.f(__builtin_fmaf(sk >= 0.0f ? hi : lo, sk, bk));
                            } else if (EPI == EPI_AVG) {
                                // mean of the four rounded fp16 values (fp32 sum,
                                // an exact quarter), rounded once to fp16
                                float sum = 0.0f;
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    sum += (float)(half_t)act.f(__builtin_fmaf(c[4 * g + e], sk, bk));
                                best = (half_t)(sum * 0.25f);
                            } else {
                                // decided on the rounded fp16 intermediate, first
                                // maximum in window order (0,0),(0,1),(1,0),(1,1)
                                best = (half_t)act.f(__builtin_fmaf(c[4 * g], sk, bk));
                                int bi = 0;
#pragma unroll
                                for (int e = 1; e < 4; ++e) {
                                    const half_t v = (half_t)act.f(__builtin_fmaf(c[4 * g + e], sk, bk));
                                    const bool gt = v > best;
                                    best = gt ? v : best;
                                    bi = gt ? e : bi;
                                }
                                const int w0 = 8 * u + 2 * g;
                                if (ab && lr < K - 32 * t && w0 < nwl) ab[olane + w0 * K + 32 * t] = (uint8_t)bi;
                            }
                            ost[(2 * gg + hh) * KP + 32 * t + lr] = best;
                        }
                    }
                    wave_lds_sync();
                    if (sr < 4) {
                        const half8 v = *srd;
                        const int w = 4 * p + sr;
                        if (w < nw && 8 * sg < K) st_out(reinterpret_cast<half8*>(yb + w * K + 8 * sg), v);
                    }
                    wave_lds_sync();   // the next pass overwrites the staging area
                }
            } else {
                // Whole output rows here too: for each (u, g) and register pair
                // e = 2eh, 2eh + 1, the two lane halves hold tile rows
                // 32u + 8g + 4hh + e of every channel 32t + lr, i.e. four
                // complete rows.  They are staged as [4][KP] fp16 (row
                // 2(e % 2) + hh) and stored by KP/8 lanes per row, 16 bytes
                // each, so every store instruction writes whole rows of y (no
                // cache line of y is written in several partial pieces).
                half_t* yb = a.y + row0 * K;
                const int nr = (int)min(64L, nrows - row0);
                const int vpr = KP / 8;               // 16-byte vectors per staged row
                const int sr = ln / vpr, sg = ln - sr * vpr;
                const lds_half8* const orw = reinterpret_cast<const lds_half8*>(ost + sr * KP + 8 * sg);
                lds_half* const owr = ost + hh * KP + lr;
                float bk[NTK], sk[NTK];
#pragma unroll
                for (int t = 0; t < NTK; ++t) {
                    bk[t] = bsl[32 * t];
                    sk[t] = ssl[32 * t];
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
#pragma unroll
                        for (int eh = 0; eh < 2; ++eh) {
#pragma unroll
                            for (int ei = 0; ei < 2; ++ei)
#pragma unroll
                                for (int t = 0; t < NTK; ++t)
                                    owr[2 * ei * KP + 32 * t] =
                                        (half_t)act.f(__builtin_fmaf(acc[u][t][4 * g + 2 * eh + ei], sk[t], bk[t]));
                            wave_lds_sync();
                            // staged row sr = 2 ei + h1 -> tile row 32u + 8g + 4 h1 + 2 eh + ei
                            const int row = 32 * u + 8 * g + 4 * (sr & 1) + 2 * eh + (sr >> 1);
                            if (sr < 4) {
                                const half8 v = *orw;
                                if (row < nr && 8 * sg < K) st_out(reinterpret_cast<half8*>(yb + row * K + 8 * sg), v);
                            }
                            wave_lds_sync();
                        }
                    }
                }
            }
        });
    };

    if constexpr (KCH > 0) {
        // One tile = KCH chunks; its chunk c sits in set (SB + c) % R, where
        // SB = (tiles done * KCH) % R takes the two values 0 and KCH % R.
        // While the tile's last PD chunks are multiplied, the next tile's
        // first PD chunks are loaded.
        // W fragments are software-pipelined one k-step (16 k) ahead: step
        // s = 4c + q uses set s % 2 while set (s + 1) % 2 is read from LDS,
        // and the first step's fragments (the same for every tile) are read
        // during the previous tile's last step.  The scheduling groups
        // interleave each step's eight MFMAs with the next step's eight LDS
        // reads, so the LDS latency hides under the matrix core.
        half8 wf[2][NTK];
        if (CONVW_WPIPE) {
#pragma unroll
            for (int t = 0; t < NTK; ++t) wf[0][t] = frag_tr_at(wlane[t], 4 * Wn.ld);
        }
        auto body = [&](auto sb) {
            constexpr int SB = decltype(sb)::value;
            // The next tile's loads are issued even when there is no next
            // tile (its rows then lie past the end, read the zero line and
            // are never used): a load under a branch would make the wait
            // counts after it assume the fewest loads in flight, i.e. wait
            // for the prefetches too.
            const long ntile = claim();
            const QRows nq = make_qrows(min(ntile, t_end));
            floatx16 acc[2][NTK];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 0; t < NTK; ++t) acc[u][t] = zero16();
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
                const int cl = c + PD;
                if (cl < KCH) load_q(qrows, cl, ring[(SB + cl) % R]);
                else load_q(nq, cl - KCH, ring[(SB + cl) % R]);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch issued here
                half8 (&cur)[2][4] = ring[(SB + c) % R];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    quad_transpose4(cur[h], lane);
#pragma unroll
                    for (int sp = 0; sp < 2; ++sp) {
                        const int q = 2 * h + sp;
                        half8 x0 = cur[h][2 * sp], x1 = cur[h][2 * sp + 1];
                        swap_halves(x0, x1);   // x0: row tile 0, x1: row tile 1; k-halves 2q, 2q + 1
                        const int st = 4 * c + q;
                        if (CONVW_WPIPE) {
                            const int sn = (st + 1) % (4 * KCH);   // next step (wraps to the next tile)
                            const int cn = sn >> 2, qn = sn & 3;
#pragma unroll
                            for (int t = 0; t < NTK; ++t)
                                wf[(st + 1) & 1][t] = frag_tr_at(wlane[t] + (64 * cn + 16 * qn) * Wn.ld, 4 * Wn.ld);
#pragma unroll
                            for (int t = 0; t < NTK; ++t) {
                                acc[0][t] = mfma32x32x16(x0, wf[st & 1][t], acc[0][t]);
                                acc[1][t] = mfma32x32x16(x1, wf[st & 1][t], acc[1][t]);
                            }
#pragma unroll
                            for (int i = 0; i < 2 * NTK; ++i) {
                                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                            }
                        } else {
                            // the fragment of column tile t + 1 is read while tile
                            // t's two MFMAs run (two fragment registers, not one:
                            // with one, every read waits out the LDS latency)
                            half8 wv = frag_tr_at(wlane[0] + 16 * st * Wn.ld, 4 * Wn.ld);
#pragma unroll
                            for (int t = 0; t < NTK; ++t) {
                                half8 wn = wv;
                                if (t + 1 < NTK) wn = frag_tr_at(wlane[t + 1] + 16 * st * Wn.ld, 4 * Wn.ld);
                                acc[0][t] = mfma32x32x16(x0, wv, acc[0][t]);
                                acc[1][t] = mfma32x32x16(x1, wv, acc[1][t]);
                                wv = wn;
                            }
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            epilogue(tile, acc);
            tile = ntile;
            qrows = nq;
        };
        while (tile < t_end) {
            body(IntC<0>{});
            if constexpr (KCH % R != 0) {
                if (tile >= t_end) break;
                body(IntC<KCH % R>{});
            }
        }
    } else {
        // Runtime chunk count: two sets, the loop unrolled by two; rows of
        // MFMA row tile u are tile rows 32u + lane%32 (operand layout loads).
        auto mma_chunk = [&](int c, const half8 (&cur)[2][4], floatx16 (&acc)[2][NTK]) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int t = 0; t < NTK; ++t) {
                    const half8 wv = frag_tr_at(wlane[t] + (64 * c + 16 * q) * Wn.ld, 4 * Wn.ld);
                    acc[0][t] = mfma32x32x16(cur[0][q], wv, acc[0][t]);
                    acc[1][t] = mfma32x32x16(cur[1][q], wv, acc[1][t]);
                }
            }
        };
        while (tile < t_end) {
            floatx16 acc[2][NTK];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 0; t < NTK; ++t) acc[u][t] = zero16();
            auto step = [&](int c, const half8 (&cur)[2][4], half8 (&nxt)[2][4]) {
                if (c + 1 < nch) {
                    ld.template load<KCH>(rows[0], c + 1, hh, nxt[0]);
                    ld.template load<KCH>(rows[1], c + 1, hh, nxt[1]);
                }
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch issued here
                mma_chunk(c, cur, acc);
            };
            for (int c = 0; c < nch; c += 2) {
                step(c, ring[0], ring[1]);
                if (c + 1 < nch) step(c + 1, ring[1], ring[0]);
            }
            // Claim the next tile and put its first chunk in flight.
            const long ntile = claim();
            Conv3x3Rows::Row nrows_[2] = {rows[0], rows[1]};
            if (ntile < t_end) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    nrows_[u] = make_row(ntile * 64 + 32 * u + lr);
                    ld.template load<KCH>(nrows_[u], 0, hh, ring[0][u]);
                }
            }
            epilogue(tile, acc);
            tile = ntile;
            rows[0] = nrows_[0];
            rows[1] = nrows_[1];
        }
    }
}

template <int NTK, int EPI, int KCH>
static hipError_t launch_convw_k(ConvWArgs a, hipStream_t st)
{
    const size_t lds = convw_lds_bytes(32 * NTK, a.Kp);
    static std::atomic<unsigned long long> lds_set{0};
    hipError_t e = allow_full_lds((const void*)k_conv_w<NTK, EPI, KCH>, &lds_set);
    if (e != hipSuccess) return e;
    const int nwaves = a.wpb > 0 ? a.wpb : convw_threads(KCH) / 64;
    long grid = device_cu_count();
    if (grid * nwaves > a.ntiles) grid = (a.ntiles + nwaves - 1) / nwaves;
    if (grid < 1) grid = 1;
    a.tiles_per_block = (a.ntiles + grid - 1) / grid;
    grid = (a.ntiles + a.tiles_per_block - 1) / a.tiles_per_block;
    hipLaunchKernelGGL((k_conv_w<NTK, EPI, KCH>), dim3((unsigned)grid), dim3(convw_threads(KCH)), lds, st, a);
    return hipGetLastError();
}

template <int NTK, int EPI>
static hipError_t launch_convw_t(ConvWArgs a, hipStream_t st)
{
    if ((a.Kp >> 6) == 9) return launch_convw_k<NTK, EPI, 9>(a, st);   // C = 64
    return launch_convw_k<NTK, EPI, 0>(a, st);
}

template <int EPI>
static hipError_t launch_convw(ConvWArgs a, hipStream_t st)
{
    switch ((a.K + 31) / 32) {
    case 1: return launch_convw_t<1, EPI>(a, st);
    case 2: return launch_convw_t<2, EPI>(a, st);
    case 3: return launch_convw_t<3, EPI>(a, st);
    case 4: return launch_convw_t<4, EPI>(a, st);
    }
    return hipErrorInvalidValue;
}

bool convw_fits(int C, int K)
{
    const int Kp = (9 * C + 63) / 64 * 64;
    return K <= 128 && convw_lds_bytes((K + 31) / 32 * 32, Kp) <= RF_LDS_LIMIT;
}

hipError_t run_conv_bias_act3x3(const half_t* x, const half_t* w, const half_t* scale, const half_t* b, int act,
                                half_t* y, int NB, int H, int W, int C, int K, hipStream_t st)
{
    ConvWArgs a;
    a.x = x; a.w = w; a.s = scale; a.b = b; a.y = y; a.argmax = nullptr;
    a.NB = NB; a.H = H; a.W = W; a.C = C; a.K = K;
    a.Kr = 9 * C; a.Kp = (9 * C + 63) / 64 * 64; a.act = act;
    a.wpb = 0;
    const long rows = (long)NB * H * W;
    if (rows == 0) return hipSuccess;
    a.ntiles = (rows + 63) / 64;
    a.fa = FastDiv::make((unsigned)H * (unsigned)W);
    a.fb = FastDiv::make((unsigned)W);
    a.fc8 = FastDiv::make((unsigned)C / 8);
    return launch_convw<EPI_STORE>(a, st);
}

hipError_t run_conv_pool_wr(const half_t* x, const half_t* w, const half_t* scale, const half_t* b, int act, bool avg,
                            half_t* y, uint8_t* argmax, int NB, int H, int W, int K, hipStream_t st);

hipError_t run_conv_pool3x3(const half_t* x, const half_t* w, const half_t* scale, const half_t* b, int act,
                            bool avg, half_t* y, uint8_t* argmax, int NB, int H, int W, int C, int K, bool regw,
                            int waves, hipStream_t st)
{
    if (regw) return run_conv_pool_wr(x, w, scale, b, act, avg, y, argmax, NB, H, W, K, st);
    ConvWArgs a;
    a.x = x; a.w = w; a.s = scale; a.b = b; a.y = y; a.argmax = argmax;
    a.NB = NB; a.H = H; a.W = W; a.C = C; a.K = K;
    a.Kr = 9 * C; a.Kp = (9 * C + 63) / 64 * 64; a.act = act;
    a.wpb = waves;
    const long rows = (long)NB * (H / 2) * (W / 2) * 4;
    if (rows == 0) return hipSuccess;
    a.ntiles = (rows + 63) / 64;
    a.fa = FastDiv::make((unsigned)(H / 2) * (unsigned)(W / 2));
    a.fb = FastDiv::make((unsigned)(W / 2));
    a.fc8 = FastDiv::make((unsigned)C / 8);
    return avg ? launch_convw<EPI_AVG>(a, st) : launch_convw<EPI_POOL>(a, st);
}

hipError_t run_chain_conv2_3x3(const half_t* x, const half_t* w0, const half_t* b0, int act, const half_t* w1,
                               const half_t* b1, half_t* y, int NB, int H, int W, int C, int K0, int K1, int waves,
                               int stages, hipStream_t st)
{
    const long M = (long)NB * H * W;
    if (M == 0) return hipSuccess;
    RfArgs a{};
    a.W0 = w0; a.b0 = b0; a.W1 = w1; a.b1 = b1; a.out = y;
    a.M = M; a.K0 = 9 * C; a.N0 = K0; a.N1 = K1;
    a.K0p = (9 * C + 63) / 64 * 64;
    a.N1p = (K1 + 63) / 64 * 64;
    a.act = act;
    a.ntiles = (M + 31) / 32;
    a.tiles_per_block = 0;
    a.wpb = waves;
    a.stages = stages;
    Conv3x3Rows ld;
    ld.x = x; ld.H = H; ld.W = W; ld.C = C; ld.M = M;
    ld.set_divisors();
    return launch_rf(ld, a, (K0 + 31) / 32, st);
}

// conv3x3 -> 1x1 (-> 1x1): the N-stage register-resident chain with the
// implicit-GEMM loader; widths[0] = 9C (the first GEMM's k), widths[i + 1] =
// output channels of stage i.  Compile-time chunk count only for C = 64.
template <int NMID>
static hipError_t launch_convN(const Conv3x3Rows& ld, const RfArgs& a, int nt0, hipStream_t st)
{
    const bool k9 = (a.K0p >> 6) == 9;
    if (k9 && a.stages == 2) {   // 8 tile-owning waves: the two-stage row ring
        switch (nt0) {
        case 1: return launch_rf_k<1, 9, Conv3x3Rows, NMID, 2>(ld, a, st);
        case 2: return launch_rf_k<2, 9, Conv3x3Rows, NMID, 2>(ld, a, st);
        case 3: return launch_rf_k<3, 9, Conv3x3Rows, NMID, 2>(ld, a, st);
        case 4: return launch_rf_k<4, 9, Conv3x3Rows, NMID, 2>(ld, a, st);
        }
    }
    switch (nt0) {
    case 1: return k9 ? launch_rf_k<1, 9, Conv3x3Rows, NMID>(ld, a, st) : launch_rf_k<1, 0, Conv3x3Rows, NMID>(ld, a, st);
    case 2: return k9 ? launch_rf_k<2, 9, Conv3x3Rows, NMID>(ld, a, st) : launch_rf_k<2, 0, Conv3x3Rows, NMID>(ld, a, st);
    case 3: return k9 ? launch_rf_k<3, 9, Conv3x3Rows, NMID>(ld, a, st) : launch_rf_k<3, 0, Conv3x3Rows, NMID>(ld, a, st);
    case 4: return k9 ? launch_rf_k<4, 9, Conv3x3Rows, NMID>(ld, a, st) : launch_rf_k<4, 0, Conv3x3Rows, NMID>(ld, a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t run_chain_convN_3x3(const half_t* x, int nst, const half_t* const* w, const half_t* const* b,
                               const int* act, const int* widths, half_t* y, int NB, int H, int W, int C,
                               hipStream_t st)
{
    const long M = (long)NB * H * W;
    if (M == 0) return hipSuccess;
    RfArgs a{};
    gemmn_args(nst, w, b, act, widths, y, M, a);
    a.stages = (a.K0p >> 6) == 9 ? 2 : 0;
    Conv3x3Rows ld;
    ld.x = x; ld.H = H; ld.W = W; ld.C = C; ld.M = M;
    ld.set_divisors();
    const int nt0 = (a.N0 + 31) / 32;
    return nst == 3 ? launch_convN<1>(ld, a, nt0, st) : launch_convN<2>(ld, a, nt0, st);
}

// ------------------------------------------------------------ max pool 2x2/2
// One thread: one output pixel x 8 channels (16-byte loads of the 4 inputs).
template <bool AVG>
__global__ __launch_bounds__(256) void k_pool2x2(const half_t* __restrict__ v, half_t* __restrict__ y,
                                                 uint8_t* __restrict__ am, int NB, int P, int Q, int K)
{
    const int PO = P >> 1, QO = Q >> 1, KB = K >> 3;
    const long total = (long)NB * PO * QO * KB;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
        const int kb = (int)(i % KB);
        const long pix = i / KB;
        const int oq = (int)(pix % QO);
        const long t = pix / QO;
        const int op = (int)(t % PO);
        const int n = (int)(t / PO);
        half8 in[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = 2 * op + (e >> 1), q = 2 * oq + (e & 1);
            in[e] = ld16(v + (((long)n * P + p) * Q + q) * K + 8 * kb);
        }
        half8 o;
        if (AVG) {
            // mean of the four fp16 values (fp32 sum, exact quarter), one rounding
#pragma unroll
            for (int c = 0; c < 8; ++c)
                o[c] = (half_t)((((float)in[0][c] + (float)in[1][c]) + (float)in[2][c] + (float)in[3][c]) * 0.25f);
            *reinterpret_cast<half8*>(y + pix * K + 8 * kb) = o;
            continue;
        }
        uint8_t ai[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float best = (float)in[0][c];
            int bi = 0;
#pragma unroll
            for (int e = 1; e < 4; ++e) {
                const float f = (float)in[e][c];
                if (f > best) { best = f; bi = e; }
            }
            o[c] = in[bi][c];
            ai[c] = (uint8_t)bi;
        }
        *reinterpret_cast<half8*>(y + pix * K + 8 * kb) = o;
        if (am) {
            uint64_t packed = 0;
#pragma unroll
            for (int c = 0; c < 8; ++c) packed |= (uint64_t)ai[c] << (8 * c);
            *reinterpret_cast<uint64_t*>(am + pix * K + 8 * kb) = packed;
        }
    }
}

hipError_t run_pool2x2(bool avg, const half_t* v, half_t* y, uint8_t* am, int NB, int P, int Q, int K,
                       hipStream_t st)
{
    const long total = (long)NB * (P / 2) * (Q / 2) * (K / 8);
    if (total == 0) return hipSuccess;
    long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (avg)
        hipLaunchKernelGGL(k_pool2x2<true>, dim3((unsigned)blocks), dim3(256), 0, st, v, y, nullptr, NB, P, Q, K);
    else
        hipLaunchKernelGGL(k_pool2x2<false>, dim3((unsigned)blocks), dim3(256), 0, st, v, y, am, NB, P, Q, K);
    return hipGetLastError();
}

// --------------------------------------------- zero padding of a middle dim
// dst[o][c][i] = c < c_in ? src[o][c][i] : 0  for a tensor viewed as
// [outer, c, inner] (NHWC channels: inner = 1; HWIO input channels:
// outer = R*S, inner = K).
__global__ __launch_bounds__(256) void k_pad_mid(const half_t* __restrict__ src, half_t* __restrict__ dst,
                                                 long outer, int c_in, int c_out, int inner)
{
    const long total = outer * c_out * (long)inner;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
        const int ii = (int)(i % inner);
        const long t = i / inner;
        const int c = (int)(t % c_out);
        const long o = t / c_out;
        dst[i] = c < c_in ? src[(o * c_in + c) * inner + ii] : (half_t)0.0f;
    }
}

hipError_t run_pad_mid(const half_t* src, half_t* dst, long outer, int c_in, int c_out, int inner, hipStream_t st)
{
    const long total = outer * c_out * (long)inner;
    if (total == 0) return hipSuccess;
    long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_pad_mid, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, outer, c_in, c_out, inner);
    return hipGetLastError();
}

}  // namespace fc
