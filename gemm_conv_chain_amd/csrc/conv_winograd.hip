// conv_winograd.hip -- 3x3 convolution by Winograd F(2x2, 3x3) fused with bias,
// activation and the 2x2 / stride-2 pool (interview page, "Conv optimisation",
// item 3: (m + r - 1)^2 = 16 products per 2x2 output tile instead of
// m^2 r^2 = 36; the transforms are those of Lavin and Gray's minimal filtering
// algorithm, since the page prints none).  A 2x2 Winograd output tile is
// exactly one pool window (the Welder notes' Conv -> ReLU -> MaxPool tile
// graph, Figure 5), so the conv output never leaves the registers.
//
//   U = G g G^T     per (c, k): k_wino_weights, once per weight tensor, in
//                   fp64 and rounded once to fp16;
//   V = B^T d B     per 4x4 input patch and channel: fp16 arithmetic, rows
//                   first (one rounding per stage);
//   M = sum_c U . V 16 channel contractions on the matrix cores (fp16 in,
//                   fp32 accumulation);
//   Y = A^T M A     in fp32, then bias, activation, pool, fp16.
//
// Work split (gfx950, 64-wide waves, 16x16x32 MFMA): a block of 8 waves runs
// persistently over batches of 2 x 8 tiles (16 tiles: the M = 16 side of the
// MFMA).  Wave w owns output channels 16w .. 16w + 15 and keeps their
// transformed weights for all 16 (xi, nu) and all C channels in registers
// (16 * C / 32 operand quadruples: 128 registers for C = 64) for the whole
// kernel, so the weights are read from HBM once per block.  A batch's input
// halo (6 x 18 pixels) arrives by LDS-DMA two batches ahead; the input
// transform is spread over all 512 threads (one tile, one 8-channel group,
// one row xi of V each) and lands in LDS as V[16][16 tiles][C], which every
// wave then reads as MFMA operand A.  Batch b + 1's V is built while batch
// b's accumulators wait for their epilogue.
#include "fc_dma.h"
#include "fc_launch.h"

namespace fc {
namespace {

constexpr int WI_THREADS = 512;   // 8 waves
constexpr int WI_TILES = 16;      // 2x2 output tiles per batch

constexpr int WI_BR = 2, WI_BC = 8;                // a batch: 2 x 8 tiles
constexpr int WI_HR = 2 * WI_BR + 2;               // its input halo: 6 rows
constexpr int WI_HC = 2 * WI_BC + 2;               // x 18 columns
constexpr int WI_HPIX = WI_HR * WI_HC;             // 108 pixels

struct WinoArgs {
    const half_t* x;     // NHWC [NB][H][W][C]
    const half_t* U;     // [16][C/8][K][8]: U[xi*4+nu][c][k] at ((xn * C/8 + c/8) * K + k) * 8 + c%8
    const half_t* b;     // [K] or null
    half_t* y;           // [NB][TH][TW][K]
    uint8_t* argmax;     // [NB][TH][TW][K] or null (max pool only)
    int NB, H, W, K, act;
    int TH, TW;          // tiles (pool windows): H/2 x W/2
    long nbatch;         // NB * ceil(TH/2) * ceil(TW/8)
    FastDiv fimg, fbw;   // by batches per image, by batches per tile row
};

__device__ __forceinline__ floatx4 mfma16x16x32(half8 a, half8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Offset (halves) of 8-channel group cg of tile tb in plane xn of a V buffer
// [16][16][C].  The 16-byte group index is XOR-ed with the tile's row of 256
// bytes so that the 16 tiles one operand read touches (same group) fall on
// 16 different 16-byte bank groups.
template <int C>
__device__ __forceinline__ int v_off(int xn, int tb, int cg)
{
    constexpr int CG = C / 8;
    constexpr int RP = 128 / C;   // tile rows per 256 bytes
    return (xn * WI_TILES + tb) * C + 8 * (cg ^ ((tb / RP) & (CG - 1)));
}

// LDS-DMA requests (64 lanes x 16 bytes) that fetch one batch's halo.
template <int C>
constexpr int wino_ndma() { return (WI_HPIX * (C / 8) + 63) / 64; }

// LDS: V double buffer [2][16][16][C], halo double buffer [2][ndma KiB]
// ([108 pixels][C] fp16, row-major over the 6 x 18 window), output staging
// [2][16][K] fp16, [2][16][K] argmax bytes, the bias [K] fp32.
template <int C>
constexpr size_t wino_lds_bytes(int K)
{
    return (size_t)2 * 16 * WI_TILES * C * 2 + (size_t)2 * wino_ndma<C>() * 1024 + (size_t)2 * WI_TILES * K * 2 +
           (size_t)2 * WI_TILES * K + (size_t)K * 4;
}

// POOL: 0 = max, 1 = average.  AM: write the argmax of the max pool.
template <int C, int POOL, bool AM>
__global__ __launch_bounds__(WI_THREADS) void k_conv_pool_wino(WinoArgs a)
{
    constexpr int CG = C / 8;           // 8-channel groups
    constexpr int KS = C / 32;          // MFMA k-steps per (xi, nu)
    constexpr int TPW = 64 / CG;        // transform: tiles per wave
    constexpr int NDMA = wino_ndma<C>();
    constexpr int HBUF = NDMA * 512;    // halves per halo buffer
    extern __shared__ __align__(16) char smem[];
    typedef FC_LDS half8 lds_half8;
    typedef FC_LDS float lds_float;
    lds_half* const vbuf = (lds_half*)smem;                                     // [2][16][16][C]
    lds_half* const hbuf = vbuf + 2 * 16 * WI_TILES * C;                        // [2][HBUF]
    lds_half* const ost = hbuf + 2 * HBUF;                                      // [2][16][K]
    FC_LDS uint8_t* const ast = (FC_LDS uint8_t*)(ost + 2 * WI_TILES * a.K);   // [2][16][K]
    lds_float* const bsl = (lds_float*)(ast + 2 * WI_TILES * a.K);            // [K]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const bool kwave = 16 * wave < a.K;          // wave computes (K % 16 == 0)
    // Per-lane values are recomputed where used from an opaque lane id
    // (lane_id_here): held across the batch loop, next to the 128 weight
    // registers, they would be spilled.

    const long lb = xcd_block(blockIdx.x, gridDim.x);
    const long b_begin = lb * a.nbatch / gridDim.x;
    const long b_end = (lb + 1) * a.nbatch / gridDim.x;
    // odd blocks walk their range backward (batch index bt -> row position
    // b_begin + b_end - 1 - bt): neighbouring ranges then reach the input rows
    // their halos share at the same time and the second fetch hits in L2
    const bool backward = lb & 1;

    if constexpr (kPoison) {
        lds_poison(smem, (int)wino_lds_bytes<C>(a.K), tid, WI_THREADS);
        __syncthreads();
    }

    // ---- transformed weights of this wave's 16 channels -> registers:
    // operand B of (xn, s): rows c = 32 s + 8 (lane / 16) + [0, 8), column
    // 16 wave + lane % 16.
    half8 uw[16][KS];
    {
        const int kcol = 16 * wave + (lane & 15);
#pragma unroll
        for (int xn = 0; xn < 16; ++xn)
#pragma unroll
            for (int s = 0; s < KS; ++s)
                uw[xn][s] = ld16_if(a.U + (((long)xn * CG + 4 * s + (lane >> 4)) * a.K + kcol) * 8, kwave);
    }
    for (int k = tid; k < a.K; k += WI_THREADS) bsl[k] = a.b ? (float)a.b[k] : 0.0f;

    // batch -> image n, tile rows 2 ib .. 2 ib + 1, tile columns 8 jb .. 8 jb + 7
    auto batch_pos = [&](long bt, unsigned& n, int& ib, int& jb) {
        n = a.fimg.div((unsigned)bt);
        const unsigned r = (unsigned)bt - n * a.fimg.d;
        const unsigned q = a.fbw.div(r);
        ib = (int)q;
        jb = (int)(r - q * a.fbw.d);
    };

    // ---- the halo of batch bt (input rows 4 ib - 1 .. 4 ib + 4, columns
    // 16 jb - 1 .. 16 jb + 16, all C channels) -> halo buffer, by LDS-DMA:
    // request m (issued by wave m % 8) moves 16-byte chunks 64 m .. 64 m + 63,
    // chunk e = pixel e / CG, channel group e % CG.  Pixels outside the image
    // (and chunks past the window) read as zero: their offsets lie outside the
    // resource, which spans the batch's image.
    auto issue_halo = [&](long bt, lds_half* hb) {
        unsigned n;
        int ib, jb;
        batch_pos(backward ? b_begin + b_end - 1 - bt : bt, n, ib, jb);
        const long img = (long)a.H * a.W * C;
        const i32x4 rs = buf_rsrc(a.x + (long)n * img, img * 2);
        const int ln = lane_id_here();
#pragma unroll
        for (int m = wave; m < NDMA; m += 8) {
            const int e = 64 * m + ln;
            const int pix = e / CG, cg = e % CG;
            const int hr = pix / WI_HC, hc = pix - hr * WI_HC;
            const int p = 4 * ib - 1 + hr, q = 16 * jb - 1 + hc;
            const bool ok = pix < WI_HPIX && p >= 0 && p < a.H && q >= 0 && q < a.W;
            const unsigned voff = ok ? (unsigned)((((long)p * a.W + q) * C + 8 * cg) * 2) : CS_OUTSIDE;
            dma16(rs, voff, hb + m * 512);
        }
    };

    // ---- input transform: thread = (tile tb of the batch, channel group cg,
    // row xi of V): t = d[ra] + sg d[rb] over the patch's 4 columns, then
    // V[xi][nu] = t B.  fp16 arithmetic; fma(b, +-1, a) rounds the exact sum
    // once, like an addition, and needs no branch.
    const int xi = wave & 3;
    const bool tactive = (wave >> 2) < CG / 4;   // C = 32: waves 4..7 idle here
    const int ra = xi == 0 ? 0 : xi == 2 ? 2 : 1;
    const int rb = xi == 0 ? 2 : xi == 1 ? 2 : xi == 2 ? 1 : 3;
    const half_t sg = (half_t)(xi == 1 ? 1.0f : -1.0f);
    auto transform = [&](const lds_half* hb, lds_half* vb) {
        const int ln = lane_id_here();
        const int tb = (wave >> 2) * TPW + ln / CG, cg = ln % CG;
        const int ti = tb / WI_BC, tj = tb % WI_BC;
        half8 d[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int bq = 0; bq < 4; ++bq)
                d[h][bq] = *reinterpret_cast<const lds_half8*>(
                    hb + ((2 * ti + (h == 0 ? ra : rb)) * WI_HC + 2 * tj + bq) * C + 8 * cg);
        // -1 as an opaque value: the compiler would fold fma(b, -1, a) back
        // into a - b, which it lowers as two scalar subtractions and a pack
        // per pair instead of one packed operation
        unsigned mone = 0xBC00BC00u;   // fp16 pair (-1, -1)
        asm volatile("" : "+s"(mone));
        const u32x4 m1w = {mone, mone, mone, mone};
        const half8 m1 = __builtin_bit_cast(half8, m1w);
        half8 sgv;
#pragma unroll
        for (int e = 0; e < 8; ++e) sgv[e] = sg;
        half8 t[4];
#pragma unroll
        for (int bq = 0; bq < 4; ++bq) t[bq] = __builtin_elementwise_fma(d[1][bq], sgv, d[0][bq]);   // rows: one rounding
        half8 v[4];   // columns: one rounding each (a - b as fma(b, -1, a))
        v[0] = __builtin_elementwise_fma(t[2], m1, t[0]);
        v[1] = t[1] + t[2];
        v[2] = __builtin_elementwise_fma(t[1], m1, t[2]);
        v[3] = __builtin_elementwise_fma(t[3], m1, t[1]);
#pragma unroll
        for (int nu = 0; nu < 4; ++nu)
            *reinterpret_cast<lds_half8*>(vb + v_off<C>(4 * xi + nu, tb, cg)) = v[nu];
    };

    // ---- a batch's outputs: tile tb = 8 ti + tj is pool output (n, 2 ib + ti,
    // 8 jb + tj); each 16-byte vector of the staged [16][K] block goes to y
    // (and the argmax) if its tile lies inside the output.
    auto store_batch = [&](long bt, int pr) {
        unsigned n;
        int ib, jb;
        batch_pos(backward ? b_begin + b_end - 1 - bt : bt, n, ib, jb);
        const int kv8 = a.K / 8;
        if (tid < WI_TILES * kv8) {
            const int tb = tid / kv8, kv = tid - tb * kv8;
            const int i = 2 * ib + tb / WI_BC, j = 8 * jb + tb % WI_BC;
            if (i < a.TH && j < a.TW) {
                const long o = (((long)n * a.TH + i) * a.TW + j) * a.K + 8 * kv;
                st_out(reinterpret_cast<half8*>(a.y + o),
                       (half8)*reinterpret_cast<const lds_half8*>(ost + pr * (WI_TILES * a.K) + tb * a.K + 8 * kv));
            }
        }
        if (AM) {
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            typedef FC_LDS const u32x2 lds_u2c;
            if (tid < WI_TILES * kv8) {
                const int tb = tid / kv8, kv = tid - tb * kv8;
                const int i = 2 * ib + tb / WI_BC, j = 8 * jb + tb % WI_BC;
                if (i < a.TH && j < a.TW) {
                    const long o = (((long)n * a.TH + i) * a.TW + j) * a.K + 8 * kv;
                    st_out(reinterpret_cast<u32x2*>(a.argmax + o),
                           (u32x2)*reinterpret_cast<lds_u2c*>(ast + pr * (WI_TILES * a.K) + tb * a.K + 8 * kv));
                }
            }
        }
    };

    // prologue: halos of the first two batches; the first batch's V
    if (b_begin < b_end) {
        issue_halo(b_begin, hbuf);
        if (b_begin + 1 < b_end) issue_halo(b_begin + 1, hbuf + HBUF);
    }
    vm_wait<0>();
    __syncthreads();
    if (b_begin < b_end && tactive) transform(hbuf, vbuf);
    __syncthreads();

    for (long bt = b_begin; bt < b_end; ++bt) {
        const int par = (int)((bt - b_begin) & 1);
        if constexpr (kPoison) {
            // released by the last barrier: the halo buffer batch bt + 2 refills,
            // the V buffer batch bt + 1's transform writes, the staging areas
            // batch bt's epilogue writes
            lds_poison(hbuf + par * HBUF, HBUF * 2, tid, WI_THREADS);
            lds_poison(vbuf + (par ^ 1) * (16 * WI_TILES * C), 16 * WI_TILES * C * 2, tid, WI_THREADS);
            lds_poison(ost + par * (WI_TILES * a.K), WI_TILES * a.K * 2, tid, WI_THREADS);
            lds_poison(ast + par * (WI_TILES * a.K), WI_TILES * a.K, tid, WI_THREADS);
            __syncthreads();
        }
        if (bt > b_begin) store_batch(bt - 1, par ^ 1);
        // batch bt + 2's halo into the buffer batch bt's transform has released
        if (bt + 2 < b_end) issue_halo(bt + 2, hbuf + par * HBUF);

        // ---- M[xn] (16 tiles x this wave's 16 channels) = V[xn] U[xn]
        floatx4 acc[16];
#pragma unroll
        for (int xn = 0; xn < 16; ++xn) acc[xn] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        if (kwave) {
            const int ln = lane_id_here();
            const lds_half* vb = vbuf + par * (16 * WI_TILES * C);
#pragma unroll
            for (int xn = 0; xn < 16; ++xn)
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const half8 av = *reinterpret_cast<const lds_half8*>(vb + v_off<C>(xn, ln & 15, 4 * s + (ln >> 4)));
                    acc[xn] = mfma16x16x32(av, uw[xn][s], acc[xn]);
                }
        }

        // batch bt + 1's V (its halo arrived during the previous batch)
        if (bt + 1 < b_end && tactive) transform(hbuf + (par ^ 1) * HBUF, vbuf + (par ^ 1) * (16 * WI_TILES * C));

        // ---- Y = A^T M A per (tile, channel) in fp32; pool; stage the batch.
        // acc[xn][r] is M[xn] of tile 4 (lane / 16) + r, channel kc.
        if (kwave) {
            const int ln = lane_id_here();
            const int kc = 16 * wave + (ln & 15);
            const float bias = bsl[kc];
            lds_half* const os = ost + par * (WI_TILES * a.K);
            FC_LDS uint8_t* const as = ast + par * (WI_TILES * a.K);
            act_dispatch(a.act, [&](auto act) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float s0[4], s1[4];
#pragma unroll
                    for (int nu = 0; nu < 4; ++nu) {
                        const float m1 = acc[4 + nu][r], m2 = acc[8 + nu][r];
                        s0[nu] = acc[nu][r] + m1 + m2;
                        s1[nu] = m1 - m2 - acc[12 + nu][r];
                    }
                    float yv[4];   // window order (0,0), (0,1), (1,0), (1,1)
                    yv[0] = s0[0] + s0[1] + s0[2];
                    yv[1] = s0[1] - s0[2] - s0[3];
                    yv[2] = s1[0] + s1[1] + s1[2];
                    yv[3] = s1[1] - s1[2] - s1[3];
                    const int idx = (4 * (ln >> 4) + r) * a.K + kc;
                    if (POOL == 0 && !AM && decltype(act)::monotone) {
                        // max of a non-decreasing function = the function of the max
                        const float m = __builtin_fmaxf(__builtin_fmaxf(yv[0], yv[1]), __builtin_fmaxf(yv[2], yv[3]));
                        os[idx] = (half_t)act.f(m + bias);
                    } else {
                        half_t v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = (half_t)act.f(yv[e] + bias);
                        if (POOL == 0) {
                            half_t best = v[0];
                            int bi = 0;
#pragma unroll
                            for (int e = 1; e < 4; ++e)
                                if ((float)v[e] > (float)best) {   // strict: the first maximum wins
                                    best = v[e];
                                    bi = e;
                                }
                            os[idx] = best;
                            if (AM) as[idx] = (uint8_t)bi;
                        } else {
                            os[idx] = (half_t)((((float)v[0] + (float)v[1]) + ((float)v[2] + (float)v[3])) * 0.25f);
                        }
                    }
                }
            });
        }
        // this wave's halo requests (batch bt + 2) and stores have landed
        // before the barrier that publishes them
        vm_wait<0>();
        __syncthreads();
    }
    if (b_begin < b_end) store_batch(b_end - 1, (int)((b_end - 1 - b_begin) & 1));
}

// fp64 -> fp16 with one rounding (to nearest even): round to fp32 toward zero
// with a sticky last bit (round-to-odd keeps the information a second
// rounding needs; fp32 has more than 11 + 2 significand bits), then one
// fp32 -> fp16 rounding.
__device__ __forceinline__ half_t f64_to_f16_rne(double x)
{
    float f = (float)x;
    if (__builtin_fabs((double)f) > __builtin_fabs(x))   // one step toward zero (f != 0 here)
        f = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, f) - 1u);
    if ((double)f != x) f = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, f) | 1u);
    return (half_t)f;
}

// U = G g G^T for every (c, k): exact in fp64 (sums of at most nine fp16
// values, halved or quartered), then one rounding to fp16.
__global__ __launch_bounds__(256) void k_wino_weights(const half_t* __restrict__ w, half_t* __restrict__ U, int C, int K)
{
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= (long)C * K) return;
    const int c = (int)(e / K), k = (int)(e - (long)c * K);
    double g[3][3];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int s = 0; s < 3; ++s) g[r][s] = (double)w[((long)(3 * r + s) * C + c) * K + k];
    // Gg (4x3): rows g0, (g0+g1+g2)/2, (g0-g1+g2)/2, g2 of the filter's rows
    double t[4][3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        t[0][s] = g[0][s];
        t[1][s] = 0.5 * (g[0][s] + g[1][s] + g[2][s]);
        t[2][s] = 0.5 * (g[0][s] - g[1][s] + g[2][s]);
        t[3][s] = g[2][s];
    }
#pragma unroll
    for (int xi = 0; xi < 4; ++xi) {
        double u[4];
        u[0] = t[xi][0];
        u[1] = 0.5 * (t[xi][0] + t[xi][1] + t[xi][2]);
        u[2] = 0.5 * (t[xi][0] - t[xi][1] + t[xi][2]);
        u[3] = t[xi][2];
#pragma unroll
        for (int nu = 0; nu < 4; ++nu)
            U[(((long)(4 * xi + nu) * (C / 8) + c / 8) * K + k) * 8 + (c & 7)] = f64_to_f16_rne(u[nu]);
    }
}

template <int C, int POOL, bool AM>
hipError_t launch_wino(const WinoArgs& a, hipStream_t st)
{
    static std::atomic<unsigned long long> lds_set{0};
    hipError_t e = allow_full_lds((const void*)k_conv_pool_wino<C, POOL, AM>, &lds_set);
    if (e != hipSuccess) return e;
    const long grid = min(a.nbatch, (long)device_cu_count());
    hipLaunchKernelGGL((k_conv_pool_wino<C, POOL, AM>), dim3((unsigned)grid), dim3(WI_THREADS),
                       wino_lds_bytes<C>(a.K), st, a);
    return hipGetLastError();
}

template <int C>
hipError_t launch_wino_c(const WinoArgs& a, bool avg, bool am, hipStream_t st)
{
    if (avg) return launch_wino<C, 1, false>(a, st);
    return am ? launch_wino<C, 0, true>(a, st) : launch_wino<C, 0, false>(a, st);
}

}  // namespace

bool wino_fits(int C, int K) { return (C == 32 || C == 64) && K % 16 == 0 && K > 0 && K <= 128; }

hipError_t run_wino_weights(const half_t* w, half_t* U, int C, int K, hipStream_t st)
{
    const long n = (long)C * K;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_wino_weights, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w, U, C, K);
    return hipGetLastError();
}

hipError_t run_conv_pool_wino(const half_t* x, const half_t* U, const half_t* b, int act, bool avg, half_t* y,
                              uint8_t* argmax, int NB, int H, int W, int C, int K, hipStream_t st)
{
    WinoArgs a;
    a.x = x;
    a.U = U;
    a.b = b;
    a.y = y;
    a.argmax = argmax;
    a.NB = NB;
    a.H = H;
    a.W = W;
    a.K = K;
    a.act = act;
    a.TH = H / 2;
    a.TW = W / 2;
    if ((long)NB * a.TH * a.TW == 0) return hipSuccess;
    const int bh = (a.TH + WI_BR - 1) / WI_BR, bw = (a.TW + WI_BC - 1) / WI_BC;
    a.nbatch = (long)NB * bh * bw;
    a.fimg = FastDiv::make((unsigned)(bh * bw));
    a.fbw = FastDiv::make((unsigned)bw);
    if (C == 64) return launch_wino_c<64>(a, avg, argmax != nullptr, st);
    return launch_wino_c<32>(a, avg, argmax != nullptr, st);
}

}  // namespace fc
