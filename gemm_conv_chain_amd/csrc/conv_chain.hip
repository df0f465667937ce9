// conv_chain.hip -- implicit-GEMM NHWC convolution chains.
//
//   conv3x3 -> bias -> act -> (fp16, registers) -> conv1x1 -> bias :
//       the register-resident chain kernel (chain_rf.h) with an implicit-GEMM
//       row loader (Conv3x3Rows).
//   conv3x3 -> bias -> ReLU -> 2x2/2 max pool (Welder's Conv+ReLU+MaxPool
//   tile graph):  k_conv_w<NTK, EPI_POOL>; the conv output tile never leaves
//   the VGPRs: the pool is a partial reduction of 4 accumulator registers.
//   conv3x3 -> bias -> act, stored (unfused baseline): k_conv_w<NTK, EPI_STORE>.
//   2x2/2 max pool of a stored tensor (unfused baseline): k_maxpool2x2.
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
// half h reads, for chunk c, the 32 consecutive k = 64c + 32h + [0, 32): a
// single (r, s) position and 32 consecutive channels (C % 32 == 0).
struct Conv3x3Rows {
    const half_t* x;
    int H, W, C;
    long M;   // N*H*W
    struct Row {
        int n, p, q;
        bool ok;
    };
    __device__ __forceinline__ Row row(long m) const
    {
        Row r;
        r.ok = m < M;
        const long mm = r.ok ? m : 0;
        const long hw = (long)H * W;
        r.n = (int)(mm / hw);
        const int rem = (int)(mm - (long)r.n * hw);
        r.p = rem / W;
        r.q = rem - r.p * W;
        return r;
    }
    __device__ __forceinline__ void load(const Row& r, int c, int hh, half8 out[4]) const
    {
        const int k0 = 64 * c + 32 * hh;
        const int rs = k0 / C;
        const int coff = k0 - rs * C;
        const int ih = r.p + rs / 3 - 1, iw = r.q + rs % 3 - 1;
        const bool ok = r.ok && rs < 9 && ih >= 0 && ih < H && iw >= 0 && iw < W;
        const half_t* p = x + (((long)r.n * H + (ok ? ih : 0)) * W + (ok ? iw : 0)) * C + coff;
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = ld16_if(p + 8 * q, ok);
    }
};

// ------------------------------------------- weights-resident conv kernel
constexpr int CW_THREADS = 512;
constexpr int CW_WAVES = CW_THREADS / 64;
enum { EPI_STORE = 0, EPI_POOL = 1 };

struct ConvWArgs {
    const half_t* x;   // [NB, H, W, C]
    const half_t* w;   // HWIO [3, 3, C, K]
    const half_t* b;   // [K] or null
    half_t* y;         // STORE: [NB, H, W, K];  POOL: [NB, H/2, W/2, K]
    uint8_t* argmax;   // POOL only, nullable: [NB, H/2, W/2, K]
    int NB, H, W, C, K;
    int Kr;            // 9*C
    int Kp;            // 9*C rounded up to 64
    int act;
    long ntiles;       // 64-row tiles
    long tiles_per_block;
};

inline size_t convw_lds_bytes(int KP, int Kp)
{
    return (size_t)Kp * wtile_ld(KP) * 2 + (size_t)KP * 4 + 16;
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
__global__ __launch_bounds__(CW_THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_conv_w(ConvWArgs a)
{
    constexpr int KP = 32 * NTK;
    extern __shared__ __align__(16) char smem[];
    typedef FC_LDS float lds_float;
    WTile Wn;   // natural layout [Kp][KP] (rows = (r, s, c))
    Wn.p = (lds_half*)smem;
    Wn.ld = wtile_ld(KP);
    Wn.swz = wtile_swz(KP);
    lds_float* bs = (lds_float*)(Wn.p + a.Kp * Wn.ld);
    FC_LDS int* next_tile = (FC_LDS int*)(bs + KP);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, hh = lane >> 5;
    const long t_begin = (long)blockIdx.x * a.tiles_per_block;
    const long t_end = min(t_begin + a.tiles_per_block, a.ntiles);
    const int nch = KCH ? KCH : a.Kp >> 6;
    const int PO = a.H >> 1, QO = a.W >> 1;
    const long nrows = EPI == EPI_POOL ? (long)a.NB * PO * QO * 4 : (long)a.NB * a.H * a.W;

    Conv3x3Rows ld;
    ld.x = a.x; ld.H = a.H; ld.W = a.W; ld.C = a.C; ld.M = (long)a.NB * a.H * a.W;

    // GEMM row -> conv output pixel
    auto make_row = [&](long gr) -> Conv3x3Rows::Row {
        Conv3x3Rows::Row r;
        r.ok = gr < nrows;
        const long g = r.ok ? gr : 0;
        if (EPI == EPI_POOL) {
            const long win = g >> 2;
            const int e = (int)(g & 3);
            const long pq = (long)PO * QO;
            r.n = (int)(win / pq);
            const int rem = (int)(win - (long)r.n * pq);
            const int i = rem / QO, j = rem - (rem / QO) * QO;
            r.p = 2 * i + (e >> 1);
            r.q = 2 * j + (e & 1);
        } else {
            const long hw = (long)a.H * a.W;
            r.n = (int)(g / hw);
            const int rem = (int)(g - (long)r.n * hw);
            r.p = rem / a.W;
            r.q = rem - r.p * a.W;
        }
        return r;
    };

    // Chunks alternate between two register sets by name (chunk c in set
    // c % 2, loop unrolled by two): no loaded register is ever copied.
    long tile = t_begin + wave;
    Conv3x3Rows::Row rows[2];
    half8 xa[2][4], xb[2][4];
    if (tile < t_end) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            rows[u] = make_row(tile * 64 + 32 * u + lr);
            ld.load(rows[u], 0, hh, xa[u]);
        }
    }

    stage_natural<8>(a.w, a.Kr, a.K, a.K, a.Kp, KP, Wn, tid, CW_THREADS);
    for (int i = tid; i < KP; i += CW_THREADS) bs[i] = (a.b && i < a.K) ? (float)a.b[i] : 0.0f;
    if (tid == 0) *next_tile = (int)(t_begin + CW_WAVES);
    __syncthreads();

    // Per-lane parts of the W fragment addresses: column k_out = 32t + lane%32,
    // rows 64c + 32hh + 8q + [0,8) (the k this lane's pixel loads cover).
    const lds_half* wlane[NTK];
#pragma unroll
    for (int t = 0; t < NTK; ++t) wlane[t] = Wn.p + frag_lane_off(Wn, 32 * t, lane) + 32 * hh * Wn.ld;

    while (tile < t_end) {
        floatx16 acc[2][NTK];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < NTK; ++t) acc[u][t] = zero16();

        auto step = [&](int c, const half8 (&cur)[2][4], half8 (&nxt)[2][4]) {
            if (c + 1 < nch) {
                ld.load(rows[0], c + 1, hh, nxt[0]);
                ld.load(rows[1], c + 1, hh, nxt[1]);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch issued here
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int t = 0; t < NTK; ++t) {
                    const half8 wv = frag_tr_at(wlane[t] + (64 * c + 8 * q) * Wn.ld, 4 * Wn.ld);
                    acc[0][t] = mfma32x32x16(cur[0][q], wv, acc[0][t]);
                    acc[1][t] = mfma32x32x16(cur[1][q], wv, acc[1][t]);
                }
            }
        };
#pragma unroll
        for (int c = 0; c < nch; c += 2) {
            step(c, xa, xb);
            if (c + 1 < nch) step(c + 1, xb, xa);
        }

        // Claim the next tile and put its first chunk in flight.
        int nt = 0;
        if (lane == 0) nt = __hip_atomic_fetch_add(next_tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        nt = __shfl(nt, 0);
        const long ntile = nt;
        Conv3x3Rows::Row nrows_[2] = {rows[0], rows[1]};
        if (ntile < t_end) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                nrows_[u] = make_row(ntile * 64 + 32 * u + lr);
                ld.load(nrows_[u], 0, hh, xa[u]);
            }
        }

        // Epilogue.  Lane holds output channel k = 32t + lr; register r of
        // tile (u, t) is GEMM row tile*64 + 32u + 8(r/4) + 4hh + (r%4).
#pragma unroll
        for (int t = 0; t < NTK; ++t) {
            const int k = 32 * t + lr;
            const float bk = bs[k];
            const bool kok = k < a.K;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const long gr0 = tile * 64 + 32 * u + 8 * g + 4 * hh;
                    if (EPI == EPI_POOL) {
                        const long win = gr0 >> 2;
                        if (!kok || gr0 >= nrows) continue;
                        // round each value to fp16 first: the pooled value and
                        // its argmax are decided on the fp16 intermediate
                        float best = (float)(half_t)act_apply(a.act, acc[u][t][4 * g] + bk);
                        int bi = 0;
#pragma unroll
                        for (int e = 1; e < 4; ++e) {
                            const float v = (float)(half_t)act_apply(a.act, acc[u][t][4 * g + e] + bk);
                            if (v > best) { best = v; bi = e; }
                        }
                        const long o = win * a.K + k;   // windows are enumerated like y's pixels
                        a.y[o] = (half_t)best;
                        if (a.argmax) a.argmax[o] = (uint8_t)bi;
                    } else {
                        if (!kok) continue;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const long gr = gr0 + e;
                            if (gr < nrows) a.y[gr * a.K + k] = (half_t)act_apply(a.act, acc[u][t][4 * g + e] + bk);
                        }
                    }
                }
            }
        }
        tile = ntile;
        rows[0] = nrows_[0];
        rows[1] = nrows_[1];
    }
}

template <int NTK, int EPI, int KCH>
static hipError_t launch_convw_k(ConvWArgs a, hipStream_t st)
{
    const size_t lds = convw_lds_bytes(32 * NTK, a.Kp);
    hipError_t e = hipFuncSetAttribute((const void*)k_conv_w<NTK, EPI, KCH>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    long grid = device_cu_count();
    if (grid * CW_WAVES > a.ntiles) grid = (a.ntiles + CW_WAVES - 1) / CW_WAVES;
    if (grid < 1) grid = 1;
    a.tiles_per_block = (a.ntiles + grid - 1) / grid;
    grid = (a.ntiles + a.tiles_per_block - 1) / a.tiles_per_block;
    hipLaunchKernelGGL((k_conv_w<NTK, EPI, KCH>), dim3((unsigned)grid), dim3(CW_THREADS), lds, st, a);
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

hipError_t run_conv_bias_act3x3(const half_t* x, const half_t* w, const half_t* b, int act, half_t* y, int NB,
                                int H, int W, int C, int K, hipStream_t st)
{
    ConvWArgs a;
    a.x = x; a.w = w; a.b = b; a.y = y; a.argmax = nullptr;
    a.NB = NB; a.H = H; a.W = W; a.C = C; a.K = K;
    a.Kr = 9 * C; a.Kp = (9 * C + 63) / 64 * 64; a.act = act;
    const long rows = (long)NB * H * W;
    if (rows == 0) return hipSuccess;
    a.ntiles = (rows + 63) / 64;
    return launch_convw<EPI_STORE>(a, st);
}

hipError_t run_conv_pool3x3(const half_t* x, const half_t* w, const half_t* b, int act, half_t* y,
                            uint8_t* argmax, int NB, int H, int W, int C, int K, hipStream_t st)
{
    ConvWArgs a;
    a.x = x; a.w = w; a.b = b; a.y = y; a.argmax = argmax;
    a.NB = NB; a.H = H; a.W = W; a.C = C; a.K = K;
    a.Kr = 9 * C; a.Kp = (9 * C + 63) / 64 * 64; a.act = act;
    const long rows = (long)NB * (H / 2) * (W / 2) * 4;
    if (rows == 0) return hipSuccess;
    a.ntiles = (rows + 63) / 64;
    return launch_convw<EPI_POOL>(a, st);
}

hipError_t run_chain_conv2_3x3(const half_t* x, const half_t* w0, const half_t* b0, int act, const half_t* w1,
                               const half_t* b1, half_t* y, int NB, int H, int W, int C, int K0, int K1,
                               hipStream_t st)
{
    const long M = (long)NB * H * W;
    if (M == 0) return hipSuccess;
    RfArgs a;
    a.W0 = w0; a.b0 = b0; a.W1 = w1; a.b1 = b1; a.out = y;
    a.M = M; a.K0 = 9 * C; a.N0 = K0; a.N1 = K1;
    a.K0p = (9 * C + 63) / 64 * 64;
    a.N1p = (K1 + 63) / 64 * 64;
    a.act = act;
    a.ntiles = (M + 31) / 32;
    a.tiles_per_block = 0;
    Conv3x3Rows ld;
    ld.x = x; ld.H = H; ld.W = W; ld.C = C; ld.M = M;
    return launch_rf(ld, a, (K0 + 31) / 32, st);
}

// ------------------------------------------------------------ max pool 2x2/2
// One thread: one output pixel x 8 channels (16-byte loads of the 4 inputs).
__global__ __launch_bounds__(256) void k_maxpool2x2(const half_t* __restrict__ v, half_t* __restrict__ y,
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

hipError_t run_maxpool2x2(const half_t* v, half_t* y, uint8_t* am, int NB, int P, int Q, int K, hipStream_t st)
{
    const long total = (long)NB * (P / 2) * (Q / 2) * (K / 8);
    if (total == 0) return hipSuccess;
    long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_maxpool2x2, dim3((unsigned)blocks), dim3(256), 0, st, v, y, am, NB, P, Q, K);
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
