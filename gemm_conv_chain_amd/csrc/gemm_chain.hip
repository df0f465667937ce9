// gemm_chain.hip -- fused back-to-back GEMM kernels and the single-GEMM
// (unfused baseline) kernel.
//
//   register-resident chain   : chain_rf.h  (N0 <= 128, weights fit in LDS)
//   LDS-resident chain        : k_gemm_lds<NT0W, true>   (N0 <= 256)
//   gemm + bias + act         : k_gemm_lds<NT0W, false>  (any N, 256-wide column blocks)
//
// The LDS-resident chain is BOLT's shared-memory-resident fusion (BOLT notes,
// "Persistent kernel (GEMM/Conv) fusion", Figure 7): when GEMM0's N is large,
// a block splits GEMM0's columns over several waves, so each wave holds only
// part of a row of the intermediate; the accumulator tile is therefore written
// to shared memory (here: LDS) by an accumulator-fragment iterator, and every
// wave of GEMM1 streams operand fragments of the whole row back from it.
#include "chain_rf.h"
#include "fc_launch.h"

namespace fc {

constexpr int LDS_THREADS = 256;   // 4 waves: 2 (rows) x 2 (columns)
constexpr int LDS_MT = 128;        // rows per block
constexpr int LDS_KC = 32;         // k per staged chunk (two MFMA k-steps)
constexpr int LDS_LDW = LDS_KC + 8;  // padded LDS row of a staged weight chunk
constexpr int LDS_N1C = 256;       // GEMM1 columns per pass (2 waves x 4 tiles x 32)

struct LdsArgs {
    const half_t* A;    // [M x K0]
    const half_t* W0;   // [K0 x N0]
    const half_t* b0;
    const half_t* W1;   // [N0 x N1]          (chain only)
    const half_t* b1;   //                    (chain only)
    half_t* out;        // [M x N1] chain, [M x N0] single GEMM
    long M;
    int K0, N0, N1;
    int act;
};

inline size_t lds_lds_bytes(int N0P, bool chain)
{
    const int wrows = chain ? (N0P > LDS_N1C ? N0P : LDS_N1C) : N0P;
    size_t b = (size_t)2 * wrows * LDS_LDW * 2;
    if (chain) b += (size_t)LDS_MT * (N0P + 8) * 2;
    return b;
}

// One block: LDS_MT rows.  Waves (wm, wn): rows 64*wm.., GEMM0 columns
// [wn*NT0W*32, +NT0W*32) and, in the chain, GEMM1 columns [wn*128, +128) of
// each 256-column pass.  Single-GEMM mode: blockIdx.y selects a block of
// 64*NT0W output columns.
template <int NT0W, bool CHAIN>
__global__ __launch_bounds__(LDS_THREADS) void k_gemm_lds(LdsArgs a)
{
    constexpr int N0P = 64 * NT0W;
    constexpr int WROWS = CHAIN ? (N0P > LDS_N1C ? N0P : LDS_N1C) : N0P;
    extern __shared__ __align__(16) char smem[];
    half_t* Wbuf0 = reinterpret_cast<half_t*>(smem);
    half_t* Wbuf1 = Wbuf0 + WROWS * LDS_LDW;
    half_t* Hs = Wbuf1 + WROWS * LDS_LDW;   // CHAIN only: [LDS_MT][N0P + 8]
    constexpr int LDH = N0P + 8;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, hh = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;
    const long m_blk = (long)blockIdx.x * LDS_MT;
    const int n_base = CHAIN ? 0 : blockIdx.y * N0P;
    const int ncols0 = a.N0 - n_base;        // columns of W0 this block reads
    const half_t* W0b = a.W0 + n_base;

    // Rows of A this lane feeds as operand B (two 32-row tiles).
    long mrow[2];
    bool mok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        mrow[u] = m_blk + 64 * wm + 32 * u + lr;
        mok[u] = mrow[u] < a.M;
    }
    auto load_a = [&](int c, half8 (&af)[2][2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int k = LDS_KC * c + 16 * hh + 8 * s;
                af[u][s] = ld16_if(a.A + (mok[u] ? mrow[u] : 0) * (long)a.K0 + k, mok[u] && k < a.K0);
            }
        }
    };

    const int nch0 = (a.K0 + LDS_KC - 1) / LDS_KC;
    const int nblk0 = (LDS_KC / 4) * (N0P / 8);   // <= LDS_THREADS
    TBlock wreg;
    half8 af[2][2];

    // Prologue: chunk 0 of A in registers, chunk 0 of W0^T in LDS.
    load_a(0, af);
    if (tid < nblk0) {
        tblock_load(W0b, a.K0, ncols0, a.N0, 0, N0P, tid, wreg);
        tblock_store<false>(Wbuf0, LDS_LDW, N0P, tid, wreg);
    }
    __syncthreads();

    floatx16 acc[NT0W][2];
#pragma unroll
    for (int t = 0; t < NT0W; ++t) {
        acc[t][0] = zero16();
        acc[t][1] = zero16();
    }

    // ---------------- GEMM0 (transposed: C0^T = W0^T A^T) ----------------
    for (int c = 0; c < nch0; ++c) {
        const bool more = c + 1 < nch0;
        half8 an[2][2];
        if (more) {
            load_a(c + 1, an);
            if (tid < nblk0) tblock_load(W0b, a.K0, ncols0, a.N0, LDS_KC * (c + 1), N0P, tid, wreg);
        }
        const half_t* wb = ((c & 1) ? Wbuf1 : Wbuf0) + (wn * NT0W * 32 + lr) * LDS_LDW + 16 * hh;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int t = 0; t < NT0W; ++t) {
                const half8 w = *reinterpret_cast<const half8*>(wb + 32 * t * LDS_LDW + 8 * s);
                acc[t][0] = mfma32x32x16(w, af[0][s], acc[t][0]);
                acc[t][1] = mfma32x32x16(w, af[1][s], acc[t][1]);
            }
        }
        if (more) {
            if (tid < nblk0) tblock_store<false>((c & 1) ? Wbuf0 : Wbuf1, LDS_LDW, N0P, tid, wreg);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                af[u][0] = an[u][0];
                af[u][1] = an[u][1];
            }
        }
        __syncthreads();
    }

    if (!CHAIN) {
        // Epilogue: bias + act + fp16, 8-byte stores of 4 consecutive columns.
#pragma unroll
        for (int t = 0; t < NT0W; ++t) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * NT0W * 32 + 32 * t + 8 * g + 4 * hh;
                const int n = n_base + nl;
                if (n >= a.N0) continue;
                float bb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) bb[e] = a.b0 ? (float)a.b0[n + e] : 0.0f;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (!mok[u]) continue;
                    half4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (half_t)act_apply(a.act, acc[t][u][4 * g + e] + bb[e]);
                    *reinterpret_cast<half4*>(a.out + mrow[u] * (long)a.N0 + n) = o;
                }
            }
        }
        return;
    }

    // ------- accumulator-fragment -> LDS iterator: H = fp16(act(C0 + b0)) -------
#pragma unroll
    for (int t = 0; t < NT0W; ++t) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n0 = wn * NT0W * 32 + 32 * t + 8 * g + 4 * hh;
            float bb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) bb[e] = (a.b0 && n0 + e < a.N0) ? (float)a.b0[n0 + e] : 0.0f;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                half4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (half_t)act_apply(a.act, acc[t][u][4 * g + e] + bb[e]);
                *reinterpret_cast<half4*>(Hs + (64 * wm + 32 * u + lr) * LDH + n0) = o;
            }
        }
    }
    // (the barrier at the end of the last GEMM0 iteration already released
    //  both weight buffers; the one below publishes H)

    // ---------------- GEMM1 (transposed: D^T = W1^T H^T) ----------------
    const int nch1 = N0P / LDS_KC;
    const int nblk1 = (LDS_KC / 4) * (LDS_N1C / 8);   // == LDS_THREADS
    for (int n1c = 0; n1c < a.N1; n1c += LDS_N1C) {
        const half_t* W1b = a.W1 + n1c;
        const int ncols1 = a.N1 - n1c;
        if (tid < nblk1) {
            tblock_load(W1b, a.N0, ncols1, a.N1, 0, LDS_N1C, tid, wreg);
            tblock_store<false>(Wbuf0, LDS_LDW, LDS_N1C, tid, wreg);
        }
        __syncthreads();
        floatx16 acc1[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            acc1[t][0] = zero16();
            acc1[t][1] = zero16();
        }
        for (int c = 0; c < nch1; ++c) {
            const bool more = c + 1 < nch1;
            if (more && tid < nblk1) tblock_load(W1b, a.N0, ncols1, a.N1, LDS_KC * (c + 1), LDS_N1C, tid, wreg);
            const half_t* wb = ((c & 1) ? Wbuf1 : Wbuf0) + (wn * 128 + lr) * LDS_LDW + 16 * hh;
            const half_t* hb = Hs + (64 * wm + lr) * LDH + LDS_KC * c + 16 * hh;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const half8 h0 = *reinterpret_cast<const half8*>(hb + 8 * s);
                const half8 h1 = *reinterpret_cast<const half8*>(hb + 32 * LDH + 8 * s);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const half8 w = *reinterpret_cast<const half8*>(wb + 32 * t * LDS_LDW + 8 * s);
                    acc1[t][0] = mfma32x32x16(w, h0, acc1[t][0]);
                    acc1[t][1] = mfma32x32x16(w, h1, acc1[t][1]);
                }
            }
            if (more && tid < nblk1) tblock_store<false>((c & 1) ? Wbuf0 : Wbuf1, LDS_LDW, LDS_N1C, tid, wreg);
            __syncthreads();
        }
        // Epilogue 1: + b1, fp16, 8-byte stores.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n1 = n1c + wn * 128 + 32 * t + 8 * g + 4 * hh;
                if (n1 >= a.N1) continue;
                float bb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) bb[e] = a.b1 ? (float)a.b1[n1 + e] : 0.0f;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (!mok[u]) continue;
                    half4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (half_t)(acc1[t][u][4 * g + e] + bb[e]);
                    *reinterpret_cast<half4*>(a.out + mrow[u] * (long)a.N1 + n1) = o;
                }
            }
        }
    }
}

// ----------------------------------------------------------------- launchers

static int g_num_cu = 0;

int device_cu_count()
{
    if (g_num_cu == 0) {
        int dev = 0;
        hipDeviceProp_t p;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess)
            g_num_cu = p.multiProcessorCount;
        if (g_num_cu <= 0) g_num_cu = 256;
    }
    return g_num_cu;
}

template <int NT0W, bool CHAIN>
static hipError_t launch_lds_t(const LdsArgs& a, hipStream_t st)
{
    const size_t lds = lds_lds_bytes(64 * NT0W, CHAIN);
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_lds<NT0W, CHAIN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const unsigned gx = (unsigned)((a.M + LDS_MT - 1) / LDS_MT);
    const unsigned gy = CHAIN ? 1u : (unsigned)((a.N0 + 64 * NT0W - 1) / (64 * NT0W));
    hipLaunchKernelGGL((k_gemm_lds<NT0W, CHAIN>), dim3(gx, gy), dim3(LDS_THREADS), lds, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- entry points

hipError_t run_chain_gemm2(const half_t* A, const half_t* W0, const half_t* b0, int act, const half_t* W1,
                           const half_t* b1, half_t* D1, long M, int K0, int N0, int N1, int variant,
                           hipStream_t st)
{
    if (M == 0) return hipSuccess;
    if (variant == VARIANT_RF) {
        RfArgs a;
        a.W0 = W0; a.b0 = b0; a.W1 = W1; a.b1 = b1; a.out = D1;
        a.M = M; a.K0 = K0; a.N0 = N0; a.N1 = N1;
        a.K0p = (K0 + 63) / 64 * 64;
        a.N1p = (N1 + 63) / 64 * 64;
        a.act = act;
        a.ntiles = (M + 31) / 32;
        a.tiles_per_block = 0;
        DenseRows ld;
        ld.A = A; ld.M = M; ld.K = K0;
        return launch_rf(ld, a, (N0 + 31) / 32, st);
    }
    LdsArgs a;
    a.A = A; a.W0 = W0; a.b0 = b0; a.W1 = W1; a.b1 = b1; a.out = D1;
    a.M = M; a.K0 = K0; a.N0 = N0; a.N1 = N1; a.act = act;
    switch ((N0 + 63) / 64) {
    case 1: return launch_lds_t<1, true>(a, st);
    case 2: return launch_lds_t<2, true>(a, st);
    case 3: return launch_lds_t<3, true>(a, st);
    case 4: return launch_lds_t<4, true>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t run_gemm_bias_act(const half_t* A, const half_t* W, const half_t* b, int act, half_t* C, long M,
                             int K, int N, hipStream_t st)
{
    if (M == 0 || N == 0) return hipSuccess;
    LdsArgs a;
    a.A = A; a.W0 = W; a.b0 = b; a.W1 = nullptr; a.b1 = nullptr; a.out = C;
    a.M = M; a.K0 = K; a.N0 = N; a.N1 = 0; a.act = act;
    if (N <= 64) return launch_lds_t<1, false>(a, st);
    if (N <= 128) return launch_lds_t<2, false>(a, st);
    return launch_lds_t<4, false>(a, st);
}

bool rf_fits(int K0, int N0, int N1)
{
    const int N0P = (N0 + 31) / 32 * 32;
    const int K0p = (K0 + 63) / 64 * 64;
    const int N1p = (N1 + 63) / 64 * 64;
    return N0P <= 128 && rf_lds_bytes(N0P, K0p, N1p) <= RF_LDS_LIMIT;
}

}  // namespace fc
