// gemm_chain.hip -- fused back-to-back GEMM kernels and the single-GEMM
// (unfused baseline) kernel.
//
//   register-resident chain   : chain_rf.h, instantiated in gemm_rf.hip (N0 <= 128, weights fit in LDS)
//   streamed-weight chain     : chain_stream.h, instantiated in gemm_stream.hip
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
#include "chain_stream.h"
#include "fc_launch.h"

namespace fc {

constexpr int LDS_THREADS = 256;   // 4 waves: 2 (rows) x 2 (columns)
constexpr int LDS_MT = 128;        // rows per block
constexpr int LDS_KC = 64;         // k per staged weight chunk (four MFMA k-steps)
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

// Weight chunks are staged in their natural row-major layout (rows = k) with
// a row stride of (columns + 32) halves: 64 bytes times an odd number modulo
// 256, which keeps the transposing fragment reads conflict-free.
__host__ __device__ constexpr int lds_wcols(int N0P, bool chain)
{
    return chain ? (N0P > LDS_N1C ? N0P : LDS_N1C) : N0P;
}

__host__ __device__ inline size_t lds_lds_bytes(int N0P, bool chain)
{
    size_t b = (size_t)2 * LDS_KC * (lds_wcols(N0P, chain) + 32) * 2;
    if (chain) b += (size_t)LDS_MT * (N0P + 8) * 2;
    b += (size_t)(N0P + (chain ? LDS_N1C : 0)) * 4;   // biases (fp32)
    return b;
}

// Copy a [LDS_KC x ncp] chunk of the row-major matrix G (rows r0.., leading
// dimension ldg) through registers into LDS (16-byte vectors, zero outside
// rows x cols).
template <int NV>
struct WChunk {
    u32x4 v[NV];
};

template <int NV>
__device__ __forceinline__ void wchunk_load(const half_t* __restrict__ G, int rows, int cols, long ldg, int r0,
                                            int ncp, int tid, WChunk<NV>& w)
{
    const int vpr = ncp >> 3;   // 16-byte vectors per row
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int v = tid + i * LDS_THREADS;
        const int r = v / vpr, c = (v - r * vpr) * 8;
        const bool ok = (r0 + r) < rows && c < cols && r < LDS_KC;
        w.v[i] = *reinterpret_cast<const u32x4*>(ok ? G + (long)(r0 + r) * ldg + c : zero_ptr());
    }
}

template <int NV>
__device__ __forceinline__ void wchunk_store(lds_half* T, int ldt, int ncp, int tid, const WChunk<NV>& w)
{
    typedef FC_LDS u32x4 lds_u32x4;
    const int vpr = ncp >> 3;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int v = tid + i * LDS_THREADS;
        const int r = v / vpr, c = (v - r * vpr) * 8;
        if (r < LDS_KC) *reinterpret_cast<lds_u32x4*>(T + r * ldt + c) = w.v[i];
    }
}

// One block: LDS_MT rows.  Waves (wm, wn): rows 64*wm + [0, 64) (two 32-row
// MFMA tiles), GEMM0 columns wn*NT0W*32 + [0, NT0W*32) and, in the chain,
// GEMM1 columns wn*128 + [0, 128) of each 256-column pass.  Single-GEMM mode:
// blockIdx.y selects a block of 64*NT0W output columns.
//   A rows stream from HBM straight into MFMA operand-B registers (two
//   chunks ahead); weight chunks are copied into LDS in their natural layout
//   (double-buffered, one chunk ahead) and read as operand-A fragments with the
//   transposing LDS load, one k-step ahead of the MFMAs that use them.
// KCH: number of 64-wide k chunks of GEMM0 when known at compile time (the
// chunk loop is then fully unrolled, which lets the compiler track exactly
// which loads each MFMA waits for; across a runtime loop's back edge it
// waits for loads that are still two chunks ahead); 0 = runtime loop.
template <int NT0W, bool CHAIN, int KCH>
__global__ __launch_bounds__(LDS_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_lds(LdsArgs a)
{
    constexpr int N0P = 64 * NT0W;
    constexpr int WC = lds_wcols(N0P, CHAIN);
    constexpr int LDW = WC + 32;
    constexpr int WBUF = LDS_KC * LDW;   // halves per weight buffer
    constexpr int LDH = N0P + 8;
    constexpr int NV0 = (LDS_KC * N0P / 8 + LDS_THREADS - 1) / LDS_THREADS;   // W0 vectors per thread
    constexpr int NV1 = LDS_KC * LDS_N1C / 8 / LDS_THREADS;                    // W1 vectors per thread
    static_assert(LDS_MT * (N0P + 8) <= 2 * WBUF, "output tile exceeds the weight buffers");
    static_assert(!CHAIN || LDS_MT * (LDS_N1C + 8) <= 2 * WBUF, "output tile exceeds the weight buffers");
    extern __shared__ __align__(16) char smem[];
    typedef FC_LDS float lds_float;
    typedef FC_LDS const floatx4 lds_float4;
    lds_half* const Wb = (lds_half*)smem;       // two weight buffers, then H
    lds_half* const Hs = Wb + 2 * WBUF;          // CHAIN only: [LDS_MT][LDH]
    lds_float* const b0s = (lds_float*)(Hs + (CHAIN ? LDS_MT * LDH : 0));   // [N0P]
    lds_float* const b1s = b0s + N0P;            // CHAIN only: [LDS_N1C] of the current pass

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, hh = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;
    const long m_blk = (long)blockIdx.x * LDS_MT;
    const int n_base = CHAIN ? 0 : blockIdx.y * N0P;
    const int ncols0 = a.N0 - n_base;        // columns of W0 this block reads
    const half_t* W0b = a.W0 + n_base;

    // A rows, quad-coalesced: lane 4i + m reads rows 4i + j (j = 0..3) of the
    // wave's 64, 16-byte segment m of each 64-byte half h of a 64-wide k
    // chunk, so every quad of lanes reads 64 contiguous bytes (the address
    // unit then takes four lanes per clock instead of one).  The in-quad
    // transpose and the half swap turn raw[h][j] into the MFMA operands
    // op[u][s] (rows 32u + lane%32, k = 64c + 16s + 8(lane/32) + [0,8)).
    const int qi = lane >> 2, qm = lane & 3;
    const half_t* arow[4];
    bool aok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const long r = m_blk + 64 * wm + 4 * qi + j;
        aok[j] = r < a.M;
        arow[j] = a.A + (aok[j] ? r : 0) * (long)a.K0 + 8 * qm;
    }
    auto load_a = [&](int c, half8 (&af)[2][4]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = LDS_KC * c + 32 * h + 8 * qm;
#pragma unroll
            for (int j = 0; j < 4; ++j) af[h][j] = ld16_if(arow[j] + LDS_KC * c + 32 * h, aok[j] && k < a.K0);
        }
    };
    auto to_operand = [&](half8 (&raw)[2][4], half8 (&op)[2][4]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            quad_transpose4(raw[h], lane);
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                half8 x0 = raw[h][2 * sp], x1 = raw[h][2 * sp + 1];
                swap_halves(x0, x1);
                op[0][2 * h + sp] = x0;
                op[1][2 * h + sp] = x1;
            }
        }
    };

    const int nch0 = KCH ? KCH : (a.K0 + LDS_KC - 1) / LDS_KC;
    // A chunks rotate through three register sets by name (chunk c lives in
    // set c % 3); the loop below is unrolled by three so no registers are
    // copied -- a copy would force a wait on the loads still in flight.
    half8 af0[2][4], af1[2][4], af2[2][4];
    WChunk<NV0> w0r;

    if constexpr (kPoison) {
        lds_poison(smem, (int)lds_lds_bytes(N0P, CHAIN), tid, LDS_THREADS);
        __syncthreads();
    }
    // Prologue: W0 chunk 0 into LDS, A chunks 0 and 1 in flight.
    load_a(0, af0);
    if (1 < nch0) load_a(1, af1);
    wchunk_load<NV0>(W0b, a.K0, ncols0, a.N0, 0, N0P, tid, w0r);
    for (int i = tid; i < N0P; i += LDS_THREADS) b0s[i] = (a.b0 && i < ncols0) ? (float)a.b0[n_base + i] : 0.0f;
    wchunk_store<NV0>(Wb, LDW, N0P, tid, w0r);
    __syncthreads();

    floatx16 acc[NT0W][2];
#pragma unroll
    for (int t = 0; t < NT0W; ++t) {
        acc[t][0] = zero16();
        acc[t][1] = zero16();
    }
    const int nb0 = wn * NT0W * 32;

    // ---------------- GEMM0 (transposed: C0^T = W0^T A^T) ----------------
    auto step0 = [&](int c, half8 (&raw)[2][4], half8 (&ld2)[2][4]) {
        const bool more = c + 1 < nch0;
        if constexpr (kPoison) {   // the buffer this step refills was released by the last barrier
            if (more) lds_poison(Wb + ((c + 1) & 1) * WBUF, WBUF * 2, tid, LDS_THREADS);
            __syncthreads();
        }
        if (more) wchunk_load<NV0>(W0b, a.K0, ncols0, a.N0, LDS_KC * (c + 1), N0P, tid, w0r);
        if (c + 2 < nch0) load_a(c + 2, ld2);
        __builtin_amdgcn_sched_barrier(0);   // keep the prefetches issued here
        half8 cur[2][4];
        to_operand(raw, cur);
        const lds_half* wb = Wb + (c & 1) * WBUF;
        half8 wf[2][NT0W];
#pragma unroll
        for (int t = 0; t < NT0W; ++t) wf[0][t] = frag_tr(wb, LDW, 0, nb0 + 32 * t, lane);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) {
#pragma unroll
                for (int t = 0; t < NT0W; ++t) wf[(s + 1) & 1][t] = frag_tr(wb, LDW, 16 * (s + 1), nb0 + 32 * t, lane);
            }
#pragma unroll
            for (int t = 0; t < NT0W; ++t) {
                acc[t][0] = mfma32x32x16(wf[s & 1][t], cur[0][s], acc[t][0]);
                acc[t][1] = mfma32x32x16(wf[s & 1][t], cur[1][s], acc[t][1]);
            }
        }
        if (more) wchunk_store<NV0>(Wb + ((c + 1) & 1) * WBUF, LDW, N0P, tid, w0r);
        __syncthreads();
    };
#pragma unroll
    for (int c = 0; c < nch0; c += 3) {
        step0(c, af0, af2);
        if (c + 1 < nch0) step0(c + 1, af1, af0);
        if (c + 2 < nch0) step0(c + 2, af2, af1);
    }

    typedef FC_LDS half4 lds_half4;
    typedef FC_LDS const half8 lds_half8;
    if (!CHAIN) {
        // Epilogue: bias + act + fp16 into an LDS tile (the weight buffers are
        // free after the last barrier), then line-coalesced row stores.
        constexpr int LDO0 = N0P + 8;
        lds_half* Ot = Wb;
        act_dispatch(a.act, [&](auto act) {
#pragma unroll
            for (int t = 0; t < NT0W; ++t) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = nb0 + 32 * t + 8 * g + 4 * hh;
                    const floatx4 bb = *reinterpret_cast<lds_float4*>(b0s + nl);
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        half4 o;
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[e] = (half_t)act.f(acc[t][u][4 * g + e] + bb[e]);
                        *reinterpret_cast<lds_half4*>(Ot + (64 * wm + 32 * u + lr) * LDO0 + nl) = o;
                    }
                }
            }
        });
        __syncthreads();
        store_tile(Ot, LDO0, LDS_MT, N0P, a.out, a.N0, m_blk, a.M, n_base, a.N0, tid, LDS_THREADS);
        return;
    }

    // Fetch W1 chunk 0 while the epilogue runs.
    WChunk<NV1> w1r;
    wchunk_load<NV1>(a.W1, a.N0, a.N1, a.N1, 0, LDS_N1C, tid, w1r);

    // ------- accumulator-fragment -> LDS iterator: H = fp16(act(C0 + b0)) -------
    act_dispatch(a.act, [&](auto act) {
#pragma unroll
        for (int t = 0; t < NT0W; ++t) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n0 = nb0 + 32 * t + 8 * g + 4 * hh;
                const floatx4 bb = *reinterpret_cast<lds_float4*>(b0s + n0);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    half4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (half_t)act.f(acc[t][u][4 * g + e] + bb[e]);
                    *reinterpret_cast<lds_half4*>(Hs + (64 * wm + 32 * u + lr) * LDH + n0) = o;
                }
            }
        }
    });
    // (the barrier closing the last GEMM0 iteration released both weight
    //  buffers; the barrier below publishes H and W1 chunk 0)

    // ---------------- GEMM1 (transposed: D^T = W1^T H^T) ----------------
    const int nch1 = N0P / LDS_KC;
    int buf = 0;
    for (int n1c = 0; n1c < a.N1; n1c += LDS_N1C) {
        const half_t* W1b = a.W1 + n1c;
        const int ncols1 = a.N1 - n1c;
        if constexpr (kPoison) {   // both weight buffers (the last output tile) and b1s are free
            lds_poison(Wb, 2 * WBUF * 2, tid, LDS_THREADS);
            lds_poison(b1s, LDS_N1C * 4, tid, LDS_THREADS);
            __syncthreads();
        }
        if (n1c > 0) wchunk_load<NV1>(W1b, a.N0, ncols1, a.N1, 0, LDS_N1C, tid, w1r);
        for (int i = tid; i < LDS_N1C; i += LDS_THREADS) b1s[i] = (a.b1 && i < ncols1) ? (float)a.b1[n1c + i] : 0.0f;
        wchunk_store<NV1>(Wb + buf * WBUF, LDW, LDS_N1C, tid, w1r);
        __syncthreads();
        floatx16 acc1[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            acc1[t][0] = zero16();
            acc1[t][1] = zero16();
        }
        for (int c = 0; c < nch1; ++c) {
            const bool more = c + 1 < nch1;
            if constexpr (kPoison) {
                if (more) lds_poison(Wb + (buf ^ 1) * WBUF, WBUF * 2, tid, LDS_THREADS);
                __syncthreads();
            }
            if (more) wchunk_load<NV1>(W1b, a.N0, ncols1, a.N1, LDS_KC * (c + 1), LDS_N1C, tid, w1r);
            __builtin_amdgcn_sched_barrier(0);
            const lds_half* wb = Wb + buf * WBUF;
            const lds_half* hb = Hs + (64 * wm + lr) * LDH + LDS_KC * c + 8 * hh;
            half8 wf[2][4], hf[2][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) wf[0][t] = frag_tr(wb, LDW, 0, wn * 128 + 32 * t, lane);
            hf[0][0] = *reinterpret_cast<lds_half8*>(hb);
            hf[0][1] = *reinterpret_cast<lds_half8*>(hb + 32 * LDH);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s < 3) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        wf[(s + 1) & 1][t] = frag_tr(wb, LDW, 16 * (s + 1), wn * 128 + 32 * t, lane);
                    hf[(s + 1) & 1][0] = *reinterpret_cast<lds_half8*>(hb + 16 * (s + 1));
                    hf[(s + 1) & 1][1] = *reinterpret_cast<lds_half8*>(hb + 32 * LDH + 16 * (s + 1));
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    acc1[t][0] = mfma32x32x16(wf[s & 1][t], hf[s & 1][0], acc1[t][0]);
                    acc1[t][1] = mfma32x32x16(wf[s & 1][t], hf[s & 1][1], acc1[t][1]);
                }
            }
            if (more) wchunk_store<NV1>(Wb + (buf ^ 1) * WBUF, LDW, LDS_N1C, tid, w1r);
            buf ^= 1;
            __syncthreads();
        }
        // Epilogue 1: + b1, fp16 into an LDS tile over the (now free) weight
        // buffers, then line-coalesced row stores.
        constexpr int LDO1 = LDS_N1C + 8;
        lds_half* Ot = Wb;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * 128 + 32 * t + 8 * g + 4 * hh;
                const floatx4 bb = *reinterpret_cast<lds_float4*>(b1s + nl);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    half4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (half_t)(acc1[t][u][4 * g + e] + bb[e]);
                    *reinterpret_cast<lds_half4*>(Ot + (64 * wm + 32 * u + lr) * LDO1 + nl) = o;
                }
            }
        }
        __syncthreads();
        store_tile(Ot, LDO1, LDS_MT, LDS_N1C, a.out, a.N1, m_blk, a.M, n1c, a.N1, tid, LDS_THREADS);
        __syncthreads();
    }
}

// ----------------------------------------------------------------- launchers

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <int NT0W, bool CHAIN, int KCH>
static hipError_t launch_lds_k(const LdsArgs& a, hipStream_t st)
{
    const size_t lds = lds_lds_bytes(64 * NT0W, CHAIN);
    static std::atomic<unsigned long long> lds_set{0};
    hipError_t e = allow_full_lds((const void*)k_gemm_lds<NT0W, CHAIN, KCH>, &lds_set);
    if (e != hipSuccess) return e;
    const unsigned gx = (unsigned)((a.M + LDS_MT - 1) / LDS_MT);
    const unsigned gy = CHAIN ? 1u : (unsigned)((a.N0 + 64 * NT0W - 1) / (64 * NT0W));
    hipLaunchKernelGGL((k_gemm_lds<NT0W, CHAIN, KCH>), dim3(gx, gy), dim3(LDS_THREADS), lds, st, a);
    return hipGetLastError();
}

// Compile-time chunk counts for the k lengths in use (64, 256, 576); others
// run the loop with a runtime trip count.
template <int NT0W, bool CHAIN>
static hipError_t launch_lds_t(const LdsArgs& a, hipStream_t st)
{
    switch ((a.K0 + LDS_KC - 1) / LDS_KC) {
    case 1: return launch_lds_k<NT0W, CHAIN, 1>(a, st);
    case 4: return launch_lds_k<NT0W, CHAIN, 4>(a, st);
    case 9: return launch_lds_k<NT0W, CHAIN, 9>(a, st);
    }
    return launch_lds_k<NT0W, CHAIN, 0>(a, st);
}

// ---------------------------------------------------------------- entry points

hipError_t run_chain_gemm2(const half_t* A, const half_t* W0, const half_t* b0, int act, const half_t* W1,
                           const half_t* b1, half_t* D1, long M, int K0, int N0, int N1, int variant, int waves,
                           int stages, hipStream_t st)
{
    if (M == 0) return hipSuccess;
    if (variant == VARIANT_RF) {
        RfArgs a{};
        a.W0 = W0; a.b0 = b0; a.W1 = W1; a.b1 = b1; a.out = D1;
        a.M = M; a.K0 = K0; a.N0 = N0; a.N1 = N1;
        a.K0p = (K0 + 63) / 64 * 64;
        a.N1p = (N1 + 63) / 64 * 64;
        a.act = act;
        a.ntiles = (M + 31) / 32;
        a.tiles_per_block = 0;
        a.wpb = waves;
        a.stages = stages;
        return run_rf_dense(A, a, 0, st);
    }
    if (variant == VARIANT_STREAM) {
        StreamArgs a;
        a.A = A; a.W0 = W0; a.b0 = b0; a.W1 = W1; a.b1 = b1; a.out = D1;
        a.M = M; a.K0 = K0; a.N0 = N0; a.N1 = N1;
        a.N1p = (N1 + CS_N1C - 1) / CS_N1C * CS_N1C;
        a.ntiles = (M + CS_MT - 1) / CS_MT;
        return run_stream(a, act, st);
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

// N-stage register-resident chain: widths[0] = K0, widths[i + 1] = output
// width of GEMM i (i < nst); every width but K0 and the last <= 128.
void gemmn_args(int nst, const half_t* const* W, const half_t* const* b, const int* act, const int* widths,
                       half_t* D, long M, RfArgs& a)
{
    const int nmid = nst - 2;
    a.W0 = W[0]; a.b0 = b[0]; a.act = act[0];
    a.W1 = W[nst - 1]; a.b1 = b[nst - 1]; a.act1 = act[nst - 1];
    a.out = D;
    a.M = M; a.K0 = widths[0]; a.N0 = widths[1]; a.N1 = widths[nst];
    a.K0p = (a.K0 + 63) / 64 * 64;
    a.N1p = (a.N1 + 63) / 64 * 64;
    for (int i = 0; i < 2; ++i) {
        const bool on = i < nmid;
        a.Wm[i] = on ? W[1 + i] : nullptr;
        a.bm[i] = on ? b[1 + i] : nullptr;
        a.Nm[i] = on ? widths[2 + i] : 0;
        a.Nmp[i] = on ? (widths[2 + i] + 63) / 64 * 64 : 0;
        a.actm[i] = on ? act[1 + i] : 0;
    }
    a.Nin1 = widths[nst - 1];
    a.Nin1p = nmid ? a.Nmp[nmid - 1] : (a.N0 + 31) / 32 * 32;
    a.ntiles = (M + 31) / 32;
    a.tiles_per_block = 0;
}

bool gemmn_fits(int nst, const int* widths)
{
    if (nst < 3 || nst > 4) return false;
    for (int i = 1; i < nst; ++i)
        if (widths[i] > 128) return false;
    const half_t* W[4] = {nullptr, nullptr, nullptr, nullptr};
    const int act[4] = {0, 0, 0, 0};
    RfArgs a{};
    gemmn_args(nst, W, W, act, widths, nullptr, 0, a);
    return rf_lds_bytes_n((a.N0 + 31) / 32 * 32, a.K0p, a.N1p, nst - 2, a.Nmp) <= RF_LDS_LIMIT;
}

hipError_t run_chain_gemmN(const half_t* A, int nst, const half_t* const* W, const half_t* const* b, const int* act,
                           const int* widths, half_t* D, long M, hipStream_t st)
{
    if (M == 0) return hipSuccess;
    RfArgs a{};
    gemmn_args(nst, W, b, act, widths, D, M, a);
    // 8 tile-owning waves per block: the two-stage row ring where it is built
    a.stages = (a.K0p >> 6) == 4 || (a.K0p >> 6) == 9 ? 2 : 0;
    return run_rf_dense(A, a, nst - 2, st);
}

bool stream_fits(int N0, int N1)
{
    return stream_fits_lds(N0, N1);
}

bool rf_fits(int K0, int N0, int N1)
{
    const int N0P = (N0 + 31) / 32 * 32;
    const int K0p = (K0 + 63) / 64 * 64;
    const int N1p = (N1 + 63) / 64 * 64;
    return N0P <= 128 && rf_lds_bytes(N0P, K0p, N1p) <= RF_LDS_LIMIT;
}

}  // namespace fc
