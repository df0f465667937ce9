// chain_rf.h -- register-resident two-stage chain kernel (GEMM -> GEMM).
//
// Computes  OUT = act(X * W0 + b0) * W1 + b1  for a row-producing operand X
// that a Loader delivers (dense GEMM rows, or implicit-GEMM conv pixels), with
// the intermediate kept in VGPRs.  This is BOLT's persistent kernel fusion
// under the threadblock-residence rule (BOLT notes, "Persistent kernel
// (GEMM/Conv) fusion": the block computing a tile of the first GEMM owns the
// FULL N of that GEMM, so the second GEMM reads its input from on-chip storage
// and never from global memory), in its register-file-resident form.
//
// Mapping to CDNA4 (one wave = 32 output rows, all N0 and all N1 columns):
//   * Both GEMMs are computed transposed, C0^T = W0^T X^T and D^T = W1^T H^T,
//     with the weights as MFMA operand A and the rows as operand B.  Operand B
//     wants, per lane, 8 consecutive k of ONE row: exactly a 16-byte global load
//     of X, so X streams from HBM straight into MFMA registers.
//   * The GEMM0 accumulator gives lane (m, h) the values of its row m at
//     n0 = 32t + 8(r/4) + 4h + (r%4).  Packed to fp16 after bias+act, 8 of them
//     form the operand-B register of GEMM1 for k-step s = 2t + r/8 -- no data
//     leaves the lane.  GEMM1's operand A (W1^T) is staged in LDS with the
//     matching permutation of its k index (PERM16 in the transposed staging).
//   * W0^T, W1^T and the biases live in LDS for the whole kernel; the grid is
//     persistent (about one block per CU), each block owning a contiguous range
//     of 32-row tiles that its waves take in turn.
//   * X is loaded in 64-wide k chunks: lane half h reads 64 contiguous bytes
//     (k = 64c + 32h + 8q + j, q = 0..3), the lane pair covers 128 contiguous
//     bytes of the row.  The next chunk (and the next tile's first chunk) is in
//     flight while the current one is multiplied.
#pragma once
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {

constexpr int RF_THREADS = 512;
constexpr int RF_WAVES = RF_THREADS / 64;

struct RfArgs {
    const half_t* W0;   // [K0 x N0] row-major
    const half_t* b0;   // [N0] or null
    const half_t* W1;   // [N0 x N1] row-major
    const half_t* b1;   // [N1] or null
    half_t* out;        // [M x N1] row-major
    long M;
    int K0, N0, N1;
    int K0p;            // K0 rounded up to 64
    int N1p;            // N1 rounded up to 64
    int act;
    long ntiles;        // ceil(M / 32)
    long tiles_per_block;
};

// LDS bytes used by the RF kernel for a given padded problem.
inline size_t rf_lds_bytes(int N0P, int K0p, int N1p)
{
    return (size_t)N0P * (K0p + 8) * 2 + (size_t)N1p * (N0P + 8) * 2 + (size_t)(N0P + N1p) * 4;
}

template <int NT0, class Loader>
__global__ __launch_bounds__(RF_THREADS) void k_chain_rf(Loader ld, RfArgs a)
{
    constexpr int N0P = 32 * NT0;
    extern __shared__ __align__(16) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, hh = lane >> 5;
    const int ldw0 = a.K0p + 8, ldw1 = N0P + 8;
    half_t* W0t = reinterpret_cast<half_t*>(smem);
    half_t* W1t = W0t + N0P * ldw0;
    float* b0s = reinterpret_cast<float*>(W1t + a.N1p * ldw1);
    float* b1s = b0s + N0P;

    const long t_begin = (long)blockIdx.x * a.tiles_per_block;
    const long t_end = min(t_begin + a.tiles_per_block, a.ntiles);
    const int nch = a.K0p >> 6;

    // Start the row stream before staging the weights so HBM is busy at once.
    long tile = t_begin + wave;
    half8 cur[4];
    typename Loader::Row row;
    if (tile < t_end) {
        row = ld.row(tile * 32 + lr);
        ld.load(row, 0, hh, cur);
    }

    stage_transposed<false>(a.W0, a.K0, a.N0, a.N0, 0, a.K0p, N0P, W0t, ldw0, tid, RF_THREADS);
    stage_transposed<true>(a.W1, a.N0, a.N1, a.N1, 0, N0P, a.N1p, W1t, ldw1, tid, RF_THREADS);
    for (int i = tid; i < N0P + a.N1p; i += RF_THREADS) {
        float v = 0.0f;
        if (i < N0P) {
            if (a.b0 && i < a.N0) v = (float)a.b0[i];
            b0s[i] = v;
        } else {
            const int j = i - N0P;
            if (a.b1 && j < a.N1) v = (float)a.b1[j];
            b1s[j] = v;
        }
    }
    __syncthreads();

    for (; tile < t_end; tile += RF_WAVES) {
        const long m = tile * 32 + lr;
        floatx16 acc0[NT0];
#pragma unroll
        for (int t = 0; t < NT0; ++t) acc0[t] = zero16();

        for (int c = 0; c < nch; ++c) {
            half8 nxt[4];
            const bool more = c + 1 < nch;
            if (more) ld.load(row, c + 1, hh, nxt);
            const half_t* wbase = W0t + lr * ldw0 + 64 * c + 32 * hh;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int t = 0; t < NT0; ++t) {
                    const half8 w = *reinterpret_cast<const half8*>(wbase + 32 * t * ldw0 + 8 * q);
                    acc0[t] = mfma32x32x16(w, cur[q], acc0[t]);
                }
            }
            if (more) {
#pragma unroll
                for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
            }
        }

        // Put the next tile's first chunk in flight before the epilogues.
        const long ntile = tile + RF_WAVES;
        typename Loader::Row nrow = row;
        if (ntile < t_end) {
            nrow = ld.row(ntile * 32 + lr);
            ld.load(nrow, 0, hh, cur);
        }

        // Epilogue 0 in registers: bias (broadcast along rows), activation,
        // one rounding to fp16.  hf[s] is GEMM1's operand B for k-step s.
        half8 hf[2 * NT0];
#pragma unroll
        for (int t = 0; t < NT0; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n0 = 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                const float v = act_apply(a.act, acc0[t][r] + b0s[n0]);
                hf[2 * t + (r >> 3)][r & 7] = (half_t)v;
            }
        }

        // GEMM1 over N1 in chunks of 64 columns (two 32x32 tiles).
        for (int n1c = 0; n1c < a.N1p; n1c += 64) {
            floatx16 acc1[2];
            acc1[0] = zero16();
            acc1[1] = zero16();
            const half_t* w1base = W1t + (n1c + lr) * ldw1 + 8 * hh;
#pragma unroll
            for (int s = 0; s < 2 * NT0; ++s) {
#pragma unroll
                for (int t1 = 0; t1 < 2; ++t1) {
                    const half8 w = *reinterpret_cast<const half8*>(w1base + 32 * t1 * ldw1 + 16 * s);
                    acc1[t1] = mfma32x32x16(w, hf[s], acc1[t1]);
                }
            }
            if (m < a.M) {
                half_t* orow = a.out + m * (long)a.N1;
#pragma unroll
                for (int t1 = 0; t1 < 2; ++t1) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n1 = n1c + 32 * t1 + 8 * g + 4 * hh;
                        if (n1 < a.N1) {
                            half4 o;
#pragma unroll
                            for (int e = 0; e < 4; ++e) o[e] = (half_t)(acc1[t1][4 * g + e] + b1s[n1 + e]);
                            *reinterpret_cast<half4*>(orow + n1) = o;
                        }
                    }
                }
            }
        }
        row = nrow;
    }
}

// Dense GEMM rows: X = A [M x K] row-major.
struct DenseRows {
    const half_t* A;
    long M;
    int K;
    struct Row {
        const half_t* p;
        bool ok;
    };
    __device__ __forceinline__ Row row(long m) const
    {
        Row r;
        r.ok = m < M;
        r.p = A + (r.ok ? m : 0) * (long)K;
        return r;
    }
    __device__ __forceinline__ void load(const Row& r, int c, int hh, half8 out[4]) const
    {
        const int k0 = 64 * c + 32 * hh;
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = ld16_if(r.p + k0 + 8 * q, r.ok && (k0 + 8 * q) < K);
    }
};

// ----------------------------------------------------------------- launch

template <int NT0, class Loader>
static hipError_t launch_rf_t(const Loader& ld, RfArgs a, hipStream_t st)
{
    const size_t lds = rf_lds_bytes(32 * NT0, a.K0p, a.N1p);
    hipError_t e = hipFuncSetAttribute((const void*)k_chain_rf<NT0, Loader>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const long per_block_min = RF_WAVES;  // at least one tile per wave
    long grid = device_cu_count();
    if (grid * per_block_min > a.ntiles) grid = (a.ntiles + per_block_min - 1) / per_block_min;
    if (grid < 1) grid = 1;
    a.tiles_per_block = (a.ntiles + grid - 1) / grid;
    grid = (a.ntiles + a.tiles_per_block - 1) / a.tiles_per_block;
    hipLaunchKernelGGL((k_chain_rf<NT0, Loader>), dim3((unsigned)grid), dim3(RF_THREADS), lds, st, ld, a);
    return hipGetLastError();
}

template <class Loader>
inline hipError_t launch_rf(const Loader& ld, const RfArgs& a, int nt0, hipStream_t st)
{
    switch (nt0) {
    case 1: return launch_rf_t<1>(ld, a, st);
    case 2: return launch_rf_t<2>(ld, a, st);
    case 3: return launch_rf_t<3>(ld, a, st);
    case 4: return launch_rf_t<4>(ld, a, st);
    }
    return hipErrorInvalidValue;
}


}  // namespace fc
