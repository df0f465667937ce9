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
//     leaves the lane.  GEMM1's operand A (W1^T) fragments are read with the
//     matching permutation of the k rows.
//   * W0, W1 (natural row-major layout, read as transposed fragments with
//     ds_read_b64_tr_b16) and the biases live in LDS for the whole kernel; the grid is
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
constexpr int RF_WB = 16;   // weight vectors (16 bytes) per thread staged ahead of the row stream

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
    int stages;         // row chunks in flight + 1 (ring depth): 0 = the default (4), or 2
    int wpb;            // waves per block that own row tiles (1..RF_WAVES; 0 = all): the block
                        // covers 32 * wpb rows per round, the other waves only stage the weights
    // N-stage chains only (kernel template NMID > 0): NMID middle GEMMs run
    // between the first and the last, each on the previous one's fp16 output
    // kept in the lane.  Middle i maps width Nin_i (N0, then Nm[0]) to Nm[i].
    const half_t* Wm[2];   // [Nin_i x Nm[i]] row-major
    const half_t* bm[2];   // [Nm[i]] or null
    int Nm[2];             // <= 128
    int Nmp[2];            // Nm rounded up to 64
    int actm[2];
    int act1;              // activation after the last GEMM
    int Nin1, Nin1p;       // input width of the last GEMM, and its padded row count in LDS
};

// Fills the N-stage fields of RfArgs (host): widths[0] = K0 of the first
// GEMM, widths[i + 1] = output width of GEMM i (i < nst).
void gemmn_args(int nst, const half_t* const* W, const half_t* const* b, const int* act, const int* widths,
                half_t* D, long M, RfArgs& a);

// Per-wave output staging tile: 32 rows x 64 columns (+8 halves of padding).
constexpr int RF_OLD = 64 + 8;
constexpr size_t RF_OSTAGE_BYTES = (size_t)RF_WAVES * 32 * RF_OLD * 2;

// LDS bytes used by the RF kernel for a given padded problem: W0 and W1 in
// their natural layout (rows = k), the biases, the per-wave output tiles.
__host__ __device__ inline size_t rf_lds_bytes(int N0P, int K0p, int N1p)
{
    return (size_t)K0p * wtile_ld(N0P) * 2 + (size_t)N0P * wtile_ld(N1p) * 2 + (size_t)(N0P + N1p) * 4 +
           RF_OSTAGE_BYTES;
}

// ... and with nmid middle GEMMs (padded widths Nmp[0..nmid-1]): their weight
// tiles sit between W0 and the last GEMM's, their biases after b1.
__host__ __device__ inline size_t rf_lds_bytes_n(int N0P, int K0p, int N1p, int nmid, const int* Nmp)
{
    size_t b = (size_t)K0p * wtile_ld(N0P) * 2;
    int nin = N0P;
    for (int i = 0; i < nmid; ++i) {
        b += (size_t)nin * wtile_ld(Nmp[i]) * 2 + (size_t)Nmp[i] * 4;
        nin = Nmp[i];
    }
    return b + (size_t)nin * wtile_ld(N1p) * 2 + (size_t)(N0P + N1p) * 4 + RF_OSTAGE_BYTES;
}

// KCH: compile-time number of 64-wide k chunks (0 = runtime loop); with a
// known count the chunk loop unrolls fully and every load is waited for
// exactly where its data is used.
// One block per CU (its LDS holds both weight matrices), 8 waves: 2 waves per
// SIMD.  Saying so lets the scheduler spend registers on loads in flight
// instead of shrinking them for an occupancy the LDS use rules out.
// NMID: middle GEMMs of an N-stage chain (0 for two GEMMs).  RD: ring depth
// (pipeline stages) of the row chunks, 0 = the default.
template <int NT0, int KCH, class Loader, int NMID = 0, int RD = 0>
__global__ __launch_bounds__(RF_THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_chain_rf(Loader ld, RfArgs a)
{
    constexpr int N0P = 32 * NT0;
    constexpr int HF = NMID ? 8 : 2 * NT0;   // k-steps of the hand-off registers (8 = 128 columns)
    extern __shared__ __align__(16) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, hh = lane >> 5;
    typedef FC_LDS float lds_float;
    typedef FC_LDS half4 lds_half4;
    // natural layouts: W0n [K0p][N0P], Wmn[i] [Nin_i][Nmp[i]], W1n [Nin1p][N1p]
    const int nin1p = NMID ? a.Nin1p : N0P;
    WTile W0n, W1n, Wmn[NMID > 0 ? NMID : 1];
    W0n.p = (lds_half*)smem;
    W0n.ld = wtile_ld(N0P);
    W0n.swz = wtile_swz(N0P);
    lds_half* wnext = W0n.p + a.K0p * W0n.ld;
    if constexpr (NMID > 0) {
#pragma unroll
        for (int i = 0; i < NMID; ++i) {
            Wmn[i].p = wnext;
            Wmn[i].ld = wtile_ld(a.Nmp[i]);
            Wmn[i].swz = wtile_swz(a.Nmp[i]);
            wnext += (i == 0 ? N0P : a.Nmp[i - 1]) * Wmn[i].ld;
        }
    }
    W1n.p = wnext;
    W1n.ld = wtile_ld(a.N1p);
    W1n.swz = wtile_swz(a.N1p);
    lds_float* b0s = (lds_float*)(W1n.p + nin1p * W1n.ld);
    lds_float* b1s = b0s + N0P;
    lds_float* bms = b1s + a.N1p;   // middle biases (NMID > 0), Nmp[0] then Nmp[1]
    lds_half* Ost = (lds_half*)(bms + (NMID > 0 ? a.Nmp[0] : 0) + (NMID > 1 ? a.Nmp[1] : 0)) + wave * 32 * RF_OLD;

    // Block ranges renumbered so that each XCD works on one contiguous stretch
    // of rows (the conv loader's 3x3 halo rows are then shared within one L2).
    const long t_begin = (long)xcd_block(blockIdx.x, gridDim.x) * a.tiles_per_block;
    const long t_end = min(t_begin + a.tiles_per_block, a.ntiles);
    const int nch = KCH ? KCH : a.K0p >> 6;

    // Row chunks are held in a ring of R register sets.  With a compile-time
    // chunk count (KCH > 0) the chunk loop is fully unrolled and chunk c lives
    // in set c % R, so the ring rotates by name: PD = R - 1 chunks are always
    // in flight ahead of the one being multiplied.  Loaded-HBM latency is far
    // longer than the MFMA work of one chunk, so the depth, not the MFMA rate,
    // sets the speed here.  (Requesting all four chunks of a K0 = 256 tile in
    // the prologue is slower: the extra requests delay the weight loads every
    // wave waits for.)  KCH == 0 (runtime chunk count) falls back to a two-set
    // ring.
    constexpr int R = (KCH > 0 && RD > 0) ? (RD < KCH ? RD : KCH) : (KCH >= 4 ? 4 : (KCH > 0 ? KCH : 2));
    constexpr int PD = R - 1;
    const int wpb = a.wpb > 0 ? a.wpb : RF_WAVES;
    long tile = wave < wpb ? t_begin + wave : t_end;
    half8 xr[R][4];
    typename Loader::Row row;
    // Prologue.  Every wave first issues its share of the weight (and bias)
    // loads, then the row loads of its first tile, and only then writes the
    // weights to LDS: the wait before those LDS writes covers the weight loads
    // alone (a wave's wait counter retires loads in issue order), and the
    // weight requests, which hit L2, are not queued behind the row stream.
    // Weights beyond one batch of RF_WB vectors per thread are staged after
    // the barrier-free first batch (their loads then wait behind the rows).
    if constexpr (kPoison) {
        lds_poison(smem, (int)(NMID ? rf_lds_bytes_n(N0P, a.K0p, a.N1p, NMID, a.Nmp) : rf_lds_bytes(N0P, a.K0p, a.N1p)),
                   tid, RF_THREADS);
        __syncthreads();
    }
    WStage2<RF_WB> ws;
    ws.G0 = a.W0; ws.rows0 = a.K0; ws.cols0 = a.N0; ws.ldg0 = a.N0; ws.nr0 = a.K0p; ws.ncp0 = N0P; ws.T0 = W0n;
    ws.G1 = a.W1; ws.rows1 = NMID ? a.Nin1 : a.N0; ws.cols1 = a.N1; ws.ldg1 = a.N1; ws.nr1 = nin1p; ws.ncp1 = a.N1p;
    ws.T1 = W1n;
    ws.init();
    ws.load(tid, RF_THREADS);
    // this thread's bias value (raw fp16; converted only after the row loads
    // are issued, so nothing waits on it early)
    const half_t* bp = zero_ptr();
    if (tid < N0P) {
        if (a.b0 && tid < a.N0) bp = a.b0 + tid;
    } else if (tid < N0P + a.N1p && a.b1 && tid - N0P < a.N1) {
        bp = a.b1 + (tid - N0P);
    }
    const half_t bias = *bp;
    if (tile < t_end) {
        row = ld.row(tile * 32 + lr);
#pragma unroll
        for (int p = 0; p < PD; ++p)
            if (p < nch) ld.template load<KCH>(row, p, hh, xr[p]);
    }
    __builtin_amdgcn_sched_barrier(0);
    ws.store(tid, RF_THREADS);
    if (tid < N0P + a.N1p) b0s[tid] = (float)bias;   // b1s follows b0s
    for (int i = tid + RF_THREADS; i < N0P + a.N1p; i += RF_THREADS) {
        float v = 0.0f;
        if (i < N0P) {
            if (a.b0 && i < a.N0) v = (float)a.b0[i];
        } else if (a.b1 && i - N0P < a.N1) {
            v = (float)a.b1[i - N0P];
        }
        b0s[i] = v;
    }
    for (int v0 = RF_WB * RF_THREADS; v0 < ws.nvt; v0 += RF_WB * RF_THREADS) {
        ws.load(tid + v0, RF_THREADS);
        ws.store(tid + v0, RF_THREADS);
    }
    if constexpr (NMID > 0) {
#pragma unroll
        for (int i = 0; i < NMID; ++i) {
            const int nin = i == 0 ? a.N0 : a.Nm[i - 1], ninp = i == 0 ? N0P : a.Nmp[i - 1];
            stage_natural<4>(a.Wm[i], nin, a.Nm[i], a.Nm[i], ninp, a.Nmp[i], Wmn[i], tid, RF_THREADS);
            lds_float* bd = bms + (i == 0 ? 0 : a.Nmp[0]);
            for (int j = tid; j < a.Nmp[i]; j += RF_THREADS) bd[j] = (a.bm[i] && j < a.Nm[i]) ? (float)a.bm[i][j] : 0.0f;
        }
    }
    __syncthreads();

    // Per-lane parts of the fragment addresses (row bases 8hh / 4hh folded in).
    const lds_half* w0lane[NT0];
#pragma unroll
    for (int t = 0; t < NT0; ++t) w0lane[t] = W0n.p + frag_lane_off(W0n, 32 * t, lane) + 8 * hh * W0n.ld;

    for (; tile < t_end; tile += wpb) {
        floatx16 acc0[NT0];
#pragma unroll
        for (int t = 0; t < NT0; ++t) acc0[t] = zero16();

        // W0^T fragment for k = 64c + 16q + 8hh + j (the rows this lane's
        // 16-byte loads of X cover) and n0 = 32t + lane%32.
        auto mma_chunk = [&](int c, const half8 (&cur)[4]) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int t = 0; t < NT0; ++t) {
                    const half8 w = frag_tr_at(w0lane[t] + (64 * c + 16 * q) * W0n.ld, 4 * W0n.ld);
                    acc0[t] = mfma32x32x16(w, cur[q], acc0[t]);
                }
            }
        };
        // Loaders whose loads do not land in operand layout move them there
        // first (in registers), just before the chunk's MFMAs.
        auto mma_raw = [&](int c, half8 (&x)[4]) {
            if constexpr (Loader::kRaw) {
                half8 op[4];
                ld.to_operand(x, op);
                mma_chunk(c, op);
            } else {
                mma_chunk(c, x);
            }
        };
        if constexpr (KCH > 0) {
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
                if (c + PD < KCH) ld.template load<KCH>(row, c + PD, hh, xr[(c + PD) % R]);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch issued here
                mma_raw(c, xr[c % R]);
            }
        } else {
            for (int c = 0; c < nch; c += 2) {
                if (c + 1 < nch) ld.template load<KCH>(row, c + 1, hh, xr[1]);
                __builtin_amdgcn_sched_barrier(0);
                mma_raw(c, xr[0]);
                if (c + 1 < nch) {
                    if (c + 2 < nch) ld.template load<KCH>(row, c + 2, hh, xr[0]);
                    __builtin_amdgcn_sched_barrier(0);
                    mma_raw(c + 1, xr[1]);
                }
            }
        }

        // Put the next tile's first chunks in flight (every set is free once
        // the last chunk's MFMAs are issued) before the epilogues.  The loads
        // are issued even when there is no next tile (its rows are then those
        // of tile ntiles, past the end, and read the zero line): loads under a
        // branch leave the ring registers to be merged after it, and that copy
        // waits for every load in flight -- the prefetch's full latency before
        // GEMM1.
        const long ntile = tile + wpb;
        const typename Loader::Row nrow = ld.row((ntile < t_end ? ntile : a.ntiles) * 32 + lr);
#pragma unroll
        for (int p = 0; p < PD; ++p)
            if (p < nch) ld.template load<KCH>(nrow, p, hh, xr[p]);

        // Epilogue 0 in registers: bias (broadcast along rows), activation,
        // one rounding to fp16.  hf[s] is GEMM1's operand B for k-step s.
        half8 hf[HF];
        act_dispatch(a.act, [&](auto act) {
#pragma unroll
            for (int t = 0; t < NT0; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n0 = 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                    hf[2 * t + (r >> 3)][r & 7] = (half_t)act.f(acc0[t][r] + b0s[n0]);
                }
            }
        });

        // Middle GEMMs of an N-stage chain: the same hand-off again.  Each
        // takes the previous fp16 output (ks k-steps of 16) as operand B and
        // produces Nmp columns in passes of 64; bias + activation + fp16 put
        // pass p's tile t into hn[2 (2p + t) + r / 8] -- again no data leaves
        // the lane.
        int ks = 2 * NT0;   // k-steps of hf
        if constexpr (NMID > 0) {
#pragma unroll
            for (int i = 0; i < NMID; ++i) {
                int lm = lane;
                asm volatile("" : "+v"(lm));
                const lds_float* bmi = bms + (i == 0 ? 0 : a.Nmp[0]);
                half8 hn[8];
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    if (64 * p < a.Nmp[i]) {
                        const lds_half* wml[2];
#pragma unroll
                        for (int t1 = 0; t1 < 2; ++t1)
                            wml[t1] = Wmn[i].p + frag_lane_off(Wmn[i], 64 * p + 32 * t1, lm) + 4 * (lm >> 5) * Wmn[i].ld;
                        floatx16 am[2];
                        am[0] = zero16();
                        am[1] = zero16();
#pragma unroll
                        for (int s2 = 0; s2 < 8; ++s2) {
                            if (s2 < ks) {
#pragma unroll
                                for (int t1 = 0; t1 < 2; ++t1) {
                                    const half8 w = frag_tr_at(wml[t1] + 16 * s2 * Wmn[i].ld, 8 * Wmn[i].ld);
                                    am[t1] = mfma32x32x16(w, hf[s2], am[t1]);
                                }
                            }
                        }
                        act_dispatch(a.actm[i], [&](auto act) {
#pragma unroll
                            for (int t1 = 0; t1 < 2; ++t1) {
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int n = 64 * p + 32 * t1 + 8 * (r >> 2) + 4 * hh + (r & 3);
                                    hn[2 * (2 * p + t1) + (r >> 3)][r & 7] = (half_t)act.f(am[t1][r] + bmi[n]);
                                }
                            }
                        });
                    }
                }
                ks = a.Nmp[i] >> 4;
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2) hf[s2] = hn[s2];
            }
        }

        // GEMM1 over N1 in chunks of 64 columns (two 32x32 tiles).
        for (int n1c = 0; n1c < a.N1p; n1c += 64) {
            // W1^T fragment bases of this 64-column chunk (the swizzle does
            // not commute with adding 64 columns); from an opaque lane index
            // so they are not hoisted out of the loop and held.
            const lds_half* w1lane[2];
            {
                int l1 = lane;
                asm volatile("" : "+v"(l1));
#pragma unroll
                for (int t1 = 0; t1 < 2; ++t1)
                    w1lane[t1] = W1n.p + frag_lane_off(W1n, n1c + 32 * t1, l1) + 4 * (l1 >> 5) * W1n.ld;
            }
            floatx16 acc1[2];
            acc1[0] = zero16();
            acc1[1] = zero16();
            // hf[s] element j holds n0 = 16s + 8(j/4) + 4hh + j%4, so the W1^T
            // fragment reads rows 16s + 4hh + [0,4) and 16s + 8 + 4hh + [0,4).
#pragma unroll
            for (int s = 0; s < HF; ++s) {
                if (NMID == 0 || s < ks) {
#pragma unroll
                    for (int t1 = 0; t1 < 2; ++t1) {
                        const half8 w = frag_tr_at(w1lane[t1] + 16 * s * W1n.ld, 8 * W1n.ld);
                        acc1[t1] = mfma32x32x16(w, hf[s], acc1[t1]);
                    }
                }
            }
            // + b1, fp16 into this wave's LDS tile, then whole-line stores:
            // each store instruction writes 8 rows x 128 contiguous bytes.
            auto out_tile = [&](auto act) {
#pragma unroll
                for (int t1 = 0; t1 < 2; ++t1) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int nl = 32 * t1 + 8 * g + 4 * hh;
                        half4 o;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            o[e] = (half_t)act.f(acc1[t1][4 * g + e] + b1s[n1c + nl + e]);
                        *reinterpret_cast<lds_half4*>(Ost + lr * RF_OLD + nl) = o;
                    }
                }
            };
            // (the two-GEMM chain has no activation after GEMM1)
            if constexpr (NMID > 0) act_dispatch(a.act1, out_tile);
            else out_tile(Act<ACT_NONE>{});
            wave_lds_sync();
            store_tile(Ost, RF_OLD, 32, 64, a.out, a.N1, tile * 32, a.M, n1c, a.N1, lane, 64);
            wave_lds_sync();
        }
        row = nrow;
    }
}

// Dense GEMM rows: X = A [M x K] row-major.
struct DenseRows {
    static constexpr bool kRaw = false;   // loads land in operand layout
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
    template <int KCH>
    __device__ __forceinline__ void load(const Row& r, int c, int hh, half8 out[4]) const
    {
        // k = 64c + 16q + 8hh + [0, 8): the MFMA's own k order, so the two
        // lanes holding a row's k-step read 32 contiguous bytes
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = 64 * c + 16 * q + 8 * hh;
            out[q] = ld16_if(r.p + k, r.ok && k < K);
        }
    }
};

// Dense GEMM rows, quad-coalesced: in load j, quad qi of the wave reads the
// 64-byte half qi >> 3 of tile row 4 (qi & 7) + j, lane qm of the quad its
// 16-byte piece qm, so every instruction reads eight whole 128-byte lines
// (non-temporal: each line is read once, by one instruction).  to_operand
// moves the data into operand layout in registers (in-quad transpose, then
// a swap of lane halves), for k = 64c + 16q + 8(lane / 32) + [0, 8).
// Measured on the 64K-row b2b GEMM: 13.8 -> 13.5 us against DenseRows (the
// same quad layout without the non-temporal hint: 14.2 us).
struct DenseRowsQ {
    static constexpr bool kRaw = true;
    const half_t* A;
    long M;
    int K;
    struct Row {
        const half_t* p;   // tile row 4 (qi & 7), this lane's piece
        unsigned ok;       // bit j: tile row 4 (qi & 7) + j exists
    };
    // m = tile * 32 + lane % 32 (the lane's operand row); the rows this lane
    // loads are other rows of the same tile, each checked against M.
    __device__ __forceinline__ Row row(long m) const
    {
        const int lane = threadIdx.x & 63, qi = lane >> 2;
        const long r0 = m - (lane & 31) + 4 * (qi & 7);
        Row r;
        r.ok = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (r0 + j < M) r.ok |= 1u << j;
        r.p = A + ((r.ok & 1u) ? r0 : 0) * (long)K + 32 * (qi >> 3) + 8 * (lane & 3);
        return r;
    }
    template <int KCH>
    __device__ __forceinline__ void load(const Row& r, int c, int, half8 out[4]) const
    {
        const int lane = threadIdx.x & 63;
        const int k = 64 * c + 32 * ((lane >> 2) >> 3) + 8 * (lane & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool ok = ((r.ok >> j) & 1u) && k < K;
            const half8* q = reinterpret_cast<const half8*>(ok ? r.p + (long)j * K + 64 * c : zero_ptr());
            out[j] = __builtin_nontemporal_load(q);
        }
    }
    __device__ __forceinline__ void to_operand(half8 (&raw)[4], half8 (&op)[4]) const
    {
        quad_transpose4(raw, threadIdx.x & 63);
        half8 x0 = raw[0], x1 = raw[1], x2 = raw[2], x3 = raw[3];
        swap_halves(x0, x1);
        swap_halves(x2, x3);
        op[0] = x0;
        op[1] = x2;
        op[2] = x1;
        op[3] = x3;
    }
};

// ----------------------------------------------------------------- launch

template <int NT0, int KCH, class Loader, int NMID = 0, int RD = 0>
static hipError_t launch_rf_k(const Loader& ld, RfArgs a, hipStream_t st)
{
    const size_t lds = NMID ? rf_lds_bytes_n(32 * NT0, a.K0p, a.N1p, NMID, a.Nmp) : rf_lds_bytes(32 * NT0, a.K0p, a.N1p);
    static std::atomic<unsigned long long> lds_set{0};
    hipError_t e = allow_full_lds((const void*)k_chain_rf<NT0, KCH, Loader, NMID, RD>, &lds_set);
    if (e != hipSuccess) return e;
    const long per_block_min = a.wpb > 0 ? a.wpb : RF_WAVES;  // at least one tile per tile-owning wave
    long grid = device_cu_count();
    if (grid * per_block_min > a.ntiles) grid = (a.ntiles + per_block_min - 1) / per_block_min;
    if (grid < 1) grid = 1;
    a.tiles_per_block = (a.ntiles + grid - 1) / grid;
    grid = (a.ntiles + a.tiles_per_block - 1) / a.tiles_per_block;
    hipLaunchKernelGGL((k_chain_rf<NT0, KCH, Loader, NMID, RD>), dim3((unsigned)grid), dim3(RF_THREADS), lds, st, ld,
                       a);
    return hipGetLastError();
}

// Compile-time chunk counts for the k lengths in use (64, 256, 576); with 4
// or 9 chunks the chains also come with a two-stage row ring (a.stages == 2:
// one chunk in flight instead of three).
template <int NT0, class Loader, int NMID = 0>
static hipError_t launch_rf_t(const Loader& ld, const RfArgs& a, hipStream_t st)
{
    if (a.stages == 2) {
        if ((a.K0p >> 6) == 4) return launch_rf_k<NT0, 4, Loader, NMID, 2>(ld, a, st);
        if ((a.K0p >> 6) == 9) return launch_rf_k<NT0, 9, Loader, NMID, 2>(ld, a, st);
    }
    switch (a.K0p >> 6) {
    case 1: return launch_rf_k<NT0, 1, Loader, NMID>(ld, a, st);
    case 4: return launch_rf_k<NT0, 4, Loader, NMID>(ld, a, st);
    case 9: return launch_rf_k<NT0, 9, Loader, NMID>(ld, a, st);
    }
    return launch_rf_k<NT0, 0, Loader, NMID>(ld, a, st);
}

template <class Loader, int NMID = 0>
inline hipError_t launch_rf(const Loader& ld, const RfArgs& a, int nt0, hipStream_t st)
{
    switch (nt0) {
    case 1: return launch_rf_t<1, Loader, NMID>(ld, a, st);
    case 2: return launch_rf_t<2, Loader, NMID>(ld, a, st);
    case 3: return launch_rf_t<3, Loader, NMID>(ld, a, st);
    case 4: return launch_rf_t<4, Loader, NMID>(ld, a, st);
    }
    return hipErrorInvalidValue;
}

// Dense-row instantiations (gemm_rf.hip): the two-GEMM chain (nmid = 0) and
// the N-stage chains (nmid = 1, 2 middle GEMMs).
hipError_t run_rf_dense(const half_t* A, const RfArgs& a, int nmid, hipStream_t st);

}  // namespace fc
