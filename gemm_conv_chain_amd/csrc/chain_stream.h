// chain_stream.h -- two-GEMM chain with the intermediate in registers and the
// weights streamed through LDS (GEMM0 widths N0 up to 256).
//
// Computes  OUT = act(A * W0 + b0) * W1 + b1  for dense rows A [M x K0].  This
// is BOLT's persistent kernel fusion (BOLT notes, "Persistent kernel
// (GEMM/Conv) fusion") for weights too large to stay resident on chip: the
// block computing a tile of GEMM0 still owns all N0 columns of that tile, so
// GEMM1 takes its operand from on-chip storage -- each wave's own registers,
// as in the register-resident chain -- and only the weights move: W0 and W1
// pass through LDS in chunks shared by the waves of the block.
//
// Mapping to CDNA4:
//   * Block = 8 waves (2 per SIMD), tile = 256 rows (32 per wave), one block
//     per CU, persistent over tiles.  A wave computes C0^T = W0^T X^T for its
//     32 rows and all N0 columns (NT0 accumulator tiles), adds the bias,
//     applies the activation, packs to fp16 straight into GEMM1's operand-B
//     registers (the register hand-off of chain_rf.h) and computes
//     D^T = W1^T H^T in passes of 128 columns.
//   * The weights form one stream of 32 KiB chunks, one per step: the W0
//     chunks of a tile (64 rows x 256 columns each), then per GEMM1 pass the
//     W1 chunks (128 rows x 128 columns), then the next tile's.  Chunks go
//     from global memory straight into LDS by the LDS-DMA load
//     (buffer_load_dwordx4 ... lds: no registers, no LDS stores) into three
//     rotating buffers, two steps ahead of the MFMAs that read them; each step
//     ends with one block barrier.  Chunks are XOR-swizzled (64-byte piece
//     ^= row & 3, the WTile layout) so the transposing fragment reads are conflict-free without
//     padding, which the DMA's contiguous 1 KiB per instruction excludes.
//   * Rows of A arrive quad-coalesced (each quad of lanes reads one 64-byte
//     segment) two steps ahead, into a ring of three register sets, and are
//     moved into operand layout in registers.  The next tile's first two
//     chunks are requested when GEMM1 starts.
//   * Each GEMM1 pass stages its output in the buffer its last step released
//     and stores whole row pieces with non-temporal stores.
//
// Memory requests and their waits.  A wave's vector-memory counter retires
// requests in issue order, and the compiler, which inserts waits for the
// loads it knows of, would count too few requests in flight (it cannot see
// the DMA ones) and wait for requests two steps early.  So every request of
// the main loop -- weight DMA, row loads, output stores -- is a buffer
// instruction issued through inline assembly, and the kernel waits itself,
// with exact counts: the group of requests issued at the start of step s
// (weights and rows for step s + 2) must be complete at the end of step s + 1,
// when only the next group may still be in flight.  Loads retire from the
// counter in issue order but stores need not (a store can complete before an
// older load), so the count never includes stores: the 8 stores of a pass
// that ended in between are waited for as well.  The waits name the row registers as
// outputs, so nothing that reads them is scheduled before the wait.  Buffer
// instructions also give the masking: offsets past a resource's size read
// zero and drop stores, so rows past M, k past K0 and columns past N0 / N1
// need no branches (a skipped instruction would break the counts).
#pragma once
#include "fc_device.h"
#include "fc_dma.h"
#include "fc_launch.h"

namespace fc {

constexpr int CS_THREADS = 512;
constexpr int CS_WAVES = CS_THREADS / 64;
constexpr int CS_MT = 32 * CS_WAVES;   // rows per tile
constexpr int CS_KC0 = 64;             // W0 rows per chunk
constexpr int CS_WC0 = 256;            // W0 chunk row width (halves; columns past N0 read zero)
constexpr int CS_KC1 = 128;            // W1 rows per chunk
constexpr int CS_N1C = 128;            // GEMM1 columns per pass (= W1 chunk row width)
constexpr int CS_BUFH = 16384;         // halves per weight buffer (32 KiB = one chunk of either kind)
constexpr int CS_NBUF = 3;
constexpr int CS_DMA_PER_WAVE = 2 * CS_BUFH / 1024 / CS_WAVES;   // 1 KiB DMA instructions per wave per chunk
static_assert(CS_KC0 * CS_WC0 == CS_BUFH && CS_KC1 * CS_N1C == CS_BUFH, "chunk sizes");

struct StreamArgs {
    const half_t* A;    // [M x K0] row-major
    const half_t* W0;   // [K0 x N0] row-major
    const half_t* b0;   // [N0] or null
    const half_t* W1;   // [N0 x N1] row-major
    const half_t* b1;   // [N1] or null
    half_t* out;        // [M x N1] row-major
    long M;
    int K0, N0, N1;
    int N1p;            // N1 rounded up to CS_N1C
    long ntiles;        // ceil(M / CS_MT)
};

// LDS bytes: three weight buffers, then the biases in fp32 (N0P + N1p).
__host__ __device__ inline size_t cs_lds_bytes(int N0P, int N1p)
{
    return (size_t)CS_NBUF * CS_BUFH * 2 + (size_t)(N0P + N1p) * 4;
}

// Rows [r0, r0 + RC) x columns [c0, c0 + WC) of the row-major G (valid rows
// x cols, leading dimension ld; zero outside) into the XOR-swizzled LDS tile
// T (row stride WC halves; element (r, c) at r * WC + (c ^ ((r & 3) << 5))):
// CS_DMA_PER_WAVE requests per wave.  A DMA instruction writes 1 KiB of
// consecutive LDS, lane i at bytes [16i, 16i + 16), so lane i fetches the
// global vector whose swizzled slot that is.  Each instruction addresses its
// rows through a resource starting at its first row, so rows past the matrix
// read zero; columns past cols get an offset outside (cols % 8 == 0 keeps
// every 16-byte vector wholly inside or outside).
template <int WC>
__device__ __forceinline__ void cs_dma_chunk(const half_t* __restrict__ G, int rows, int cols, int ld, int r0,
                                             int c0, lds_half* T, int wave, int lane)
{
    constexpr int VPR = WC / 8;                    // vectors per row
    constexpr int RPI = 64 / VPR;                  // rows per instruction
    constexpr int RSTEP = RPI * CS_WAVES;          // rows between a wave's instructions
    const int rloc = RPI * wave + lane / VPR;      // row (within the instruction's group) of this lane
    // the WTile swizzle of a width that is a multiple of 128 (rloc & 3 is the
    // same in every instruction)
    static_assert(WC % 128 == 0, "chunk rows are swizzled as 128-column multiples");
    const int col = ((lane % VPR) * 8) ^ ((rloc & 3) << 5);
    const unsigned voff = c0 + col < cols ? (unsigned)(rloc * ld + col) * 2u : CS_OUTSIDE;
    // The resources depend only on kernel arguments; computed from an opaque
    // r0 they stay here instead of being hoisted (and spilled) for every step.
    asm volatile("" : "+s"(r0));
#pragma unroll
    for (int i = 0; i < CS_DMA_PER_WAVE; ++i) {
        const int rb = r0 + RSTEP * i;             // first row of this instruction's group
        const i32x4 rs = buf_rsrc(G + (long)rb * ld + c0, ((long)(rows - rb) * ld - c0) * 2);
        if constexpr (kPoison)   // poison first: a read the real DMA has not reached yet sees it
            dma16(buf_rsrc(&fc_poison_line, sizeof(PoisonLine)), 16u * (unsigned)lane, T + (wave + CS_WAVES * i) * 512);
        dma16(rs, voff, T + (wave + CS_WAVES * i) * 512);
    }
}

template <int NT0, int KCH, int ACT>
__global__ __launch_bounds__(CS_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_chain_stream(StreamArgs a)
{
    constexpr int N0P = 32 * NT0;
    constexpr int KS1 = 2 * NT0;                                     // GEMM1 k-steps
    constexpr int NJ = (N0P + CS_KC1 - 1) / CS_KC1;                  // W1 chunks per pass
    constexpr int NDMA = CS_DMA_PER_WAVE * kDmaFactor;   // DMA requests per wave per chunk
    extern __shared__ __align__(16) char smem[];
    typedef FC_LDS float lds_float;
    lds_half* bufs[CS_NBUF];
#pragma unroll
    for (int i = 0; i < CS_NBUF; ++i) bufs[i] = (lds_half*)smem + i * CS_BUFH;
    lds_float* const b0s = (lds_float*)((lds_half*)smem + CS_NBUF * CS_BUFH);
    lds_float* const b1s = b0s + N0P;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nch = KCH ? KCH : (a.K0 + CS_KC0 - 1) / CS_KC0;
    const int np = a.N1p / CS_N1C;
    const int S = nch + np * NJ;                                     // stream steps per tile
    if constexpr (kPoison) {
        lds_poison(smem, (int)cs_lds_bytes(N0P, a.N1p), tid, CS_THREADS);
        __syncthreads();
    }

    // Biases in fp32 (zero past N0 / N1), once per block, before any request
    // of the stream is in flight.
    for (int i = tid; i < N0P + a.N1p; i += CS_THREADS) {
        float v = 0.0f;
        if (i < N0P) {
            if (a.b0 && i < a.N0) v = (float)a.b0[i];
        } else if (a.b1 && i - N0P < a.N1) {
            v = (float)a.b1[i - N0P];
        }
        b0s[i] = v;   // b1s follows b0s
    }

    // Weight chunk of tile step tau (0 <= tau < S) into T.
    auto dma_step = [&](int tau, lds_half* T) {
        if (tau < nch) {
            cs_dma_chunk<CS_WC0>(a.W0, a.K0, a.N0, a.N0, CS_KC0 * tau, 0, T, wave, lane);
        } else {
            const int u = tau - nch, p = u / NJ, j = u - p * NJ;
            cs_dma_chunk<CS_N1C>(a.W1, a.N0, a.N1, a.N1, CS_KC1 * j, CS_N1C * p, T, wave, lane);
        }
    };

    // Quad-coalesced rows: in load j, quad qi reads half (qi >> 3) (64 bytes)
    // of row 4 (qi & 7) + j of the wave's 32, lane qm of the quad its 16-byte
    // piece qm.  quad_transpose4 leaves lane L with pieces 0..3 of half L / 32
    // of row L % 32; two lane-half swaps give the operands of k-steps 0..3.
    // Rows are addressed through a per-wave resource that ends at row M.
    const int qi = lane >> 2, qm = lane & 3;
    const int koff = 32 * (qi >> 3) + 8 * qm;
    auto a_rsrc = [&](long tile) {
        const long r0 = tile * CS_MT + 32 * wave;
        return buf_rsrc(a.A + r0 * (long)a.K0, (a.M - r0) * (long)a.K0 * 2);
    };
    // (the row offsets are rebuilt from an opaque copy at every chunk: the
    // compiler would otherwise keep one set per unrolled chunk alive)
    auto load_a = [&](const i32x4& rs, int c, half8 (&raw)[4]) {
        int kq = koff, rq = 4 * (qi & 7);
        asm volatile("" : "+v"(kq), "+v"(rq));
        const int k = CS_KC0 * c + kq;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const unsigned vo = k < a.K0 ? (unsigned)((rq + j) * a.K0 + k) * 2u : CS_OUTSIDE;
            bload16(raw[j], rs, vo);
        }
    };
    auto to_operand = [&](half8 (&raw)[4], half8 (&op)[4]) {
        quad_transpose4(raw, lane);
        half8 x0 = raw[0], x1 = raw[1], x2 = raw[2], x3 = raw[3];
        swap_halves(x0, x1);
        swap_halves(x2, x3);
        op[0] = x0;
        op[1] = x2;
        op[2] = x1;
        op[3] = x3;
    };
    // Buffer of the current step is bufs[0]; rotate after every step.
    auto rotate = [&]() {
        lds_half* t = bufs[0];
        bufs[0] = bufs[1];
        bufs[1] = bufs[2];
        bufs[2] = t;
    };

    half8 ring[3][4];
    long tile = blockIdx.x;
    i32x4 rsA = a_rsrc(tile);
    // Prologue: the groups of the pseudo-steps -2 and -1 (steps 0 and 1).
    dma_step(0, bufs[0]);
    load_a(rsA, 0, ring[0]);
    if (S > 1) dma_step(1, bufs[1]);
    if (nch > 1) load_a(rsA, 1, ring[1]);
    if (nch > 1) vm_wait<NDMA + 4>();
    else if (S > 1) vm_wait<NDMA>();
    else vm_wait<0>();
    settle(ring[0]);
    __syncthreads();
    bool first = true;

    for (; tile < a.ntiles; tile += gridDim.x) {
        // Frag offsets from an opaque lane index: hoisted out of the tile
        // loop they would be spilled.
        int lo = lane;
        asm volatile("" : "+v"(lo));
        const int hho = lo >> 5;
        int ow0[NT0];
        {
            WTile t0;
            t0.ld = CS_WC0;
            t0.swz = wtile_swz(CS_WC0);
#pragma unroll
            for (int t = 0; t < NT0; ++t) ow0[t] = frag_lane_off(t0, 32 * t, lo) + 8 * hho * CS_WC0;
        }
        floatx16 acc0[NT0];
#pragma unroll
        for (int t = 0; t < NT0; ++t) acc0[t] = zero16();
        const long ntile = tile + gridDim.x;

        // GEMM0 step c: chunk c (ring set c % 3) against W0 rows 64c.. in
        // bufs[0]; issues the group of step c + 2.
        auto step0 = [&](int c, auto SC) {
            constexpr int sc = decltype(SC)::value;
            dma_step(c + 2 < S ? c + 2 : c + 2 - S, bufs[2]);
            const bool pa = c + 2 < nch;
            if (pa) load_a(rsA, c + 2, ring[(sc + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);
            half8 op[4];
            to_operand(ring[sc], op);
            // MFMA i = (k-step i / NT0, tile i % NT0); fragments two ahead
            constexpr int NM = 4 * NT0;
            auto wfrag = [&](int i) {
                return frag_tr_at(bufs[0] + ow0[i % NT0] + 16 * (i / NT0) * CS_WC0, 4 * CS_WC0);
            };
            half8 wf[3];
            wf[0] = wfrag(0);
            wf[1] = wfrag(1);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                if (i + 2 < NM) wf[(i + 2) % 3] = wfrag(i + 2);
                acc0[i % NT0] = mfma32x32x16(wf[i % 3], op[i / NT0], acc0[i % NT0]);
            }
            // the group of step c - 1 is complete once at most this step's
            // group remains (at c == 0 of a later tile the previous tile's
            // last stores are waited for too: a store may complete before an
            // older load, so only loads issued after the needed ones may stay
            // in flight.  The first of the two waits there is implied by the
            // second; without it this branch is scheduled differently and
            // the NT0 = 8 kernels spill registers.)
            if (c == 0 && !first) {
                if (pa) {
                    vm_wait<NDMA + 4 + 8>();
                    vm_wait<NDMA + 4>();
                } else {
                    vm_wait<NDMA + 8>();
                    vm_wait<NDMA>();
                }
            } else {
                if (pa) vm_wait<NDMA + 4>();
                else vm_wait<NDMA>();
            }
            // the rows of chunk c + 1 were in the completed group (for c == 0
            // of a later tile they were completed during GEMM1)
            if ((c > 0 || first) && c + 1 < nch) settle(ring[(sc + 1) % 3]);
            __syncthreads();
            rotate();
        };
        if constexpr (KCH > 0) {
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
                if (c % 3 == 0) step0(c, IntC<0>{});
                else if (c % 3 == 1) step0(c, IntC<1>{});
                else step0(c, IntC<2>{});
            }
        } else {
            for (int c0 = 0; c0 < nch; c0 += 3) {
                step0(c0, IntC<0>{});
                if (c0 + 1 < nch) step0(c0 + 1, IntC<1>{});
                if (c0 + 2 < nch) step0(c0 + 2, IntC<2>{});
            }
        }
        first = false;

        // bias + activation + fp16: hf[s] is GEMM1's operand B for k-step s
        // (element j of hf[2t + r/8] holds n0 = 32t + 8(r/4) + 4hh + r%4).
        half8 hf[KS1];
#pragma unroll
        for (int t = 0; t < NT0; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n0 = 32 * t + 8 * (r >> 2) + 4 * hho + (r & 3);
                hf[2 * t + (r >> 3)][r & 7] = (half_t)Act<ACT>::f(acc0[t][r] + b0s[n0]);
            }
        }

        // GEMM1 in passes of 128 output columns; chunk j of a pass holds W1
        // rows 128j.. (k-steps 8j..8j+7) of the pass's columns.
        const i32x4 rsAn = a_rsrc(ntile);
        const long grow0 = tile * CS_MT + 32 * wave;
        const i32x4 rsO = buf_rsrc(a.out + grow0 * a.N1, (a.M - grow0) * (long)a.N1 * 2);
        for (int p = 0; p < np; ++p) {
            int l1 = lane;
            asm volatile("" : "+v"(l1));
            int ow1[4];
            {
                WTile t1;
                t1.ld = CS_N1C;
                t1.swz = wtile_swz(CS_N1C);
#pragma unroll
                for (int t = 0; t < 4; ++t) ow1[t] = frag_lane_off(t1, 32 * t, l1) + 4 * (l1 >> 5) * CS_N1C;
            }
            floatx16 acc1[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) acc1[t] = zero16();
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int tau = nch + p * NJ + j;
                dma_step(tau + 2 < S ? tau + 2 : tau + 2 - S, bufs[2]);
                if (p == 0 && j == 0) {
                    // the next tile's first chunks (rows past M read zero)
                    load_a(rsAn, 0, ring[0]);
                    if (nch > 1) load_a(rsAn, 1, ring[1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // MFMA i = (k-step 8j + i / 4, tile i % 4), fragments two ahead
                const int KSJ = (KS1 - 8 * j) < 8 ? (KS1 - 8 * j) : 8;
                const int NM = 4 * KSJ;
                auto wfrag = [&](int i) {
                    return frag_tr_at(bufs[0] + ow1[i % 4] + 16 * (i / 4) * CS_N1C, 8 * CS_N1C);
                };
                half8 wf[3];
                wf[0] = wfrag(0);
                wf[1] = wfrag(1);
#pragma unroll
                for (int i = 0; i < NM; ++i) {
                    if (i + 2 < NM) wf[(i + 2) % 3] = wfrag(i + 2);
                    acc1[i % 4] = mfma32x32x16(wf[i % 3], hf[8 * j + i / 4], acc1[i % 4]);
                }
                // in flight may remain: this step's group and, at the first
                // step, the next tile's prefetched rows (loads issued after
                // the group of the previous step; the previous pass's stores
                // are not counted -- a store may complete before an older
                // load -- so they are waited for)
                if (j == 0 && p == 0) {
                    // (with a single GEMM1 step the prefetch is needed at the
                    // very next step: wait for it here)
                    if (S == nch + 1) vm_wait<0>();
                    else if (nch > 1) vm_wait<NDMA + 8>();
                    else vm_wait<NDMA + 4>();
                } else {
                    vm_wait<NDMA>();
                }
                // the prefetch group completes at the step after it
                if (p * NJ + j == 1 || S == nch + 1) {
                    settle(ring[0]);
                    if (nch > 1) settle(ring[1]);
                }
                __syncthreads();
                rotate();
            }
            // + b1, fp16, staged 64 columns at a time in this wave's 4 KiB of
            // the buffer the last step released (bufs[2] after the rotation;
            // rows XOR-swizzled by 8-half groups), then 16-byte reads and
            // row-contiguous non-temporal stores: 8 per wave per pass.
            const int lro = l1 & 31;
            lds_half* const st = bufs[2] + wave * (32 * 64);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = 32 * t + 8 * g + 4 * (l1 >> 5);
                        half4 o;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            o[e] = (half_t)(acc1[2 * u + t][4 * g + e] + b1s[CS_N1C * p + 64 * u + n + e]);
                        *reinterpret_cast<FC_LDS half4*>(st + lro * 64 + (n ^ ((lro & 7) << 3))) = o;
                    }
                }
                wave_lds_sync();
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int row = 8 * it + (l1 >> 3);
                    const int col = 8 * (l1 & 7);
                    const u32x4 v = *reinterpret_cast<FC_LDS const u32x4*>(st + row * 64 + (col ^ ((row & 7) << 3)));
                    const int gc = CS_N1C * p + 64 * u + col;
                    bstore16_nt(v, rsO, gc < a.N1 ? (unsigned)(row * a.N1 + gc) * 2u : CS_OUTSIDE);
                }
                wave_lds_sync();   // the next round overwrites the staging area
            }
            __syncthreads();   // the next step's DMA refills this buffer
        }
        rsA = rsAn;
    }
    // Requests for a tile past the end are still in flight: drain them.
    vm_wait<0>();
}

// N0 is padded to 64, 128 or 256 columns (zero weights, zero bias).  The
// biases must fit in LDS beside the three weight buffers.
inline bool stream_fits_lds(int N0, int N1)
{
    const int N0P = N0 <= 64 ? 64 : (N0 <= 128 ? 128 : 256);
    const long N1p = ((long)N1 + CS_N1C - 1) / CS_N1C * CS_N1C;
    return N0 <= 256 && (long)cs_lds_bytes(N0P, 0) + 4 * N1p <= (long)RF_LDS_LIMIT;
}

// Instantiated in gemm_stream.hip.
hipError_t run_stream(const StreamArgs& a, int act, hipStream_t st);

}  // namespace fc
