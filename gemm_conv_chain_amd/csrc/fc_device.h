// fc_device.h -- device-side building blocks shared by the fused-chain kernels
// (gfx950 / CDNA4, wave64, fp16 MFMA with fp32 accumulation).
//
// MFMA operand conventions used throughout (v_mfma_f32_32x32x16_f16):
//   operand A (32 x 16): lane l supplies row (l % 32), k-group (l / 32);
//   operand B (16 x 32): lane l supplies column (l % 32), k-group (l / 32);
//   a k-group is 8 consecutive fp16 values packed in one 16-byte register
//   quadruple.  Which 8 k indices a k-group stands for is the kernels' choice:
//   the hardware pairs A and B element by element, so any assignment that both
//   operands share computes the same sum.
//   result D (32 x 32): lane l, accumulator register r holds
//       D[8*(r/4) + 4*(l/32) + (r%4)][l % 32].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fc {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Pointers into LDS carry address space 3 explicitly, so every access compiles
// to a ds_* instruction (a generic pointer would be a flat access or need a
// null-checked cast at each use).
#define FC_LDS __attribute__((address_space(3)))
typedef FC_LDS half_t lds_half;

enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2, ACT_HARDSWISH = 3 };

__device__ __forceinline__ floatx16 mfma32x32x16(half8 a, half8 b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 zero8()
{
    half8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (half_t)0.0f;
    return z;
}

__device__ __forceinline__ floatx16 zero16()
{
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// 16-byte global load (global_load_dwordx4); the caller guarantees alignment.
__device__ __forceinline__ half8 ld16(const half_t* p)
{
    return *reinterpret_cast<const half8*>(p);
}

// 64 bytes of zeros in device (global) memory: masked-off lanes load from
// here.  Never written; non-const so that it lives in the global address space
// like the tensors (a pointer select between address spaces would turn the
// loads into flat loads, which also occupy the LDS wait counter).
static __device__ __align__(64) unsigned int fc_zero_line[16];

__device__ __forceinline__ const half_t* zero_ptr()
{
    return reinterpret_cast<const half_t*>(fc_zero_line);
}

// Branch-free masked 16-byte load: lanes with !ok read the zero line instead
// of p.  The choice is made on the address, before the load, so nothing
// consumes the loaded value early: the load stays in flight until the MFMA
// that needs it (a select on the VALUE would force a wait right after the
// load and expose its full latency).
__device__ __forceinline__ half8 ld16_if(const half_t* p, bool ok)
{
    return ld16(ok ? p : zero_ptr());
}

// Final outputs are stored with the non-temporal hint (global_store ... nt):
// they are not read again by the kernel, and without the hint they pile up as
// dirty L2 lines that are written back only when the kernel ends, after the
// last input has arrived.  Measured on the 64K-row b2b GEMM (reads 33 MB,
// writes 17 MB): 16.6 -> 13.6 us.  (Non-temporal LOADS are slower there: the
// operand layout reads each 128-byte line in four 32-byte pieces, and with
// the hint the line is not kept in L2 between them.)
template <class V>
__device__ __forceinline__ void st_out(V* p, const V& v)
{
    __builtin_nontemporal_store(v, p);
}

// Element-wise activation in fp32 (the epilogue's element-wise operator),
// fixed at compile time so that an epilogue is straight-line code the
// scheduler can interleave.  GELU, tanh form: 0.5 x (1 + tanh(u)) with
// u = sqrt(2/pi) (x + 0.044715 x^3).  Since 0.5 (1 + tanh(u)) = 1/(1 + e^{-2u}),
// this evaluates x / (1 + 2^q) with q = -2 log2(e) sqrt(2/pi) x (1 + 0.044715 x^2)
// by the hardware base-2 exponential and reciprocal: no cancellation near 0,
// and the exponential saturating to 0 or infinity gives x or 0 at the extremes.
template <int ACT> struct Act;
// `monotone`: f is non-decreasing, so max_i f(v_i) = f(max_i v_i) (used by
// the max-pool epilogue; GELU and Hardswish dip below zero and are not).
template <> struct Act<ACT_NONE> {
    static constexpr bool monotone = true;
    __device__ static __forceinline__ float f(float x) { return x; }
};
template <> struct Act<ACT_RELU> {
    static constexpr bool monotone = true;
    __device__ static __forceinline__ float f(float x) { return x > 0.0f ? x : 0.0f; }
};
template <> struct Act<ACT_GELU_TANH> {
    static constexpr bool monotone = false;
    __device__ static __forceinline__ float f(float x)
    {
        const float c1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;   // -2 sqrt(2/pi) log2(e)
        const float c3 = c1 * 0.044715f;
        const float q = x * __builtin_fmaf(x * x, c3, c1);
        return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(q));
    }
};

// Hardswish x * min(max(x + 3, 0), 6) / 6 (the fused Conv2D + BiasAdd +
// Hardswish epilogue of the BOLT notes, "Enabling deeper operator fusion").
template <> struct Act<ACT_HARDSWISH> {
    static constexpr bool monotone = false;
    __device__ static __forceinline__ float f(float x)
    {
        const float r6 = __builtin_fminf(__builtin_fmaxf(x + 3.0f, 0.0f), 6.0f);
        return x * r6 * (1.0f / 6.0f);
    }
};

// Unsigned division by a runtime constant d >= 1 without a divide sequence:
// magic = floor(2^32 / d) (2^32 - 1 for d = 1) gives q0 = mulhi(x, magic) in
// {x/d - 1, x/d}, and one comparison fixes it (exact for every 32-bit x).
struct FastDiv {
    unsigned d, magic;
    static FastDiv make(unsigned dd)
    {
        FastDiv f;
        f.d = dd;
        f.magic = dd > 1 ? (unsigned)(0x100000000ull / dd) : 0xffffffffu;
        return f;
    }
    __device__ __forceinline__ unsigned div(unsigned x) const
    {
        unsigned q = __umulhi(x, magic);
        if (x - q * d >= d) ++q;
        return q;
    }
};

template <int V> struct IntC {
    static constexpr int value = V;
};

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8), and each XCD has its own L2.  This renumbering gives every XCD a
// contiguous range of block indices, so neighbouring tiles (which share halo
// rows or weights) meet in the same L2.  A bijection of [0, n) when 8 | n;
// the identity otherwise.
__device__ __forceinline__ unsigned xcd_block(unsigned b, unsigned n)
{
    return (n & 7u) ? b : (b & 7u) * (n >> 3) + (b >> 3);
}

// ---- quad-coalesced MFMA operand loads -------------------------------------
// The texture addresser takes a 16-byte-per-lane load at four lanes per clock
// when each group of four consecutive lanes reads one 64-byte segment, and at
// one lane per clock otherwise.  MFMA operand layouts put a different row in
// every lane of a quad, so rows are loaded quad-wise (lane 4i + m reads
// segment m of row group i) and moved into operand layout in registers: a 4x4
// transpose inside every quad (two DPP exchange stages), then a swap of lane
// halves between two registers.

__device__ __forceinline__ unsigned dpp_quad_xor2(unsigned v)
{
    return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
}
__device__ __forceinline__ unsigned dpp_quad_xor1(unsigned v)
{
    return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
}

// In every quad (lanes 4i..4i+3): a[r] at quad lane j  ->  a[j] at quad lane r.
__device__ __forceinline__ void quad_transpose4(half8 (&a)[4], int lane)
{
    const bool b1 = (lane >> 1) & 1, b0 = lane & 1;
    u32x4 x[4], y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = __builtin_bit_cast(u32x4, a[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const unsigned o = dpp_quad_xor2(x[r ^ 2][d]);
            y[r][d] = (b1 == (bool)((r >> 1) & 1)) ? x[r][d] : o;
        }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const unsigned o = dpp_quad_xor1(y[r ^ 1][d]);
            x[r][d] = (b0 == (bool)(r & 1)) ? y[r][d] : o;
        }
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = __builtin_bit_cast(half8, x[r]);
}

// lo = [lo lanes 0-31 | hi lanes 0-31], hi = [lo lanes 32-63 | hi lanes 32-63].
__device__ __forceinline__ void swap_halves(half8& lo, half8& hi)
{
    u32x4 x = __builtin_bit_cast(u32x4, lo), y = __builtin_bit_cast(u32x4, hi);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const auto p = __builtin_amdgcn_permlane32_swap(x[d], y[d], false, false);
        x[d] = p[0];
        y[d] = p[1];
    }
    lo = __builtin_bit_cast(half8, x);
    hi = __builtin_bit_cast(half8, y);
}

// Calls f(Act<act>{}) with the activation as a compile-time type: the branch
// on the (wave-uniform) activation is taken once per epilogue, not per element.
template <class F>
__device__ __forceinline__ void act_dispatch(int act, F&& f)
{
    if (act == ACT_GELU_TANH) f(Act<ACT_GELU_TANH>{});
    else if (act == ACT_RELU) f(Act<ACT_RELU>{});
    else if (act == ACT_HARDSWISH) f(Act<ACT_HARDSWISH>{});
    else f(Act<ACT_NONE>{});
}

// Transposed staging of a row-major fp16 matrix G [rows x cols] (leading
// dimension ldg) into LDS:  T[c * ldt + slot(r - r0)] = G[r][c]  for the rows
// [r0, r0 + nr) and columns [0, ncp); entries outside [0, rows) x [0, cols) are
// zero.  nr must be a multiple of 4, ncp a multiple of 8, and cols a multiple
// of 8 so that every 16-byte column block is fully inside or fully outside.
// Work unit ("block"): 4 rows x 8 columns = four 16-byte global loads, written
// as eight 8-byte LDS stores of four consecutive slots.  PERM16 applies, inside
// each group of 16 slots, the quad swap 0-3,4-7,8-11,12-15 -> 0-3,8-11,4-7,12-15:
// the order in which a 32x32 accumulator hands rows to a lane (the
// register-resident hand-off of the chain kernels).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct TBlock {
    u32x4 v[4];   // four rows of 8 fp16, two per dword (low half = even column)
};

__device__ __forceinline__ void tblock_load(const half_t* __restrict__ G, int rows, int cols, long ldg,
                                            int r0, int ncp, int blk, TBlock& b)
{
    const int nbc = ncp >> 3;
    const int br = blk / nbc, bc = blk - br * nbc;
    const int c0 = bc * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = r0 + br * 4 + i;
        const bool ok = r < rows && c0 < cols;
        b.v[i] = *reinterpret_cast<const u32x4*>(ok ? G + (long)r * ldg + c0 : zero_ptr());
    }
}

template <bool PERM16>
__device__ __forceinline__ void tblock_store(lds_half* T, int ldt, int ncp, int blk, const TBlock& b)
{
    const int nbc = ncp >> 3;
    const int br = blk / nbc, bc = blk - br * nbc;
    const int rl = br * 4, c0 = bc * 8;
    int slot = rl;
    if (PERM16) {
        const int q = rl & 15;  // quad start inside its 16-group: 0, 4, 8 or 12
        slot = (rl & ~15) + 8 * ((q >> 2) & 1) + 4 * (q >> 3);
    }
    // column c of the block = halves c of rows 0..3; v_perm_b32 pairs the low
    // (even c) or high (odd c) halves of two dwords.
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        u32x2 lo, hi;
        lo.x = __builtin_amdgcn_perm(b.v[1][d], b.v[0][d], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(b.v[3][d], b.v[2][d], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(b.v[1][d], b.v[0][d], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(b.v[3][d], b.v[2][d], 0x07060302u);
        *reinterpret_cast<FC_LDS u32x2*>(T + (c0 + 2 * d) * ldt + slot) = lo;
        *reinterpret_cast<FC_LDS u32x2*>(T + (c0 + 2 * d + 1) * ldt + slot) = hi;
    }
}

template <bool PERM16>
__device__ __forceinline__ void stage_transposed(const half_t* __restrict__ G, int rows, int cols, long ldg,
                                                 int r0, int nr, int ncp, lds_half* T, int ldt,
                                                 int tid, int nthreads)
{
    const int nblk = (nr >> 2) * (ncp >> 3);
    for (int blk = tid; blk < nblk; blk += nthreads) {
        TBlock b;
        tblock_load(G, rows, cols, ldg, r0, ncp, blk, b);
        tblock_store<PERM16>(T, ldt, ncp, blk, b);
    }
}

// ---------------------------------------------------------------------------
// MFMA operand fragment read from a row-major LDS tile with the gfx950
// transposing LDS load (ds_read_b64_tr_b16).  The tile T holds k along its rows
// (T[k][n], row stride ldt halves), as weights arrive from HBM.  The fragment
// is that of a 32x32x16 operand whose lane l stands for index nb + (l % 32)
// (a row of operand A or a column of operand B) and k-group h = l / 32:
//     element j (0..7) = T[k0 + 8h + j][nb + l % 32].
// Measured behaviour of the instruction: inside each group of 16 lanes, lane i
// receives element (i % 4) of the 8-byte chunks addressed by lanes
// 4e + i/4, e = 0..3.  So lane j of a group addresses row k0 + 8h + j/4 (+4 for
// the second read), columns nb + 16*(group & 1) + 4*(j % 4) .. +3.
// Conflict-free when the row stride is 64 bytes (times an odd number) modulo
// 256: the four rows each 32-lane half reads then fill all 64 banks.
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef FC_LDS fp16x4_t lds_fp16x4_t;

__device__ __forceinline__ half8 frag_tr(const lds_half* T, int ldt, int k0, int nb, int lane)
{
    const int g = lane >> 4, i = lane & 15;
    const lds_half* p = T + (k0 + 8 * (g >> 1) + (i >> 2)) * ldt + nb + 16 * (g & 1) + 4 * (i & 3);
    const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t*)(p));
    const fp16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t*)(p + 4 * ldt));
    half8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (half_t)lo[e];
        r[e + 4] = (half_t)hi[e];
    }
    return r;
}

// A natural (row-major, rows = k) weight tile in LDS, optionally XOR-swizzled.
//
// Bank geometry (measured on gfx950 with the LDS bank-conflict counter): a
// transposing 8-byte read of 64 lanes is served at 256 bytes per clock, i.e.
// 64 four-byte banks, when the 32 lanes of each half touch 256 distinct bank
// bytes.  Such a half reads 4 rows x 32 columns (64 bytes per row) of the
// tile, so the four rows' 64-byte pieces must sit at four different offsets
// modulo 256 bytes.
//   N % 64 == 32: the row stride (64 * odd bytes) already separates them.
//   N % 128 == 64: rows 2q and 2q+1 differ by 128 bytes; rows 2,3 (mod 4)
//                  flip the 64-byte piece (XOR 32 halves).
//   N % 128 == 0:  every row starts at the same bank; row r (mod 4) takes
//                  piece r (XOR 32 (r % 4) halves).
// Both XORs keep 8-half (16-byte) vectors whole and commute with adding a
// multiple of 128 columns (not 64).
struct WTile {
    lds_half* p;
    int ld;      // row stride in halves
    int swz;     // 0: none; 1: XOR columns with 32 (row % 4); 2: XOR with 32 ((row / 2) % 2)
    __device__ __forceinline__ int off(int r, int c) const
    {
        const int m = swz == 1 ? (r & 3) << 5 : swz == 2 ? ((r >> 1) & 1) << 5 : 0;
        return r * ld + (c ^ m);
    }
};

// Row stride / swizzle for a natural [rows x N] fp16 tile (N % 32 == 0): no
// padding, the swizzle chosen from N as above.
__host__ __device__ constexpr int wtile_ld(int N) { return N; }
__host__ __device__ constexpr int wtile_swz(int N) { return N % 128 == 0 ? 1 : N % 64 == 0 ? 2 : 0; }

// Lane part of a transposing fragment read from a WTile: the offset (in
// halves) of this lane's 8-byte chunk for rows starting at 0 and the column
// block nb (nb % 32 == 0; pass the full column: the swizzle does not commute
// with adding 64 columns).  Add row * ld for the row base with a row offset
// that is a multiple of 4 (the swizzle depends on row % 4); the second read
// of a fragment is 4 (or 8) rows further down.
__device__ __forceinline__ int frag_lane_off(const WTile& T, int nb, int lane)
{
    const int g = lane >> 4, i = lane & 15;
    return T.off(i >> 2, nb + 16 * (g & 1) + 4 * (i & 3));
}

__device__ __forceinline__ half8 frag_tr_at(const lds_half* p, int hi_off)
{
    const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t*)(p));
    const fp16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_t*)(p + hi_off));
    half8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (half_t)lo[e];
        r[e + 4] = (half_t)hi[e];
    }
    return r;
}

// Copy rows [0, nr) x columns [0, ncp) of the row-major G (leading dimension
// ldg; zero outside rows x cols) into the natural tile T, 16-byte vectors,
// NB vectors per thread per batch (all loads of a batch are issued before its
// stores).
template <int NB>
__device__ __forceinline__ void stage_natural(const half_t* __restrict__ G, int rows, int cols, long ldg, int nr,
                                              int ncp, const WTile& T, int tid, int nthreads)
{
    typedef FC_LDS u32x4 lds_u32x4;
    const int vpr = ncp >> 3;
    const int nv = nr * vpr;
    for (int v0 = 0; v0 < nv; v0 += NB * nthreads) {
        u32x4 x[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int v = v0 + tid + i * nthreads;
            const int r = v / vpr, c = (v - r * vpr) * 8;
            const bool ok = v < nv && r < rows && c < cols;
            x[i] = *reinterpret_cast<const u32x4*>(ok ? G + (long)r * ldg + c : zero_ptr());
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int v = v0 + tid + i * nthreads;
            const int r = v / vpr, c = (v - r * vpr) * 8;
            if (v < nv) *reinterpret_cast<lds_u32x4*>(T.p + T.off(r, c)) = x[i];
        }
    }
}

// Two-phase staging of up to two natural weight tiles into LDS: load()
// issues this thread's share of the global loads into registers, store()
// writes them to LDS.  Between the two a kernel may issue its own streaming
// loads: the wait before store() then covers only the staging loads (a wave's
// wait counter retires loads in issue order).  Vector v (16 bytes) of matrix m
// is row v / vpr, column 8 (v % vpr); thread tid handles v = tid + i*nthreads,
// whose (row, column) advance by a fixed step -- no division per vector.
template <int NV>
struct WStage2 {
    u32x4 x[NV];
    // matrix 0 and matrix 1 (kept as separate fields: a runtime-indexed
    // array would be placed in scratch memory)
    const half_t* G0;
    const half_t* G1;
    int rows0, cols0, nr0, ncp0, rows1, cols1, nr1, ncp1;
    long ldg0, ldg1;
    WTile T0, T1;
    int nv0, nvt;    // vectors of matrix 0; of both
    bool dense;      // both matrices fill their tiles exactly and are contiguous in memory

    __device__ __forceinline__ void init()
    {
        nv0 = nr0 * (ncp0 >> 3);
        nvt = nv0 + nr1 * (ncp1 >> 3);
        dense = rows0 == nr0 && cols0 == ncp0 && ldg0 == cols0 && rows1 == nr1 && cols1 == ncp1 && ldg1 == cols1;
    }
    template <bool STORE>
    __device__ __forceinline__ void walk(int v0, int nthreads)
    {
        typedef FC_LDS u32x4 lds_u32x4;
        const int step = nthreads * 8;
        // position in matrix 0 (one division per call)
        const int vpr0 = ncp0 >> 3, vpr1 = ncp1 >> 3;
        int m = v0 >= nv0;
        int vv = m ? v0 - nv0 : v0;
        int r = vv / (m ? vpr1 : vpr0);
        int c = (vv - r * (m ? vpr1 : vpr0)) * 8;
        const int dr0 = step / ncp0, dc0 = step - dr0 * ncp0;
        const int dr1 = step / ncp1, dc1 = step - dr1 * ncp1;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = v0 + i * nthreads;
            if (v - (int)(threadIdx.x & 63) >= nvt) break;   // the whole wave is past the end
            if (!m && v >= nv0) {   // crossed into matrix 1 (once)
                m = 1;
                vv = v - nv0;
                r = vv / vpr1;
                c = (vv - r * vpr1) * 8;
            }
            const int ncp = m ? ncp1 : ncp0;
            if (STORE) {
                if (v < nvt) {
                    lds_half* dst = m ? T1.p + T1.off(r, c) : T0.p + T0.off(r, c);
                    *reinterpret_cast<lds_u32x4*>(dst) = x[i];
                }
            } else {
                const bool ok = v < nvt && r < (m ? rows1 : rows0) && c < (m ? cols1 : cols0);
                const half_t* src = m ? G1 + (long)r * ldg1 + c : G0 + (long)r * ldg0 + c;
                x[i] = *reinterpret_cast<const u32x4*>(ok ? src : zero_ptr());
            }
            c += m ? dc1 : dc0;
            r += m ? dr1 : dr0;
            if (c >= ncp) {
                c -= ncp;
                ++r;
            }
        }
    }
    // Loads: vector v of a dense pair is simply the 8 halves at G0 + 8v (or
    // G1 + 8(v - nv0)), a few operations per vector instead of the walk.
    __device__ __forceinline__ void load(int v0, int nthreads)
    {
        if (!dense) {
            walk<false>(v0, nthreads);
            return;
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = v0 + i * nthreads;
            if (v - (int)(threadIdx.x & 63) >= nvt) break;   // the whole wave is past the end
            const half_t* src = v < nv0 ? G0 + 8L * v : G1 + 8L * (v - nv0);
            x[i] = *reinterpret_cast<const u32x4*>(v < nvt ? src : zero_ptr());
        }
    }
    __device__ __forceinline__ void store(int v0, int nthreads) { walk<true>(v0, nthreads); }
};

// Line-coalesced store of an fp16 tile held in LDS: T [rows x cols] (row
// stride ldt halves, cols % 8 == 0) -> out[(row0 + r) * ldo + col0 + c] for
// row0 + r < nrows and col0 + c < ncols.  Consecutive threads write consecutive
// 16-byte pieces of a row, so every store instruction covers whole 128-byte
// lines (partial-line stores are written back to HBM several times over).
__device__ __forceinline__ void store_tile(const lds_half* T, int ldt, int rows, int cols, half_t* out, long ldo,
                                           long row0, long nrows, int col0, int ncols, int tid, int nthreads)
{
    typedef FC_LDS const u32x4 lds_u32x4;
    const int vpr = cols >> 3;
    for (int v = tid; v < rows * vpr; v += nthreads) {
        const int r = v / vpr, c = (v - r * vpr) * 8;
        if (row0 + r < nrows && col0 + c < ncols)
            st_out(reinterpret_cast<u32x4*>(out + (row0 + r) * ldo + col0 + c), (u32x4)*reinterpret_cast<lds_u32x4*>(T + r * ldt + c));
    }
}

// Orders this wave's LDS accesses around a hand-off through LDS between its
// own lanes (LDS instructions of one wave execute in order; this also keeps
// the compiler from moving accesses across it).
// The lane id, computed where it is used (v_mbcnt over a full mask): the asm
// block has no inputs and is volatile, so the compiler can neither hoist it
// out of a loop nor keep an earlier copy alive across the loop (a per-lane
// value held across a register-bound main loop gets spilled, and its reload
// waits for every load in flight).
__device__ __forceinline__ int lane_id_here()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

__device__ __forceinline__ void wave_lds_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------ LDS poison
// Debug build (-DFC_DEBUG_POISON: libfusedchain_poison.so).  A kernel fills
// its LDS with a poison pattern when it starts, and the kernels that reuse LDS
// buffers (DMA rings, double buffers) poison each buffer again after the
// barrier that releases it and before its next producer writes it.  A read
// that is not ordered after its producer -- a missing barrier, a memory-counter
// wait that retires too few requests -- then returns poison instead of stale
// but plausible data.  The pattern is the fp16 pair (65504, 65504): finite, so
// a read whose products are multiplied by zero stays harmless, and large enough
// that a poisoned operand sends the outputs out of tolerance or to infinity;
// as bytes (0xFF, 0x7B) it is no valid pool index.  In the product build
// kPoison is false and every poison step compiles to nothing.
#ifdef FC_DEBUG_POISON
constexpr bool kPoison = true;
#else
constexpr bool kPoison = false;
#endif
constexpr unsigned kPoisonWord = 0x7BFF7BFFu;

// Fill `bytes` (a multiple of 16) of LDS at p (an LDS pointer, or the
// kernel's dynamic LDS array) with the poison; the threads tid = 0 ..
// nthreads - 1 of the caller take 16-byte pieces in turn.
template <class P>
__device__ __forceinline__ void lds_poison(P p, int bytes, int tid, int nthreads)
{
    typedef FC_LDS u32x4 lds_u32x4;
    const u32x4 v = {kPoisonWord, kPoisonWord, kPoisonWord, kPoisonWord};
    lds_u32x4* q = (lds_u32x4*)p;
    for (int i = tid; i < bytes / 16; i += nthreads) q[i] = v;
}

}  // namespace fc
