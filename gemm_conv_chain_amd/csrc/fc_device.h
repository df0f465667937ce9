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
typedef float floatx4 __attribute__((ext_vector_type(4)));

enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2 };

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

__device__ __forceinline__ half8 ld16_if(const half_t* p, bool ok)
{
    return ok ? ld16(p) : zero8();
}

// Element-wise activation in fp32 (the epilogue's element-wise operator).
// GELU, tanh form: 0.5 x (1 + tanh(u)) with u = sqrt(2/pi) (x + 0.044715 x^3).
// Since 0.5 (1 + tanh(u)) = 1 / (1 + e^{-2u}), this evaluates
// x / (1 + 2^{-2u log2 e}) with the hardware base-2 exponential and
// reciprocal: no cancellation near 0, and the exponential saturating to 0 or
// infinity gives x or 0 at the extremes.
__device__ __forceinline__ float act_apply(int act, float x)
{
    if (act == ACT_RELU) return x > 0.0f ? x : 0.0f;
    if (act == ACT_GELU_TANH) {
        const float k2 = 2.0f * 0.7978845608028654f * 1.4426950408889634f;  // 2 sqrt(2/pi) log2(e)
        float u = x + 0.044715f * x * x * x;
        float e = __builtin_amdgcn_exp2f(-k2 * u);
        return x * __builtin_amdgcn_rcpf(1.0f + e);
    }
    return x;
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
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
        b.v[i] = ok ? *reinterpret_cast<const u32x4*>(G + (long)r * ldg + c0) : u32x4{0u, 0u, 0u, 0u};
    }
}

template <bool PERM16>
__device__ __forceinline__ void tblock_store(half_t* T, int ldt, int ncp, int blk, const TBlock& b)
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
        *reinterpret_cast<u32x2*>(T + (c0 + 2 * d) * ldt + slot) = lo;
        *reinterpret_cast<u32x2*>(T + (c0 + 2 * d + 1) * ldt + slot) = hi;
    }
}

template <bool PERM16>
__device__ __forceinline__ void stage_transposed(const half_t* __restrict__ G, int rows, int cols, long ldg,
                                                 int r0, int nr, int ncp, half_t* T, int ldt,
                                                 int tid, int nthreads)
{
    const int nblk = (nr >> 2) * (ncp >> 3);
    for (int blk = tid; blk < nblk; blk += nthreads) {
        TBlock b;
        tblock_load(G, rows, cols, ldg, r0, ncp, blk, b);
        tblock_store<PERM16>(T, ldt, ncp, blk, b);
    }
}

}  // namespace fc
