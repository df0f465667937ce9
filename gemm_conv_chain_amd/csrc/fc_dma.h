// fc_dma.h -- raw buffer resources, LDS-DMA requests and explicit
// vector-memory waits (gfx950), shared by the kernels that stream operands
// into LDS.  Requests issued through inline assembly are invisible to the
// compiler's own wait-count bookkeeping, so the kernels that use them wait
// for them explicitly (vm_wait).
#pragma once
#include "fc_device.h"

namespace fc {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (stride 0) for the bytes [p, p + nbytes): loads at
// offsets past nbytes return zero and stores there are dropped.  The flags
// word is the gfx9 raw-buffer format.  Offsets of 2^31 and more are always
// outside (nbytes is capped below that).
__device__ __forceinline__ i32x4 buf_rsrc(const void* p, long nbytes)
{
    const unsigned long long u = (unsigned long long)p;
    nbytes = nbytes < 0 ? 0 : (nbytes > 0x7fffffffL ? 0x7fffffffL : nbytes);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)u);
    r[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(u >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
    r[3] = 0x00020000;
    return r;
}
constexpr unsigned CS_OUTSIDE = 0x80000000u;   // an offset outside every resource

// 16-byte LDS-DMA request: bytes at voff (per lane) of the resource to LDS
// at dst + 16 * lane (dst wave-uniform, in M0; one wait state after the M0
// write).
__device__ __forceinline__ void dma16(i32x4 rsrc, unsigned voff, const lds_half* dst)
{
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(size_t)dst);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(m0)
                 : "memory", "m0");
}

// Poison (debug builds): 1 KiB of the poison pattern in global memory, the
// source of the poison LDS-DMA requests of the streamed kernels (a DMA fills
// LDS without the registers an LDS store loop would take).
struct PoisonLine {
    unsigned w[256];
};
__host__ __device__ constexpr PoisonLine make_poison_line()
{
    PoisonLine p{};
    for (int i = 0; i < 256; ++i) p.w[i] = kPoisonWord;
    return p;
}
static __device__ __align__(16) PoisonLine fc_poison_line = make_poison_line();

// DMA requests per real one: 2 in the poison build (each 1 KiB DMA is
// preceded by one that writes the poison to the same LDS bytes).
constexpr int kDmaFactor = kPoison ? 2 : 1;

// 16-byte load into registers (the kernel waits for it with vm_wait).
// Non-temporal: each row line is read once, by one instruction (quad layout).
__device__ __forceinline__ void bload16(half8& dst, i32x4 rsrc, unsigned voff)
{
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen nt" : "=v"(dst) : "v"(voff), "s"(rsrc));
}

// 16-byte non-temporal store.
__device__ __forceinline__ void bstore16_nt(const u32x4& v, i32x4 rsrc, unsigned voff)
{
    asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen nt" ::"v"(v), "v"(voff), "s"(rsrc) : "memory");
}

// Wait until at most N of this wave's vector-memory requests are in flight.
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// After a vm_wait that completed the loads of x: names x as redefined here,
// so nothing that reads it is scheduled before the wait (volatile asm keeps
// its order), while slots still in flight stay untouched.
__device__ __forceinline__ void settle(half8 (&x)[4])
{
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}

}  // namespace fc
