// probe.hip -- measurement aids, not part of any chain: the matrix-core rate
// and the shader clock this GPU sustains, and the rate at which it streams a
// buffer from memory, for reading the chains' fractions of peak against what
// the hardware actually delivers.
//
// Every wave issues `iters` rounds of eight independent fp16 MFMAs
// (32x32x16, fp32 accumulate) on operands held in registers -- no memory
// traffic, no LDS -- and the first wave of each block records the shader
// clock counter (s_memtime) and the fixed 100 MHz counter (s_memrealtime)
// around its loop, so the host can derive the clock while the matrix cores
// are saturated.
#include "../../include/fusedchain.h"
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {

template <int WPS>
__global__ __launch_bounds__(256 * WPS) __attribute__((amdgpu_waves_per_eu(WPS, WPS)))
void k_mfma_probe(int iters, unsigned long long* __restrict__ stamps, float* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    half8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (half_t)(0.001f * (float)(lane + i));
        b[i] = (half_t)(0.002f * (float)(lane - i));
    }
    floatx16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = zero16();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mfma32x32x16(a, b, acc[j]);
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    // one value per block keeps the MFMAs live; per-lane addresses (vector stores)
    if (threadIdx.x == 0) sink[blockIdx.x] = s;
    if (threadIdx.x < 4) {
        const unsigned long long v = threadIdx.x == 0 ? t0 : threadIdx.x == 1 ? t1 : threadIdx.x == 2 ? r0 : r1;
        stamps[4 * (long)blockIdx.x + threadIdx.x] = v;
    }
}

// Streams n16 16-byte vectors of p once: consecutive threads read consecutive
// vectors (whole cache lines per wave), four independent loads in flight per
// thread per round, grid-stride; the XOR of everything read goes to
// sink[block] so that no load is dead.
__global__ __launch_bounds__(256) void k_read_probe(const u32x4* __restrict__ p, long n16, unsigned* __restrict__ sink)
{
    u32x4 acc = {0u, 0u, 0u, 0u};
    const long stride = (long)gridDim.x * 256;
    long i = (long)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    unsigned v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v ^= (unsigned)__shfl_xor((int)v, o);
    __shared__ unsigned part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace fc

extern "C" fc_status fc_probe_read(const void* buf, int64_t nbytes, uint32_t* sink, int32_t capacity,
                                   int32_t* blocks, void* stream)
{
    if (!buf || !sink || !blocks) return FC_E_NULL;
    if (nbytes < 16 || nbytes % 16) return FC_E_SHAPE;
    if (((uintptr_t)buf & 15u) || ((uintptr_t)sink & 3u)) return FC_E_ALIGN;
    const long n16 = (long)(nbytes / 16);
    // two blocks per CU (the fastest of 2..16 blocks per CU and 4..16 loads in
    // flight per thread on a 75.5 MB stream), or fewer for small buffers
    long grid = 2L * fc::device_cu_count();
    if (grid > (n16 + 255) / 256) grid = (n16 + 255) / 256;
    if (grid < 1) return FC_E_HIP;
    if (grid > capacity) return FC_E_SHAPE;
    hipLaunchKernelGGL(fc::k_read_probe, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const fc::u32x4*>(buf), n16, reinterpret_cast<unsigned*>(sink));
    if (hipGetLastError() != hipSuccess) return FC_E_HIP;
    *blocks = (int32_t)grid;
    return FC_OK;
}

extern "C" fc_status fc_probe_mfma(int32_t waves_per_simd, int32_t iters, uint64_t* stamps, float* sink,
                                   int32_t capacity, int32_t* blocks, void* stream)
{
    if (!stamps || !sink || !blocks) return FC_E_NULL;
    if ((waves_per_simd != 1 && waves_per_simd != 2) || iters < 1 || iters > (1 << 20)) return FC_E_SHAPE;
    if (((uintptr_t)stamps & 7u) || ((uintptr_t)sink & 3u)) return FC_E_ALIGN;
    const int grid = fc::device_cu_count();
    if (grid < 1) return FC_E_HIP;
    if (grid > capacity) return FC_E_SHAPE;   // the buffers hold fewer blocks than the grid
    hipStream_t st = (hipStream_t)stream;
    unsigned long long* sp = reinterpret_cast<unsigned long long*>(stamps);
    if (waves_per_simd == 1)
        hipLaunchKernelGGL(fc::k_mfma_probe<1>, dim3(grid), dim3(256), 0, st, (int)iters, sp, sink);
    else
        hipLaunchKernelGGL(fc::k_mfma_probe<2>, dim3(grid), dim3(512), 0, st, (int)iters, sp, sink);
    if (hipGetLastError() != hipSuccess) return FC_E_HIP;
    *blocks = grid;
    return FC_OK;
}
