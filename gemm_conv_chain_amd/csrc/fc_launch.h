// fc_launch.h -- host-side launch functions behind the C ABI (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <atomic>

namespace fc {

typedef _Float16 half_t;

enum { VARIANT_AUTO = 0, VARIANT_RF = 1, VARIANT_LDS = 2, VARIANT_STREAM = 3, VARIANT_PIPE = 4 };

// LDS a block may use (gfx950: 160 KiB per CU; one block of the persistent
// kernels per CU).
constexpr size_t RF_LDS_LIMIT = 160 * 1024;

// Lets kernel f use the whole LDS on the current device.  The attribute is
// set once per device (bit d of *done); launches then need no extra call,
// which also keeps them capturable in a HIP graph.
inline hipError_t allow_full_lds(const void* f, std::atomic<unsigned long long>* done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
    if (bit && (done->load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)RF_LDS_LIMIT);
    if (e == hipSuccess && bit) done->fetch_or(bit, std::memory_order_relaxed);
    return e;
}

int device_cu_count();
bool rf_fits(int K0, int N0, int N1);
bool stream_fits(int N0, int N1);
bool gemmn_fits(int nst, const int* widths);
hipError_t run_chain_gemmN(const half_t* A, int nst, const half_t* const* W, const half_t* const* b, const int* act,
                           const int* widths, half_t* D, long M, hipStream_t st);

// waves: tile-owning waves per block of the register-resident variant (0 = all);
// stages: its row-chunk ring depth (0 = the default 4, or 2)
hipError_t run_chain_gemm2(const half_t* A, const half_t* W0, const half_t* b0, int act, const half_t* W1,
                           const half_t* b1, half_t* D1, long M, int K0, int N0, int N1, int variant, int waves,
                           int stages, hipStream_t st);
hipError_t run_gemm_bias_act(const half_t* A, const half_t* W, const half_t* b, int act, half_t* C, long M,
                             int K, int N, hipStream_t st);

}  // namespace fc
