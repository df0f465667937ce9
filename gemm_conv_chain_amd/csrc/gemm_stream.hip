// gemm_stream.hip -- instantiations of the streamed-weight chain kernel
// (chain_stream.h).  Kept apart from the other kernels so that the sources
// compile in parallel.
#include "chain_stream.h"

namespace fc {

// ----------------------------------------------------------------- launch

template <int NT0, int KCH, int ACT>
static hipError_t launch_stream_k(const StreamArgs& a, hipStream_t st)
{
    const size_t lds = cs_lds_bytes(32 * NT0, a.N1p);
    static std::atomic<unsigned long long> lds_set{0};
    hipError_t e = allow_full_lds((const void*)k_chain_stream<NT0, KCH, ACT>, &lds_set);
    if (e != hipSuccess) return e;
    long grid = device_cu_count();
    if (grid > a.ntiles) grid = a.ntiles;
    hipLaunchKernelGGL((k_chain_stream<NT0, KCH, ACT>), dim3((unsigned)grid), dim3(CS_THREADS), lds, st, a);
    return hipGetLastError();
}

template <int NT0, int ACT>
static hipError_t launch_stream_a(const StreamArgs& a, hipStream_t st)
{
    switch ((a.K0 + CS_KC0 - 1) / CS_KC0) {
    case 1: return launch_stream_k<NT0, 1, ACT>(a, st);
    case 4: return launch_stream_k<NT0, 4, ACT>(a, st);
    case 9: return launch_stream_k<NT0, 9, ACT>(a, st);
    }
    return launch_stream_k<NT0, 0, ACT>(a, st);
}

template <int NT0>
static hipError_t launch_stream_n(const StreamArgs& a, int act, hipStream_t st)
{
    if (act == ACT_GELU_TANH) return launch_stream_a<NT0, ACT_GELU_TANH>(a, st);
    if (act == ACT_HARDSWISH) return launch_stream_a<NT0, ACT_HARDSWISH>(a, st);
    if (act == ACT_RELU) return launch_stream_a<NT0, ACT_RELU>(a, st);
    return launch_stream_a<NT0, ACT_NONE>(a, st);
}

static hipError_t launch_stream(const StreamArgs& a, int act, hipStream_t st)
{
    if (a.N0 <= 64) return launch_stream_n<2>(a, act, st);
    if (a.N0 <= 128) return launch_stream_n<4>(a, act, st);
    if (a.N0 <= 256) return launch_stream_n<8>(a, act, st);
    return hipErrorInvalidValue;
}

hipError_t run_stream(const StreamArgs& a, int act, hipStream_t st) { return launch_stream(a, act, st); }

}  // namespace fc
