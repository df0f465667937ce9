// gemm_stream.hip -- instantiations of the streamed-weight chain kernel
// (chain_stream.h).  Kept apart from the other kernels so that the sources
// compile in parallel.
#include "chain_stream.h"

namespace fc {

hipError_t run_stream(const StreamArgs& a, int act, hipStream_t st) { return launch_stream(a, act, st); }

}  // namespace fc
