// gemm_rf.hip -- instantiations of the register-resident chain kernel
// (chain_rf.h) for dense rows: the two-GEMM chain (RF variant) and the
// N-stage chains.  Kept apart from the other kernels so that the sources
// compile in parallel.
#include "chain_rf.h"

namespace fc {

hipError_t run_rf_dense(const half_t* A, const RfArgs& a, int nmid, hipStream_t st)
{
    const int nt0 = (a.N0 + 31) / 32;
    if (a.K0 == 64 || a.K0 == 256 || a.K0 == 576) {   // compile-time chunk counts: quad-coalesced rows
        DenseRowsQ ld;
        ld.A = A; ld.M = a.M; ld.K = a.K0;
        if (nmid == 0) return launch_rf(ld, a, nt0, st);
        return nmid == 1 ? launch_rf<DenseRowsQ, 1>(ld, a, nt0, st) : launch_rf<DenseRowsQ, 2>(ld, a, nt0, st);
    }
    DenseRows ld;
    ld.A = A; ld.M = a.M; ld.K = a.K0;
    if (nmid == 0) return launch_rf(ld, a, nt0, st);
    return nmid == 1 ? launch_rf<DenseRows, 1>(ld, a, nt0, st) : launch_rf<DenseRows, 2>(ld, a, nt0, st);
}

}  // namespace fc
