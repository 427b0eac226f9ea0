// Instantiations of the skinny kernel: (rows, columns, waves splitting K).
#include "internal.hpp"

namespace dg {
namespace {
template <int DT, int MR, int NB, int W>
hipError_t go(const GemmArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.nblk + NB - 1) / NB));
    if (a.ep.on)
        return launch_args(&gemm_skinny_kernel<DT, MR, NB, W, true>, grid, dim3(64 * W), a, s);
    return launch_args(&gemm_skinny_kernel<DT, MR, NB, W, false>, grid, dim3(64 * W), a, s);
}

template <int DT>
hipError_t dispatch(int tm, int tn, int waves, const GemmArgs& a, hipStream_t s)
{
#define DG_CASE(M_, N_, W_) \
    if (tm == M_ && tn == N_ && waves == W_) return go<DT, M_ / 16, N_ / 16, W_>(a, s);
    DG_SKINNY_LADDER(DG_CASE)
#undef DG_CASE
    return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_skinny(int dt, int tm, int tn, int waves, const GemmArgs& a, hipStream_t s)
{
    return dt == DT_BF16 ? dispatch<DT_BF16>(tm, tn, waves, a, s)
                         : dispatch<DT_FP8>(tm, tn, waves, a, s);
}
}  // namespace dg
