#include "internal.hpp"

namespace dg {
namespace {
template <int DT, int MR, int NB>
hipError_t go(const GemmArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.nblk + NB - 1) / NB));
    return launch_args(&gemm_skinny_kernel<DT, MR, NB>, grid, dim3(256), a, s);
}

template <int DT>
hipError_t dispatch(int tm, int tn, const GemmArgs& a, hipStream_t s)
{
#define DG_CASE(M_, N_) if (tm == M_ && tn == N_) return go<DT, M_ / 16, N_ / 16>(a, s);
    DG_CASE(16, 16) DG_CASE(16, 32) DG_CASE(16, 64)
    DG_CASE(32, 16) DG_CASE(32, 32) DG_CASE(32, 64)
    DG_CASE(48, 16) DG_CASE(48, 32) DG_CASE(48, 64)
    DG_CASE(64, 16) DG_CASE(64, 32) DG_CASE(64, 64)
#undef DG_CASE
    return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_skinny(int dt, int tm, int tn, const GemmArgs& a, hipStream_t s)
{
    return dt == DT_BF16 ? dispatch<DT_BF16>(tm, tn, a, s) : dispatch<DT_FP8>(tm, tn, a, s);
}
}  // namespace dg
