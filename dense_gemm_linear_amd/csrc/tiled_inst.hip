// Instantiations of the tiled kernels for one (element type, variant,
// family), chosen by the build: DG_INST_DT (DT_BF16 / DT_FP8), DG_INST_MODE
// (MODE_PLAIN / MODE_SPLIT / MODE_EPI / MODE_SK) and DG_INST_FAMILY (0: the tiled
// ladder, 1: the A+B and ping-pong ladders).  The build compiles this file
// once per combination, in parallel; each defines launch_inst_<dt>_<mode>_<family>,
// which launches rung idx of its ladders.
#include "internal.hpp"

#if !defined(DG_INST_DT) || !defined(DG_INST_MODE) || !defined(DG_INST_FAMILY)
#error "tiled_inst.hip is compiled with -DDG_INST_DT, -DDG_INST_MODE and -DDG_INST_FAMILY"
#endif

#define DG_INST_PASTE_(d, m, f) launch_inst_##d##_##m##_##f
#define DG_INST_PASTE(d, m, f) DG_INST_PASTE_(d, m, f)
#define DG_INST_FN DG_INST_PASTE(DG_INST_DT, DG_INST_MODE, DG_INST_FAMILY)

namespace dg {
namespace {
constexpr int DT = DG_INST_DT;
constexpr int MODE = DG_INST_MODE;

// split-K: tiles x slices workgroups; stream-K: a persistent grid, one
// workgroup per CU (a.splits carries the grid size)
dim3 grid_of(const GemmArgs& a)
{
    if (MODE == MODE_SK)
        return dim3((unsigned)a.splits);
    return dim3((unsigned)(a.tiles_m * a.tiles_n * (MODE == MODE_SPLIT ? a.splits : 1)));
}

// Stream-K instances exist for outputs of 128 x 128 to 128 x 256 only
// (sk_rung), and e4m3 16 x 16 atoms (128 K bytes per MFMA) only with
// 128-byte k-tiles (atom_fits); other rungs answer hipErrorInvalidValue.

#if DG_INST_FAMILY == 0
template <int TM, int TN, int WM, int ST, int R, int KTB>
hipError_t go(const GemmArgs& a, hipStream_t s)
{
    if constexpr ((MODE == MODE_SK && !sk_rung(TM, TN)) || !atom_fits<DT, R, KTB>()) {
        return hipErrorInvalidValue;
    } else {
        return launch_args(&gemm_tiled_kernel<DT, TM, TN, WM, ST, R, KTB, MODE>, grid_of(a),
                           dim3(TiledShape<TM, TN, WM, ST, R, KTB>::THREADS), a, s);
    }
}
#else
// The 4-wave 256 x 256 e4m3 rung with 32 x 32 atoms and four 64-byte stages
// runs its plain and fused-epilogue launches on the kernel with whole-line A
// loads (same results bit for bit: the same MFMAs in the same order).
template <int TM, int TN, int WM, int WN, int ST, int R, int KTB>
constexpr bool ab_line_rung()
{
    return DT == DT_FP8 && TM == 256 && TN == 256 && WM == 2 && WN == 2 && ST == 4 && R == 32 &&
           KTB == 64 && (MODE == MODE_PLAIN || MODE == MODE_EPI);
}

template <int TM, int TN, int WM, int WN, int ST, int R, int KTB>
hipError_t go_ab(const GemmArgs& a, hipStream_t s)
{
    if constexpr ((MODE == MODE_SK && !sk_rung(TM, TN)) || !atom_fits<DT, R, KTB>()) {
        return hipErrorInvalidValue;
    } else if constexpr (ab_line_rung<TM, TN, WM, WN, ST, R, KTB>()) {
        return launch_args(&gemm_ab_line_kernel<DT, R, WM, WN, MODE == MODE_EPI>, grid_of(a),
                           dim3(64 * WM * WN), a, s);
    } else {
        return launch_args(&gemm_ab_kernel<DT, TM, TN, WM, WN, ST, R, KTB, MODE>, grid_of(a),
                           dim3(ABShape<TM, TN, WM, WN, ST, R, KTB>::THREADS), a, s);
    }
}
template <int TM, int TN, int ST, int R, int KTB>
hipError_t go_pp(const GemmArgs& a, hipStream_t s)
{
    if constexpr (MODE == MODE_SK) {
        return hipErrorInvalidValue;
    } else {
        return launch_args(&gemm_pp_kernel<DT, TM, TN, ST, R, KTB, MODE>, grid_of(a), dim3(512), a,
                           s);
    }
}
#endif
}  // namespace

hipError_t DG_INST_FN(int kernel, int idx, const GemmArgs& a, hipStream_t s)
{
    int i = 0;
#if DG_INST_FAMILY == 0
    (void)kernel;
#define DG_CASE(M_, N_, W_, ST_, R_, KTB_) \
    if (idx == i++) return go<M_, N_, W_ / 4, ST_, R_, KTB_>(a, s);
    DG_TILED_LADDER(DG_CASE)
#undef DG_CASE
#else
    if (kernel == GEMM_KERNEL_TILED_AB) {
#define DG_CASE(M_, N_, WM_, WN_, ST_, R_, KTB_) \
    if (idx == i++) return go_ab<M_, N_, WM_, WN_, ST_, R_, KTB_>(a, s);
        DG_AB_LADDER(DG_CASE)
#undef DG_CASE
    } else {
#define DG_CASE(M_, N_, ST_, R_, KTB_) \
    if (idx == i++) return go_pp<M_, N_, ST_, R_, KTB_>(a, s);
        DG_PP_LADDER(DG_CASE)
#undef DG_CASE
    }
#endif
    return hipErrorInvalidValue;
}
}  // namespace dg
