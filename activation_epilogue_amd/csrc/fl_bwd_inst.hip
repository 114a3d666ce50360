// fl_bwd_inst.hip -- instantiates the backward-epilogue kernels for one
// 16-bit dtype: D = A @ B^T with B given as (N, K) row-major, dX = D *
// act'(Xs), the gate's dY = D * Xs, dbias += column sums of dX.  The 8-wave
// 256x256 tile, and 256x128 where the forward choice would take a narrower
// tile.  Built once per dtype with -DFL_INST_DTYPE=<fl_dtype value>.
#include "fl_kernels.hpp"
#include "fl_dma16.hpp"

#ifndef FL_INST_DTYPE
#error "define FL_INST_DTYPE"
#endif

namespace fl {
namespace {

template <int DT, int ACT, int BN, int WAVES_N, bool M16>
void launch_bwd(const GemmArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((fused_linear_bwd_kernel<DT, ACT, 64, BN, WAVES_N, M16>), dim3(grid),
                       dim3(Dma16<DT, ACT, 64, BN, WAVES_N>::THREADS), 0, s, a);
}

template <int DT, int BN, int WAVES_N, bool M16 = false>
fused_launcher pick_bwd_act(int act) {
    switch (act) {
    case FL_ACT_NONE: return launch_bwd<DT, FL_ACT_NONE, BN, WAVES_N, M16>;
    case FL_ACT_RELU: return launch_bwd<DT, FL_ACT_RELU, BN, WAVES_N, M16>;
    case FL_ACT_GELU_TANH: return launch_bwd<DT, FL_ACT_GELU_TANH, BN, WAVES_N, M16>;
    default: return launch_bwd<DT, FL_ACT_GLU, BN, WAVES_N, M16>;
    }
}

}  // namespace

template <>
fused_launcher pick_bwd_for<FL_INST_DTYPE>(int act, int variant) {
    constexpr int DT = FL_INST_DTYPE;
    static_assert(DT != FL_F32, "the backward epilogue is built for the 16-bit dtypes");
    switch (variant) {
    case kDirect64x256W8: return pick_bwd_act<DT, 256, 4>(act);
    case kDirect64x128: return pick_bwd_act<DT, 128, 2>(act);
    case kDirect64x256W8M16: return pick_bwd_act<DT, 256, 4, true>(act);
    case kDirect64x128M16: return pick_bwd_act<DT, 128, 2, true>(act);
    default: return nullptr;
    }
}

}  // namespace fl
