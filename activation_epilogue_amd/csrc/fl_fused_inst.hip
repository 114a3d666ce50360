// fl_fused_inst.hip -- instantiates the fused GEMM kernels of one dtype.
// Built once per dtype with -DFL_INST_DTYPE=<fl_dtype value>.
#include "fl_kernels.hpp"
#include "fl_dma16.hpp"

#ifndef FL_INST_DTYPE
#error "define FL_INST_DTYPE"
#endif

namespace fl {
namespace {

template <int DT, int ACT, bool V>
void launch(const GemmArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((fused_linear_kernel<DT, ACT, V>), dim3(grid), dim3(kThreads), 0, s, a);
}

}  // namespace

template <int DT, int ACT, int BK, int BN, int WAVES_N, int OCC, bool RES, bool M16>
void launch_dma(const GemmArgs &a, int grid, hipStream_t s) {
    if constexpr (DT != FL_F32)
        hipLaunchKernelGGL((fused_linear_dma16_kernel<DT, ACT, BK, BN, WAVES_N, kCopySpread, OCC, RES, -1, DT, M16>),
                           dim3(grid), dim3(Dma16<DT, ACT, BK, BN, WAVES_N, 1, 1, false, -1, DT, false, M16>::THREADS),
                           0, s, a);
}

template <int DT, int BK, int BN, int WAVES_N, int OCC, bool RES, bool M16>
fused_launcher pick_dma_res(int act) {
    switch (act) {
    case FL_ACT_NONE: return launch_dma<DT, FL_ACT_NONE, BK, BN, WAVES_N, OCC, RES, M16>;
    case FL_ACT_RELU: return launch_dma<DT, FL_ACT_RELU, BK, BN, WAVES_N, OCC, RES, M16>;
    case FL_ACT_GELU_TANH: return launch_dma<DT, FL_ACT_GELU_TANH, BK, BN, WAVES_N, OCC, RES, M16>;
    default: return launch_dma<DT, FL_ACT_GLU, BK, BN, WAVES_N, OCC, RES, M16>;
    }
}

template <int DT, int BK, int BN, int WAVES_N = 2, int OCC = 1, bool M16 = false>
fused_launcher pick_dma(int act, bool residual) {
    return residual ? pick_dma_res<DT, BK, BN, WAVES_N, OCC, true, M16>(act)
                    : pick_dma_res<DT, BK, BN, WAVES_N, OCC, false, M16>(act);
}

template <>
fused_launcher pick_fused_for<FL_INST_DTYPE>(int act, bool vec, int variant, bool residual) {
    constexpr int DT = FL_INST_DTYPE;
    if constexpr (DT != FL_F32) {
        switch (variant) {
        case kDirect64x256: return pick_dma<DT, 64, 256>(act, residual);
        case kDirect32x256: return pick_dma<DT, 32, 256>(act, residual);
        case kDirect64x128: return pick_dma<DT, 64, 128>(act, residual);
        case kDirect64x256W8: return pick_dma<DT, 64, 256, 4>(act, residual);
        case kDirect32x128Occ2: return pick_dma<DT, 32, 128, 2, 2>(act, residual);
        case kDirect64x192: return pick_dma<DT, 64, 192>(act, residual);
        case kDirect32x192: return pick_dma<DT, 32, 192>(act, residual);
        case kDirect64x256M16: return pick_dma<DT, 64, 256, 2, 1, true>(act, residual);
        case kDirect64x256W8M16: return pick_dma<DT, 64, 256, 4, 1, true>(act, residual);
        case kDirect64x192M16: return pick_dma<DT, 64, 192, 2, 1, true>(act, residual);
        case kDirect64x128M16: return pick_dma<DT, 64, 128, 2, 1, true>(act, residual);
        case kDirect32x256M16: return pick_dma<DT, 32, 256, 2, 1, true>(act, residual);
        case kDirect32x256W8M16: return pick_dma<DT, 32, 256, 4, 1, true>(act, residual);
        case kDirect64x192W8M16: return pick_dma<DT, 64, 192, 4, 1, true>(act, residual);
        default: break;
        }
    }
    switch (act) {
    case FL_ACT_NONE: return vec ? launch<DT, FL_ACT_NONE, true> : launch<DT, FL_ACT_NONE, false>;
    case FL_ACT_RELU: return vec ? launch<DT, FL_ACT_RELU, true> : launch<DT, FL_ACT_RELU, false>;
    case FL_ACT_GELU_TANH: return vec ? launch<DT, FL_ACT_GELU_TANH, true> : launch<DT, FL_ACT_GELU_TANH, false>;
    default: return vec ? launch<DT, FL_ACT_GLU, true> : launch<DT, FL_ACT_GLU, false>;
    }
}

}  // namespace fl
