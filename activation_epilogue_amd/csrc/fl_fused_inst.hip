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

template <int DT, int ACT, int BK>
void launch_dma(const GemmArgs &a, int grid, hipStream_t s) {
    if constexpr (DT != FL_F32)
        hipLaunchKernelGGL((fused_linear_dma16_kernel<DT, ACT, BK>), dim3(grid), dim3(kThreads), 0, s, a);
}

template <int DT, int ACT>
void launch_stg(const GemmArgs &a, int grid, hipStream_t s) {
    if constexpr (DT != FL_F32)
        hipLaunchKernelGGL((fused_linear_stg16_kernel<DT, ACT>), dim3(grid), dim3(kThreads), 0, s, a);
}

template <>
fused_launcher pick_fused_for<FL_INST_DTYPE>(int act, bool vec, int variant) {
    constexpr int DT = FL_INST_DTYPE;
    // fp16/bf16 with 16-byte aligned operands use the direct-to-LDS kernel
    // (64-deep K stages, or 32-deep with variant 2) unless the register-staged
    // one is requested (variant 1).
    if (DT != FL_F32 && vec && variant == 3) {
        switch (act) {
        case FL_ACT_NONE: return launch_stg<DT, FL_ACT_NONE>;
        case FL_ACT_RELU: return launch_stg<DT, FL_ACT_RELU>;
        case FL_ACT_GELU_TANH: return launch_stg<DT, FL_ACT_GELU_TANH>;
        default: return launch_stg<DT, FL_ACT_GLU>;
        }
    }
    if (DT != FL_F32 && vec && variant != 1) {
        const bool bk32 = variant == 2;
        switch (act) {
        case FL_ACT_NONE: return bk32 ? launch_dma<DT, FL_ACT_NONE, 32> : launch_dma<DT, FL_ACT_NONE, 64>;
        case FL_ACT_RELU: return bk32 ? launch_dma<DT, FL_ACT_RELU, 32> : launch_dma<DT, FL_ACT_RELU, 64>;
        case FL_ACT_GELU_TANH:
            return bk32 ? launch_dma<DT, FL_ACT_GELU_TANH, 32> : launch_dma<DT, FL_ACT_GELU_TANH, 64>;
        default: return bk32 ? launch_dma<DT, FL_ACT_GLU, 32> : launch_dma<DT, FL_ACT_GLU, 64>;
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
