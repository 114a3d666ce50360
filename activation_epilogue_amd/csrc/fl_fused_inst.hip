// fl_fused_inst.hip -- instantiates the fused GEMM kernels of one dtype.
// Built once per dtype with -DFL_INST_DTYPE=<fl_dtype value>.
#include "fl_kernels.hpp"

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

template <>
fused_launcher pick_fused_for<FL_INST_DTYPE>(int act, bool vec) {
    constexpr int DT = FL_INST_DTYPE;
    switch (act) {
    case FL_ACT_NONE: return vec ? launch<DT, FL_ACT_NONE, true> : launch<DT, FL_ACT_NONE, false>;
    case FL_ACT_RELU: return vec ? launch<DT, FL_ACT_RELU, true> : launch<DT, FL_ACT_RELU, false>;
    case FL_ACT_GELU_TANH: return vec ? launch<DT, FL_ACT_GELU_TANH, true> : launch<DT, FL_ACT_GELU_TANH, false>;
    default: return vec ? launch<DT, FL_ACT_GLU, true> : launch<DT, FL_ACT_GLU, false>;
    }
}

}  // namespace fl
