// fl_fp8_inst.hip -- instantiates the FP8-input fused kernels for one 16-bit
// output dtype (A and B as OCP E4M3 codes, the scaled FP8 MFMAs, K stages of
// 128 so that an A row is the same 128 bytes as a 64-deep 16-bit stage; the
// two-per-CU kernel: stages of 64, 64-byte A rows as in its 16-bit form).
// Built once per output dtype with -DFL_INST_DTYPE=<fl_dtype value>.
#include "fl_kernels.hpp"
#include "fl_dma16.hpp"

#ifndef FL_INST_DTYPE
#error "define FL_INST_DTYPE"
#endif

namespace fl {
namespace {

template <int DT, int ACT, int BN, int WAVES_N, bool M16, int BK, int OCC>
void launch_f8(const GemmArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((fused_linear_dma16_kernel<DT, ACT, BK, BN, WAVES_N, kCopySpread, OCC, false, -1, kInFp8, M16>),
                       dim3(grid), dim3(Dma16<DT, ACT, BK, BN, WAVES_N, 1, OCC, false, -1, kInFp8, false, M16>::THREADS),
                       0, s, a);
}

template <int DT, int BN, int WAVES_N, bool M16 = false, int BK = 128, int OCC = 1>
fused_launcher pick_f8_act(int act) {
    switch (act) {
    case FL_ACT_NONE: return launch_f8<DT, FL_ACT_NONE, BN, WAVES_N, M16, BK, OCC>;
    case FL_ACT_RELU: return launch_f8<DT, FL_ACT_RELU, BN, WAVES_N, M16, BK, OCC>;
    case FL_ACT_GELU_TANH: return launch_f8<DT, FL_ACT_GELU_TANH, BN, WAVES_N, M16, BK, OCC>;
    default: return launch_f8<DT, FL_ACT_GLU, BN, WAVES_N, M16, BK, OCC>;
    }
}

}  // namespace

template <>
fused_launcher pick_fp8_for<FL_INST_DTYPE>(int act, int variant) {
    constexpr int DT = FL_INST_DTYPE;
    static_assert(DT != FL_F32, "FP8 inputs produce fp16 or bf16 outputs");
    switch (variant) {
    case kDirect64x256W8: return pick_f8_act<DT, 256, 4>(act);
    case kDirect64x256: return pick_f8_act<DT, 256, 2>(act);
    case kDirect64x128: return pick_f8_act<DT, 128, 2>(act);
    case kDirect64x128M16: return pick_f8_act<DT, 128, 2, true>(act);
    case kDirect64x192: return pick_f8_act<DT, 192, 2>(act);
    case kDirect32x128Occ2: return pick_f8_act<DT, 128, 2, false, 64, 2>(act);
    default: return nullptr;
    }
}

}  // namespace fl
