// fl_quant_inst.hip -- instantiates the quantized-output fused kernels of one
// 16-bit dtype (the direct-to-LDS kernels the automatic tile choice uses).
// Built once per dtype with -DFL_INST_DTYPE=<fl_dtype value>.
#include "fl_kernels.hpp"
#include "fl_dma16.hpp"

#ifndef FL_INST_DTYPE
#error "define FL_INST_DTYPE"
#endif

namespace fl {
namespace {

template <int DT, int ACT, int BK, int BN, int WAVES_N, int OCC, int QF, bool M16>
void launch_q(const GemmArgs &a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((fused_linear_dma16_kernel<DT, ACT, BK, BN, WAVES_N, kCopySpread, OCC, false, QF, DT, M16>),
                       dim3(grid), dim3(Dma16<DT, ACT, BK, BN, WAVES_N, 1, 1, false, QF, DT, false, M16>::THREADS), 0,
                       s, a);
}

template <int DT, int BK, int BN, int WAVES_N, int OCC, int QF, bool M16>
fused_launcher pick_q_act(int act) {
    switch (act) {
    case FL_ACT_NONE: return launch_q<DT, FL_ACT_NONE, BK, BN, WAVES_N, OCC, QF, M16>;
    case FL_ACT_RELU: return launch_q<DT, FL_ACT_RELU, BK, BN, WAVES_N, OCC, QF, M16>;
    case FL_ACT_GELU_TANH: return launch_q<DT, FL_ACT_GELU_TANH, BK, BN, WAVES_N, OCC, QF, M16>;
    default: return launch_q<DT, FL_ACT_GLU, BK, BN, WAVES_N, OCC, QF, M16>;
    }
}

template <int DT, int BK, int BN, int WAVES_N, int OCC, bool M16 = false>
fused_launcher pick_q(int act, int qfmt) {
    return qfmt == FL_Q_INT8 ? pick_q_act<DT, BK, BN, WAVES_N, OCC, FL_Q_INT8, M16>(act)
                             : pick_q_act<DT, BK, BN, WAVES_N, OCC, FL_Q_FP8_E4M3, M16>(act);
}

}  // namespace

template <>
fused_launcher pick_quant_for<FL_INST_DTYPE>(int act, int variant, int qfmt) {
    constexpr int DT = FL_INST_DTYPE;
    static_assert(DT != FL_F32, "quantized output is built for the 16-bit input dtypes");
    switch (variant) {
    case kDirect64x256W8: return pick_q<DT, 64, 256, 4, 1>(act, qfmt);
    case kDirect64x128: return pick_q<DT, 64, 128, 2, 1>(act, qfmt);
    case kDirect32x128Occ2: return pick_q<DT, 32, 128, 2, 2>(act, qfmt);
    case kDirect64x192: return pick_q<DT, 64, 192, 2, 1>(act, qfmt);
    case kDirect64x256W8M16: return pick_q<DT, 64, 256, 4, 1, true>(act, qfmt);
    case kDirect64x128M16: return pick_q<DT, 64, 128, 2, 1, true>(act, qfmt);
    case kDirect64x192M16: return pick_q<DT, 64, 192, 2, 1, true>(act, qfmt);
    case kDirect64x192W8M16: return pick_q<DT, 64, 192, 4, 1, true>(act, qfmt);
    default: return nullptr;
    }
}

}  // namespace fl
