// mfma_probe.hip -- sustained MFMA rate of this GPU, for the roofline.
//
// A measurement aid, separate from the fused-linear library: every wave runs
// back-to-back v_mfma_f32_32x32x16_f16 on operands held in registers, with
// no memory traffic inside the loop, so the achieved rate is the matrix
// cores' sustained throughput at the clock the chip holds under that load.
// The operands are either small constants (few toggling bits) or random
// fp16 values with full mantissas; the matrix unit's power, and so the
// clock the chip can hold, depends on how many operand bits toggle.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 4 waves per workgroup, each with a 4x4 grid of 32x32 accumulators
// (16 independent MFMAs per iteration).
__global__ void __launch_bounds__(256, 1) mfma_probe_kernel(float *out, int iters, int random) {
    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    // xorshift32 per lane for the random operands
    uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 12345u;
    auto next = [&]() -> float {
        h ^= h << 13;
        h ^= h >> 17;
        h ^= h << 5;
        return ((float)(h & 0xffffu) / 32768.0f - 1.0f) * 0.0625f;
    };
    f16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float c = (float)((threadIdx.x + i + e) & 3) * 0.001f;
            a[i][e] = (_Float16)(random ? next() : c);
            b[i][e] = (_Float16)(random ? next() : c);
        }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[i][j][e];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Launches `grid` workgroups of 256 threads, each wave issuing 16*iters
// MFMAs (32*32*16*2 flop each).  out: device buffer of grid*256 floats
// (written once per thread so the work is not removed).  Returns 0, or the
// hipError_t of the launch.  Flops per launch: grid * 4 * 16 * iters * 32768.
int fl_probe_mfma(void *out, int grid, int iters, int random, void *stream) {
    if (!out || grid <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<float *>(out), iters, random);
    return (int)hipGetLastError();
}

}  // extern "C"
