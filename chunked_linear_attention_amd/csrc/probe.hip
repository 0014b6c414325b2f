// Measurement helper (not part of the TTT path): a loop of independent bf16
// matrix-core products, from which a benchmark reads the dense bf16 MFMA
// rate this part reaches, to quote roofline fractions against a measured peak
// beside the published one.
#include "../../include/ttt.h"
#include "ttt_device.h"

namespace tttk {

// Every wave keeps four independent 32x32x16 accumulations in flight, so the
// matrix pipe never waits on a dependent result (on gfx950 this shape reaches
// about 1.6x the rate of the 16x16x32 one, measured with the same loop, so it
// is the one that shows the part's dense bf16 ceiling).  Operands come from
// the lane index (never zero, so nothing is folded away); the sum of the
// accumulators is written so the loop cannot be removed.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) void probe_mfma_loop(float *out, int iters)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(1.0f + 0.001f * (lane + j));
        b[j] = (__bf16)(1.0f - 0.001f * (lane + 2 * j));
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace tttk

extern "C" ttt_status ttt_probe_mfma_bf16(float *out, int blocks, int iters, void *stream)
{
    if (!out || blocks < 1 || iters < 1 || blocks > (1 << 20)) return TTT_EINVAL;
    tttk::probe_mfma_loop<<<dim3(blocks), dim3(256), 0, (hipStream_t)stream>>>(out, iters);
    return hipGetLastError() == hipSuccess ? TTT_OK : TTT_EHIP;
}
