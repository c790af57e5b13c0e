// combine.hip - FP32 combination of split partials into FP16 rows.
//
// Design note "DFlash2 E4M3 attention with FP32 state", first section: the
// partition numerators stay unnormalised in FP32 with a separate FP32 max and
// sum, and the combination is FP32; the final activation is FP16.  The V
// dequantisation scale is applied here, once, as the output scale (vLLM PR
// "Qwen4Exp: fp8_e4m3 main KV cache on the QSA path", review thread on
// host-side KV scales).
//
// One workgroup per output row; thread d owns column d.  Split weights are
// w_s = 2^(m_s - M) with M the largest max among non-empty splits, so an
// empty split (m = -inf, l = 0) is skipped and -inf - -inf never forms.
#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void combine_kernel(const float *__restrict__ acc,
                                                           const float *__restrict__ mx,
                                                           const float *__restrict__ sm,
                                                           int S, int R, int D,
                                                           float out_scale,
                                                           uint16_t *__restrict__ out)
{
    const int r = blockIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) {
        float l = sm[(int64_t)s * R + r];
        float m = mx[(int64_t)s * R + r];
        if (l > 0.0f && m > M)
            M = m;
    }
    for (int d = threadIdx.x; d < D; d += kThreads) {
        float num = 0.0f, den = 0.0f;
        for (int s = 0; s < S; ++s) {
            int64_t k = (int64_t)s * R + r;
            float l = sm[k];
            if (!(l > 0.0f))
                continue;
            float w = exp2f(mx[k] - M);
            den += w * l;
            num += w * acc[k * D + d];
        }
        float o = den > 0.0f ? (num / den) * out_scale : 0.0f;
        out[(int64_t)r * D + d] = __builtin_bit_cast(uint16_t, (_Float16)o);
    }
}

}  // namespace

hipError_t launch_combine(const float *acc, const float *mx, const float *sm, int num_splits,
                          int num_rows, int head_dim, float out_scale, uint16_t *out,
                          hipStream_t stream)
{
    if (num_rows == 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3(num_rows), dim3(kThreads), 0, stream, acc, mx, sm,
                       num_splits, num_rows, head_dim, out_scale, out);
    return hipGetLastError();
}

}  // namespace pa
