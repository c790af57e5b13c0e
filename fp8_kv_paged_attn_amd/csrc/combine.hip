// combine.hip - FP32 combination of split partials into FP16 rows.
//
// Design note "DFlash2 E4M3 attention with FP32 state", first section: the
// partition numerators stay unnormalised in FP32 with a separate FP32 max and
// sum, and the combination is FP32; the final activation is FP16.  The V
// dequantisation scale is applied here, once, as the output scale (vLLM PR
// "Qwen4Exp: fp8_e4m3 main KV cache on the QSA path", review thread on
// host-side KV scales).
//
// For a row with split partials (m_s, l_s, acc_s) (base-2 max, sum and
// numerator relative to m_s), the result is
//     M = max over non-empty splits (l_s > 0) of m_s
//     o = out_scale * sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// with empty splits weighted 0 (so -inf - -inf never forms) and o = 0 when
// every split is empty.
//
// One workgroup per (row, 64-column chunk): 16 float4 column lanes x 16 split
// groups.  Split group k takes splits k, k+16, k+32, ...; all of a thread's
// loads are issued before any is used (one memory round trip), and the thread
// merges its splits online against its own running max.  The 16 groups are
// then merged through LDS in a fixed order.  All arithmetic is FP32.
#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kLanes = 16;                 // float4 column lanes: 64 columns
constexpr int kGroups = kThreads / kLanes; // split groups
constexpr int kBatch = 16;                 // splits per group loaded at once

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void combine_kernel(const float *__restrict__ acc,
                                                           const float *__restrict__ mx,
                                                           const float *__restrict__ sm,
                                                           int S, int R, int D,
                                                           float out_scale,
                                                           uint16_t *__restrict__ out)
{
    __shared__ float gm[kGroups][kLanes];
    __shared__ float gl[kGroups][kLanes];
    __shared__ f32x4 gn[kGroups][kLanes];

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid % kLanes, grp = tid / kLanes;
    const int d0 = blockIdx.y * (4 * kLanes) + 4 * lane;
    const bool col_ok = d0 < D;          // D is a multiple of 4

    // running state of this thread's splits: max m, sum l, numerator num
    float m = -INFINITY, l = 0.0f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = grp; s0 < S; s0 += kGroups * kBatch) {
        float ms[kBatch], ls[kBatch];
        f32x4 vs[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int s = s0 + k * kGroups;
            ms[k] = -INFINITY;
            ls[k] = 0.0f;
            vs[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (s < S) {
                const int64_t i = (int64_t)s * R + r;
                ms[k] = mx[i];
                ls[k] = sm[i];
                if (col_ok)
                    vs[k] = *(const f32x4 *)(acc + i * D + d0);
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (ls[k] > 0.0f) {
                const float mn = fmaxf(m, ms[k]);
                const float a = exp2f(m - mn);        // 0 while m = -inf
                const float b = exp2f(ms[k] - mn);
                l = l * a + ls[k] * b;
                num = num * a + vs[k] * b;
                m = mn;
            }
        }
    }
    gm[grp][lane] = m;
    gl[grp][lane] = l;
    gn[grp][lane] = num;
    __syncthreads();
    if (grp == 0 && col_ok) {
        float M = gm[0][lane];
#pragma unroll
        for (int k = 1; k < kGroups; ++k)
            M = fmaxf(M, gm[k][lane]);
        float den = 0.0f;
        f32x4 tot = {0.f, 0.f, 0.f, 0.f};
        if (M != -INFINITY) {
#pragma unroll
            for (int k = 0; k < kGroups; ++k) {
                const float w = exp2f(gm[k][lane] - M);   // 0 for empty groups
                den += w * gl[k][lane];
                tot += w * gn[k][lane];
            }
        }
        uint16_t h[4];
        for (int k = 0; k < 4; ++k) {
            const float o = den > 0.0f ? (tot[k] / den) * out_scale : 0.0f;
            h[k] = __builtin_bit_cast(uint16_t, (_Float16)o);
        }
        uint2 packed = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
        *(uint2 *)(out + (int64_t)r * D + d0) = packed;
    }
}

}  // namespace

hipError_t launch_combine(const float *acc, const float *mx, const float *sm, int num_splits,
                          int num_rows, int head_dim, float out_scale, uint16_t *out,
                          hipStream_t stream)
{
    if (num_rows == 0)
        return hipSuccess;
    if (head_dim % 4 != 0)
        return hipErrorInvalidValue;
    dim3 grid(num_rows, (head_dim + 4 * kLanes - 1) / (4 * kLanes));
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, stream, acc, mx, sm, num_splits,
                       num_rows, head_dim, out_scale, out);
    return hipGetLastError();
}

}  // namespace pa
