// combine.hip - FP32 combination of split partials into FP16 rows.
//
// Design note "DFlash2 E4M3 attention with FP32 state", first section: the
// partition numerators stay unnormalised in FP32 with a separate FP32 max and
// sum, and the combination is FP32; the final activation is FP16.  The V
// dequantisation scale is applied here, once, as the output scale (vLLM PR
// "Qwen4Exp: fp8_e4m3 main KV cache on the QSA path", review thread on
// host-side KV scales).
//
// Split weights are w_s = 2^(m_s - M) with M the largest max among non-empty
// splits (l_s > 0); empty splits get weight 0 and are skipped, so -inf - -inf
// never forms, and a row whose splits are all empty is written as 0.
//
// One workgroup per (row, 64-column chunk): 16 column lanes x 16 split groups.
// The weights of 256 splits at a time are computed once into LDS, each thread
// accumulates float4 columns over its splits, and the 16 split groups are
// summed through LDS.  The split sums are plain FP32 sums in a fixed order.
#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kLanes = 16;                 // float4 column lanes: 64 columns
constexpr int kGroups = kThreads / kLanes; // split groups

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void combine_kernel(const float *__restrict__ acc,
                                                           const float *__restrict__ mx,
                                                           const float *__restrict__ sm,
                                                           int S, int R, int D,
                                                           float out_scale,
                                                           uint16_t *__restrict__ out)
{
    __shared__ float red[kThreads];
    __shared__ float wts[kThreads];
    __shared__ f32x4 part[kGroups][kLanes];

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid % kLanes, grp = tid / kLanes;
    const int d0 = blockIdx.y * (4 * kLanes) + 4 * lane;

    // M = max over non-empty splits
    float m = -INFINITY;
    for (int s = tid; s < S; s += kThreads) {
        const int64_t k = (int64_t)s * R + r;
        if (sm[k] > 0.0f)
            m = fmaxf(m, mx[k]);
    }
    red[tid] = m;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (tid < off)
            red[tid] = fmaxf(red[tid], red[tid + off]);
        __syncthreads();
    }
    const float M = red[0];
    __syncthreads();

    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    float den_part = 0.0f;
    const bool col_ok = d0 < D;          // D is a multiple of 4
    for (int s0 = 0; s0 < S; s0 += kThreads) {
        const int s = s0 + tid;
        float w = 0.0f;
        if (s < S) {
            const int64_t k = (int64_t)s * R + r;
            const float l = sm[k];
            if (l > 0.0f) {
                w = exp2f(mx[k] - M);
                den_part += w * l;
            }
        }
        wts[tid] = w;
        __syncthreads();
        const int cnt = min(kThreads, S - s0);
        if (col_ok) {
            for (int j = grp; j < cnt; j += kGroups) {
                const float wj = wts[j];
                if (wj != 0.0f) {
                    const f32x4 v = *(const f32x4 *)(acc + ((int64_t)(s0 + j) * R + r) * D + d0);
                    num += wj * v;
                }
            }
        }
        __syncthreads();
    }
    red[tid] = den_part;
    part[grp][lane] = num;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (tid < off)
            red[tid] += red[tid + off];
        __syncthreads();
    }
    if (grp == 0 && col_ok) {
        f32x4 tot = part[0][lane];
        for (int gq = 1; gq < kGroups; ++gq)
            tot += part[gq][lane];
        const float den = red[0];
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
