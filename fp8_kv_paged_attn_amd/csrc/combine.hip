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
//     M = max over non-empty splits (l_s != 0) of m_s
//     o = out_scale * sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// with empty splits (l_s = 0) weighted 0, so -inf - -inf never forms, and
// o = 0 when every split is empty.  A split whose sum is NaN (NaN bytes at
// positions a row sees) is not empty: the NaN reaches the row, as it does in
// the unsplit definition.
//
// A thread owns one float4 of columns of one row and a group of its splits
// (splits g, g + GROUPS, ...).  A workgroup of 256 threads covers 64 columns of
// 16 / GROUPS rows.  All loads of a batch are issued before any is used (one
// memory round trip per batch of BATCH splits).  The thread takes the batch's
// largest max first and then weights every split against it, so the
// exponentials of a batch are independent of each other instead of forming
// one chain of pairwise merges.  The GROUPS states of a row's float4 are
// combined the same way through LDS: the row max over the groups, each group
// rescaled to it, and the rescaled sums added in group order.  GROUPS is
// chosen on the host so that the grid has about 128 K threads: many splits
// over few rows (one request, long context) get 16 groups; many rows over few
// splits (a batch of sparse requests) get 1 or 2.  All arithmetic is FP32.
//
// The same kernel can also write the unrounded FP32 output and the base-2 LSE
// of each row, M + log2(sum_s w_s l_s), for a merge across ranks (1Cat-vLLM PR
// "Qualify calibrated E4M3 and disk PLE with QSA DCP2": base-2 LSE and FP32
// partial output exported for cross-rank merging).
//
// Partials come in one of two layouts.  Uniform: split s of output row r is
// element s * R + r.  Ragged (a batch whose splits follow the lengths):
// output row r = (b, i, h) belongs to KV unit u = b * Hkv + h / G as unit row
// ru = i * G + h % G; its splits are index[u] .. index[u + 1] - 1, and split
// s is element s * (q_rows * G) + ru.
#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kLanes = 16;                 // float4 column lanes: 64 columns
constexpr int kTargetThreads = 131072;

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct RaggedRows {
    const int32_t *index;   // null: uniform layout
    int q_rows, heads, group, hkv;
};

template <int GROUPS, int BATCH>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float *__restrict__ acc,
                                                           const float *__restrict__ mx,
                                                           const float *__restrict__ sm,
                                                           int S, int R, int D,
                                                           float out_scale,
                                                           uint16_t *__restrict__ out,
                                                           float *__restrict__ out32,
                                                           float *__restrict__ lse,
                                                           RaggedRows rg)
{
    constexpr int kRowsPerWG = kThreads / (kLanes * GROUPS);
    __shared__ float gm[GROUPS > 1 ? kThreads : 1];
    __shared__ float gl[GROUPS > 1 ? kThreads : 1];
    __shared__ f32x4 gn[GROUPS > 1 ? kThreads : 1];

    const int tid = threadIdx.x;
    const int lane = tid % kLanes;
    const int grp = (tid / kLanes) % GROUPS;
    const int rsub = tid / (kLanes * GROUPS);
    const int r = blockIdx.x * kRowsPerWG + rsub;
    const int d0 = blockIdx.y * (4 * kLanes) + 4 * lane;
    const bool ok = r < R && d0 < D;          // D is a multiple of 4

    // this row's splits: first, count, and the element stride and offset
    int first = 0, count = S, stride = R, rrow = r;
    if (rg.index && ok) {
        const int per_req = rg.q_rows * rg.heads;
        const int rb = r / per_req, rem = r - rb * per_req;
        const int i = rem / rg.heads, h = rem - i * rg.heads;
        const int u = rb * rg.hkv + h / rg.group;
        first = rg.index[u];
        count = rg.index[u + 1] - first;
        stride = rg.q_rows * rg.group;
        rrow = i * rg.group + h % rg.group;
    }

    // running state of this thread's splits: max m, sum l, numerator num
    float m = -INFINITY, l = 0.0f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    if (ok) {
        for (int s0 = grp; s0 < count; s0 += GROUPS * BATCH) {
            float ms[BATCH], ls[BATCH];
            f32x4 vs[BATCH];
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const int s = s0 + k * GROUPS;
                ms[k] = -INFINITY;
                ls[k] = 0.0f;
                vs[k] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (s < count) {
                    const int64_t i = (int64_t)(first + s) * stride + rrow;
                    ms[k] = mx[i];
                    ls[k] = sm[i];
                    vs[k] = *(const f32x4 *)(acc + i * D + d0);
                }
            }
            // the batch's largest max among non-empty splits (empty: l = 0; a
            // NaN sum is kept), then every split weighted against it at once
            // (an empty split's numerator is never multiplied, whatever it holds)
            float bm = m;
#pragma unroll
            for (int k = 0; k < BATCH; ++k)
                bm = ls[k] != 0.0f ? fmaxf(bm, ms[k]) : bm;
            const float a = (m == -INFINITY) ? 0.0f : exp2f(m - bm);
            l *= a;
            num *= a;
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const float wk = (ms[k] == -INFINITY) ? 0.0f : exp2f(ms[k] - bm);
                if (ls[k] != 0.0f) {
                    l += wk * ls[k];
                    num += wk * vs[k];
                }
            }
            m = bm;
        }
    }
    if (GROUPS > 1) {
        // the row's max over the groups, each group rescaled to it, and the
        // rescaled sums added in group order
        const int base = rsub * kLanes * GROUPS + lane;
        gm[tid] = m;
        __syncthreads();
        float M = gm[base];
#pragma unroll
        for (int k = 1; k < GROUPS; ++k)
            M = fmaxf(M, gm[base + k * kLanes]);
        const float f = (m == -INFINITY) ? 0.0f : exp2f(m - M);
        gl[tid] = l * f;
        gn[tid] = num * f;
        __syncthreads();
        if (grp != 0)
            return;
        m = M;
        l = gl[base];
        num = gn[base];
#pragma unroll
        for (int k = 1; k < GROUPS; ++k) {
            l += gl[base + k * kLanes];
            num += gn[base + k * kLanes];
        }
    }
    if (ok) {
        f32x4 o;
        for (int k = 0; k < 4; ++k)
            o[k] = l != 0.0f ? (num[k] / l) * out_scale : 0.0f;
        if (out) {
            uint16_t h[4];
            for (int k = 0; k < 4; ++k)
                h[k] = __builtin_bit_cast(uint16_t, (_Float16)o[k]);
            uint2 packed = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
            *(uint2 *)(out + (int64_t)r * D + d0) = packed;
        }
        if (out32)
            *(f32x4 *)(out32 + (int64_t)r * D + d0) = o;
        // every column chunk of the row holds the same (m, l); chunk 0 writes
        if (lse && blockIdx.y == 0 && lane == 0)
            lse[r] = l != 0.0f ? m + log2f(l) : -INFINITY;
    }
}

template <int GROUPS, int BATCH>
hipError_t launch_g(const float *acc, const float *mx, const float *sm, int num_splits,
                    int num_rows, int head_dim, float out_scale, uint16_t *out, float *out32,
                    float *lse, RaggedRows rg, hipStream_t stream)
{
    constexpr int kRowsPerWG = kThreads / (kLanes * GROUPS);
    dim3 grid((num_rows + kRowsPerWG - 1) / kRowsPerWG, (head_dim + 4 * kLanes - 1) / (4 * kLanes));
    hipLaunchKernelGGL((combine_kernel<GROUPS, BATCH>), grid, dim3(kThreads), 0, stream, acc, mx,
                       sm, num_splits, num_rows, head_dim, out_scale, out, out32, lse, rg);
    return hipGetLastError();
}

// splits_per_row: the splits one row combines (ragged: an estimate, the
// total over the units' count), which sizes the split groups
hipError_t launch_any(const float *acc, const float *mx, const float *sm, int num_splits,
                      int splits_per_row, int num_rows, int head_dim, float out_scale,
                      uint16_t *out, float *out32, float *lse, RaggedRows rg, hipStream_t stream)
{
    if (num_rows == 0)
        return hipSuccess;
    if (head_dim % 4 != 0)
        return hipErrorInvalidValue;
    // split groups per (row, float4): double while the grid stays under the
    // target thread count and every group has a split
    const int64_t base = (int64_t)num_rows * ((head_dim + 63) / 64) * kLanes;
    int groups = 1;
    while (groups < 16 && groups < splits_per_row && base * groups * 2 <= kTargetThreads)
        groups *= 2;
    const bool big = (splits_per_row + groups - 1) / groups > 8;   // splits per thread
#define PA_COMBINE(G)                                                                          \
    return big ? launch_g<G, 16>(acc, mx, sm, num_splits, num_rows, head_dim, out_scale, out,  \
                                 out32, lse, rg, stream)                                       \
               : launch_g<G, 8>(acc, mx, sm, num_splits, num_rows, head_dim, out_scale, out,   \
                                out32, lse, rg, stream)
    switch (groups) {
    case 1: PA_COMBINE(1);
    case 2: PA_COMBINE(2);
    case 4: PA_COMBINE(4);
    case 8: PA_COMBINE(8);
    default: PA_COMBINE(16);
    }
#undef PA_COMBINE
}

}  // namespace

hipError_t launch_combine(const float *acc, const float *mx, const float *sm, int num_splits,
                          int num_rows, int head_dim, float out_scale, uint16_t *out,
                          float *out32, float *lse, hipStream_t stream)
{
    return launch_any(acc, mx, sm, num_splits, num_splits, num_rows, head_dim, out_scale, out,
                      out32, lse, RaggedRows{nullptr, 0, 0, 0, 0}, stream);
}

hipError_t launch_combine_ragged(const float *acc, const float *mx, const float *sm,
                                 const int32_t *index, int num_splits, int batch, int q_rows,
                                 int num_heads, int num_kv_heads, int head_dim, float out_scale,
                                 uint16_t *out, float *out32, float *lse, hipStream_t stream)
{
    const int64_t rows = (int64_t)batch * q_rows * num_heads;
    const int64_t units = (int64_t)batch * num_kv_heads;
    const int per_row = (int)((num_splits + units - 1) / units);
    return launch_any(acc, mx, sm, num_splits, per_row < 1 ? 1 : per_row, (int)rows, head_dim,
                      out_scale, out, out32, lse,
                      RaggedRows{index, q_rows, num_heads, num_heads / num_kv_heads, num_kv_heads},
                      stream);
}

}  // namespace pa
