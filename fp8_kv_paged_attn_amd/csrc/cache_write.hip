// cache_write.hip - FP16 K/V tokens into E4M3 pages by slot.
//
// The cache is stored as uint8 E4M3 and written with the layer's per-tensor
// scales (vLLM PR "Qwen4Exp: fp8_e4m3 main KV cache on the QSA path": the
// uint8 cache written by the unchanged write path with per-tensor scales).
// Element x of token t, KV head g becomes E4M3(fp32(x) / scale): the nearest
// code, ties to even, saturating at +-448, NaN to 0x7F, -0 to 0x80.  Token t
// goes to page slot / page_size, row slot % page_size of both planes.
//
// One thread per 16 elements of a token: two 16-byte FP16 loads and one
// 16-byte store per plane.  The encoder is exact: the quotient is scaled by a power of two so
// that the code's step is 1, then rounded half to even (v_rndne).
#include "pa_internal.h"

#include <hip/hip_fp16.h>
#include <math.h>

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 256 * 8;

// FP32 -> E4M3FN code: nearest, ties to even, saturating; NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float x)
{
    const uint32_t sign = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
    const float a = fabsf(x);
    if (!(a == a))
        return 0x7Fu;
    if (a >= 448.0f)                       // also +-inf
        return sign | 0x7Eu;
    uint32_t code;
    if (a < 0.015625f) {
        // below 2^-6 the codes are m * 2^-9, m = 0..7 (m = 8 is the first normal)
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        // 2^e <= a < 2^(e+1), e = -6..8: a * 2^(3-e) in [8, 16), the code's
        // mantissa step is 1; rounding up to 16 carries into the exponent
        const int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFFu) - 127;
        const uint32_t m8 = (uint32_t)rintf(ldexpf(a, 3 - e));
        code = ((uint32_t)(e + 7) << 3) + m8 - 8u;
    }
    return sign | code;
}

// 16 FP16 values (32 bytes) -> 16 E4M3 codes (16 bytes), each divided by scale.
__device__ __forceinline__ uint4 encode16(uint4 in0, uint4 in1, float scale)
{
    const uint32_t w[8] = {in0.x, in0.y, in0.z, in0.w, in1.x, in1.y, in1.z, in1.w};
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint16_t bits = (uint16_t)(w[j] >> (16 * h));
            const float x = (float)__builtin_bit_cast(_Float16, bits);
            const uint32_t c = e4m3_code(__fdiv_rn(x, scale));
            out[j >> 1] |= c << (8 * (2 * (j & 1) + h));
        }
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// Thread layout: a token's chunks (num_kv_heads x head_dim/16 of them) are
// consecutive threads; a workgroup covers 256 / chunks tokens per iteration
// (chunks <= 256), and loops over chunks itself when a token has more.
__global__ __launch_bounds__(kThreads) void cache_write_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, int64_t num_tokens,
    int num_kv_heads, int head_dim, const int64_t *__restrict__ slots, uint8_t *__restrict__ kp,
    uint8_t *__restrict__ vp, int64_t page_stride, int64_t token_stride, int64_t head_stride,
    int page_size, int64_t num_slots, float k_scale, float v_scale)
{
    const int per_head = head_dim / 16;
    const int chunks = num_kv_heads * per_head;          // 16-element chunks per token
    const int tpw = chunks <= kThreads ? kThreads / chunks : 1;   // tokens per iteration
    const int tt = chunks <= kThreads ? (int)threadIdx.x / chunks : 0;
    const int c0 = chunks <= kThreads ? (int)threadIdx.x - tt * chunks : (int)threadIdx.x;
    const int cstep = chunks <= kThreads ? chunks : kThreads;
    if (tt >= tpw)
        return;
    for (int64_t t = (int64_t)blockIdx.x * tpw + tt; t < num_tokens; t += (int64_t)gridDim.x * tpw) {
        const int64_t slot = slots[t];
        if (slot < 0 || slot >= num_slots)
            continue;
        const int64_t page = slot / page_size, row = slot - page * page_size;
        const int64_t base = page * page_stride + row * token_stride;
        for (int c = c0; c < chunks; c += cstep) {
            const int g = c / per_head, e = 16 * (c - g * per_head);
            const int64_t src = (t * num_kv_heads + g) * head_dim + e;
            const uint4 *ks = (const uint4 *)(k + src);
            const uint4 *vs = (const uint4 *)(v + src);
            const uint4 k0 = ks[0], k1 = ks[1], v0 = vs[0], v1 = vs[1];
            const int64_t dst = base + g * head_stride + e;
            *(uint4 *)(kp + dst) = encode16(k0, k1, k_scale);
            *(uint4 *)(vp + dst) = encode16(v0, v1, v_scale);
        }
    }
}

}  // namespace

hipError_t launch_cache_write(const uint16_t *k, const uint16_t *v, int64_t num_tokens,
                              int num_kv_heads, int head_dim, const int64_t *slots, uint8_t *kp,
                              uint8_t *vp, int64_t page_stride, int64_t token_stride,
                              int64_t head_stride, int page_size, int64_t num_slots,
                              float k_scale, float v_scale, hipStream_t stream)
{
    if (num_tokens == 0)
        return hipSuccess;
    const int chunks = num_kv_heads * (head_dim / 16);
    const int64_t tpw = chunks <= kThreads ? kThreads / chunks : 1;
    int64_t blocks = (num_tokens + tpw - 1) / tpw;
    if (blocks > kMaxBlocks)
        blocks = kMaxBlocks;
    hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, k, v,
                       num_tokens, num_kv_heads, head_dim, slots, kp, vp, page_stride,
                       token_stride, head_stride, page_size, num_slots, k_scale, v_scale);
    return hipGetLastError();
}

}  // namespace pa
