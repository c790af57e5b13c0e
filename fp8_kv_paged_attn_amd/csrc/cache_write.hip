// cache_write.hip - FP16 K/V tokens into E4M3 pages by slot.
//
// The cache is stored as uint8 E4M3 and written with the layer's per-tensor
// scales (vLLM PR "Qwen4Exp: fp8_e4m3 main KV cache on the QSA path": the
// uint8 cache written by the unchanged write path with per-tensor scales).
// Element x of token t, KV head g becomes E4M3(fp32(x) / scale): the nearest
// code, ties to even, saturating at +-448, NaN to 0x7F, -0 to 0x80.  Token t
// goes to page slot / page_size, row slot % page_size of both planes.
//
// One thread per 8 elements: a 16-byte FP16 load and an 8-byte store per
// plane.  The encoder is exact: the quotient is scaled by a power of two so
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

// 8 FP16 values (16 bytes) -> 8 E4M3 codes (8 bytes), each divided by scale.
__device__ __forceinline__ uint2 encode8(uint4 in, float scale)
{
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint16_t bits = (uint16_t)(w[j] >> (16 * h));
            const float x = (float)__builtin_bit_cast(_Float16, bits);
            const uint32_t c = e4m3_code(__fdiv_rn(x, scale));
            out[j >> 1] |= c << (8 * (2 * (j & 1) + h));
        }
    }
    return make_uint2(out[0], out[1]);
}

__global__ __launch_bounds__(kThreads) void cache_write_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, int64_t num_tokens,
    int num_kv_heads, int head_dim, const int64_t *__restrict__ slots, uint8_t *__restrict__ kp,
    uint8_t *__restrict__ vp, int64_t page_stride, int64_t token_stride, int64_t head_stride,
    int page_size, int64_t num_slots, float k_scale, float v_scale)
{
    const int chunks = head_dim / 8;
    const int64_t per_token = (int64_t)num_kv_heads * chunks;
    const int64_t total = num_tokens * per_token;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t t = i / per_token;
        const int rem = (int)(i - t * per_token);
        const int g = rem / chunks, c = rem - g * chunks;
        const int64_t slot = slots[t];
        if (slot < 0 || slot >= num_slots)
            continue;
        const int64_t page = slot / page_size, row = slot - page * page_size;
        const int64_t src = ((t * num_kv_heads + g) * head_dim) + 8 * c;
        const int64_t dst = page * page_stride + row * token_stride + g * head_stride + 8 * c;
        const uint4 kin = *(const uint4 *)(k + src);
        const uint4 vin = *(const uint4 *)(v + src);
        *(uint2 *)(kp + dst) = encode8(kin, k_scale);
        *(uint2 *)(vp + dst) = encode8(vin, v_scale);
    }
}

}  // namespace

hipError_t launch_cache_write(const uint16_t *k, const uint16_t *v, int64_t num_tokens,
                              int num_kv_heads, int head_dim, const int64_t *slots, uint8_t *kp,
                              uint8_t *vp, int64_t page_stride, int64_t token_stride,
                              int64_t head_stride, int page_size, int64_t num_slots,
                              float k_scale, float v_scale, hipStream_t stream)
{
    const int64_t total = num_tokens * num_kv_heads * (head_dim / 8);
    if (total == 0)
        return hipSuccess;
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > kMaxBlocks)
        blocks = kMaxBlocks;
    hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, k, v,
                       num_tokens, num_kv_heads, head_dim, slots, kp, vp, page_stride,
                       token_stride, head_stride, page_size, num_slots, k_scale, v_scale);
    return hipGetLastError();
}

}  // namespace pa
