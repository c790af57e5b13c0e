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
// 16-byte device-scope store per plane.  The quotient is the correctly rounded FP32
// division, formed from the scale's reciprocal with one FMA correction; the
// hardware FP8 conversion rounds it to nearest even after a clamp to the
// largest finite code.
#include "pa_internal.h"

#include <hip/hip_fp16.h>
#include <math.h>

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 256 * 8;

// Two FP32 values -> two E4M3FN codes, written into bytes 0-1 (HI false) or 2-3
// (HI true) of `old`: nearest, ties to even, saturating at +-448.  The values
// are clamped to [-448, 448] first (so infinities and values past the largest
// code saturate, as the rounding of a clamped value does) and the hardware
// conversion rounds to nearest even.  A NaN passes through unclamped and comes
// out as a NaN code (0xFF on gfx950, whatever its sign); nan_to_7f makes every
// NaN code 0x7F.
template <bool HI>
__device__ __forceinline__ int e4m3_pair(float a, float b, int old)
{
    a = (a == a) ? __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f) : a;
    b = (b == b) ? __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f) : b;
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Bytes 0xFF of w become 0x7F.  0xFF is a NaN code and no finite value
// encodes to it (the most negative finite code is 0xFE), so this only gives
// every NaN the single code 0x7F.
__device__ __forceinline__ uint32_t nan_to_7f(uint32_t w)
{
    const uint32_t t = ~w;                                        // 0xFF bytes -> 0x00
    // high bit of each byte of t that is nonzero; the byte sums cannot carry
    const uint32_t nz = ((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t;
    return w ^ (~nz & 0x80808080u);
}

// The correctly rounded FP32 quotient a / b from y = RN(1/b) (Markstein's
// correction): q = RN(a y) lies within an ulp of a / b, r = a - q b is exact
// with an FMA, and RN(q + r y) = RN(a / b) when nothing under- or overflows.
// Used for FP16 a and b in [2^-110, 2^126], where a y cannot overflow; a
// quotient small enough to underflow lies far below the smallest E4M3 code,
// and the copysign keeps its sign (and that of a zero).  Infinite and NaN a
// take q = a y.
__device__ __forceinline__ float div_by(float a, float b, float y)
{
    const float q = a * y;
    const float r = __builtin_fmaf(-q, b, a);
    const float c = __builtin_copysignf(__builtin_fmaf(r, y, q), a);
    return __builtin_isfinite(a) ? c : q;
}

// 16 FP16 values (32 bytes) -> 16 E4M3 codes (16 bytes), each divided by scale:
// with div_by (FAST, y = RN(1 / scale)) or the library's correctly rounded
// division.
template <bool FAST>
__device__ __forceinline__ uint4 encode16(uint4 in0, uint4 in1, float scale, float y)
{
    const uint32_t w[8] = {in0.x, in0.y, in0.z, in0.w, in1.x, in1.y, in1.z, in1.w};
    float q[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint16_t bits = (uint16_t)(w[j] >> (16 * h));
            const float x = (float)__builtin_bit_cast(_Float16, bits);
            q[2 * j + h] = FAST ? div_by(x, scale, y) : __fdiv_rn(x, scale);
        }
    }
    int out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        out[i] = e4m3_pair<true>(q[4 * i + 2], q[4 * i + 3],
                                 e4m3_pair<false>(q[4 * i], q[4 * i + 1], 0));
    return make_uint4(nan_to_7f((uint32_t)out[0]), nan_to_7f((uint32_t)out[1]),
                      nan_to_7f((uint32_t)out[2]), nan_to_7f((uint32_t)out[3]));
}

// A 16-byte store at device scope (SC1).  Each XCD of the chip has its own
// L2, and such a store is written through to memory as it is issued; an
// ordinary store stays dirty in the L2 until the write-back that ends the
// kernel, which then holds the kernel's completion (up to the L2 capacity of
// the written bytes).  The compiler offers no device-scope 16-byte store, so
// it is inline asm with a 64-bit address.  The compiler's hazard checks do not
// see into the asm: a VALU write of the VGPRs holding the data of a store of
// more than 8 bytes needs two wait states after it, which the s_nop provides.
// Nothing in the kernel reads what it stores, so no wait for it is needed.
__device__ __forceinline__ void store16_device(uint8_t *p, uint4 v)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = {v.x, v.y, v.z, v.w};
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(x) : "memory");
}

// Thread layout: a token's chunks (num_kv_heads x head_dim/16 of them) are
// consecutive threads; a workgroup covers 256 / chunks tokens per iteration
// (chunks <= 256), and loops over chunks itself when a token has more.
template <bool FAST>
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
    const float ky = FAST ? __fdiv_rn(1.0f, k_scale) : 0.0f;
    const float vy = FAST ? __fdiv_rn(1.0f, v_scale) : 0.0f;
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
            store16_device(kp + dst, encode16<FAST>(k0, k1, k_scale, ky));
            store16_device(vp + dst, encode16<FAST>(v0, v1, v_scale, vy));
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
    // the reciprocal-based division where both scales keep it exact
    const auto in_range = [](float s) { return s >= 0x1p-110f && s <= 0x1p126f; };
    if (in_range(k_scale) && in_range(v_scale))
        hipLaunchKernelGGL(cache_write_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, k, v, num_tokens, num_kv_heads, head_dim, slots, kp, vp,
                           page_stride, token_stride, head_stride, page_size, num_slots, k_scale,
                           v_scale);
    else
        hipLaunchKernelGGL(cache_write_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, k, v, num_tokens, num_kv_heads, head_dim, slots, kp, vp,
                           page_stride, token_stride, head_stride, page_size, num_slots, k_scale,
                           v_scale);
    return hipGetLastError();
}

}  // namespace pa
