// verify_simple.hip - straightforward FP32 verify kernel (dense, and sparse over
// selected blocks or selected token ids).
//
// One workgroup per (split, KV unit).  Each 64-position tile of the split is
// gathered into LDS as raw E4M3 bytes, scores are FP32 dot products, the
// online softmax keeps a per-row FP32 max and sum, and P.V accumulates in FP32
// registers, one output column per thread.  A position a row does not see
// adds nothing to that row's P.V (selected out, not multiplied by 0), so a
// NaN byte reaches exactly the rows that see it.  It is the plain form of the
// computation (design note "DFlash2 E4M3 attention with FP32 state", first
// section: FP32 unnormalised partition numerators, separate FP32 max/sum),
// kept as the A/B baseline of the MFMA kernel and for shapes it does not take.
#include "pa_verify.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kMaxRows = 48;

// E4M3 -> float.  The 7 magnitude bits, shifted under an FP16 exponent field,
// form an FP16 number equal to the E4M3 value times 2^-8 for every finite code
// (subnormals included); the factor is undone exactly in FP32.  The two NaN
// codes S.1111.111 decode to NaN.
__device__ inline float e4m3_to_float(uint32_t byte)
{
    uint16_t h = (uint16_t)(((byte & 0x7Fu) << 7) | ((byte & 0x80u) << 8));
    const float f = (float)__builtin_bit_cast(_Float16, h) * 256.0f;
    return (byte & 0x7Fu) == 0x7Fu ? __builtin_nanf("") : f;
}

__device__ inline float fp16_to_float(uint16_t bits)
{
    return (float)__builtin_bit_cast(_Float16, bits);
}

__device__ inline float bf16_to_float(uint16_t bits)
{
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
}

// List position -> (logical token, byte offset of its K/V head row).  False for
// an empty selection slot or a token no row of this unit sees.  lmax is at
// most the table's capacity, so a token below it has a table entry.
template <int MODE>
__device__ inline bool resolve(const VerifyArgs &a, int b, int g, int pos, int lmax,
                               int32_t &t, int64_t &off)
{
    const int ps = a.page_size;
    int blk, u;
    if (MODE == kModeDense) {
        t = pos;
        blk = pos / ps;
        u = pos - blk * ps;
        if (t >= lmax)
            return false;
        off = (int64_t)a.block_table[(int64_t)b * a.table_stride + blk] * a.page_stride;
    } else if (MODE == kModeTokens) {
        t = a.sel[((int64_t)b * a.num_kv_heads + g) * a.topk + pos];
        if (t < 0 || t >= lmax)
            return false;
        blk = t / ps;
        u = t - blk * ps;
        off = (int64_t)a.block_table[(int64_t)b * a.table_stride + blk] * a.page_stride;
    } else {
        int j = pos / ps;
        u = pos - j * ps;
        blk = a.sel[((int64_t)b * a.num_kv_heads + g) * a.topk + j];
        if (blk < 0)
            return false;
        t = blk * ps + u;
        if (t >= lmax)
            return false;
        off = (int64_t)a.block_table[(int64_t)b * a.table_stride + blk] * a.page_stride;
    }
    off += (int64_t)u * a.token_stride + (int64_t)g * a.head_stride;
    return true;
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void verify_simple_kernel(VerifyArgs a)
{
    __shared__ float q_s[kMaxRows][D];
    __shared__ __attribute__((aligned(16))) uint8_t k_s[kTile][D];
    __shared__ __attribute__((aligned(16))) uint8_t v_s[kTile][D];
    __shared__ float p_s[kMaxRows][kTile + 1];
    __shared__ int32_t tok_s[kTile];
    __shared__ float m_s[kMaxRows], l_s[kMaxRows], alpha_s[kMaxRows];
    __shared__ int32_t len_s[16];

    const int tid = threadIdx.x;
    // the split of a KV unit this workgroup reads and its span (a ragged batch
    // derives them from every row length, the same in every wave)
    int split = blockIdx.x, unit = blockIdx.y, tps = a.tokens_per_split;
    if (a.ragged) {
        const RaggedPos rp = ragged_locate(a, blockIdx.x, tid & 63,
                                           blockIdx.x == 0 && blockIdx.z == 0 && tid < 64);
        if (rp.unit < 0)
            return;
        split = rp.local;
        unit = rp.unit;
        tps = rp.span;
    }
    const int b = unit / a.num_kv_heads, g = unit - b * a.num_kv_heads;
    // rows of a KV unit beyond 48 go to further workgroups (grid z)
    const int row0 = blockIdx.z * kMaxRows;
    const int R = min(a.rows - row0, kMaxRows), G = a.group;

    if (tid < a.q_rows) {
        int L = a.row_lens[(int64_t)b * a.q_rows + tid];
        len_s[tid] = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
    }
    for (int idx = tid; idx < R * D; idx += kThreads) {
        int r = idx / D, d = idx - r * D;
        int i = (row0 + r) / G, h = g * G + (row0 + r - i * G);
        uint16_t bits = a.q[(((int64_t)b * a.q_rows + i) * a.num_heads + h) * D + d];
        q_s[r][d] = MODE != kModeDense ? bf16_to_float(bits) : fp16_to_float(bits);
    }
    if (tid < R) {
        m_s[tid] = -INFINITY;
        l_s[tid] = 0.0f;
    }
    __syncthreads();
    int lmax = 0;
    for (int i = 0; i < a.q_rows; ++i)
        lmax = max(lmax, len_s[i]);

    const int lo = split * tps;
    int hi = min(lo + tps, a.list_len);
    if (MODE == kModeDense)
        hi = min(hi, lmax);

    float acc[kMaxRows];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r)
        acc[r] = 0.0f;

    constexpr int kChunks = D / 16;
    for (int p0 = lo; p0 < hi; p0 += kTile) {
        for (int c = tid; c < kTile * kChunks; c += kThreads) {
            int j = c / kChunks, piece = c - j * kChunks;
            int pos = p0 + j;
            int32_t t = -1;
            int64_t off = 0;
            bool ok = pos < hi && resolve<MODE>(a, b, g, pos, lmax, t, off);
            uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
            if (ok) {
                kv = *(const uint4 *)(a.k_pool + off + piece * 16);
                vv = *(const uint4 *)(a.v_pool + off + piece * 16);
            }
            *(uint4 *)&k_s[j][piece * 16] = kv;
            *(uint4 *)&v_s[j][piece * 16] = vv;  // zero bytes for unseen positions
            if (piece == 0)
                tok_s[j] = ok ? t : -1;
        }
        __syncthreads();
        for (int idx = tid; idx < R * kTile; idx += kThreads) {
            int r = idx / kTile, j = idx - r * kTile;
            int t = tok_s[j];
            float s = -INFINITY;
            if (t >= 0 && t < len_s[(row0 + r) / G]) {
                float dot = 0.0f;
                for (int d = 0; d < D; ++d)
                    dot += q_s[r][d] * e4m3_to_float(k_s[j][d]);
                s = dot * a.logit_scale;
            }
            p_s[r][j] = s;
        }
        __syncthreads();
        if (tid < R) {
            float mx = m_s[tid];
            for (int j = 0; j < kTile; ++j)
                mx = fmaxf(mx, p_s[tid][j]);
            float alpha = (mx == -INFINITY) ? 1.0f : exp2f(m_s[tid] - mx);
            // a position the row does not see (score -inf) is marked p = -1
            float sum = 0.0f;
            for (int j = 0; j < kTile; ++j) {
                float s = p_s[tid][j];
                float p = (s == -INFINITY) ? -1.0f : exp2f(s - mx);
                p_s[tid][j] = p;
                sum += (p < 0.0f) ? 0.0f : p;
            }
            l_s[tid] = l_s[tid] * alpha + sum;
            m_s[tid] = mx;
            alpha_s[tid] = alpha;
        }
        __syncthreads();
        if (tid < D) {
#pragma unroll
            for (int r = 0; r < kMaxRows; ++r) {
                if (r < R) {
                    float s = acc[r] * alpha_s[r];
                    for (int j = 0; j < kTile; ++j) {
                        const float p = p_s[r][j];
                        s += (p < 0.0f) ? 0.0f : p * e4m3_to_float(v_s[j][tid]);
                    }
                    acc[r] = s;
                }
            }
        }
        __syncthreads();
    }

    // workspace rows: (b, i, h) of the output, or [split][row of the unit]
    const int64_t ws_base =
        a.ragged ? (int64_t)blockIdx.x * a.rows : (int64_t)split * a.total_rows;
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
        if (r < R && tid < D) {
            int i = (row0 + r) / G, h = g * G + (row0 + r - i * G);
            int64_t orow = a.ragged ? (int64_t)(row0 + r)
                                    : ((int64_t)b * a.q_rows + i) * a.num_heads + h;
            a.ws_acc[(ws_base + orow) * D + tid] = acc[r];
        }
    }
    if (tid < R) {
        int i = (row0 + tid) / G, h = g * G + (row0 + tid - i * G);
        int64_t orow = a.ragged ? (int64_t)(row0 + tid)
                                : ((int64_t)b * a.q_rows + i) * a.num_heads + h;
        a.ws_max[ws_base + orow] = m_s[tid];
        a.ws_sum[ws_base + orow] = l_s[tid];
    }
}

}  // namespace

hipError_t launch_verify_simple(const VerifyArgs &a, int head_dim, VerifyMode mode,
                                hipStream_t stream, const hipEvent_t *ev)
{
    dim3 grid(a.num_splits, a.ragged ? 1 : a.batch * a.num_kv_heads,
              (a.rows + kMaxRows - 1) / kMaxRows);
    dim3 block(kThreads);
    hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
#define PA_SIMPLE(D, M)                                                                        \
    hipExtLaunchKernelGGL((verify_simple_kernel<D, M>), grid, block, 0, stream, e0, e1, 0, a)
    if (head_dim == 256 && mode == kModeDense)
        PA_SIMPLE(256, kModeDense);
    else if (head_dim == 128 && mode == kModeDense)
        PA_SIMPLE(128, kModeDense);
    else if (head_dim == 256 && mode == kModeBlocks)
        PA_SIMPLE(256, kModeBlocks);
    else if (head_dim == 128 && mode == kModeBlocks)
        PA_SIMPLE(128, kModeBlocks);
    else if (head_dim == 256 && mode == kModeTokens)
        PA_SIMPLE(256, kModeTokens);
    else if (head_dim == 128 && mode == kModeTokens)
        PA_SIMPLE(128, kModeTokens);
    else
        return hipErrorInvalidValue;
#undef PA_SIMPLE
    return hipGetLastError();
}

}  // namespace pa
