// pa_verify.h - the verify kernels' argument block and launchers.
// Internal to libpaged_attn_e4m3; the public interface is include/paged_attn_e4m3.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// How a list position maps to a token.
enum VerifyMode : int {
    kModeDense = 0,     // position p of request b is token p
    kModeBlocks = 1,    // position p is row p % page of selected block sel[p / page]
    kModeTokens = 2,    // position p is token sel[p] (-1: empty)
};

// Everything a verify kernel needs, resolved on the host.  One struct serves
// the dense path and both sparse selections.
struct VerifyArgs {
    const uint16_t *q;          // fp16 (dense) or bf16 (sparse) bits [B][q_rows][H][D]
    const uint8_t *k_pool;
    const uint8_t *v_pool;
    int64_t page_stride;
    int64_t token_stride;
    int64_t head_stride;
    int32_t page_size;
    const int32_t *block_table; // [B][table_stride] (one request: [entries])
    int32_t table_stride;       // entries per request (one dense request: 0)
    const int32_t *sel;         // sparse: [B][Hkv][topk] blocks or token ids; dense: nullptr
    int32_t topk;
    const int32_t *row_lens;    // [B][q_rows]
    int32_t len_cap;            // lengths are clamped to [0, len_cap]
    int32_t list_len;           // positions per KV unit (dense: max_tokens; blocks:
                                // topk*page; tokens: topk)
    int32_t batch, q_rows, num_heads, num_kv_heads, group;  // group = H / Hkv
    int32_t rows;               // rows per KV unit = q_rows * group
    int32_t num_splits, tokens_per_split;
    int32_t total_rows;         // rows of the workspace = B * q_rows * H
    float logit_scale;          // sm_scale * k_scale * log2(e)
    float *ws_acc, *ws_max, *ws_sum;
    int32_t split_by_length;    // 1: a unit's splits share its longest row length
                                // (split_span), 0: split s covers s*T .. s*T + T - 1
};

// Positions per split of a KV unit whose longest (clamped) row length is lmax,
// when splits follow the length: ceil(lmax / S) rounded up to the 64-token
// tile, so never more than the plan's T (S * T covers every length).
__host__ __device__ inline int split_span(int lmax, int num_splits)
{
    const int t = (lmax + num_splits - 1) / num_splits;
    return t > 0 ? (t + 63) / 64 * 64 : 64;
}

// Page slots (token ids: list entries) the MFMA kernel keeps per workgroup in
// LDS.  A split of T positions in pages of P tokens needs (T - 1) / P + 2 of
// them; a split of T token ids needs T.
__host__ __device__ constexpr int mfma_max_slots(int head_dim)
{
    return head_dim == 256 ? 1024 : 2048;
}

__host__ __device__ inline long long mfma_slots_needed(int tokens_per_split, int page_size,
                                                       bool token_ids)
{
    return token_ids ? (long long)tokens_per_split
                     : (long long)(tokens_per_split - 1) / page_size + 2;
}

// Launchers return hipSuccess or the launch error.  Grid = (num_splits, units,
// row chunks of 48).
// `ev`, when not null, is a (begin, end) pair of HIP events bound to the
// kernel's own dispatch (hipExtLaunchKernel), for the kernel timer.
hipError_t launch_verify_simple(const VerifyArgs &a, int head_dim, VerifyMode mode,
                                hipStream_t stream, const hipEvent_t *ev = nullptr);
hipError_t launch_verify_mfma(const VerifyArgs &a, int head_dim, VerifyMode mode,
                              hipStream_t stream, const hipEvent_t *ev = nullptr);
}  // namespace pa
