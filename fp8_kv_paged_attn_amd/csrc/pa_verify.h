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
    int32_t chunk_rows;         // rows of a KV unit one MFMA workgroup takes: 16, 32
                                // or 48 (grid z counts the chunks; ragged: 48); it
                                // sits in the alignment gap before the table pointer,
                                // so the other fields keep their offsets
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
    // 0: the grid is (num_splits, units, row chunks), split s of every unit
    // covers positions [s*T, s*T + T) and writes workspace rows (b, i, h).
    // 1 (a batch of requests): the grid is (num_splits, 1, row chunks), and
    // ragged_locate() gives each workgroup its unit, its split of that unit
    // and the span from all row lengths; it writes workspace rows
    // [s][row of its unit], and split_index[u] is the first split of unit u
    // (split_index[units] the number of splits used).
    int32_t ragged;
    int32_t *split_index;
};

// Query rows per request of a ragged batch (the batched entry's limit).
constexpr int kRaggedMaxQRows = 16;

// Longest clamped row length of request b (all its KV heads see the same).
// The loop is unrolled to the row limit, so that every length load is issued
// before the first is waited for: one memory round trip, not one per row.
__device__ inline int request_len(const VerifyArgs &a, int b)
{
    const int32_t *lens = a.row_lens + (int64_t)b * a.q_rows;
    int raw[kRaggedMaxQRows];
#pragma unroll
    for (int i = 0; i < kRaggedMaxQRows; ++i)
        raw[i] = i < a.q_rows ? lens[i] : 0;
    int L = 0;
#pragma unroll
    for (int i = 0; i < kRaggedMaxQRows; ++i) {
        const int l = raw[i] < 0 ? 0 : (raw[i] > a.len_cap ? a.len_cap : raw[i]);
        L = l > L ? l : L;
    }
    return L;
}

struct RaggedPos {
    int unit;    // -1: no split of the batch falls on this workgroup
    int local;   // split index within the unit
    int span;    // positions per split, the same for the whole batch
};

// Where workgroup s of a ragged batch works.  Called by every lane of a wave
// (lane = 0..63); the result is the same in all lanes.  With U = batch *
// num_kv_heads units, L_u the longest row length of unit u, and S the
// number of splits, the span is T = ceil(sum_u L_u / (S - U)) on the 64-token
// tile (at most the plan's tokens_per_split, which also serves when S <= U),
// so that unit u takes S_u = ceil(L_u / T) splits and sum_u S_u <= S: splits
// follow the lengths, a long request gets more of them than a short one, and
// every workgroup that works reads about T tokens.  Units take consecutive
// splits in order; with write_index the workgroup writes split_index.
__device__ inline RaggedPos ragged_locate(const VerifyArgs &a, int s, int lane, bool write_index)
{
    const int B = a.batch, Hkv = a.num_kv_heads, S = a.num_splits;
    const int64_t U = (int64_t)B * Hkv;
    // the first 64 requests' lengths are kept for the second pass (one round
    // trip for a batch of up to 64 requests)
    const int L0 = lane < B ? request_len(a, lane) : 0;
    int64_t total = L0;
    for (int b0 = 64; b0 < B; b0 += 64)
        total += (b0 + lane < B) ? request_len(a, b0 + lane) : 0;
    for (int o = 32; o >= 1; o >>= 1)
        total += __shfl_xor(total, o, 64);
    total *= Hkv;
    int64_t T = a.tokens_per_split;
    if (S > U) {
        // the span ceil(total / (S - U)): a 32-bit division when the sum of
        // the lengths allows (a 64-bit one takes several times as many
        // instructions), both on wave-uniform values
        const int64_t d = S - U;
        int64_t t;
        if (total + d <= (int64_t)INT32_MAX)
            t = (int64_t)(((uint32_t)total + (uint32_t)d - 1u) / (uint32_t)d);
        else
            t = (total + d - 1) / d;
        t = (t + 63) / 64 * 64;
        T = t < 64 ? 64 : (t < T ? t : T);
    }
    RaggedPos pos = {-1, 0, (int)T};
    int base = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int b = b0 + lane;
        const int L = b0 == 0 ? L0 : (b < B ? request_len(a, b) : 0);
        // L + T - 1 < 2^31: a batch plan keeps the capacity plus its span in int32
        const int sb = (int)((uint32_t)(L + (int)T - 1) / (uint32_t)T);
        const int cnt = Hkv * sb;
        int incl = cnt;                               // inclusive scan over lanes
        for (int o = 1; o < 64; o <<= 1) {
            const int up = __shfl_up(incl, o, 64);
            incl += lane >= o ? up : 0;
        }
        const int excl = incl - cnt;
        if (write_index && b < B)
            for (int g = 0; g < Hkv; ++g)
                a.split_index[(int64_t)b * Hkv + g] = base + excl + g * sb;
        const bool hit = b < B && s >= base + excl && s < base + incl;
        const uint64_t m = __ballot(hit);
        if (m) {
            const int j = __builtin_ctzll(m);
            const int sj = __shfl(sb, j, 64), ej = __shfl(excl, j, 64);
            const int d = s - base - ej;
            pos.unit = (b0 + j) * Hkv + d / sj;
            pos.local = d % sj;
        }
        base += __shfl(incl, 63, 64);
    }
    if (write_index && lane == 0)
        a.split_index[U] = base;
    return pos;
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
