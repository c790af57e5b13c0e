// pa_internal.h - declarations shared by the sources of libpaged_attn_e4m3.
// Internal; the public interface is include/paged_attn_e4m3.h.
#pragma once

#include "pa_verify.h"

namespace pa {

// Streaming read of bytes (a multiple of 16) from a 16-byte aligned buffer.
hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t stream);
// FP16 K/V tokens [num_tokens][num_kv_heads][head_dim] into the E4M3 pool by
// slot; slots < 0 or >= num_slots are skipped.  head_dim a multiple of 16.
hipError_t launch_cache_write(const uint16_t *k, const uint16_t *v, int64_t num_tokens,
                              int num_kv_heads, int head_dim, const int64_t *slots, uint8_t *kp,
                              uint8_t *vp, int64_t page_stride, int64_t token_stride,
                              int64_t head_stride, int page_size, int64_t num_slots,
                              float k_scale, float v_scale, hipStream_t stream);
// Any of out (FP16), out32 (FP32) and lse (base-2 LSE per row) may be null.
hipError_t launch_combine(const float *acc, const float *mx, const float *sm, int num_splits,
                          int num_rows, int head_dim, float out_scale, uint16_t *out,
                          float *out32, float *lse, hipStream_t stream);
// The combine of a ragged batch's partials (VerifyArgs::ragged) into FP16
// rows (b, i, h); index[u] .. index[u + 1] - 1 are unit u's splits.
hipError_t launch_combine_ragged(const float *acc, const float *mx, const float *sm,
                                 const int32_t *index, int num_splits, int batch, int q_rows,
                                 int num_heads, int num_kv_heads, int head_dim, float out_scale,
                                 uint16_t *out, float *out32, float *lse, hipStream_t stream);

}  // namespace pa
