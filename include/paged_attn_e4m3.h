/* paged_attn_e4m3.h - multi-row verify attention over a paged FP8-E4M3 KV
 * cache, for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What the library computes.  For a query row i of head h, whose KV head is
 * g = h / (num_heads / num_kv_heads), and the tokens t that row sees:
 *
 *     s_t = sm_scale * k_scale * sum_d q[i][h][d] * K_t[g][d]
 *     o[i][h][:] = v_scale * sum_t softmax(s)_t * V_t[g][:]
 *
 * with K_t and V_t the exact values of the E4M3 bytes stored for token t.
 * Sources:
 *   [DN]  1Cat-vLLM design note "DFlash2 E4M3 attention with FP32 state",
 *         first section: single-request verification of q2-8 draft rows with
 *         H6/Hkv1/D256 grouped heads over E4M3 pages, live per-query lengths
 *         including zero padding, FP32 unnormalised partition numerators,
 *         separate FP32 max/sum, FP32 combination, FP16 activations; page
 *         size is a runtime stride, not a template ("revision 4" paragraph).
 *   [QSA] vLLM PR "[Model] Qwen4Exp: fp8_e4m3 main KV cache on the QSA path":
 *         the sparse split-K paged GQA kernel over selected blocks, which
 *         dequantises E4M3 on load; k_scale folded into the softmax scale on
 *         the host and v_scale used as the kernel's output scale (review
 *         thread on host-side KV scales); scale validation before launch
 *         (CodeRabbit finding).
 *   [NB]  1Cat-vLLM PR "[Model] Qualify calibrated E4M3 and disk PLE with QSA
 *         DCP2": rows that no query attends must not reach P.V even when the
 *         null block decodes to NaN (commit fixing the grouped-page4 NaN);
 *         strided (packed) page views read like unpacked ones.
 *
 * Conventions for every entry point:
 *   - Buffers are device pointers unless marked (host).  The caller owns all
 *     memory; the library never allocates, never frees, keeps no state
 *     between calls except a per-device record of whether it is a gfx950
 *     (and the kernel timer's events, below, once a caller arms it), never
 *     synchronises (but in paged_attn_timer_read) and never copies host
 *     memory to the device.  Work
 *     is enqueued on `stream` (a hipStream_t; NULL = the null stream), so
 *     calls can be captured into a HIP graph.
 *   - A problem the host can see (null pointer, bad shape, misalignment, a
 *     plan that does not fit the call, a workspace that is too small)
 *     returns a negative status and enqueues nothing.  A failed kernel
 *     launch returns PA_EHIP.  There is no fallback to another precision.
 *   - Device-resident data is not inspected on the host.  Row lengths are
 *     clamped on the device; block-table and selection entries must name
 *     pages inside the pool (precondition; reading outside is undefined).
 *   - Workspace buffers are reused by successive calls on one stream only.
 *   - Calls are thread-safe.
 */
#ifndef PAGED_ATTN_E4M3_H
#define PAGED_ATTN_E4M3_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Revision of this interface.  A caller built against another revision must
 * refuse the library rather than run it ([DN] revision gate: the wrapper
 * requires the revision it was written for, so new workspace layouts never
 * reach an older binary).  Revision 2: the planner takes the page size and
 * the selection kind, and plans carry them. */
#define PA_ABI_VERSION 3

enum pa_status {
    PA_OK = 0,
    PA_EINVAL = -1,        /* null pointer, bad shape or count, bad scale */
    PA_EUNSUPPORTED = -2,  /* valid but not built: head_dim, rows per KV head,
                              more than 65,536 heads */
    PA_EWORKSPACE = -3,    /* workspace smaller than the plan needs */
    PA_EALIGN = -4,        /* pointer or stride not 16-byte aligned */
    PA_EDEVICE = -5,       /* no HIP device, or not gfx950 */
    PA_EHIP = -6,          /* a HIP call or kernel launch failed */
    PA_EPLAN = -7,         /* plan does not cover this call */
    PA_ESCRATCH = -8       /* plan needs more than the fixed scratch of
                              paged_attn_verify_noalloc_e4m3 */
};

/* PA_ABI_VERSION of the built library. */
int32_t paged_attn_abi_version(void);

/* Static, never-NULL identifier of the sources the library was built from: the
 * first 16 hex digits of a SHA-256 over its HIP sources, its headers and its
 * code-generation flags, computed by the build and compiled in.  A harness
 * compares it with the same hash of the sources it holds to know that the
 * binary it loaded is the one those sources describe. */
const char *paged_attn_build_id(void);

/* Static, never-NULL description of a status code. */
const char *paged_attn_status_string(int32_t status);

/* (host) Paged K/V pool.  Byte (page p, token u, KV head g, element d) of the
 * K plane is k_pool[p*page_stride + u*token_stride + g*head_stride + d]; the
 * V plane uses the same strides.  Elements of one head are contiguous.
 * page_stride, token_stride, head_stride and both base pointers must be
 * multiples of 16 bytes; any page_size >= 1 is accepted.  Strided views of a
 * larger interleaved allocation ("packed pages") are ordinary pools here. */
typedef struct pa_kv_pool {
    const uint8_t *k_pool;
    const uint8_t *v_pool;
    int64_t page_stride;
    int64_t token_stride;
    int64_t head_stride;
    int32_t num_pages;
    int32_t page_size;
} pa_kv_pool;

/* Kernel choice carried by a plan (an A/B switch; both compute the same
 * function, with different FP32 rounding).  Neither falls back to the other:
 * a plan the chosen kernel cannot run is refused with PA_EPLAN. */
enum pa_kernel {
    PA_KERNEL_AUTO = 0,            /* the MFMA kernel */
    PA_KERNEL_SIMPLE = 1,          /* plain FP32 kernel (A/B baseline, any plan) */
    PA_KERNEL_MFMA = 2             /* the MFMA kernel */
};

/* What a list position of a KV unit names (the entry point a plan is for). */
enum pa_selection {
    PA_SEL_DENSE = 0,              /* paged_attn_verify_e4m3 (and its allocation-free form) */
    PA_SEL_BLOCKS = 1,             /* qsa_sparse_verify_e4m3 */
    PA_SEL_TOKENS = 2,             /* qsa_sparse_verify_tokens_e4m3 */
    PA_SEL_BATCH = 3               /* paged_attn_verify_batch_e4m3: splits shared by a batch */
};

/* (host) Split plan: the token axis of each KV unit (one KV head of one
 * request) is cut into num_splits ranges of tokens_per_split tokens; range s
 * is one workgroup.  Filled by paged_attn_plan; the other fields record what
 * the plan was made for and are checked by the compute entry points
 * (PA_EPLAN when they differ from the call).  The fields past num_splits and
 * tokens_per_split, and the workspace struct below, add to the pages' bare
 * "split count + FP32 workspace" what the library checks before a launch. */
typedef struct pa_plan {
    int32_t num_splits;
    int32_t tokens_per_split;      /* multiple of 64 */
    int32_t kernel;                /* enum pa_kernel; paged_attn_plan sets PA_KERNEL_AUTO */
    int32_t max_tokens;            /* tokens per KV unit the plan covers */
    int32_t rows_per_kv_unit;      /* query rows x heads sharing one KV head */
    int32_t num_kv_units;          /* KV heads x requests */
    int32_t head_dim;
    int32_t page_size;             /* tokens per page (per selected block) */
    int32_t selection;             /* enum pa_selection */
    int64_t ws_acc_bytes;          /* FP32 [num_splits][rows][head_dim] */
    int64_t ws_stat_bytes;         /* FP32 [num_splits][rows], each of max and sum */
    int64_t ws_index_bytes;        /* int32 [num_kv_units + 1] (PA_SEL_BATCH), else 0 */
    int32_t rows_per_workgroup;    /* rows of a KV unit one MFMA workgroup takes: 16, 32
                                      or 48 (0 reads as 48); PA_SEL_BATCH: 48.  The
                                      workspace layout does not depend on it; the values
                                      may differ in FP32 rounding (a row block's lazy
                                      reference max follows all of its rows).  The plain
                                      kernel always takes 48 */
} pa_plan;

/* (host) FP32 split workspace written by the verify entry points and read by
 * paged_attn_combine_fp32.  Row r of split s holds, for the tokens of that
 * split that the row sees ([DN]: FP32 unnormalised partition numerators with
 * a separate FP32 max and sum), with y_t = s_t * log2(e):
 *     max[s][r]    = m = max_t y_t            (-inf when the split is empty)
 *     sum[s][r]    = l = sum_t 2^(y_t - m)    (0 when empty)
 *     acc[s][r][d] = sum_t 2^(y_t - m) * V_t[g][d]   (no v_scale; the MFMA kernel
 *                    leaves it unwritten when the split is empty, since the
 *                    combine never uses an empty split's numerator)
 * Rows are numbered like the output (rows = (i, h), or (b, i, h) for a batch
 * of requests), so the combine works row by row; a ragged batch
 * (paged_attn_verify_batch_e4m3) numbers them per KV unit instead. */
typedef struct pa_workspace {
    float *acc;
    float *max;
    float *sum;
    int64_t acc_bytes;             /* capacity of acc */
    int64_t stat_bytes;            /* capacity of each of max and sum */
    int32_t *index;                /* split index of a ragged batch (PA_SEL_BATCH plans);
                                      NULL elsewhere */
    int64_t index_bytes;           /* capacity of index */
} pa_workspace;

/* (host, integer) Choose the split of max_tokens list positions (tokens for
 * the dense entries, topk*page_size for selected blocks, the list length for
 * token ids) for num_kv_units units of rows_per_kv_unit rows, read in pages of
 * page_size tokens with the given selection (enum pa_selection).
 * num_cus = compute units to fill; <= 0 takes the current device's count
 * (queried once per device and kept), or 256 (the MI355X count) when no
 * device can be queried.  requested_splits > 0 asks for that split count; 0
 * picks one: at most one workgroup per compute unit over all units (a unit of more
 * than 48 rows counts once per 48-row chunk, each chunk being a workgroup),
 * but no split shorter than 128 tokens, so that the FP32 partial each split
 * writes stays small against its K/V bytes (the pages tune split counts per
 * device and region, [QSA] sm_120 retune commit).  When that leaves each
 * workgroup fewer than two 128-token steps (short lists), the rows of a unit
 * are cut finer (rows_per_workgroup 16, else 32) if that still fills at most
 * num_cus workgroups, with splits of at most 3 steps (16 rows) or 4 (32 rows)
 * and a count of (split, unit) pairs that is a multiple of 8: more compute
 * units read the list, each does less per token, and the chunks of a split
 * run on one XCD.  A requested count keeps 48-row chunks.
 * Either count is then
 * clamped to what the token count allows and raised where a split would
 * otherwise cover more pages (token ids: entries) than the MFMA kernel keeps
 * per workgroup, 1,024 at head_dim 256 and 2,048 at 128, so that every plan
 * it returns runs on that kernel.  PA_SEL_BATCH plans a ragged batch instead:
 * num_splits counts the splits of all num_kv_units units together (one
 * workgroup per compute unit and 48-row chunk, or as requested), raised to
 * num_kv_units * ceil(max_tokens / T) so that every unit fits at full length,
 * with T (tokens_per_split) the longest split the MFMA kernel takes for the
 * page size; the kernels shorten the span from the row lengths.  Returns PA_EINVAL for non-positive sizes or
 * an unknown selection, PA_EUNSUPPORTED when the count would pass 65,535. */
int32_t paged_attn_plan(int32_t max_tokens, int32_t rows_per_kv_unit, int32_t num_kv_units,
                        int32_t head_dim, int32_t page_size, int32_t selection,
                        int32_t num_cus, int32_t requested_splits, pa_plan *out);

/* Dense verify of one request ([DN] first section), writing split partials.
 *   q_fp16       [q_rows][num_heads][head_dim] FP16, contiguous, 16-byte aligned
 *   kv           (host) the pool; head_dim bytes per token and head
 *   block_table  [num_table_entries] int32: logical page -> physical page
 *   row_lens     [q_rows] int32: row i sees tokens t < clamp(len_i, 0, max_tokens);
 *                zero is allowed and gives an empty row
 *   max_tokens   (host) bound on the lengths, <= num_table_entries*page_size;
 *                must equal plan->max_tokens
 *   q_rows 1..8; num_heads % num_kv_heads == 0; q_rows*num_heads/num_kv_heads
 *   <= 48 rows per KV head; head_dim 128 or 256
 *   sm_scale, k_scale (host) both > 0 and finite; the logit scale
 *                sm_scale*k_scale*log2(e) is folded on the host ([QSA]) and must
 *                be a positive normal FP32 number (PA_EINVAL otherwise)
 *   plan         (host) from paged_attn_plan(max_tokens, q_rows*num_heads/num_kv_heads,
 *                num_kv_heads, head_dim, kv->page_size, PA_SEL_DENSE, ...); besides
 *                the checks of its fields (PA_EPLAN), its splits must satisfy
 *                (int64)num_splits*tokens_per_split <= INT32_MAX and leave no
 *                split wholly past max_tokens ((num_splits-1)*tokens_per_split
 *                < max(max_tokens, 1)), and the MFMA kernel (PA_KERNEL_AUTO or
 *                _MFMA) needs (tokens_per_split-1)/page_size + 2 pages per split
 *                to fit its 1,024 (head_dim 256) or 2,048 (128) page slots
 *   ws           (host) workspace of at least plan->ws_*_bytes
 * Tokens a row does not see never reach that row's P.V: their scores are
 * replaced by -inf with selects, and in a block that some row does not see
 * whole the V bytes are cleared of NaN codes before P.V, so NaN bytes in
 * padding pages or page tails have no effect ([NB] null-block fix).  NaN bytes
 * at positions a row sees (not specified by the pages) give what the
 * definition gives: a NaN K byte makes every row that sees its token NaN, a
 * NaN V byte makes its column NaN in exactly the rows that see its token. */
int32_t paged_attn_verify_e4m3(const void *q_fp16, const pa_kv_pool *kv,
                               const int32_t *block_table, int32_t num_table_entries,
                               const int32_t *row_lens, int32_t max_tokens, int32_t q_rows,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               float sm_scale, float k_scale, const pa_plan *plan,
                               const pa_workspace *ws, void *stream);

/* Dense verify of a batch of independent requests ([DN] first section: shapes
 * outside the single-request q2-8 route -- independent-request batches, q16,
 * other grouped shapes -- take a path with FP32 accumulation and the FP32
 * split workspace), writing split partials for paged_attn_combine_batch_fp32.
 *   q_fp16       [batch][q_rows][num_heads][head_dim] FP16, contiguous, 16-byte aligned
 *   block_table  [batch][max_blocks_per_req] int32: request b's logical page ->
 *                physical page; entries up to the longest row of each request
 *                must name pages in the pool
 *   row_lens     [batch][q_rows] int32: row i of request b sees its tokens
 *                t < clamp(len, 0, max_blocks_per_req*page_size); zero allowed
 *   q_rows 1..16; num_heads % num_kv_heads == 0; q_rows*num_heads/num_kv_heads
 *   <= 96 rows per KV head (more than 48 run as two row chunks, each reading
 *   the unit's K/V); batch*num_kv_heads <= 65535; head_dim 128 or 256
 *   plan         (host) from paged_attn_plan(max_blocks_per_req*page_size,
 *                q_rows*num_heads/num_kv_heads, batch*num_kv_heads, head_dim,
 *                page_size, PA_SEL_BATCH, ...)
 *   ws           (host) acc [num_splits][rows_per_unit][head_dim], max and sum
 *                [num_splits][rows_per_unit] with rows_per_unit =
 *                q_rows*num_heads/num_kv_heads (unit row i*G + h%G for query
 *                row i, head h), and index [batch*num_kv_heads + 1]
 * Splits follow the lengths over the whole batch (a ragged plan): with U =
 * batch*num_kv_heads units, L_u the longest row length of unit u (after the
 * clamp; the KV heads of a request share it) and S = plan->num_splits, every
 * split spans T = ceil(sum_u L_u / (S - U)) positions on the 64-token tile
 * (plan->tokens_per_split when that is smaller or S <= U), unit u takes
 * S_u = ceil(L_u / T) consecutive splits, unit 0 first, and its split k covers
 * tokens [k*T, (k+1)*T).  index[u] is unit u's first split and index[U] the
 * splits used; splits past it write nothing.  A long request thus gets more
 * workgroups than a short one, and every working workgroup reads about T
 * tokens.  This is computed on the device from row_lens, so a captured call
 * replays with new lengths.
 * Other arguments, masking and errors as for paged_attn_verify_e4m3. */
int32_t paged_attn_verify_batch_e4m3(const void *q_fp16, const pa_kv_pool *kv,
                                     const int32_t *block_table, int32_t max_blocks_per_req,
                                     const int32_t *row_lens, int32_t batch, int32_t q_rows,
                                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                     float sm_scale, float k_scale, const pa_plan *plan,
                                     const pa_workspace *ws, void *stream);

/* Allocation-free dense verify of one request: paged_attn_verify_e4m3 followed
 * by paged_attn_combine_fp32 (the same kernels, so the same output bits), with
 * the FP32 split partials kept in a fixed device array of the library instead
 * of a caller workspace.  For callers that cannot allocate device memory or
 * manage a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The entry itself allocates and frees
 * nothing.
 *   Arguments as for paged_attn_verify_e4m3, plus
 *   v_scale      (host) finite; the combine's output scale
 *   out_fp16     [q_rows][num_heads][head_dim] FP16, 8-byte aligned
 * Limit: the partials, num_splits*rows*(head_dim + 2)*4 bytes with rows =
 * q_rows*num_heads (each of the three parts rounded up to 256 bytes), must fit
 * PA_NOALLOC_SCRATCH_BYTES (16 MiB; 256 splits of 48 rows at head_dim 256
 * take 12.7 MB); a larger plan returns PA_ESCRATCH before anything is
 * enqueued.  The array is a file-scope __device__ variable: every device the
 * library runs on holds its own copy until the process ends.  Its device
 * address is looked up on the first call on each device (PA_EHIP if that
 * fails).  Every call overwrites all the partials it reads, so nothing needs
 * clearing between calls; but all calls on one device share the one array,
 * so calls that may overlap on one device (other streams, other threads)
 * race and must be ordered by the caller. */
#define PA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int32_t paged_attn_verify_noalloc_e4m3(const void *q_fp16, const pa_kv_pool *kv,
                                       const int32_t *block_table, int32_t num_table_entries,
                                       const int32_t *row_lens, int32_t max_tokens,
                                       int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, float sm_scale, float k_scale,
                                       float v_scale, const pa_plan *plan, void *out_fp16,
                                       void *stream);

/* The FP32 combination (as paged_attn_combine_fp32) of the partials that
 * paged_attn_verify_batch_e4m3 wrote with the same plan and workspace: row
 * (b, i, h) merges the splits index[u] .. index[u+1]-1 of its unit u = b*Hkv
 * + h/G into out_fp16 [batch][q_rows][num_heads][head_dim] (8-byte aligned).
 * PA_EPLAN for a plan not made for this shape with PA_SEL_BATCH. */
int32_t paged_attn_combine_batch_fp32(const pa_workspace *ws, const pa_plan *plan,
                                      int32_t batch, int32_t q_rows, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, float out_scale,
                                      void *out_fp16, void *stream);

/* The batch combine for a merge across ranks ([NB] commit exposing an optional
 * base-2 LSE and FP32 partial output for cross-rank merging): the combination
 * of paged_attn_combine_batch_fp32, writing any of
 *   out_fp16 [batch][q_rows][num_heads][head_dim]  as paged_attn_combine_batch_fp32
 *   out_fp32 the same shape                        the values before FP16 rounding
 *   lse      [batch][q_rows][num_heads]            the base-2 log of each row's whole
 *                                                  softmax sum, -inf for a row whose
 *                                                  splits are all empty
 * with the meanings of paged_attn_combine_fp32_lse.  Null outputs are skipped; at
 * least one must be given (PA_EINVAL otherwise); out_fp16 8-byte, out_fp32
 * 16-byte, lse 4-byte aligned (PA_EALIGN otherwise).  Other arguments and errors
 * as for paged_attn_combine_batch_fp32. */
int32_t paged_attn_combine_batch_fp32_lse(const pa_workspace *ws, const pa_plan *plan,
                                          int32_t batch, int32_t q_rows, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          float out_scale, void *out_fp16, float *out_fp32,
                                          float *lse, void *stream);

/* FP32 combination of split partials into FP16 rows ([DN] first section):
 *   M = max over non-empty splits of max[s][r],  w_s = 2^(max[s][r] - M),
 *   out[r][d] = fp16_rne(out_scale * sum_s w_s acc[s][r][d] / sum_s w_s sum[s][r]),
 * and out[r][:] = 0 when every split of row r is empty.  A split is empty when
 * its sum is exactly 0; a NaN sum (NaN bytes at positions the row sees) is not
 * empty and makes the row NaN, as the unsplit definition does.  out_scale is the
 * V dequantisation scale ([QSA] output scale).  ws_* as written by a verify
 * call with num_splits splits and num_rows rows; out_fp16 [num_rows][head_dim]
 * (= [q_rows][num_heads][head_dim], or [batch][q_rows][num_heads][head_dim]).
 * head_dim is a multiple of 4 (<= 4096); ws_acc is 16-byte aligned and
 * out_fp16 8-byte aligned (PA_EALIGN otherwise). */
int32_t paged_attn_combine_fp32(const float *ws_acc, const float *ws_max, const float *ws_sum,
                                int32_t num_splits, int32_t num_rows, int32_t head_dim,
                                float out_scale, void *out_fp16, void *stream);

/* Combine for a merge across ranks ([NB] commit exposing an optional base-2
 * LSE and FP32 partial output for cross-rank merging, with the output gate
 * applied after the merge): the FP32 combination of paged_attn_combine_fp32,
 * writing any of
 *   out_fp16 [num_rows][head_dim]  as paged_attn_combine_fp32
 *   out_fp32 [num_rows][head_dim]  the same values before FP16 rounding
 *   lse      [num_rows]            M + log2(sum_s w_s sum[s][r]): the base-2 log
 *                                  of the row's whole softmax sum,
 *                                  log2 sum_t 2^(y_t), y_t = s_t * log2(e);
 *                                  -inf for a row whose splits are all empty
 * Null outputs are skipped; at least one must be given (PA_EINVAL otherwise).
 * out_fp16 8-byte, out_fp32 16-byte, lse 4-byte aligned (PA_EALIGN otherwise).
 * Two ranks holding disjoint tokens of the same rows merge as
 *   LSE = log2(2^lse_1 + 2^lse_2),  o = 2^(lse_1 - LSE) o_1 + 2^(lse_2 - LSE) o_2.
 * Other arguments as for paged_attn_combine_fp32. */
int32_t paged_attn_combine_fp32_lse(const float *ws_acc, const float *ws_max,
                                    const float *ws_sum, int32_t num_splits, int32_t num_rows,
                                    int32_t head_dim, float out_scale, void *out_fp16,
                                    float *out_fp32, float *lse, void *stream);

/* Sparse (QSA) verify of a batch over selected blocks ([QSA] sparse split-K
 * paged GQA kernel), writing split partials.  A block is one page.
 *   q_bf16       [batch][q_rows][num_heads][head_dim] BF16, contiguous
 *   block_table  [batch][max_blocks_per_req] int32: logical block -> physical page
 *   sel_blocks   [batch][num_kv_heads][topk] int32 logical block ids; -1 = empty
 *                slot (skipped); repeated ids are attended as often as listed
 *   row_lens     [batch][q_rows] int32: row i of request b sees logical tokens
 *                t < clamp(len, 0, max_blocks_per_req*page_size), which masks
 *                the newest block causally
 *   plan         (host) from paged_attn_plan(topk*page_size, q_rows*num_heads/num_kv_heads,
 *                batch*num_kv_heads, head_dim, page_size, PA_SEL_BLOCKS, ...);
 *                split s covers selection
 *                list positions [s*T, (s+1)*T), position p naming slot
 *                p / page_size and in-block token p % page_size
 *   rows of the workspace and of the combined output: (b, i, h).
 * Other arguments as for paged_attn_verify_e4m3. */
int32_t qsa_sparse_verify_e4m3(const void *q_bf16, const pa_kv_pool *kv,
                               const int32_t *block_table, int32_t max_blocks_per_req,
                               const int32_t *sel_blocks, int32_t topk,
                               const int32_t *row_lens, int32_t batch, int32_t q_rows,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               float sm_scale, float k_scale, const pa_plan *plan,
                               const pa_workspace *ws, void *stream);

/* Sparse (QSA) verify of a batch over selected token ids: the token-id
 * selection with -1 padding that [NB] keeps for its DCP2 operator.  The pages
 * name this interface without spelling it out; the reading taken here: each
 * (request, KV head) carries a list of logical token ids.
 *   sel_tokens   [batch][num_kv_heads][num_sel] int32 token ids; -1 = empty
 *                entry (skipped).  Id t is row t % page_size of logical block
 *                t / page_size of the request (through block_table).  Ids
 *                >= max_blocks_per_req*page_size are never seen and never
 *                index the table; repeated ids are attended as often as listed.
 *   row_lens     [batch][q_rows] int32: row i of request b sees the ids
 *                t < clamp(len, 0, max_blocks_per_req*page_size), so each row
 *                has its own mask at any position of the list
 *   plan         (host) from paged_attn_plan(num_sel, q_rows*num_heads/num_kv_heads,
 *                batch*num_kv_heads, head_dim, page_size, PA_SEL_TOKENS, ...);
 *                split s covers list entries [s*T, (s+1)*T).  The MFMA kernel
 *                takes T <= 1024 (head_dim 256) or <= 2048 (head_dim 128), which
 *                the planner keeps; a hand-made plan with a longer split runs
 *                only on PA_KERNEL_SIMPLE (PA_EPLAN otherwise).
 * Other arguments, the workspace rows and the errors as for
 * qsa_sparse_verify_e4m3.  A block selection written out as its token ids
 * (block s -> ids s*page_size .. s*page_size + page_size - 1, an empty slot
 * -> page_size entries of -1) attends the same tokens in the same list
 * order. */
int32_t qsa_sparse_verify_tokens_e4m3(const void *q_bf16, const pa_kv_pool *kv,
                                      const int32_t *block_table, int32_t max_blocks_per_req,
                                      const int32_t *sel_tokens, int32_t num_sel,
                                      const int32_t *row_lens, int32_t batch, int32_t q_rows,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float sm_scale, float k_scale, const pa_plan *plan,
                                      const pa_workspace *ws, void *stream);

/* E4M3 cache write ([QSA]: the uint8 cache is written with the layer's
 * per-tensor scales through the write path): FP16 K/V tokens into the pool's
 * pages by slot.  This entry writes the bytes of kv->k_pool and kv->v_pool.
 *   k_fp16, v_fp16 [num_tokens][num_kv_heads][head_dim] FP16, contiguous,
 *                16-byte aligned; head_dim a multiple of 16 (the pool's
 *                layout must hold head_dim bytes per head; it is the caller's)
 *   slot_mapping [num_tokens] int64: token t goes to page slot / page_size,
 *                row slot % page_size; slots < 0 or >= num_pages*page_size are
 *                skipped (nothing is written for them)
 *   kv           (host) the pool layout, as for the verify entries
 *   k_scale, v_scale (host) finite and > 0 (PA_EINVAL otherwise)
 * Each element x becomes E4M3(fp32(x) / scale), the quotient rounded once in
 * FP32: the nearest code, ties to even, saturating at +-448 (also for +-inf),
 * NaN to 0x7F, -0 to 0x80.  Tokens with equal slots race (last writer wins in
 * no defined order). */
int32_t paged_attn_cache_write_e4m3(const void *k_fp16, const void *v_fp16, int64_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim,
                                    const int64_t *slot_mapping, const pa_kv_pool *kv,
                                    float k_scale, float v_scale, void *stream);

/* Kernel timer, for measurement harnesses; no result depends on it.
 *
 * paged_attn_timer_arm(n), 0 <= n <= PA_TIMER_MAX_LAUNCHES: the next n verify
 * launches (any of the four verify entry points, any stream) made
 * with the current device current get a pair of HIP events passed with the
 * kernel's dispatch (hipExtLaunchKernel): the interval runs from the point the
 * launch is processed on the stream to the kernel's completion, so it adds no
 * marker commands to the stream but includes the dispatch delay after the
 * previous command.  n = 0 disarms.  The first
 * arm creates 2 * PA_TIMER_MAX_LAUNCHES events on the current device, kept
 * until the process ends; arming later on another device gives PA_EDEVICE.
 *
 * paged_attn_timer_read(ms, cap, count): (host) *count = launches timed since
 * the arm; waits for each of the first min(count, cap) and writes its kernel
 * time in milliseconds to ms[i], in launch order; disarms.  PA_EHIP if an
 * event cannot be read (for example a launch that failed).
 *
 * Arm, launches and read must not interleave with another thread's. */
#define PA_TIMER_MAX_LAUNCHES 1024
int32_t paged_attn_timer_arm(int32_t n);
int32_t paged_attn_timer_read(float *ms, int32_t cap, int32_t *count);

/* Streaming read probe, for measurement harnesses; no result depends on it.
 * Reads bytes (>= 0, a multiple of 16) from buf (16-byte aligned) once, with
 * 16-byte loads spread over every compute unit, and keeps nothing (sink, one
 * uint32, is written only in a case that zero-filled buffers never reach).
 * The bandwidth it reaches on a buffer much larger than the 256 MB Infinity
 * Cache is the practical HBM read ceiling of the device.  PA_EINVAL for a null
 * pointer or a bad size, PA_EALIGN for a misaligned buffer. */
int32_t paged_attn_stream_read_probe(const void *buf, int64_t bytes, uint32_t *sink,
                                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_E4M3_H */
