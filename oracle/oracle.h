/* oracle.h - FP64 CPU oracle for multi-row verify attention over a paged
 * FP8-E4M3 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.
 *
 * Sources (the three pages this work follows):
 *   [DN]  1Cat-vLLM design note "DFlash2 E4M3 attention with FP32 state"
 *         (sections "DFlash2 E4M3 attention with FP32 state",
 *          "Observability and reproduction", "Rebuilt operator results").
 *   [QSA] vLLM PR "[Model] Qwen4Exp: fp8_e4m3 main KV cache on the QSA path"
 *         (review threads, CodeRabbit finding, commits, description).
 *   [NB]  1Cat-vLLM PR "[Model] Qualify calibrated E4M3 and disk PLE with
 *         QSA DCP2" (commit fixing the grouped-page4 null-block NaN, and the
 *         commit adding the DCP merge with a base-2 LSE).
 *
 * All functions return 0 on success and a negative value when an input
 * violates a precondition (an out-of-range page id or selection); they never
 * read outside the arrays described by their arguments.
 */
#ifndef ORACLE_H
#define ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Closed-form values of the 256 E4M3FN codes (NaN for 0x7F and 0xFF). */
void orc_e4m3_table(double tab[256]);
/* Nearest E4M3 code to x, ties to the even code, |x| saturated at 448, NaN
 * to 0x7F, sign kept (so -0.0 gives 0x80). */
uint8_t orc_e4m3_encode(double x);
void orc_e4m3_encode_array(const double *x, int64_t n, uint8_t *out);

/* Cache write of FP16 K/V tokens into E4M3 pages by slot: each element x
 * becomes E4M3(fp32(x) / fp32(scale)) (nearest code, ties to even, saturating
 * at 448, NaN to 0x7F).  Slots < 0 are skipped; -1 if a slot is out of range. */
int orc_cache_write(const uint16_t *k, const uint16_t *v, int64_t num_tokens,
                    int32_t num_kv_heads, int32_t head_dim, const int64_t *slot_mapping,
                    uint8_t *k_pool, uint8_t *v_pool, int64_t page_stride, int64_t token_stride,
                    int64_t head_stride, int32_t num_pages, int32_t page_size, float k_scale,
                    float v_scale);
/* Closed-form values of IEEE binary16 / bfloat16 bit patterns. */
double orc_fp16_value(uint16_t bits);
double orc_bf16_value(uint16_t bits);

/* Dense verify for one request.
 *   q        [q_rows][num_heads][head_dim] fp16 bit patterns
 *   k_pool/v_pool: byte (p, u, g, d) at p*page_stride + u*token_stride
 *            + g*head_stride + d
 *   block_table[num_entries]: logical page -> physical page
 *   row_lens[q_rows]: row i sees tokens t < clamp(len_i, 0, max_tokens)
 *   out      [q_rows][num_heads][head_dim] FP64 */
int orc_verify_dense(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                     int64_t page_stride, int64_t token_stride, int64_t head_stride,
                     int32_t num_pages, int32_t page_size,
                     const int32_t *block_table, int32_t num_entries,
                     const int32_t *row_lens, int32_t max_tokens,
                     int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                     int32_t head_dim, double sm_scale, double k_scale, double v_scale,
                     int32_t nthreads, double *out);

/* Split partials of the dense verify: split s covers tokens
 * [s*T, min((s+1)*T, L_i)).  Rows are ordered like the output, (i, h).
 *   ws_acc [S][q_rows*num_heads][head_dim]  sum of 2^(y_t - m_s) * v(t)
 *   ws_max [S][q_rows*num_heads]            m_s = max y_t, y_t = s_t*log2(e)
 *   ws_sum [S][q_rows*num_heads]            l_s = sum of 2^(y_t - m_s)
 * An empty split gives m = -inf, l = 0, acc = 0.  v_scale is not applied. */
int orc_verify_dense_split(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                           int64_t page_stride, int64_t token_stride, int64_t head_stride,
                           int32_t num_pages, int32_t page_size,
                           const int32_t *block_table, int32_t num_entries,
                           const int32_t *row_lens, int32_t max_tokens,
                           int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, double sm_scale, double k_scale,
                           int32_t num_splits, int32_t tokens_per_split, int32_t nthreads,
                           double *ws_acc, double *ws_max, double *ws_sum);

/* Merge of split partials: o = v_scale * sum_s w_s acc_s / sum_s w_s l_s with
 * w_s = 2^(m_s - M), M the largest m_s over non-empty splits; 0 when every
 * split is empty.  The _f32 form reads an FP32 workspace. */
int orc_combine(const double *ws_acc, const double *ws_max, const double *ws_sum,
                int32_t num_splits, int32_t num_rows, int32_t head_dim, double v_scale,
                double *out);
int orc_combine_f32(const float *ws_acc, const float *ws_max, const float *ws_sum,
                    int32_t num_splits, int32_t num_rows, int32_t head_dim, double v_scale,
                    double *out);

/* The same merge, also writing lse[r] = M + log2(sum_s w_s l_s): the base-2
 * log of the row's whole softmax sum, log2 sum_t 2^(y_t) with y_t the logit
 * times log2(e); -inf for a row whose splits are all empty.  Two disjoint token
 * sets of one row merge as LSE = log2(2^lse_1 + 2^lse_2),
 * o = 2^(lse_1 - LSE) o_1 + 2^(lse_2 - LSE) o_2 (1Cat-vLLM PR "Qualify
 * calibrated E4M3 and disk PLE with QSA DCP2": base-2 LSE and FP32 partial
 * output exported for the merge across ranks). */
int orc_combine_lse(const double *ws_acc, const double *ws_max, const double *ws_sum,
                    int32_t num_splits, int32_t num_rows, int32_t head_dim, double v_scale,
                    double *out, double *lse);
int orc_combine_lse_f32(const float *ws_acc, const float *ws_max, const float *ws_sum,
                        int32_t num_splits, int32_t num_rows, int32_t head_dim,
                        double v_scale, double *out, double *lse);

/* Sparse (QSA) verify over selected blocks, a batch of requests.
 *   q          [batch][q_rows][num_heads][head_dim] bfloat16 bit patterns
 *   block_table[batch][max_blocks]: logical block -> physical page (block = page)
 *   sel        [batch][num_kv_heads][topk]: logical block ids, -1 = empty
 *   row_lens   [batch][q_rows]: row i of request b sees logical tokens
 *              t < clamp(len, 0, max_blocks*page_size)
 *   out        [batch][q_rows][num_heads][head_dim] FP64
 * The token set of (b, g) is the multiset union of the selected blocks. */
int orc_qsa_verify(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                   int64_t page_stride, int64_t token_stride, int64_t head_stride,
                   int32_t num_pages, int32_t page_size,
                   const int32_t *block_table, int32_t max_blocks,
                   const int32_t *sel, int32_t topk, const int32_t *row_lens,
                   int32_t batch, int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                   int32_t head_dim, double sm_scale, double k_scale, double v_scale,
                   int32_t nthreads, double *out);

/* Split partials of the sparse verify.  The list position p in
 * [0, topk*page_size) names selection entry p / page_size and in-block token
 * p % page_size; split s covers positions [s*T, (s+1)*T).  Rows are ordered
 * (b, i, h). */
int orc_qsa_split(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                  int64_t page_stride, int64_t token_stride, int64_t head_stride,
                  int32_t num_pages, int32_t page_size,
                  const int32_t *block_table, int32_t max_blocks,
                  const int32_t *sel, int32_t topk, const int32_t *row_lens,
                  int32_t batch, int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                  int32_t head_dim, double sm_scale, double k_scale,
                  int32_t num_splits, int32_t tokens_per_split, int32_t nthreads,
                  double *ws_acc, double *ws_max, double *ws_sum);

/* Sparse verify over selected token ids (the token-id selection with -1
 * padding that 1Cat-vLLM PR "Qualify calibrated E4M3 and disk PLE with QSA
 * DCP2" keeps): sel_tokens [batch][num_kv_heads][num_sel] logical token ids,
 * -1 = empty.  Entry j with id t >= 0 is token t of request b: block t /
 * page_size through block_table, row t % page_size.  Row i keeps the entries
 * with t < clamp(len, 0, max_blocks*page_size), so each row gets its own mask
 * in any block.  Other arguments as for orc_qsa_verify; the split form splits
 * by list entry: split s covers entries [s*T, (s+1)*T). */
int orc_qsa_tokens_verify(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                          int64_t page_stride, int64_t token_stride, int64_t head_stride,
                          int32_t num_pages, int32_t page_size,
                          const int32_t *block_table, int32_t max_blocks,
                          const int32_t *sel_tokens, int32_t num_sel, const int32_t *row_lens,
                          int32_t batch, int32_t q_rows, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, double sm_scale,
                          double k_scale, double v_scale, int32_t nthreads, double *out);
int orc_qsa_tokens_split(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                         int64_t page_stride, int64_t token_stride, int64_t head_stride,
                         int32_t num_pages, int32_t page_size,
                         const int32_t *block_table, int32_t max_blocks,
                         const int32_t *sel_tokens, int32_t num_sel, const int32_t *row_lens,
                         int32_t batch, int32_t q_rows, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, double sm_scale,
                         double k_scale, int32_t num_splits, int32_t tokens_per_split,
                         int32_t nthreads, double *ws_acc, double *ws_max, double *ws_sum);

#ifdef __cplusplus
}
#endif
#endif
