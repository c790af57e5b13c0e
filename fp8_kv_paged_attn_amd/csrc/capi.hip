// capi.hip - the C ABI of libpaged_attn_e4m3: argument checks, the split
// planner and kernel dispatch.  Host code only; the kernels live in the other
// sources of this directory.
//
// Every check here runs before anything is enqueued, so a rejected call
// leaves the stream untouched (design note "DFlash2 E4M3 attention with FP32
// state": an incompatible call raises instead of silently using another
// precision; vLLM PR "Qwen4Exp: fp8_e4m3 main KV cache on the QSA path",
// CodeRabbit finding: scales are validated before the launch).
#include "paged_attn_e4m3.h"
#include "pa_internal.h"

#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>

#ifndef PA_BUILD_ID
#error "PA_BUILD_ID (the source hash) is defined by the build"
#endif

namespace {

constexpr int kTileTokens = 64;
constexpr int kMaxRowsPerUnit = 48;
constexpr int kMaxQRows = 8;
// the verify kernel stores a KV unit's partial rows by 32-bit byte offsets from
// the unit's first row: q_rows * num_heads * head_dim * 4 must stay below 2^31
constexpr int kMaxHeads = 65536;
// the batched entry: up to 16 query rows, up to 96 rows per KV unit (two
// 48-row chunks, one workgroup each)
constexpr int kMaxRowsPerUnitBatch = 96;
constexpr int kMaxQRowsBatch = pa::kRaggedMaxQRows;
constexpr int kDefaultCUs = 256;
// Fewest tokens a split should read, so that the FP32 partial it writes
// (rows x (head_dim + 2) x 4 bytes) stays small against its K/V bytes.
constexpr int kMinTokensPerSplit = 128;
// Tokens of one step of an MFMA workgroup (four waves of 32-token blocks).
constexpr int kChunkStepTokens = 128;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned16(int64_t v) { return (v & 15) == 0; }

// Per-device record: 0 unknown, 1 gfx950, -1 something else.
std::atomic<int> g_device_ok[64];
// Per-device compute-unit count: 0 unknown.
std::atomic<int> g_device_cus[64];

// Compute units of the current device, queried once per device; kDefaultCUs
// when no device can be queried (a host without a GPU).
int device_cus()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return kDefaultCUs;
    if (dev < 64) {
        const int known = g_device_cus[dev].load(std::memory_order_relaxed);
        if (known > 0)
            return known;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
        return kDefaultCUs;
    if (dev < 64)
        g_device_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

int32_t check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return PA_EDEVICE;
    if (dev < 64) {
        int known = g_device_ok[dev].load(std::memory_order_relaxed);
        if (known != 0)
            return known > 0 ? PA_OK : PA_EDEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return PA_EDEVICE;
    bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64)
        g_device_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? PA_OK : PA_EDEVICE;
}

int32_t check_pool(const pa_kv_pool *kv)
{
    if (!kv || !kv->k_pool || !kv->v_pool)
        return PA_EINVAL;
    if (kv->page_size < 1 || kv->num_pages < 1 || kv->page_stride < 0 || kv->token_stride < 0 ||
        kv->head_stride < 0)
        return PA_EINVAL;
    if (!aligned16(kv->k_pool) || !aligned16(kv->v_pool) || !aligned16(kv->page_stride) ||
        !aligned16(kv->token_stride) || !aligned16(kv->head_stride))
        return PA_EALIGN;
    return PA_OK;
}

int32_t check_shape(int32_t q_rows, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t *rows_per_unit, int32_t max_q_rows = kMaxQRows,
                    int32_t max_rows = kMaxRowsPerUnit)
{
    if (q_rows < 1 || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0)
        return PA_EINVAL;
    if (q_rows > max_q_rows || num_heads > kMaxHeads)
        return PA_EUNSUPPORTED;
    if (head_dim != 128 && head_dim != 256)
        return PA_EUNSUPPORTED;
    int64_t rows = (int64_t)q_rows * (num_heads / num_kv_heads);
    if (rows > max_rows)
        return PA_EUNSUPPORTED;
    *rows_per_unit = (int32_t)rows;
    return PA_OK;
}

// The folded logit scale sm_scale * k_scale * log2(e) must be a positive normal
// FP32 number: the kernels take row maxima on raw scores and scale afterwards.
int32_t check_scales(float sm_scale, float k_scale)
{
    if (!std::isfinite(sm_scale) || !std::isfinite(k_scale) || !(sm_scale > 0.0f) ||
        !(k_scale > 0.0f))
        return PA_EINVAL;
    const float c = (float)((double)sm_scale * (double)k_scale * 1.4426950408889634);
    if (!std::isnormal(c))
        return PA_EINVAL;
    return PA_OK;
}

// Rows of a KV unit one MFMA workgroup takes (a plan's 0 reads as 48).
int32_t chunk_rows(const pa_plan *plan)
{
    return plan->rows_per_workgroup == 0 ? kMaxRowsPerUnit : plan->rows_per_workgroup;
}

// A plan fits a call when it was made for the call's sizes, page size and
// selection, its splits cover the list without a split wholly past it and
// without 32-bit overflow of a split's bounds, and -- for the MFMA kernel --
// every split's page slots fit that kernel's LDS slot cache.
int32_t check_plan(const pa_plan *plan, int32_t list_len, int32_t rows_per_unit,
                   int32_t units, int32_t head_dim, int32_t page_size, int32_t selection)
{
    if (!plan)
        return PA_EINVAL;
    if (plan->max_tokens != list_len || plan->rows_per_kv_unit != rows_per_unit ||
        plan->num_kv_units != units || plan->head_dim != head_dim ||
        plan->page_size != page_size || plan->selection != selection)
        return PA_EPLAN;
    if (plan->num_splits < 1 || plan->tokens_per_split < kTileTokens ||
        plan->tokens_per_split % kTileTokens != 0 || plan->num_splits > 65535)
        return PA_EPLAN;
    if (plan->kernel < PA_KERNEL_AUTO || plan->kernel > PA_KERNEL_MFMA)
        return PA_EPLAN;
    const int32_t ch = chunk_rows(plan);
    if (ch != 16 && ch != 32 && ch != kMaxRowsPerUnit)
        return PA_EPLAN;
    if (selection == PA_SEL_BATCH && ch != kMaxRowsPerUnit)
        return PA_EPLAN;
    if (plan->kernel != PA_KERNEL_SIMPLE &&
        pa::mfma_slots_needed(plan->tokens_per_split, page_size, selection == PA_SEL_TOKENS) >
            pa::mfma_max_slots(head_dim))
        return PA_EPLAN;
    if (selection == PA_SEL_BATCH) {
        // a ragged batch: its splits are shared by all units, and there must be
        // enough of them for every unit at full length at the plan's span (so
        // the span the kernels derive from the lengths always fits them all)
        const int64_t T = plan->tokens_per_split;
        if ((int64_t)list_len + T > INT32_MAX)
            return PA_EPLAN;
        if ((int64_t)plan->num_splits < (int64_t)units * ((list_len + T - 1) / T))
            return PA_EPLAN;
        return PA_OK;
    }
    const int64_t span = (int64_t)plan->num_splits * plan->tokens_per_split;
    if (span < (int64_t)list_len || span > INT32_MAX)
        return PA_EPLAN;
    if ((int64_t)(plan->num_splits - 1) * plan->tokens_per_split >=
        (int64_t)(list_len > 1 ? list_len : 1))
        return PA_EPLAN;
    return PA_OK;
}

// total_rows: rows of one split's partials (all output rows, or for a ragged
// batch the rows of one unit); index_entries: split-index entries a ragged
// batch writes (0: none)
int32_t check_ws(const pa_workspace *ws, const pa_plan *plan, int64_t total_rows,
                 int32_t head_dim, int64_t index_entries = 0)
{
    if (!ws || !ws->acc || !ws->max || !ws->sum)
        return PA_EINVAL;
    int64_t need_acc = (int64_t)plan->num_splits * total_rows * head_dim * 4;
    int64_t need_stat = (int64_t)plan->num_splits * total_rows * 4;
    if (ws->acc_bytes < need_acc || ws->stat_bytes < need_stat)
        return PA_EWORKSPACE;
    if (index_entries > 0) {
        if (!ws->index)
            return PA_EINVAL;
        if (ws->index_bytes < index_entries * 4)
            return PA_EWORKSPACE;
    }
    return PA_OK;
}

// Checks shared by the combine entry points; any of the three outputs may be
// null (the caller checks that one is not).
int32_t combine_checked(const float *ws_acc, const float *ws_max, const float *ws_sum,
                        int32_t num_splits, int32_t num_rows, int32_t head_dim, float out_scale,
                        void *out_fp16, float *out_fp32, float *lse, void *stream)
{
    if (!ws_acc || !ws_max || !ws_sum)
        return PA_EINVAL;
    if (num_splits < 1 || num_rows < 0 || head_dim < 4 || head_dim > 4096 ||
        head_dim % 4 != 0 || !std::isfinite(out_scale))
        return PA_EINVAL;
    if (!aligned16(ws_acc) || (reinterpret_cast<uintptr_t>(out_fp16) & 7u) != 0 ||
        !aligned16(out_fp32) || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
        return PA_EALIGN;
    if (num_rows > 0x7FFFFFFF / 2)
        return PA_EINVAL;
    int32_t rc = check_device();
    if (rc != PA_OK)
        return rc;
    hipError_t err = pa::launch_combine(ws_acc, ws_max, ws_sum, num_splits, num_rows, head_dim,
                                        out_scale, static_cast<uint16_t *>(out_fp16), out_fp32,
                                        lse, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PA_OK : PA_EHIP;
}

// Kernel timer: (begin, end) event pairs handed to the next `armed` verify
// launches on the device the timer was armed on, passed with the dispatch.
struct KernelTimer {
    std::mutex mu;
    hipEvent_t ev[2 * PA_TIMER_MAX_LAUNCHES] = {};
    bool created = false;
    int device = -1;
    int armed = 0, used = 0;
};
KernelTimer g_timer;

// The event pair for this launch, or nullptr when the timer is not armed.
const hipEvent_t *timer_take()
{
    std::lock_guard<std::mutex> lock(g_timer.mu);
    if (g_timer.used >= g_timer.armed)
        return nullptr;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != g_timer.device)
        return nullptr;
    return &g_timer.ev[2 * g_timer.used++];
}

int32_t dispatch(const pa::VerifyArgs &a, const pa_plan *plan, int head_dim,
                 pa::VerifyMode mode, hipStream_t stream)
{
    int32_t rc = check_device();
    if (rc != PA_OK)
        return rc;
    const hipEvent_t *ev = timer_take();
    hipError_t err;
    if (plan->kernel == PA_KERNEL_SIMPLE) {
        err = pa::launch_verify_simple(a, head_dim, mode, stream, ev);
    } else {
        // AUTO is the MFMA kernel; check_plan has made sure it takes the plan,
        // and nothing falls back to the plain kernel
        err = pa::launch_verify_mfma(a, head_dim, mode, stream, ev);
        if (err == hipErrorNotSupported)
            return PA_EPLAN;
    }
    return err == hipSuccess ? PA_OK : PA_EHIP;
}

// The two sparse entries: a selection list of blocks (positions topk * page)
// or of token ids (positions topk), -1 = empty.
int32_t sparse_verify(pa::VerifyMode mode, const void *q_bf16, const pa_kv_pool *kv,
                      const int32_t *block_table, int32_t max_blocks_per_req,
                      const int32_t *sel, int32_t topk, const int32_t *row_lens,
                      int32_t batch, int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                      int32_t head_dim, float sm_scale, float k_scale, const pa_plan *plan,
                      const pa_workspace *ws, void *stream)
{
    int32_t rc, rows_per_unit = 0;
    if (!q_bf16 || !block_table || !sel || !row_lens)
        return PA_EINVAL;
    if ((rc = check_pool(kv)) != PA_OK)
        return rc;
    if ((rc = check_shape(q_rows, num_heads, num_kv_heads, head_dim, &rows_per_unit)) != PA_OK)
        return rc;
    if (!aligned16(q_bf16))
        return PA_EALIGN;
    if (batch < 1 || max_blocks_per_req < 1 || topk < 1)
        return PA_EINVAL;
    const int64_t list_len =
        mode == pa::kModeTokens ? (int64_t)topk : (int64_t)topk * kv->page_size;
    const int64_t cap = (int64_t)max_blocks_per_req * kv->page_size;
    if (list_len > 0x7FFFFFFF || cap > 0x7FFFFFFF)
        return PA_EINVAL;
    if ((int64_t)batch * num_kv_heads > 65535)
        return PA_EUNSUPPORTED;
    if ((rc = check_scales(sm_scale, k_scale)) != PA_OK)
        return rc;
    if ((rc = check_plan(plan, (int32_t)list_len, rows_per_unit, batch * num_kv_heads,
                         head_dim, kv->page_size,
                         mode == pa::kModeTokens ? PA_SEL_TOKENS : PA_SEL_BLOCKS)) != PA_OK)
        return rc;
    const int64_t total_rows = (int64_t)batch * q_rows * num_heads;
    if (total_rows > 0x7FFFFFFF)
        return PA_EINVAL;
    if ((rc = check_ws(ws, plan, total_rows, head_dim)) != PA_OK)
        return rc;

    pa::VerifyArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = static_cast<const uint16_t *>(q_bf16);
    a.k_pool = kv->k_pool;
    a.v_pool = kv->v_pool;
    a.page_stride = kv->page_stride;
    a.token_stride = kv->token_stride;
    a.head_stride = kv->head_stride;
    a.page_size = kv->page_size;
    a.block_table = block_table;
    a.table_stride = max_blocks_per_req;
    a.sel = sel;
    a.topk = topk;
    a.row_lens = row_lens;
    a.len_cap = (int32_t)cap;
    a.list_len = (int32_t)list_len;
    a.batch = batch;
    a.q_rows = q_rows;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_heads / num_kv_heads;
    a.rows = rows_per_unit;
    a.chunk_rows = chunk_rows(plan);
    a.num_splits = plan->num_splits;
    a.tokens_per_split = plan->tokens_per_split;
    a.total_rows = (int32_t)total_rows;
    a.logit_scale = (float)((double)sm_scale * (double)k_scale * 1.4426950408889634);
    a.ws_acc = ws->acc;
    a.ws_max = ws->max;
    a.ws_sum = ws->sum;
    return dispatch(a, plan, head_dim, mode, static_cast<hipStream_t>(stream));
}

// Checks and kernel arguments of one dense request (everything but the
// workspace), shared by the dense entry points.
int32_t dense_args(const void *q_fp16, const pa_kv_pool *kv, const int32_t *block_table,
                   int32_t num_table_entries, const int32_t *row_lens, int32_t max_tokens,
                   int32_t q_rows, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                   float sm_scale, float k_scale, const pa_plan *plan, pa::VerifyArgs *out)
{
    int32_t rc, rows_per_unit = 0;
    if (!q_fp16 || !block_table || !row_lens)
        return PA_EINVAL;
    if ((rc = check_pool(kv)) != PA_OK)
        return rc;
    if ((rc = check_shape(q_rows, num_heads, num_kv_heads, head_dim, &rows_per_unit)) != PA_OK)
        return rc;
    if (!aligned16(q_fp16))
        return PA_EALIGN;
    if (num_table_entries < 0 || max_tokens < 0 ||
        (int64_t)max_tokens > (int64_t)num_table_entries * kv->page_size)
        return PA_EINVAL;
    if ((rc = check_scales(sm_scale, k_scale)) != PA_OK)
        return rc;
    if ((int64_t)q_rows * num_heads > INT32_MAX)
        return PA_EINVAL;
    if (num_kv_heads > 65535)
        return PA_EUNSUPPORTED;
    if ((rc = check_plan(plan, max_tokens, rows_per_unit, num_kv_heads, head_dim, kv->page_size,
                         PA_SEL_DENSE)) != PA_OK)
        return rc;
    pa::VerifyArgs &a = *out;
    std::memset(&a, 0, sizeof a);
    a.q = static_cast<const uint16_t *>(q_fp16);
    a.k_pool = kv->k_pool;
    a.v_pool = kv->v_pool;
    a.page_stride = kv->page_stride;
    a.token_stride = kv->token_stride;
    a.head_stride = kv->head_stride;
    a.page_size = kv->page_size;
    a.block_table = block_table;
    a.table_stride = 0;
    a.sel = nullptr;
    a.topk = 0;
    a.row_lens = row_lens;
    a.len_cap = max_tokens;
    a.list_len = max_tokens;
    a.batch = 1;
    a.q_rows = q_rows;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_heads / num_kv_heads;
    a.rows = rows_per_unit;
    a.chunk_rows = chunk_rows(plan);
    a.num_splits = plan->num_splits;
    a.tokens_per_split = plan->tokens_per_split;
    a.total_rows = q_rows * num_heads;
    a.logit_scale = (float)((double)sm_scale * (double)k_scale * 1.4426950408889634);
    return PA_OK;
}

int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

// Scratch of the allocation-free entry point: the FP32 split partials of one
// call, in a fixed array of every device the library runs on (held until the
// process ends).  Host code never uses the array's name as an address: its
// device address is looked up once per device, with that device current, and
// kept.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
uint8_t *g_scratch_base[64] = {};

int32_t scratch_base(uint8_t **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return PA_EDEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_base[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return PA_EHIP;
        g_scratch_base[dev] = static_cast<uint8_t *>(p);
    }
    *out = g_scratch_base[dev];
    return PA_OK;
}

}  // namespace

extern "C" {

int32_t paged_attn_abi_version(void) { return PA_ABI_VERSION; }

const char *paged_attn_build_id(void) { return PA_BUILD_ID; }

const char *paged_attn_status_string(int32_t status)
{
    switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument (null pointer, shape, count or scale)";
    case PA_EUNSUPPORTED: return "unsupported shape (head_dim, query rows or rows per KV head)";
    case PA_EWORKSPACE: return "workspace smaller than the plan requires";
    case PA_EALIGN: return "pointer or stride not 16-byte aligned";
    case PA_EDEVICE: return "no usable gfx950 device";
    case PA_EHIP: return "HIP launch failed";
    case PA_EPLAN: return "plan does not match this call";
    case PA_ESCRATCH:
        return "plan needs more partials than the allocation-free entry's fixed scratch holds";
    default: return "unknown status";
    }
}

int32_t paged_attn_plan(int32_t max_tokens, int32_t rows_per_kv_unit, int32_t num_kv_units,
                        int32_t head_dim, int32_t page_size, int32_t selection,
                        int32_t num_cus, int32_t requested_splits, pa_plan *out)
{
    if (!out || max_tokens < 0 || rows_per_kv_unit < 1 || num_kv_units < 1 || head_dim < 1 ||
        requested_splits < 0 || page_size < 1 || selection < PA_SEL_DENSE ||
        selection > PA_SEL_BATCH)
        return PA_EINVAL;
    const int64_t cus = num_cus > 0 ? num_cus : device_cus();
    const int64_t tiles = max_tokens > 0 ? (max_tokens + kTileTokens - 1) / kTileTokens : 1;
    const int64_t slots = pa::mfma_max_slots(head_dim);
    if (selection == PA_SEL_BATCH) {
        // a ragged batch: num_splits counts the splits of all units together,
        // one workgroup per compute unit and 48-row chunk (or as requested),
        // but at least enough for every unit at full length at the longest
        // span the MFMA kernel takes
        const int64_t chunks = ((int64_t)rows_per_kv_unit + 47) / 48;
        int64_t T = (slots - 1) * (int64_t)page_size / kTileTokens * kTileTokens;
        if (T > tiles * kTileTokens)
            T = tiles * kTileTokens;
        int64_t splits = requested_splits > 0 ? requested_splits : (cus + chunks - 1) / chunks;
        const int64_t need = (int64_t)num_kv_units * (((int64_t)max_tokens + T - 1) / T);
        if (splits < need)
            splits = need;
        if (splits < 1)
            splits = 1;
        if (splits > 65535 || (int64_t)max_tokens + T > INT32_MAX)
            return PA_EUNSUPPORTED;
        std::memset(out, 0, sizeof *out);
        out->num_splits = (int32_t)splits;
        out->tokens_per_split = (int32_t)T;
        out->kernel = PA_KERNEL_AUTO;
        out->max_tokens = max_tokens;
        out->rows_per_kv_unit = rows_per_kv_unit;
        out->num_kv_units = num_kv_units;
        out->head_dim = head_dim;
        out->page_size = page_size;
        out->selection = selection;
        out->ws_acc_bytes = splits * rows_per_kv_unit * head_dim * 4;
        out->ws_stat_bytes = splits * rows_per_kv_unit * 4;
        out->ws_index_bytes = ((int64_t)num_kv_units + 1) * 4;
        out->rows_per_workgroup = kMaxRowsPerUnit;
        return PA_OK;
    }
    // longest split whose page slots (token ids: entries) fit the MFMA
    // kernel's cache: (T - 1) / page + 2 <= slots, i.e. T <= (slots - 1) * page
    int64_t tcap = selection == PA_SEL_TOKENS ? slots : (slots - 1) * (int64_t)page_size;
    tcap = tcap / kTileTokens * kTileTokens;
    // the split length for a wanted split count: whole tiles, within the
    // cache, and the count that length needs
    struct Shape {
        int64_t splits, tps;
    };
    auto shape_for = [&](int64_t want) -> Shape {
        if (want > tiles)
            want = tiles;
        if (want > 65535)
            want = 65535;
        int64_t tps = (tiles + want - 1) / want * kTileTokens;
        if (tps > tcap)
            tps = tcap;
        return {max_tokens > 0 ? ((int64_t)max_tokens + tps - 1) / tps : 1, tps};
    };
    // no split shorter than kMinTokensPerSplit tokens
    int64_t min_cap = ((int64_t)max_tokens + kMinTokensPerSplit - 1) / kMinTokensPerSplit;
    if (min_cap < 1)
        min_cap = 1;
    Shape sh;
    int64_t chunk = kMaxRowsPerUnit;
    if (requested_splits > 0) {
        sh = shape_for(requested_splits);
    } else {
        // at most one workgroup per compute unit over all units, a unit of
        // more than 48 rows taking one workgroup per 48-row chunk (a count
        // rounded up would leave a few workgroups for a second round: three
        // KV heads at 64K with 86 splits, 258 workgroups, took 49.8 us per
        // call against 32.4 with 79) ...
        const int64_t wgs = (int64_t)num_kv_units * (((int64_t)rows_per_kv_unit + 47) / 48);
        int64_t want = cus / wgs > 1 ? cus / wgs : 1;
        // ... but no split shorter than kMinTokensPerSplit tokens
        sh = shape_for(want < min_cap ? want : min_cap);
        // A short list leaves each 48-row workgroup fewer than two 128-token
        // steps (at most one block per wave, some waves idle) beside a fixed
        // cost of the same order.  Smaller row chunks then put more compute
        // units on the list, with longer splits and less work per token each
        // (the chunks of a split read the same K/V, mostly from L2): 16 rows
        // with splits of at most three steps, else 32 rows with at most four,
        // within one workgroup per compute unit.  (MI355X, q8 rows of six
        // heads, per call: 8K 14.8 us at 48 rows against 11.5 at 16; 24K 18.8
        // against 14.7 at 16; 48K 21.4 against 17.7 at 32.  From two steps
        // on, at 64K and up, 48 rows gave the faster verify kernel.)  The
        // count of (split, unit) pairs is kept a multiple of 8, so that the
        // chunks of a pair, whose workgroup ids differ by a multiple of it,
        // run on one XCD and share its L2 (79 splits instead of 64 at 64K
        // took 23.8 against 21.6 us per call).
        if (sh.tps < 2 * kChunkStepTokens) {
            const int64_t chunk_rows[2] = {16, 32}, max_steps[2] = {3, 4};
            bool found = false;
            for (int k = 0; k < 2 && !found; ++k) {
                const int64_t c = chunk_rows[k];
                if (rows_per_kv_unit <= c)
                    continue;   // one chunk of the unit either way
                const int64_t per = (int64_t)num_kv_units * (((int64_t)rows_per_kv_unit + c - 1) / c);
                int64_t w = cus / per;
                if (w > min_cap)
                    w = min_cap;
                for (; w >= 1; --w) {
                    const Shape sc = shape_for(w);
                    if (sc.tps > max_steps[k] * kChunkStepTokens)
                        break;   // fewer splits only make them longer
                    const int64_t pairs = sc.splits * num_kv_units;
                    if (sc.splits * per <= cus && (pairs % 8 == 0 || pairs < 8)) {
                        sh = sc;
                        chunk = c;
                        found = true;
                        break;
                    }
                }
            }
        }
    }
    const int64_t splits = sh.splits, tps = sh.tps;
    if (splits > 65535 || splits * tps > INT32_MAX)
        return PA_EUNSUPPORTED;
    const int64_t rows = (int64_t)rows_per_kv_unit * num_kv_units;
    std::memset(out, 0, sizeof *out);
    out->num_splits = (int32_t)splits;
    out->tokens_per_split = (int32_t)tps;
    out->kernel = PA_KERNEL_AUTO;
    out->max_tokens = max_tokens;
    out->rows_per_kv_unit = rows_per_kv_unit;
    out->num_kv_units = num_kv_units;
    out->head_dim = head_dim;
    out->page_size = page_size;
    out->selection = selection;
    out->ws_acc_bytes = splits * rows * head_dim * 4;
    out->ws_stat_bytes = splits * rows * 4;
    out->rows_per_workgroup = (int32_t)chunk;
    return PA_OK;
}

int32_t paged_attn_verify_e4m3(const void *q_fp16, const pa_kv_pool *kv,
                               const int32_t *block_table, int32_t num_table_entries,
                               const int32_t *row_lens, int32_t max_tokens, int32_t q_rows,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               float sm_scale, float k_scale, const pa_plan *plan,
                               const pa_workspace *ws, void *stream)
{
    pa::VerifyArgs a;
    int32_t rc = dense_args(q_fp16, kv, block_table, num_table_entries, row_lens, max_tokens,
                            q_rows, num_heads, num_kv_heads, head_dim, sm_scale, k_scale, plan,
                            &a);
    if (rc != PA_OK)
        return rc;
    if ((rc = check_ws(ws, plan, a.total_rows, head_dim)) != PA_OK)
        return rc;
    a.ws_acc = ws->acc;
    a.ws_max = ws->max;
    a.ws_sum = ws->sum;
    return dispatch(a, plan, head_dim, pa::kModeDense, static_cast<hipStream_t>(stream));
}

int32_t paged_attn_verify_noalloc_e4m3(const void *q_fp16, const pa_kv_pool *kv,
                                       const int32_t *block_table, int32_t num_table_entries,
                                       const int32_t *row_lens, int32_t max_tokens,
                                       int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, float sm_scale, float k_scale,
                                       float v_scale, const pa_plan *plan, void *out_fp16,
                                       void *stream)
{
    pa::VerifyArgs a;
    int32_t rc = dense_args(q_fp16, kv, block_table, num_table_entries, row_lens, max_tokens,
                            q_rows, num_heads, num_kv_heads, head_dim, sm_scale, k_scale, plan,
                            &a);
    if (rc != PA_OK)
        return rc;
    if (!out_fp16)
        return PA_EINVAL;
    if ((reinterpret_cast<uintptr_t>(out_fp16) & 7u) != 0)
        return PA_EALIGN;
    if (!std::isfinite(v_scale))
        return PA_EINVAL;
    // the partials' layout in the scratch array: acc, then max, then sum,
    // each starting on a 256-byte boundary
    const int64_t cells = (int64_t)plan->num_splits * a.total_rows;
    const int64_t acc_bytes = align256(cells * head_dim * 4);
    const int64_t stat_bytes = align256(cells * 4);
    if (acc_bytes + 2 * stat_bytes > PA_NOALLOC_SCRATCH_BYTES)
        return PA_ESCRATCH;
    if ((rc = check_device()) != PA_OK)
        return rc;
    uint8_t *base = nullptr;
    if ((rc = scratch_base(&base)) != PA_OK)
        return rc;
    a.ws_acc = reinterpret_cast<float *>(base);
    a.ws_max = reinterpret_cast<float *>(base + acc_bytes);
    a.ws_sum = reinterpret_cast<float *>(base + acc_bytes + stat_bytes);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = dispatch(a, plan, head_dim, pa::kModeDense, st)) != PA_OK)
        return rc;
    // the verify kernel has written every (split, row) of the partials it
    // combines, so nothing in the array needs clearing between calls
    const hipError_t err = pa::launch_combine(a.ws_acc, a.ws_max, a.ws_sum, plan->num_splits,
                                              a.total_rows, head_dim, v_scale,
                                              static_cast<uint16_t *>(out_fp16), nullptr,
                                              nullptr, st);
    return err == hipSuccess ? PA_OK : PA_EHIP;
}

int32_t paged_attn_verify_batch_e4m3(const void *q_fp16, const pa_kv_pool *kv,
                                     const int32_t *block_table, int32_t max_blocks_per_req,
                                     const int32_t *row_lens, int32_t batch, int32_t q_rows,
                                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                     float sm_scale, float k_scale, const pa_plan *plan,
                                     const pa_workspace *ws, void *stream)
{
    int32_t rc, rows_per_unit = 0;
    if (!q_fp16 || !block_table || !row_lens)
        return PA_EINVAL;
    if ((rc = check_pool(kv)) != PA_OK)
        return rc;
    if ((rc = check_shape(q_rows, num_heads, num_kv_heads, head_dim, &rows_per_unit,
                          kMaxQRowsBatch, kMaxRowsPerUnitBatch)) != PA_OK)
        return rc;
    if (!aligned16(q_fp16))
        return PA_EALIGN;
    if (batch < 1 || max_blocks_per_req < 1)
        return PA_EINVAL;
    const int64_t cap = (int64_t)max_blocks_per_req * kv->page_size;
    if (cap > 0x7FFFFFFF)
        return PA_EINVAL;
    if ((int64_t)batch * num_kv_heads > 65535)
        return PA_EUNSUPPORTED;
    if ((rc = check_scales(sm_scale, k_scale)) != PA_OK)
        return rc;
    if ((rc = check_plan(plan, (int32_t)cap, rows_per_unit, batch * num_kv_heads, head_dim,
                         kv->page_size, PA_SEL_BATCH)) != PA_OK)
        return rc;
    const int64_t total_rows = (int64_t)batch * q_rows * num_heads;
    if (total_rows > 0x7FFFFFFF)
        return PA_EINVAL;
    if ((rc = check_ws(ws, plan, rows_per_unit, head_dim,
                       (int64_t)batch * num_kv_heads + 1)) != PA_OK)
        return rc;

    pa::VerifyArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = static_cast<const uint16_t *>(q_fp16);
    a.k_pool = kv->k_pool;
    a.v_pool = kv->v_pool;
    a.page_stride = kv->page_stride;
    a.token_stride = kv->token_stride;
    a.head_stride = kv->head_stride;
    a.page_size = kv->page_size;
    a.block_table = block_table;
    a.table_stride = max_blocks_per_req;
    a.sel = nullptr;
    a.topk = 0;
    a.row_lens = row_lens;
    a.len_cap = (int32_t)cap;
    a.list_len = (int32_t)cap;
    a.batch = batch;
    a.q_rows = q_rows;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_heads / num_kv_heads;
    a.rows = rows_per_unit;
    a.chunk_rows = chunk_rows(plan);
    a.num_splits = plan->num_splits;
    a.tokens_per_split = plan->tokens_per_split;
    a.total_rows = (int32_t)total_rows;
    a.logit_scale = (float)((double)sm_scale * (double)k_scale * 1.4426950408889634);
    a.ragged = 1;
    a.split_index = ws->index;
    a.ws_acc = ws->acc;
    a.ws_max = ws->max;
    a.ws_sum = ws->sum;
    return dispatch(a, plan, head_dim, pa::kModeDense, static_cast<hipStream_t>(stream));
}

namespace {

// The batch combine's checks and launch, writing any of the three outputs.
int32_t combine_batch_checked(const pa_workspace *ws, const pa_plan *plan, int32_t batch,
                              int32_t q_rows, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, float out_scale, void *out_fp16,
                              float *out_fp32, float *lse, void *stream)
{
    int32_t rc, rows_per_unit = 0;
    if (!plan || (!out_fp16 && !out_fp32 && !lse))
        return PA_EINVAL;
    if ((rc = check_shape(q_rows, num_heads, num_kv_heads, head_dim, &rows_per_unit,
                          kMaxQRowsBatch, kMaxRowsPerUnitBatch)) != PA_OK)
        return rc;
    if (batch < 1 || !std::isfinite(out_scale))
        return PA_EINVAL;
    if ((int64_t)batch * num_kv_heads > 65535)
        return PA_EUNSUPPORTED;
    if (plan->selection != PA_SEL_BATCH || plan->num_kv_units != batch * num_kv_heads ||
        plan->rows_per_kv_unit != rows_per_unit || plan->head_dim != head_dim ||
        plan->num_splits < 1)
        return PA_EPLAN;
    if ((rc = check_ws(ws, plan, rows_per_unit, head_dim,
                       (int64_t)batch * num_kv_heads + 1)) != PA_OK)
        return rc;
    if (!aligned16(ws->acc) || (reinterpret_cast<uintptr_t>(out_fp16) & 7u) != 0 ||
        !aligned16(out_fp32) || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
        return PA_EALIGN;
    if ((rc = check_device()) != PA_OK)
        return rc;
    const hipError_t err = pa::launch_combine_ragged(
        ws->acc, ws->max, ws->sum, ws->index, plan->num_splits, batch, q_rows, num_heads,
        num_kv_heads, head_dim, out_scale, static_cast<uint16_t *>(out_fp16), out_fp32, lse,
        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PA_OK : PA_EHIP;
}

}  // namespace

int32_t paged_attn_combine_batch_fp32(const pa_workspace *ws, const pa_plan *plan,
                                      int32_t batch, int32_t q_rows, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, float out_scale,
                                      void *out_fp16, void *stream)
{
    if (!out_fp16)
        return PA_EINVAL;
    return combine_batch_checked(ws, plan, batch, q_rows, num_heads, num_kv_heads, head_dim,
                                 out_scale, out_fp16, nullptr, nullptr, stream);
}

int32_t paged_attn_combine_batch_fp32_lse(const pa_workspace *ws, const pa_plan *plan,
                                          int32_t batch, int32_t q_rows, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          float out_scale, void *out_fp16, float *out_fp32,
                                          float *lse, void *stream)
{
    return combine_batch_checked(ws, plan, batch, q_rows, num_heads, num_kv_heads, head_dim,
                                 out_scale, out_fp16, out_fp32, lse, stream);
}

int32_t paged_attn_combine_fp32(const float *ws_acc, const float *ws_max, const float *ws_sum,
                                int32_t num_splits, int32_t num_rows, int32_t head_dim,
                                float out_scale, void *out_fp16, void *stream)
{
    if (!out_fp16)
        return PA_EINVAL;
    return combine_checked(ws_acc, ws_max, ws_sum, num_splits, num_rows, head_dim, out_scale,
                           out_fp16, nullptr, nullptr, stream);
}

int32_t paged_attn_combine_fp32_lse(const float *ws_acc, const float *ws_max,
                                    const float *ws_sum, int32_t num_splits, int32_t num_rows,
                                    int32_t head_dim, float out_scale, void *out_fp16,
                                    float *out_fp32, float *lse, void *stream)
{
    if (!out_fp16 && !out_fp32 && !lse)
        return PA_EINVAL;
    return combine_checked(ws_acc, ws_max, ws_sum, num_splits, num_rows, head_dim, out_scale,
                           out_fp16, out_fp32, lse, stream);
}

int32_t qsa_sparse_verify_e4m3(const void *q_bf16, const pa_kv_pool *kv,
                               const int32_t *block_table, int32_t max_blocks_per_req,
                               const int32_t *sel_blocks, int32_t topk,
                               const int32_t *row_lens, int32_t batch, int32_t q_rows,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               float sm_scale, float k_scale, const pa_plan *plan,
                               const pa_workspace *ws, void *stream)
{
    return sparse_verify(pa::kModeBlocks, q_bf16, kv, block_table, max_blocks_per_req,
                         sel_blocks, topk, row_lens, batch, q_rows, num_heads, num_kv_heads,
                         head_dim, sm_scale, k_scale, plan, ws, stream);
}

int32_t qsa_sparse_verify_tokens_e4m3(const void *q_bf16, const pa_kv_pool *kv,
                                      const int32_t *block_table, int32_t max_blocks_per_req,
                                      const int32_t *sel_tokens, int32_t num_sel,
                                      const int32_t *row_lens, int32_t batch, int32_t q_rows,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float sm_scale, float k_scale, const pa_plan *plan,
                                      const pa_workspace *ws, void *stream)
{
    return sparse_verify(pa::kModeTokens, q_bf16, kv, block_table, max_blocks_per_req,
                         sel_tokens, num_sel, row_lens, batch, q_rows, num_heads, num_kv_heads,
                         head_dim, sm_scale, k_scale, plan, ws, stream);
}

int32_t paged_attn_cache_write_e4m3(const void *k_fp16, const void *v_fp16, int64_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim,
                                    const int64_t *slot_mapping, const pa_kv_pool *kv,
                                    float k_scale, float v_scale, void *stream)
{
    int32_t rc;
    if (!k_fp16 || !v_fp16 || !slot_mapping)
        return PA_EINVAL;
    if ((rc = check_pool(kv)) != PA_OK)
        return rc;
    if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 16 || head_dim % 16 != 0)
        return PA_EINVAL;
    if (num_tokens > ((int64_t)1 << 40) / ((int64_t)num_kv_heads * head_dim))
        return PA_EINVAL;
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.0f) ||
        !(v_scale > 0.0f))
        return PA_EINVAL;
    if (!aligned16(k_fp16) || !aligned16(v_fp16))
        return PA_EALIGN;
    rc = check_device();
    if (rc != PA_OK)
        return rc;
    // the verify entries only read the pool (const in pa_kv_pool); this one writes it
    hipError_t err = pa::launch_cache_write(
        static_cast<const uint16_t *>(k_fp16), static_cast<const uint16_t *>(v_fp16), num_tokens,
        num_kv_heads, head_dim, slot_mapping, const_cast<uint8_t *>(kv->k_pool),
        const_cast<uint8_t *>(kv->v_pool), kv->page_stride, kv->token_stride, kv->head_stride,
        kv->page_size, (int64_t)kv->num_pages * kv->page_size, k_scale, v_scale,
        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PA_OK : PA_EHIP;
}

int32_t paged_attn_stream_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *stream)
{
    if (!buf || !sink || bytes < 0 || bytes % 16 != 0)
        return PA_EINVAL;
    if (!aligned16(buf))
        return PA_EALIGN;
    int32_t rc = check_device();
    if (rc != PA_OK)
        return rc;
    hipError_t err = pa::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PA_OK : PA_EHIP;
}

int32_t paged_attn_timer_arm(int32_t n)
{
    if (n < 0 || n > PA_TIMER_MAX_LAUNCHES)
        return PA_EINVAL;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return PA_EDEVICE;
    std::lock_guard<std::mutex> lock(g_timer.mu);
    if (n > 0 && g_timer.created && dev != g_timer.device)
        return PA_EDEVICE;
    if (n > 0 && !g_timer.created) {
        for (int i = 0; i < 2 * PA_TIMER_MAX_LAUNCHES; ++i) {
            if (hipEventCreate(&g_timer.ev[i]) != hipSuccess) {
                for (int k = 0; k < i; ++k)
                    (void)hipEventDestroy(g_timer.ev[k]);
                return PA_EHIP;
            }
        }
        g_timer.created = true;
        g_timer.device = dev;
    }
    g_timer.armed = n;
    g_timer.used = 0;
    return PA_OK;
}

int32_t paged_attn_timer_read(float *ms, int32_t cap, int32_t *count)
{
    if (!count || cap < 0 || (cap > 0 && !ms))
        return PA_EINVAL;
    std::lock_guard<std::mutex> lock(g_timer.mu);
    const int used = g_timer.used;
    g_timer.armed = g_timer.used = 0;
    *count = used;
    for (int i = 0; i < used && i < cap; ++i) {
        if (hipEventSynchronize(g_timer.ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms[i], g_timer.ev[2 * i], g_timer.ev[2 * i + 1]) != hipSuccess)
            return PA_EHIP;
    }
    return PA_OK;
}

}  // extern "C"
