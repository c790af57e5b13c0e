// verify_mfma.hip - MFMA verify kernel for gfx950 (CDNA4).
//
// What it computes is the function in include/paged_attn_e4m3.h: per query row,
// softmax attention over the E4M3 K/V tokens it sees, as split partials with
// FP32 unnormalised numerators and a separate FP32 max and sum (design note
// "DFlash2 E4M3 attention with FP32 state", first section).  How it computes it
// on an MI355X:
//
//  * One workgroup per (split, KV unit): four waves, one per SIMD.  The split
//    is cut into 32-token blocks dealt to the waves in turn; each wave runs the
//    whole attention (S = Q K^T, online softmax, O += P V over all D columns)
//    on its own blocks, with its own running max and sum.  The main loop has
//    no barrier and no exchange between waves; the four partial states are
//    merged once, through LDS, at the end of the split.
//  * K/V bytes move HBM -> LDS with direct-to-LDS 16-byte loads (no VGPRs),
//    into two stages per plane per wave, one block ahead, on a fixed issue
//    schedule so that the wait counts are the same every step.  Keeping the
//    per-CU queue of loads short matters more than depth: a wave whose load
//    issue finds the queue full stalls, and with two blocks ahead every wave
//    sat in the issue of the first burst while its first block had landed.  The 16-byte
//    chunks of each token row are XOR-swizzled so that the MFMA operand reads
//    are free of LDS bank conflicts.
//  * E4M3 -> FP16 (or BF16 for a BF16 query) with the hardware converter,
//    which is exact for every finite code.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_{f16,bf16}: K is the A operand (one
//    ds_read_b64 per lane per 32 dims), Q^T the B operand, in registers for the
//    whole kernel.  The 16 tokens of each MFMA are ordered so that each lane's
//    8 scores of a 32-token block are exactly the 8 P^T elements it provides to
//    P.V, so P never leaves the registers.
//  * O^T += V^T P^T: V^T fragments come straight from LDS with ds_read_tr8_b64
//    (the transposing read).  P is split into FP16 hi + lo parts and both are
//    multiplied ("compensated probabilities", design note first section);
//    every product is exact in FP32.  A wave's FP32 accumulator is 16 RB rows x
//    D, RB = 1, 2 or 3 the row blocks of the workgroup's chunk of the unit's
//    rows (a kernel instance per chunk size: 16, 32 or 48 rows).
//  * Row blocks (16 rows) in which no row sees any token are skipped: the main
//    loop is instantiated for 1 .. RB row blocks.
//  * The running reference max of a row moves only when a block exceeds it by
//    more than 2^8, so P <= 2^14 in FP16 and accumulator rescales are rare;
//    the partial written out uses the exact row max.
//  * Tokens a row must not see get score -inf by select.  In a block that
//    some live row does not see whole, the V bytes are sanitised in registers
//    before P.V (NaN codes become 0, so p = 0 times a NaN byte cannot reach a
//    row that does not see it), and the (row, column) pairs whose row sees a
//    NaN V byte in that column are recorded and set to NaN before the split's
//    merge: every row gets what the unsplit definition gives it, and NaN bytes
//    in padding pages cannot leak (null-block fix of 1Cat-vLLM PR #702).
#include "pa_verify.h"

#include <math.h>
#include <stdint.h>

#include <type_traits>

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSub = 32;                  // tokens of one wave block
constexpr int kMacro = kSub * kWaves;     // tokens per macro-step (all waves)
constexpr int kRowBlocks = 3;             // 48 rows
constexpr float kLazy = 8.0f;             // reference-max slack (log2 units)
constexpr float kPLog2 = 6.0f;            // P is carried as 2^6 * p (FP16 normal range)
constexpr float kPUnscale = 1.0f / 64.0f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef int int4v __attribute__((ext_vector_type(4)));

// Unsigned division by the page size: q = (n * m) >> s for 0 <= n < 2^31.
struct DivMagic {
    uint32_t m;
    uint32_t s;
};

__device__ __forceinline__ int divp(int n, DivMagic dm)
{
    return (int)(((uint64_t)(uint32_t)n * dm.m) >> dm.s);
}

// XOR swizzle of the 16-byte chunks of token row r (0..31 within a wave block).
// D = 256: a row spans all 64 banks, so rows read together need distinct chunk
// offsets.  D = 128: two rows share the bank range; (row parity, offset) must
// differ.  Both hold for the K reads (16 rows 8(m/4) + 4b + m%4) and the
// transposing V reads (rows 8g + j).
template <int D>
__device__ __forceinline__ int swz(int r)
{
    if (D == 256)
        return (r + 4 * (r >> 4)) & 15;
    return ((r >> 1) + 2 * (r >> 4)) & 7;
}

// Wait until at most N vector-memory loads of this wave are in flight.  Inline
// asm on purpose: the compiler does not see the direct-to-LDS loads (also asm),
// so it would consider a builtin s_waitcnt redundant and may delete it.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier for LDS data that this wave wrote with ordinary LDS
// stores or read with LDS loads: they complete first (lgkmcnt 0).  Unlike
// __syncthreads() it does not wait for direct-to-LDS loads still in flight.
__device__ __forceinline__ void barrier_lds()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
}

// One 16-byte-per-lane direct-to-LDS load: lane l's 16 bytes from gaddr land at
// LDS byte lds_base + 16 l.  Issued as inline asm so that the compiler does not
// track it: its own tracking of these loads is conservative (it drains every
// load in flight before LDS reads it cannot disambiguate).  Completion is
// waited for explicitly with wait_vmcnt, on a fixed per-step issue schedule.
//
// The compiler's hazard recognizer does not see into inline asm, so the asm
// carries the wait states gfx9 requires before these loads itself: one after
// an SALU write of M0 (the LDS destination) and five after a VALU write of an
// SGPR that the load reads (the readfirstlane that forms an SGPR base).
__device__ __forceinline__ void dma16(const void *gaddr, uint32_t lds_base)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 : : "v"(gaddr), "{m0}"(lds_base) : "memory");
}

// The same load addressed as a wave-uniform SGPR base plus a per-lane 32-bit
// offset, which needs no per-lane address arithmetic.  The base goes through
// readfirstlane so that it is held in SGPRs; FIRST marks the first load after
// the base was formed, which must wait out the VALU-to-SGPR hazard.
template <bool FIRST>
__device__ __forceinline__ void dma16_s(const void *base, uint32_t voff, uint32_t lds_base)
{
    const uint64_t u = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    const void *sbase = (const void *)(((uint64_t)hi << 32) | lo);
    if (FIRST)
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                     : : "v"(voff), "s"(sbase), "{m0}"(lds_base) : "memory");
    else
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     : : "v"(voff), "s"(sbase), "{m0}"(lds_base) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Stores of the split partials at device scope (the SC1 cache-policy bit).
// Each XCD of the chip has its own L2, so such a store is written through to
// memory when it is issued.  An ordinary store stays dirty in the L2 until
// the write-back that ends the kernel, and every workgroup writes its
// partials in its last microseconds, so that write-back would delay the end
// of the kernel.  The stores go through a raw buffer resource: a uniform
// base, a 32-bit byte offset below 2^31 per lane, and the 32-bit data format.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStoreDeviceScope = 16;      // cache-policy operand: SC1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(float *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ void store_ws(__amdgpu_buffer_rsrc_t rs, uint32_t off, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0,
                                           kStoreDeviceScope);
}

__device__ __forceinline__ void store_ws(__amdgpu_buffer_rsrc_t rs, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, off, 0,
                                          kStoreDeviceScope);
}

template <bool BF16>
struct Frag;
template <>
struct Frag<false> {
    typedef half8 T;
};
template <>
struct Frag<true> {
    typedef bf16x8 T;
};

// 8 E4M3 bytes -> 8 FP16 values, in byte order.
__device__ __forceinline__ half8 dec_f16(int2v raw)
{
    half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw.x, 1.0f, false);
    half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw.x, 1.0f, true);
    half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw.y, 1.0f, false);
    half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw.y, 1.0f, true);
    half8 r = {a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
    return r;
}

__device__ __forceinline__ bf16x8 dec_bf16(int2v raw)
{
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, true);
    bf16x8 r = {a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
    return r;
}

__device__ __forceinline__ f32x4 mfma_qk(half8 a, half8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_qk(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Lanes n, n+16, n+32, n+48 hold the same row.  The permlane swaps give every
// lane {v[l], v[l^32]} and then {v[l], v[l^16]}, each pair in the same order on
// all four lanes of a row, so the results are bitwise equal across the row.
// Both halves of a swap are copied to scalars before any bit_cast: clang's
// __builtin_bit_cast of a vector element reads element 0 whatever the index.
__device__ __forceinline__ void swap32(float v, float &x0, float &x1)
{
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    x0 = __builtin_bit_cast(float, r0);
    x1 = __builtin_bit_cast(float, r1);
}

__device__ __forceinline__ void swap16(float v, float &x0, float &x1)
{
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    x0 = __builtin_bit_cast(float, r0);
    x1 = __builtin_bit_cast(float, r1);
}

// Maxima of scores as plain v_max_f32 / v_max3_f32.  fmaxf makes the compiler
// quiet each operand it cannot prove quiet (MFMA results, lane swaps) with a
// v_max(x, x) first, which doubles the softmax's maxima.  The instructions
// drop a quiet NaN operand as maxnum does; the scores never hold a signalling
// NaN (they come out of the MFMA), so the result is the same.
__device__ __forceinline__ float max2(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ float max3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// p - h[i] for the FP16 pair h, in one v_fma_mix_f32 (p * 1 - h[i], one
// rounding): the FP16 operand is read in place, where a conversion to FP32
// and a subtraction would take two instructions.
__device__ __forceinline__ float sub_half(float p, half2v h, int i)
{
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    float r;
    if (i == 0)
        asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(r) : "v"(p), "v"(hb));
    else
        asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "=v"(r) : "v"(p), "v"(hb));
    return r;
}

__device__ __forceinline__ float max_over_groups(float v)
{
    float a, b;
    swap32(v, a, b);
    swap16(max2(a, b), a, b);
    return max2(a, b);
}

__device__ __forceinline__ float sum_over_groups(float v)
{
    float a, b;
    swap32(v, a, b);
    swap16(a + b, a, b);
    return a + b;
}

__device__ __forceinline__ uint32_t or_over_groups(uint32_t v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    const auto t = __builtin_amdgcn_permlane16_swap(r0 | r1, r0 | r1, false, false);
    const uint32_t t0 = t[0], t1 = t[1];
    return t0 | t1;
}

// Bit 7 of each byte of the result is set where that byte of x is an E4M3 NaN
// code (S.1111.111): (x & 0x7F) + 1 carries into bit 7 of a byte exactly when
// its low seven bits are all ones, and never into the next byte.
__device__ __forceinline__ uint32_t nan_byte_marks(uint32_t x)
{
    return ((x & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
}

// The NaN codes of the four bytes of x become 0x00; returns a 4-bit mask of
// the bytes that were NaN.
__device__ __forceinline__ uint32_t drop_nan_bytes(int &x)
{
    const uint32_t u = (uint32_t)x;
    const uint32_t hit = nan_byte_marks(u);
    x = (int)(u & ~((hit >> 7) * 0xFFu));
    return ((hit >> 7) & 1u) | ((hit >> 14) & 2u) | ((hit >> 21) & 4u) | ((hit >> 28) & 8u);
}

// x *= f, one accumulator fragment at a time: the volatile asm keeps the
// compiler from reading a whole accumulator array out of AGPRs at once.
__device__ __forceinline__ void scale_in_place(f32x4 &x, float f)
{
    f32x4 t = x;
    asm volatile("" : "+v"(t));
    t *= f;
    asm volatile("" : "+v"(t));
    x = t;
}

// Reductions over each row of 16 lanes by DPP rotations within the row
// (row_ror 8, 4, 2, 1): every lane ends with its row's result, with no LDS
// round trip (a shuffle through ds_bpermute costs one per step).
template <int ROR>
__device__ __forceinline__ int row_ror(int v)
{
    return __builtin_amdgcn_update_dpp(v, v, 0x120 + ROR, 0xF, 0xF, false);
}

__device__ __forceinline__ int row16_max(int v)
{
    v = max(v, row_ror<8>(v));
    v = max(v, row_ror<4>(v));
    v = max(v, row_ror<2>(v));
    return max(v, row_ror<1>(v));
}

__device__ __forceinline__ int row16_min(int v)
{
    v = min(v, row_ror<8>(v));
    v = min(v, row_ror<4>(v));
    v = min(v, row_ror<2>(v));
    return min(v, row_ror<1>(v));
}

// Max over lanes 0..15 (the row lengths of one request), broadcast to the wave.
__device__ __forceinline__ int max16_broadcast(int v)
{
    return __builtin_amdgcn_readfirstlane(row16_max(v));
}

// Max over the whole wave: each row of 16, then across the four rows.
__device__ __forceinline__ int wave_max(int v)
{
    v = row16_max(v);
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    const int r0 = r[0], r1 = r[1];
    const auto t = __builtin_amdgcn_permlane16_swap(max(r0, r1), max(r0, r1), false, false);
    const int t0 = t[0], t1 = t[1];
    return max(t0, t1);
}

template <int D>
struct Cfg {
    static constexpr int KB = D / 32;                 // QK k-blocks
    static constexpr int DB = D / 16;                 // PV d-blocks (all of D per wave)
    static constexpr int DQ = DB / kWaves;            // d-blocks of one output quarter
    static constexpr int BLOCK = kSub * D;            // bytes of one wave's 32 rows
    static constexpr int DMA = BLOCK / 1024;          // 1 KB direct loads per stage
    static constexpr int ROWS_PER_DMA = 1024 / D;
    static constexpr int LANES_PER_ROW = D / 16;
    static constexpr int STAGES = 2 * 2 * kWaves * BLOCK;           // K and V, two stages
    // end-of-split merge: each wave leaves its three foreign output quarters
    static constexpr int QUARTER = kRowBlocks * DQ * 64 * 16;       // bytes per (wave, quarter)
    static constexpr int MERGE = kWaves * (kWaves - 1) * QUARTER;
    static constexpr int SHARED = STAGES > MERGE ? STAGES : MERGE;
    // Each wave leaves its quarters in a private area: its own four stage
    // slots (K and V of both stages: no other wave's loads target them) and a
    // 1/kWaves share of the space past the stages, in 1 KB chunks.
    static constexpr int SLOT_CHUNKS = BLOCK / 1024;
    static constexpr int EXTRA = (SHARED - STAGES) / kWaves;
    static_assert((kWaves - 1) * QUARTER == 4 * BLOCK + EXTRA && EXTRA % 1024 == 0,
                  "a wave's three quarters fill its stage slots and its extra share");
};

template <int D>
constexpr int max_slots()
{
    return mfma_max_slots(D);
}

template <int D, int MODE, int RB>
__global__ __launch_bounds__(kThreads, 1) void verify_mfma_kernel(VerifyArgs a, DivMagic dm,
                                                                   DivMagic hm, uint32_t g_magic)
{
    // SPARSE: bf16 queries and a selection list (blocks or token ids); TOK:
    // the list holds token ids, one slot per position, and dm divides by the
    // page size to place a token (in the other modes positions are divided)
    constexpr bool SPARSE = MODE != kModeDense;
    constexpr bool TOK = MODE == kModeTokens;
    typedef Cfg<D> C;
    typedef typename Frag<SPARSE>::T QFrag;
    constexpr int kSlots = max_slots<D>();
    constexpr int kEnt = (kSlots + kThreads - 1) / kThreads;

    // K/V stages during the split, the merge area after it.  Stage layout:
    // [K0 | K1 | V0 | V1], each [wave][32 rows][D] with swizzled chunks.
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::SHARED];
    __shared__ int2v slots[kSlots];                 // (physical page, first token) per slot
    __shared__ __attribute__((aligned(16))) int32_t tok_s[kWaves][2][kSub];   // sparse tokens
    __shared__ int32_t blk_tmax[kWaves][2];         // sparse: last token of an all-valid block
    __shared__ float xm[kWaves][16 * RB];   // merge: per-wave row max
    __shared__ float xl[kWaves][16 * RB];   // merge: per-wave row sum
    __shared__ float xr[kWaves][16 * RB];   // merge: per-wave accumulator reference

    // The argument block spans four 64-byte scalar-cache lines; one word of
    // each, read at entry, brings them all in with one miss, where reading the
    // fields as they are needed takes a miss per line, in sequence.
    {
        const uint32_t *kp = (const uint32_t *)__builtin_amdgcn_kernarg_segment_ptr();
        const uint32_t t0 = kp[0], t1 = kp[16], t2 = kp[32], t3 = kp[48];
        asm volatile("" : : "s"(t0), "s"(t1), "s"(t2), "s"(t3));
    }
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    // the split of a KV unit this workgroup reads and its span; a ragged batch
    // derives them from every row length of the batch (the same in every
    // wave), and a workgroup no split falls on has nothing to do
    int split = blockIdx.x, unit = blockIdx.y, tps = a.tokens_per_split;
    if (a.ragged) {
        const RaggedPos rp =
            ragged_locate(a, blockIdx.x, lane, blockIdx.x == 0 && blockIdx.z == 0 && w == 0);
        if (rp.unit < 0)
            return;
        split = __builtin_amdgcn_readfirstlane(rp.local);
        unit = __builtin_amdgcn_readfirstlane(rp.unit);
        tps = __builtin_amdgcn_readfirstlane(rp.span);
    }
    const int b = divp(unit, hm);              // unit / num_kv_heads
    const int kvh = unit - b * a.num_kv_heads;
    // the rows of a KV unit are taken in chunks of 16 RB rows (one workgroup
    // each, grid z): this one takes rows row0 .. row0 + R - 1 of the unit
    const int row0 = blockIdx.z * (16 * RB);
    const int R = min(a.rows - row0, 16 * RB), G = a.group;
    // row / G for a row of the KV unit (row < rows <= 96, G <= rows, so
    // row * G < 2^16): (row * g_magic) >> 16 with g_magic = ceil(2^16 / G)
    // (from the host) is exact, one 24-bit multiply and a shift where a
    // division takes about twenty instructions, several of them at quarter
    // rate.  The divisions by the page size and by the KV head count are
    // multiply-shifts from the host too (dm, hm).
    auto div_g = [&](int row) __attribute__((always_inline)) {
        return (int)(__umul24((uint32_t)row, g_magic) >> 16);
    };
    const int ps = a.page_size;

    uint8_t *const k_st = smem;                               // [2][kWaves][BLOCK]
    uint8_t *const v_st = smem + 2 * kWaves * C::BLOCK;       // [2][kWaves][BLOCK]

    // With pages of at least 32 tokens a 32-row block spans at most two page
    // slots and is loaded from one page lookup (two_slot).
    const bool two_slot = !TOK && ps >= kSub && a.token_stride < (1 << 25);

    // ---- one round trip: Q (to LDS), row lengths, page table ----------------
    // Q is fetched once per workgroup with direct-to-LDS loads into the K0
    // stage (free until the first K/V loads), rows of 2D bytes with their
    // 16-byte chunks XOR-swizzled by row, and read into registers from there.
    // Q row r of this KV unit is query row r / G, head kvh*G + r % G: it lies
    // r + (r / G)(H - G) rows past the unit's first Q row.
    uint8_t *const q_st = k_st;
    constexpr int kQRowsPerDma = 1024 / (2 * D);
    constexpr int kQLanesPerRow = 2 * D / 16;
    {
        const int nq = (R * 2 * D + 1023) / 1024;          // 1 KB loads for R rows
        const int r_in = lane / kQLanesPerRow, c = lane % kQLanesPerRow;
        const uint8_t *qb =
            (const uint8_t *)(a.q + ((int64_t)b * a.q_rows * a.num_heads + (int64_t)kvh * G) * D);
        for (int i = w; i < nq; i += kWaves) {
            const int r = i * kQRowsPerDma + r_in;
            if (r < R) {
                const int row = row0 + r;
                const int qrow = row + div_g(row) * (a.num_heads - G);
                dma16(qb + (int64_t)qrow * (2 * D) + 16 * (c ^ (r & 15)),
                      __builtin_amdgcn_readfirstlane(lds_addr(q_st + i * 1024)));
            }
        }
    }
    // lane i < q_rows: length of query row i, clamped where it is first
    // needed (after the table reads are issued; the empty asm statement keeps
    // the clamp there instead of right after the load, where the compiler
    // would wait for it)
    int lraw = 0;
    if (lane < a.q_rows)
        lraw = a.row_lens[(int64_t)b * a.q_rows + lane];
    auto clamp_len = [&](int l) __attribute__((always_inline)) {
        return l < 0 ? 0 : (l > a.len_cap ? a.len_cap : l);
    };
    const int lo = split * tps;
    const int hi_list = min(lo + tps, a.list_len);
    const int32_t *table = a.block_table + (int64_t)b * a.table_stride;
    int slot0 = 0, nslots = 0;
    if (hi_list > lo) {
        slot0 = TOK ? lo : divp(lo, dm);
        nslots = min(TOK ? hi_list - lo : divp(hi_list - 1, dm) + 1 - slot0, kSlots);
    }
    // table entries of this split's slots (dense), its selected blocks or its
    // selected token ids (sparse)
    int ent[kEnt];
#pragma unroll
    for (int k = 0; k < kEnt; ++k) {
        const int i = tid + k * kThreads;
        ent[k] = -1;
        if (i < nslots)
            ent[k] = SPARSE ? a.sel[((int64_t)b * a.num_kv_heads + kvh) * a.topk + slot0 + i]
                            : table[slot0 + i];
    }
    // the longest row length and the split's end, known once the lengths
    // are in (the addressing helpers below read them only after that)
    int lmax = 0, hi = hi_list;
    const int64_t head_off = (int64_t)kvh * a.head_stride;

    // Position -> (byte offset of the K/V head row, token, valid).  Branch-free;
    // the slot cache is the only table read.
    auto resolve = [&](int pos, int64_t &off, int &t) __attribute__((always_inline)) -> bool {
        if (TOK) {
            const int2v e = slots[min(max(pos - slot0, 0), kSlots - 1)];
            t = e.y;
            const bool ok = pos < hi && e.x >= 0;
            const int u = t - divp(t, dm) * ps;
            off = ok ? (int64_t)e.x * a.page_stride + (int64_t)u * a.token_stride + head_off : 0;
            return ok;
        }
        const int slot = divp(pos, dm);
        const int u = pos - slot * ps;
        const int si = min(max(slot - slot0, 0), kSlots - 1);
        const int2v e = slots[si];
        t = SPARSE ? e.y + u : pos;
        bool ok = pos < hi && e.x >= 0;
        if (SPARSE)
            ok = ok && t < lmax;
        off = ok ? (int64_t)e.x * a.page_stride + (int64_t)u * a.token_stride + head_off : 0;
        return ok;
    };

    // Direct-to-LDS loads of this wave's block j into one stage.  Lane l loads,
    // in load i, row r_i = i*ROWS_PER_DMA + l/LANES_PER_ROW, swizzled chunk
    // position l%LANES_PER_ROW.  With pages of at least 32 tokens a block spans
    // at most two page slots, so the page lookup is done once per block
    // (wave-uniform) and a lane only adds its precomputed row offset; small
    // pages, very large token strides and token-id lists take the per-row
    // resolve.  Positions past the end load an in-bounds dummy address, so that
    // every step issues the same number of loads.  tokst (sparse, V loads only)
    // receives the token of each row, INT32_MAX for rows no query sees, and
    // blk_tmax the largest of them when it is known (INT32_MAX otherwise).
    const int cp = lane % C::LANES_PER_ROW;
    int32_t loff[C::DMA];
#pragma unroll
    for (int i = 0; i < C::DMA; ++i) {
        const int r = i * C::ROWS_PER_DMA + lane / C::LANES_PER_ROW;
        loff[i] = two_slot ? r * (int32_t)a.token_stride + 16 * (cp ^ swz<D>(r)) : 0;
    }
    // Page lookup of block j of this wave (wave-uniform), done once for its K
    // and V loads.  With pages of at least 32 tokens the block spans at most
    // two page slots: rows [0, end_a) come from the first at base_a + row
    // offset, rows [na, end_b) from the second at base_b + row offset.
    struct BlockRef {
        int na, ua, end_a, end_b, tb_a, tb_b, phys_a, phys_b;
        int64_t base_a, base_b;
    };
    // The page reference of a 32-row block at position pos0 whose rows
    // [0, na) lie in page phys_a (first token tb_a) and the rest in phys_b
    // (first token tb_b), rows at or past end loading the dummy address.
    auto make_ref = [&](int pos0, int end, int phys_a, int tb_a, int phys_b,
                        int tb_b) __attribute__((always_inline)) -> BlockRef {
        BlockRef br;
        const int sa = divp(pos0, dm);
        br.ua = pos0 - sa * ps;
        br.na = min(kSub, ps - br.ua);
        br.phys_a = phys_a;
        br.phys_b = phys_b;
        br.tb_a = tb_a;
        br.tb_b = tb_b;
        const int hip = end - pos0;
        br.end_a = min(br.na, hip);
        br.end_b = hip;
        br.base_a = (int64_t)phys_a * a.page_stride + (int64_t)br.ua * a.token_stride + head_off;
        br.base_b = (int64_t)phys_b * a.page_stride - (int64_t)br.na * a.token_stride + head_off;
        return br;
    };
    auto lookup = [&](int j) __attribute__((always_inline)) -> BlockRef {
        BlockRef br = {};
        if (two_slot) {
            const int pos0 = lo + (j * kWaves + w) * kSub;
            const int sa = divp(pos0, dm);
            const int2v ea = slots[min(max(sa - slot0, 0), kSlots - 1)];
            const int2v eb = slots[min(max(sa + 1 - slot0, 0), kSlots - 1)];
            br = make_ref(pos0, hi, __builtin_amdgcn_readfirstlane(ea.x),
                          __builtin_amdgcn_readfirstlane(ea.y),
                          __builtin_amdgcn_readfirstlane(eb.x),
                          __builtin_amdgcn_readfirstlane(eb.y));
            if (SPARSE) {
                br.end_a = br.phys_a >= 0 ? min(br.end_a, lmax - (br.tb_a + br.ua)) : 0;
                br.end_b = br.phys_b >= 0 ? min(br.end_b, br.na + lmax - br.tb_b) : 0;
            }
        }
        return br;
    };
    auto issue_plane = [&](const BlockRef &br, int j, const uint8_t *pool, uint8_t *stage,
                           int32_t *tokst) __attribute__((always_inline)) {
        int32_t *tmaxp = &blk_tmax[w][j & 1];
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(stage + w * C::BLOCK));
        // the stage being refilled was read by this wave's previous use of it
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        if (two_slot) {
            if (br.na == kSub && br.end_a == kSub) {
                // the whole block is valid and inside one page: SGPR base + lane offset
                const uint8_t *sb = pool + br.base_a;
#pragma unroll
                for (int i = 0; i < C::DMA; ++i) {
                    if (i == 0)
                        dma16_s<true>(sb, (uint32_t)loff[i], dst);
                    else
                        dma16_s<false>(sb, (uint32_t)loff[i], dst + i * 1024);
                }
                if (SPARSE && tokst != nullptr && cp == 0) {
#pragma unroll
                    for (int i = 0; i < C::DMA; ++i) {
                        const int r = i * C::ROWS_PER_DMA + lane / C::LANES_PER_ROW;
                        tokst[r] = br.tb_a + br.ua + r;
                    }
                }
                if (SPARSE && tokst != nullptr && lane == 0)
                    *tmaxp = br.tb_a + br.ua + kSub - 1;
            } else {
#pragma unroll
                for (int i = 0; i < C::DMA; ++i) {
                    const int r = i * C::ROWS_PER_DMA + lane / C::LANES_PER_ROW;
                    const bool in_b = r >= br.na;
                    const bool ok = in_b ? (r < br.end_b) : (r < br.end_a);
                    const int64_t src = ok ? (in_b ? br.base_b : br.base_a) + loff[i] : 0;
                    dma16(pool + src, dst + i * 1024);
                    if (SPARSE && tokst != nullptr && cp == 0)
                        tokst[r] = ok ? (in_b ? br.tb_b - br.na + r : br.tb_a + br.ua + r) : INT32_MAX;
                }
                if (SPARSE && tokst != nullptr && lane == 0)
                    *tmaxp = INT32_MAX;
            }
        } else {
            const int pos0 = lo + (j * kWaves + w) * kSub;
            int tm = 0;
#pragma unroll
            for (int i = 0; i < C::DMA; ++i) {
                const int row = i * C::ROWS_PER_DMA + lane / C::LANES_PER_ROW;
                int64_t off;
                int t;
                const bool ok = resolve(pos0 + row, off, t);
                const int64_t src = ok ? off + 16 * (cp ^ swz<D>(row)) : 0;
                dma16(pool + src, dst + i * 1024);
                if (SPARSE && tokst != nullptr && cp == 0)
                    tokst[row] = ok ? t : INT32_MAX;
                tm = max(tm, ok ? t : INT32_MAX);
            }
            if (TOK && tokst != nullptr)
                tm = wave_max(tm);   // token ids are unordered: the block's largest
            if (SPARSE && tokst != nullptr && lane == 0)
                *tmaxp = TOK ? tm : INT32_MAX;
        }
    };

    asm volatile("" : "+v"(lraw));
    const int lmine = clamp_len(lraw);
    lmax = max16_broadcast(lmine);
    int lrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = rb * 16 + n;
        const int lr = __shfl(lmine, r < R ? div_g(row0 + r) : 0, 64);
        lrow[rb] = r < R ? lr : 0;
    }
    // row blocks up to the last one with a row that sees a token
    int nrb = 1;
#pragma unroll
    for (int rb = 1; rb < RB; ++rb)
        if (__any(lrow[rb] > 0))
            nrb = rb + 1;
    if (!SPARSE)
        hi = min(hi, lmax);
    // Per row block, the smallest length among the rows that can see tokens of
    // this split (dense: length past the split start; sparse: nonzero).  A
    // block whose tokens all lie below it is seen whole by every such row, and
    // is processed without masks; rows that see nothing of the split are reset
    // to the empty state at the end.
    // Dense blocks are never unmasked past hi, where the K bytes may be NaN.
    int minl[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int v = SPARSE ? INT32_MAX : hi;
        if (rb * 16 + n < R && lrow[rb] > (SPARSE ? 0 : lo))
            v = SPARSE ? lrow[rb] : min(lrow[rb], hi);
        minl[rb] = __builtin_amdgcn_readfirstlane(row16_min(v));   // rows of lanes share n
    }
#pragma unroll
    for (int k = 0; k < kEnt; ++k) {
        const int i = tid + k * kThreads;
        if (i < nslots) {
            int phys = -1, tb = 0;
            if (!SPARSE) {
                phys = ent[k];
                tb = (slot0 + i) * ps;
            } else if (TOK) {
                // a token no row sees keeps phys -1; lmax <= the table's
                // capacity, so a token below it has a table entry
                const int t = ent[k];
                if (t >= 0 && t < lmax) {
                    phys = table[divp(t, dm)];
                    tb = t;
                }
            } else {
                const int blk = ent[k];
                if (blk >= 0 && (int64_t)blk * ps < lmax) {
                    phys = table[blk];
                    tb = blk * ps;
                }
            }
            slots[i] = int2v{phys, tb};
        }
    }
    wait_vmcnt<0>();   // this wave's Q loads
    __syncthreads();

    // Q^T is the B operand of S^T = K Q^T: lane (n, g) holds row 16rb + n.
    // The head dimension is walked in a permuted order that both operands
    // share: MFMA k-block kb = 2t + e, lane group g covers dims
    // 64t + 16g + 8e .. +7 (16-byte chunk 8t + 2g + e of the row), so that one
    // 16-byte LDS chunk of K (dims 64t + 16g .. +15) feeds two consecutive
    // k-blocks.
    QFrag qf[RB][C::KB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = rb * 16 + n;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
            int4v v = int4v{0, 0, 0, 0};
            if (r < R && rb < nrb) {          // row blocks past nrb are never used
                const int c = 8 * (kb >> 1) + 2 * g + (kb & 1);
                v = *(const int4v *)(q_st + r * 2 * D + 16 * (c ^ (r & 15)));
            }
            qf[rb][kb] = __builtin_bit_cast(QFrag, v);
        }
    }
    barrier_lds();     // everyone has its Q before its stage is refilled

    // this wave's blocks: positions lo + 32 (4j + w), j = 0 .. nms-1
    const int nms = hi > lo ? (hi - lo + kMacro - 1) / kMacro : 0;

    // ---- per-wave state ------------------------------------------------------
    f32x4 acc[RB][C::DB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int d = 0; d < C::DB; ++d)
            acc[rb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_true[RB], m_ref[RB], l_part[RB];
    // per row block, (d-block, k) pairs of this lane whose row saw a NaN V byte
    uint64_t nan_hit[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_true[rb] = -INFINITY;
        m_ref[rb] = -INFINITY;
        l_part[rb] = 0.0f;
        nan_hit[rb] = 0;
    }
    const float c = a.logit_scale;

    // Per-lane parts of the LDS read addresses.  Stage bases are multiples of
    // the block size, so a 16-byte chunk index can be XORed into an address.
    //  K (A operand of QK): lane (n, g) reads rows 8(n/4) + 4bb + n%4 (MFMA row
    //    n of token block bb), chunk 4t + g, i.e. dims 64t + 16g .. +15.
    //  V^T (A operand of P.V): the transposing read's supplier lane (n, g)
    //    points at row 8g + n/2, byte 8(n%2) of d-block db's chunk.
    uint32_t koff[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const int krow = 8 * (n >> 2) + 4 * bb + (n & 3);
        koff[bb] = krow * D + ((g ^ swz<D>(krow)) << 4);
    }
    const int vrow = 8 * g + (n >> 1);
    const uint32_t voff = vrow * D + (swz<D>(vrow) << 4) + ((n & 1) << 3);

    // One block of this wave (step j) with NRB live row blocks.  Block j uses K
    // stage j%2 and V stage j%2.  Issue order: K0 V0 (prologue), then in step
    // j: K(j+1) after QK(j) (its stage held K(j-1)), V(j+1) after P.V(j) (its
    // stage held V(j-1)); blocks past the last step are not loaded.  Before
    // QK(j) the only group issued after K(j) is V(j); before P.V(j) it is
    // K(j+1), if block j+1 exists.  Loads complete in issue order, so
    // allowing exactly that many groups in flight means the awaited group has
    // landed.
    auto wait_groups = [&](int groups) __attribute__((always_inline)) {
        if (groups >= 3)
            wait_vmcnt<3 * C::DMA>();
        else if (groups == 2)
            wait_vmcnt<2 * C::DMA>();
        else if (groups == 1)
            wait_vmcnt<C::DMA>();
        else
            wait_vmcnt<0>();
    };
    // The page reference of block j of this wave from that of its block j - 1
    // (dense lists): with both blocks whole inside one page, block j is the
    // same page 128 positions on, and its base moves by 128 token strides
    // (a few scalar operations instead of the slot-cache reads, their wait and
    // the 64-bit address arithmetic of a lookup).  Otherwise the full lookup.
    auto next_ref = [&](const BlockRef &prev, int j) __attribute__((always_inline)) -> BlockRef {
        if (!SPARSE && two_slot) {
            const int pos0 = lo + (j * kWaves + w) * kSub;
            if (prev.na == kSub && prev.end_a == kSub && prev.ua + kMacro + kSub <= ps &&
                pos0 + kSub <= hi) {
                BlockRef br = prev;       // same page: phys, first tokens and na stay
                br.ua = prev.ua + kMacro;
                br.base_a = prev.base_a + (int64_t)kMacro * a.token_stride;
                br.end_a = kSub;
                br.end_b = hi - pos0;
                return br;
            }
        }
        return lookup(j);
    };
    BlockRef bcur = {};   // the reference of this wave's current block
    auto step = [&](auto nrb_c, int j) __attribute__((always_inline)) {
        constexpr int NRB = decltype(nrb_c)::value;
        const int st = j & 1;
        uint8_t *kst = k_st + st * (kWaves * C::BLOCK);
        uint8_t *vst = v_st + st * (kWaves * C::BLOCK);
        int32_t *tok = &tok_s[w][st][0];
        const int pos0 = lo + (j * kWaves + w) * kSub;
        const bool any = pos0 < hi;                  // wave-uniform
        // block 0's V is issued once its K is in: the first burst of the grid
        // carries K alone, so that the first QK can start sooner
        if (j == 0) {
            wait_groups(0);                          // K(0)
            issue_plane(bcur, 0, a.v_pool, v_st, &tok_s[w][0][0]);
        } else {
            wait_groups(1);                          // K(j); V(j) may be in flight
        }

        // ---- S^T = K Q^T on this wave's 32 tokens --------------------------
        // (the first k-block's MFMAs take a zero accumulator operand, so the
        // scores need no initialisation; they are only read when any)
        f32x4 s[NRB][2];
        if (any) {
            const uint32_t kbase = lds_addr(kst + w * C::BLOCK);
            // all K reads of the block first, so that their latencies overlap
            int4v kraw[C::KB / 2][2];
#pragma unroll
            for (int t = 0; t < C::KB / 2; ++t)
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
                    kraw[t][bb] = *(const __attribute__((address_space(3))) int4v *)(uintptr_t)(
                        (kbase + koff[bb]) ^ (uint32_t)(t << 6));
            __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of their uses
#pragma unroll
            for (int t = 0; t < C::KB / 2; ++t) {
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) {
                    const int4v raw = kraw[t][bb];
                    QFrag k0, k1;
                    if (SPARSE) {
                        k0 = __builtin_bit_cast(QFrag, dec_bf16(int2v{raw.x, raw.y}));
                        k1 = __builtin_bit_cast(QFrag, dec_bf16(int2v{raw.z, raw.w}));
                    } else {
                        k0 = __builtin_bit_cast(QFrag, dec_f16(int2v{raw.x, raw.y}));
                        k1 = __builtin_bit_cast(QFrag, dec_f16(int2v{raw.z, raw.w}));
                    }
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb)
                        s[rb][bb] = mfma_qk(k0, qf[rb][2 * t],
                                            t == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[rb][bb]);
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb)
                        s[rb][bb] = mfma_qk(k1, qf[rb][2 * t + 1], s[rb][bb]);
                }
            }
        }
        BlockRef bnext = {};
        if (j + 1 < nms) {
            bnext = next_ref(bcur, j + 1);
            issue_plane(bnext, j + 1, a.k_pool, k_st + (st ^ 1) * (kWaves * C::BLOCK), nullptr);
        }

        // ---- visibility, online softmax, P = hi + lo -------------------------
        half8 ph[NRB], pl[NRB];
        // every live row block sees every token of this block (wave-uniform)
        bool all_full = true;
        if (any) {
            // row blocks that see every token of this block (wave-uniform)
            const int tmax = SPARSE ? blk_tmax[w][st] : 0;
            bool full[NRB];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                full[rb] = SPARSE ? (tmax < minl[rb]) : (pos0 + kSub <= minl[rb]);
                all_full = all_full && full[rb];
            }
            // this lane's 8 scores are tokens at positions pos0 + 8g + jj
            const int tfirst = pos0 + 8 * g;
            int tk[8];
            if (SPARSE && !all_full) {
                const int4v t0 = *(const int4v *)&tok[8 * g];
                const int4v t1 = *(const int4v *)&tok[8 * g + 4];
                tk[0] = t0.x; tk[1] = t0.y; tk[2] = t0.z; tk[3] = t0.w;
                tk[4] = t1.x; tk[5] = t1.y; tk[6] = t1.z; tk[7] = t1.w;
            }
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                // this lane's 8 raw scores; in a block not seen whole, the ones
                // its row must not see become -inf (c > 0 keeps them -inf)
                float sv[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    sv[jj] = s[rb][jj >> 2][jj & 3];
                if (!full[rb]) {
                    uint32_t vis;
                    if (!SPARSE) {
                        const int nv = min(max(min(lrow[rb], hi) - tfirst, 0), 8);
                        vis = (1u << nv) - 1u;
                    } else {
                        vis = 0;
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj)
                            vis |= (tk[jj] < lrow[rb]) ? (1u << jj) : 0u;   // invalid = INT32_MAX
                    }
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        sv[jj] = ((vis >> jj) & 1u) ? sv[jj] : -INFINITY;
                }
                // c > 0, so the largest logit comes from the largest raw score
                const float mloc = max2(max3(sv[0], sv[1], sv[2]),
                                        max3(sv[3], sv[4], max3(sv[5], sv[6], sv[7])));
                const float mt = max2(m_true[rb], max_over_groups(mloc) * c);
                m_true[rb] = mt;
                if (__any(mt > m_ref[rb] + kLazy)) {
                    // rare: move the reference and rescale what was accumulated.
                    // A row that has seen nothing keeps -inf (and zero state).
                    // While no row of the row block has a reference yet (its first
                    // block: every accumulator and sum is still exactly zero) the
                    // rescale is skipped; it would multiply 16 x D zeros.
                    if (__any(m_ref[rb] != -INFINITY)) {
                        const float alpha = (mt == -INFINITY) ? 1.0f : exp2f(m_ref[rb] - mt);
                        l_part[rb] *= alpha;
#pragma unroll
                        for (int d = 0; d < C::DB; ++d)
                            scale_in_place(acc[rb][d], alpha);
                    }
                    m_ref[rb] = mt;
                }
                // p = 2^(logit - m_ref + 6) = exp2(fma(s, c, 6 - m_ref)): P carries 2^6
                const float bias = kPLog2 - ((m_ref[rb] == -INFINITY) ? 0.0f : m_ref[rb]);
                half8 hh8, ll8;
                float lsum = 0.0f;
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[jj], c, bias));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[jj + 1], c, bias));
                    lsum += p0 + p1;
                    // hi = p rounded toward zero to FP16 (its first 11 bits), lo =
                    // p - hi, exact in FP32, rounded toward zero to FP16
                    const half2v hh = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(p0, p1));
                    const float l0 = sub_half(p0, hh, 0), l1 = sub_half(p1, hh, 1);
                    const half2v ll = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(l0, l1));
                    hh8[jj] = hh.x;
                    hh8[jj + 1] = hh.y;
                    ll8[jj] = ll.x;
                    ll8[jj + 1] = ll.y;
                }
                l_part[rb] += lsum;
                ph[rb] = hh8;
                pl[rb] = ll8;
            }
        }
        wait_groups(j + 1 < nms ? 1 : 0);            // V(j); K(j+1) may be in flight

        // ---- O^T += V^T P^T over the wave's 32 tokens, all D columns ---------
        if (any) {
            const uint32_t vaddr = lds_addr(vst + w * C::BLOCK) + voff;
            // all V^T reads of the block first, so that their latencies overlap
            int2v vraw[C::DB];
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
                vraw[db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) int2v *)(uintptr_t)(vaddr ^ (uint32_t)(db << 4)));
            __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of their uses
            // Lane (n, g) holds V[token 8g + j][column 16 db + n] in byte j of
            // vraw[db].  In a block that some live row does not see whole, a
            // NaN byte would reach rows that mask its token (p = 0 times NaN):
            // such a block is checked for NaN codes, and only if it holds any
            // are they replaced by 0 and their positions recorded as one
            // 32-bit token mask per column ([D] words, byte g from lane group
            // g) in this wave's K stage, which holds nothing until K(j+2).
            uint8_t *const nanw = kst + w * C::BLOCK;
            bool has_nan = false;
            if (__builtin_expect(!all_full, 0)) {
                uint32_t hit = 0;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
                    hit |= nan_byte_marks((uint32_t)vraw[db].x) | nan_byte_marks((uint32_t)vraw[db].y);
                has_nan = __any(hit != 0);
            }
            if (__builtin_expect(has_nan, 0)) {
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    int x = vraw[db].x, y = vraw[db].y;
                    const uint32_t lo4 = drop_nan_bytes(x);
                    const uint32_t hi4 = drop_nan_bytes(y);
                    vraw[db] = int2v{x, y};
                    nanw[(16 * db + n) * 4 + g] = (uint8_t)(lo4 | (hi4 << 4));
                }
            }
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const half8 vf = dec_f16(vraw[db]);
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)
                    acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph[rb], acc[rb][db], 0, 0, 0);
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)
                    acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl[rb], acc[rb][db], 0, 0, 0);
            }
            if (__builtin_expect(has_nan, 0)) {
                // acc[rb][db] lane (n, g) holds row 16 rb + n, columns
                // 16 db + 4 g + k; bit 4 db + k of nan_hit[rb] records that the
                // row sees a NaN byte of that column.  Row visibility over the
                // block's 32 tokens: dense, the prefix below the row's length;
                // sparse, the tokens below it (INT32_MAX: no row sees it).
                uint32_t vis32[NRB];
                int tk8[8];
                if (SPARSE) {
                    const int4v t0 = *(const int4v *)&tok[8 * g];
                    const int4v t1 = *(const int4v *)&tok[8 * g + 4];
                    tk8[0] = t0.x; tk8[1] = t0.y; tk8[2] = t0.z; tk8[3] = t0.w;
                    tk8[4] = t1.x; tk8[5] = t1.y; tk8[6] = t1.z; tk8[7] = t1.w;
                }
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    if (SPARSE) {
                        uint32_t v8 = 0;
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj)
                            v8 |= (tk8[jj] < lrow[rb]) ? (1u << jj) : 0u;
                        vis32[rb] = or_over_groups(v8 << (8 * g));
                    } else {
                        const int nv = min(max(min(lrow[rb], hi) - pos0, 0), kSub);
                        vis32[rb] = nv >= kSub ? 0xFFFFFFFFu : (1u << nv) - 1u;
                    }
                }
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    const int4v nm = *(const int4v *)(nanw + (16 * db + 4 * g) * 4);
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            nan_hit[rb] |= ((uint32_t)nm[k] & vis32[rb]) ? (1ull << (4 * db + k)) : 0ull;
                }
            }
        }
        if (j + 1 < nms)
            issue_plane(bnext, j + 1, a.v_pool, v_st + (st ^ 1) * (kWaves * C::BLOCK),
                        &tok_s[w][st ^ 1][0]);
        bcur = bnext;
    };

    auto main_loop = [&](auto nrb_c) __attribute__((always_inline)) {
        for (int j = 0; j < nms; ++j)
            step(nrb_c, j);
    };

    if (nms > 0) {
        bcur = lookup(0);
        issue_plane(bcur, 0, a.k_pool, k_st, nullptr);
        if constexpr (RB == 1) {
            main_loop(std::integral_constant<int, 1>());
        } else if constexpr (RB == 2) {
            if (nrb == 1)
                main_loop(std::integral_constant<int, 1>());
            else
                main_loop(std::integral_constant<int, 2>());
        } else {
            if (nrb == 1)
                main_loop(std::integral_constant<int, 1>());
            else if (nrb == 2)
                main_loop(std::integral_constant<int, 2>());
            else
                main_loop(std::integral_constant<int, 3>());
        }
    }

    // ---- merge the four waves' states and write the split's partial --------
    // Wave w owns output quarter w: d-blocks [w*DQ, (w+1)*DQ).  Every wave
    // leaves its accumulators of the three other quarters in its private part
    // of LDS, relative to its own reference; the owner adds them with weights
    // 2^(m_ref - M), M the exact row max over the split.
    wait_vmcnt<0>();   // this wave's loads no longer target its stage slots
    // rows that see no token of this split may have accumulated values in
    // blocks processed without masks: they get the empty state
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        if (lrow[rb] <= (SPARSE ? 0 : lo)) {
            m_true[rb] = -INFINITY;
            m_ref[rb] = -INFINITY;
            l_part[rb] = 0.0f;
        }
    }
    // NaN V bytes seen by a row (rare; only blocks not seen whole record them)
    bool any_nan = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        any_nan = any_nan || nan_hit[rb] != 0;
    if (__builtin_expect(__any(any_nan), 0)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int d = 0; d < C::DB; ++d) {
                f32x4 x = acc[rb][d];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    x[k] = ((nan_hit[rb] >> (4 * d + k)) & 1ull) ? __builtin_nanf("") : x[k];
                acc[rb][d] = x;
            }
    }
    float lw[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        lw[rb] = sum_over_groups(l_part[rb]);
    // Chunk c (1 KB) of wave v's private merge area.  The wave's own loads
    // are done (the wait above), and no other wave writes there, so it
    // exports without waiting for the others to finish their blocks.
    auto xchunk = [&](int v, int c) __attribute__((always_inline)) -> uint8_t * {
        return c < 4 * C::SLOT_CHUNKS
                   ? smem + ((c / C::SLOT_CHUNKS) * kWaves + v) * C::BLOCK +
                         (c % C::SLOT_CHUNKS) * 1024
                   : smem + C::STAGES + v * C::EXTRA + (c - 4 * C::SLOT_CHUNKS) * 1024;
    };
    // per wave and row: running max, accumulator reference and row sum
    if (g == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            xm[w][rb * 16 + n] = m_true[rb];
            xr[w][rb * 16 + n] = m_ref[rb];
            xl[w][rb * 16 + n] = lw[rb];
        }
    }
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
        if (q == w)
            continue;
        const int qi = q < w ? q : q - 1;    // this quarter among the wave's three
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            if (rb < nrb)     // row blocks past nrb were never accumulated: zero
#pragma unroll
                for (int d = 0; d < C::DQ; ++d)
                    *(f32x4 *)(xchunk(w, (qi * RB + rb) * C::DQ + d) + lane * 16) =
                        acc[rb][q * C::DQ + d];
    }
    __syncthreads();
    // Every wave derives all four weights 2^(m_ref_v - M) itself, so that one
    // barrier separates the exchange from its use.
    // workspace rows: (b, i, h) of the output, or [split][row of the unit].
    // Row r of the unit is output row unit_row + r + (r / G)(H - G), so the
    // stores are addressed from the unit's first row.
    const int64_t ws_base =
        a.ragged ? (int64_t)blockIdx.x * a.rows
                 : (int64_t)split * a.total_rows +
                       ((int64_t)b * a.q_rows * a.num_heads + (int64_t)kvh * G);
    const __amdgpu_buffer_rsrc_t rs_acc = ws_rsrc(a.ws_acc + ws_base * D);
    const __amdgpu_buffer_rsrc_t rs_max = ws_rsrc(a.ws_max + ws_base);
    const __amdgpu_buffer_rsrc_t rs_sum = ws_rsrc(a.ws_sum + ws_base);
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
        if (q != w)
            continue;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = rb * 16 + n;
            // the three foreign partials of this quarter: all LDS reads first
            f32x4 xs[kWaves - 1][C::DQ];
            if (rb < nrb) {
#pragma unroll
                for (int vi = 0; vi < kWaves - 1; ++vi) {
                    const int v = vi < q ? vi : vi + 1;
                    const int qi = q < v ? q : q - 1;   // quarter q among wave v's three
#pragma unroll
                    for (int d = 0; d < C::DQ; ++d)
                        xs[vi][d] = *(const f32x4 *)(
                            xchunk(v, (qi * RB + rb) * C::DQ + d) + lane * 16);
                }
            }
            float mv[kWaves], rv[kWaves], lv[kWaves];
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                mv[v] = xm[v][r];
                rv[v] = xr[v][r];
                lv[v] = xl[v][r];
            }
            float M = mv[0];
#pragma unroll
            for (int v = 1; v < kWaves; ++v)
                M = fmaxf(M, mv[v]);
            float fv[kWaves];
            float L = 0.0f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                // rv <= M: the hardware exp2 (a weight below 2^-126 may
                // flush to zero, a negligible contribution)
                const float f = (rv[v] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(rv[v] - M);
                L += lv[v] * f;
                fv[v] = f * kPUnscale;
            }
            const int orow = a.ragged ? row0 + r : row0 + r + div_g(row0 + r) * (a.num_heads - G);
#pragma unroll
            for (int d = 0; d < C::DQ; ++d) {
                f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
                if (rb < nrb) {
                    o = acc[rb][q * C::DQ + d] * fv[q];
#pragma unroll
                    for (int vi = 0; vi < kWaves - 1; ++vi)
                        o += xs[vi][d] * fv[vi < q ? vi : vi + 1];
                }
                // lane (n, g) of d-block db holds d = 16 db + 4 g + k.  A row
                // that sees nothing of the split (sum 0) writes no numerator:
                // the combine never uses an empty split's numerator, and what
                // its accumulators took up unmasked is not part of it.
                if (r < R && L != 0.0f)
                    store_ws(rs_acc, (uint32_t)(orow * D + 16 * (q * C::DQ + d) + 4 * g) * 4u, o);
            }
            if (q == 0 && g == 0 && r < R) {
                store_ws(rs_max, (uint32_t)orow * 4u, M);
                store_ws(rs_sum, (uint32_t)orow * 4u, L * kPUnscale);
            }
        }
    }
}

DivMagic make_magic(int d)
{
    // l = ceil(log2 d); m = floor(2^(31+l) / d) + 1 is exact for 0 <= n < 2^31.
    int l = 0;
    while ((1ll << l) < d)
        ++l;
    DivMagic dm;
    dm.m = (uint32_t)(((uint64_t)1 << (31 + l)) / (uint64_t)d + 1);
    dm.s = (uint32_t)(31 + l);
    return dm;
}

template <int D, int MODE, int RB>
hipError_t launch_rb(const VerifyArgs &a, hipStream_t stream, const hipEvent_t *ev)
{
    // every split's page slots (token ids: positions) must fit the LDS slot cache
    if (mfma_slots_needed(a.tokens_per_split, a.page_size, MODE == kModeTokens) > max_slots<D>())
        return hipErrorNotSupported;
    // grid z: the row chunks of a KV unit
    // (a ragged batch's splits are shared by its units: grid y is 1)
    dim3 grid(a.num_splits, a.ragged ? 1 : a.batch * a.num_kv_heads,
              (a.rows + a.chunk_rows - 1) / a.chunk_rows);
    const uint32_t g_magic = (65536u + (uint32_t)a.group - 1u) / (uint32_t)a.group;
    hipExtLaunchKernelGGL((verify_mfma_kernel<D, MODE, RB>), grid, dim3(kThreads), 0, stream,
                          ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0, a,
                          make_magic(a.page_size), make_magic(a.num_kv_heads), g_magic);
    return hipGetLastError();
}

// One instance per row-chunk size, so that a chunk of 16 or 32 rows carries
// no code or registers for the row blocks it never has.
template <int D, int MODE>
hipError_t launch_t(const VerifyArgs &a, hipStream_t stream, const hipEvent_t *ev)
{
    switch (a.chunk_rows) {
    case 16: return launch_rb<D, MODE, 1>(a, stream, ev);
    case 32: return launch_rb<D, MODE, 2>(a, stream, ev);
    case 16 * kRowBlocks: return launch_rb<D, MODE, kRowBlocks>(a, stream, ev);
    default: return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_verify_mfma(const VerifyArgs &a, int head_dim, VerifyMode mode,
                              hipStream_t stream, const hipEvent_t *ev)
{
    if (a.chunk_rows != 16 && a.chunk_rows != 32 && a.chunk_rows != 16 * kRowBlocks)
        return hipErrorNotSupported;
    if (a.ragged && a.chunk_rows != 16 * kRowBlocks)
        return hipErrorNotSupported;
    if (a.rows < 1 || a.rows > 65535 * a.chunk_rows)
        return hipErrorNotSupported;
    // the partial stores' byte offsets from a KV unit's first row are 32-bit
    const int64_t span = a.ragged ? a.rows : (int64_t)a.q_rows * a.num_heads;
    if (span * head_dim * 4 >= ((int64_t)1 << 31))
        return hipErrorNotSupported;
    switch (head_dim * 4 + mode) {
    case 256 * 4 + kModeDense: return launch_t<256, kModeDense>(a, stream, ev);
    case 256 * 4 + kModeBlocks: return launch_t<256, kModeBlocks>(a, stream, ev);
    case 256 * 4 + kModeTokens: return launch_t<256, kModeTokens>(a, stream, ev);
    case 128 * 4 + kModeDense: return launch_t<128, kModeDense>(a, stream, ev);
    case 128 * 4 + kModeBlocks: return launch_t<128, kModeBlocks>(a, stream, ev);
    case 128 * 4 + kModeTokens: return launch_t<128, kModeTokens>(a, stream, ev);
    default: return hipErrorNotSupported;
    }
}

}  // namespace pa
