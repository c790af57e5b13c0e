// verify_mfma.hip - MFMA verify kernel for gfx950 (CDNA4).
//
// What it computes is the function in include/paged_attn_e4m3.h: per query row,
// softmax attention over the E4M3 K/V tokens it sees, as split partials with
// FP32 unnormalised numerators and a separate FP32 max and sum (design note
// "DFlash2 E4M3 attention with FP32 state", first section).  How it computes it
// on an MI355X:
//
//  * One workgroup per (split, KV unit): four waves, one per SIMD.  The split
//    is walked in macro-steps of 128 tokens.  Wave w owns tokens [32w, 32w+32)
//    of each macro-step for S = Q K^T and owns d-quarter w of the output for
//    P.V, so the FP32 accumulator of a wave is 48 rows x D/4 columns (48
//    registers at D = 256) and no end-of-kernel reduction of accumulators is
//    needed.  P and the per-row step maxima are exchanged through LDS.
//  * K/V bytes move HBM -> LDS with direct-to-LDS 16-byte loads (no VGPRs).
//    Two stages per plane; K is prefetched two macro-steps ahead, V one.
//    16-byte chunks of each token row are XOR-swizzled so that the MFMA
//    operand reads are free of LDS bank conflicts.
//  * E4M3 -> FP16 (or BF16 for a BF16 query) with the hardware converter,
//    which is exact for every finite code.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_{f16,bf16}: K is the A operand (one
//    ds_read_b64 per lane per 32 dims), Q^T the B operand, in registers for the
//    whole kernel.  The 16 tokens of each MFMA are ordered so that each lane's
//    8 scores of a 32-token block are exactly the 8 P^T elements it provides to
//    P.V: the P^T fragments are written to LDS as they are, 16 bytes per lane.
//  * O^T += V^T P^T: V^T fragments come straight from LDS with ds_read_tr8_b64
//    (the transposing read).  P is split into FP16 hi + lo parts and both are
//    multiplied ("compensated probabilities", design note first section);
//    every product is exact in FP32.
//  * The running reference max of a row moves only when a step exceeds it by
//    more than 2^8, so P <= 2^8 and accumulator rescales are rare; the partial
//    written out uses the exact row max.
//  * Tokens a row must not see get score -inf by select, and V bytes of
//    positions no row sees are zeroed by select before P.V, so NaN bytes in
//    padding pages cannot leak (null-block fix of 1Cat-vLLM PR #702).
#include "pa_internal.h"

#include <math.h>
#include <stdint.h>

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSub = 32;                  // tokens per wave per macro-step
constexpr int kMacro = kSub * kWaves;     // tokens per macro-step
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
typedef __attribute__((address_space(3))) void lds_void;

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

// Workgroup barrier for LDS data.  __syncthreads() (and any release fence on
// LDS) makes the compiler drain every in-flight direct-to-LDS load first, which
// would empty the prefetch pipeline at each barrier.  Here the wave's own LDS
// stores are completed (lgkmcnt 0), the direct loads that other waves will read
// are waited for explicitly by the caller, and the asm memory clobber keeps the
// compiler from moving memory accesses across the barrier.
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

__device__ __forceinline__ float max_over_groups(float v)
{
    float a, b;
    swap32(v, a, b);
    swap16(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}

__device__ __forceinline__ float sum_over_groups(float v)
{
    float a, b;
    swap32(v, a, b);
    swap16(a + b, a, b);
    return a + b;
}

template <int D>
struct Cfg {
    static constexpr int KB = D / 32;                 // QK k-blocks
    static constexpr int DBW = D / 16 / kWaves;       // PV d-blocks per wave
    static constexpr int BLOCK = kSub * D;            // bytes of one wave's 32 rows
    static constexpr int DMA = BLOCK / 1024;          // 1 KB direct loads per plane
    static constexpr int ROWS_PER_DMA = 1024 / D;
    static constexpr int LANES_PER_ROW = D / 16;
};

constexpr int kMaxSlotsD256 = 512;
constexpr int kMaxSlotsD128 = 1024;

template <int D>
constexpr int max_slots()
{
    return D == 256 ? kMaxSlotsD256 : kMaxSlotsD128;
}

template <int D, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void verify_mfma_kernel(VerifyArgs a, DivMagic dm)
{
    typedef Cfg<D> C;
    typedef typename Frag<SPARSE>::T QFrag;
    constexpr int kSlots = max_slots<D>();

    // stage planes: [wave block][32 rows][D], swizzled
    __shared__ __attribute__((aligned(16))) uint8_t k_s0[kWaves * C::BLOCK];
    __shared__ __attribute__((aligned(16))) uint8_t k_s1[kWaves * C::BLOCK];
    __shared__ __attribute__((aligned(16))) uint8_t v_s0[kWaves * C::BLOCK];
    __shared__ __attribute__((aligned(16))) uint8_t v_s1[kWaves * C::BLOCK];
    // P^T fragments: [token block kk][row block][hi, lo][64 lanes] x 16 bytes
    __shared__ __attribute__((aligned(16))) int4v p_s[kWaves][kRowBlocks][2][64];
    __shared__ int2v slots[kSlots];                 // (physical page, first token) per slot
    __shared__ __attribute__((aligned(16))) int32_t tok_s[2][kMacro];   // sparse: token per position
    __shared__ float xmax[kWaves][16 * kRowBlocks];
    __shared__ float xl[kWaves][16 * kRowBlocks];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int split = blockIdx.x;
    const int unit = blockIdx.y;
    const int b = unit / a.num_kv_heads;
    const int kvh = unit - b * a.num_kv_heads;
    const int R = a.rows, G = a.group;
    const int ps = a.page_size;

    // ---- query fragments: B operand of S^T = K Q^T (issued first, so their
    //      latency overlaps the length and page-table reads) ------------------
    QFrag qf[kRowBlocks][C::KB];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        const int r = rb * 16 + n;
        const bool live = r < R;
        const int i = live ? r / G : 0;
        const int h = kvh * G + (live ? r - i * G : 0);
        const uint16_t *qrow = a.q + (((int64_t)b * a.q_rows + i) * a.num_heads + h) * D;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (live)
                v = *(const uint4 *)(qrow + kb * 32 + g * 8);
            qf[rb][kb] = __builtin_bit_cast(QFrag, v);
        }
    }

    // ---- lengths -----------------------------------------------------------
    int lmax = 0;
    int lrow[kRowBlocks] = {0, 0, 0};
    for (int i = 0; i < a.q_rows; ++i) {
        int L = a.row_lens[(int64_t)b * a.q_rows + i];
        L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
        lmax = max(lmax, L);
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
            const int r = rb * 16 + n;
            if (r < R && r / G == i)
                lrow[rb] = L;
        }
    }
    const int lo = split * a.tokens_per_split;
    int hi = min(lo + a.tokens_per_split, a.list_len);
    if (!SPARSE)
        hi = min(hi, lmax);

    // ---- page slots of this split (the host guarantees they fit) -----------
    const int32_t *table = SPARSE ? a.block_table + (int64_t)b * a.table_stride : a.block_table;
    int slot0 = 0, nslots = 0;
    if (hi > lo) {
        slot0 = divp(lo, dm);
        nslots = min(divp(hi - 1, dm) + 1 - slot0, kSlots);
    }
    for (int i = tid; i < nslots; i += kThreads) {
        const int slot = slot0 + i;
        int phys = -1, tb = 0;
        if (!SPARSE) {
            phys = table[slot];
            tb = slot * ps;
        } else {
            const int blk = a.sel[((int64_t)b * a.num_kv_heads + kvh) * a.topk + slot];
            if (blk >= 0 && (int64_t)blk * ps < lmax) {
                phys = table[blk];
                tb = blk * ps;
            }
        }
        slots[i] = int2v{phys, tb};
    }

    // Q and the slot table are in before any direct-to-LDS load is issued, so no
    // later wait on them can also drain the K/V pipeline.  Q only ever feeds
    // MFMA as the B operand: it is kept in AGPRs, leaving the VGPRs to the
    // accumulators and the per-step working set.
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
            asm volatile("" : "+a"(qf[rb][kb]));
    wait_vmcnt<0>();
    __syncthreads();

    const int64_t head_off = (int64_t)kvh * a.head_stride;
    const int nms = hi > lo ? (hi - lo + kMacro - 1) / kMacro : 0;  // macro-steps

    // Position -> (byte offset of the K/V head row, token, valid).  Branch-free;
    // the slot cache is the only table read.
    auto resolve = [&](int pos, int64_t &off, int &t) __attribute__((always_inline)) -> bool {
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

    // Direct-to-LDS loads of this wave's 32 rows of macro-step j into one plane.
    // Lane l loads, in load i, row r_i = i*ROWS_PER_DMA + l/LANES_PER_ROW, swizzled
    // chunk position l%LANES_PER_ROW.  With pages of at least 32 tokens a wave's
    // block spans at most two page slots, so the page lookup is done once per
    // block (wave-uniform) and a lane only adds its precomputed row offset; small
    // pages or very large token strides take the per-row resolve.
    const int cp = lane % C::LANES_PER_ROW;
    const bool two_slot = ps >= kSub && a.token_stride < (1 << 25);
    int32_t loff[C::DMA];
#pragma unroll
    for (int i = 0; i < C::DMA; ++i) {
        const int r = i * C::ROWS_PER_DMA + lane / C::LANES_PER_ROW;
        loff[i] = two_slot ? r * (int32_t)a.token_stride + 16 * (cp ^ swz<D>(r)) : 0;
    }
    auto issue_plane = [&](int j, const uint8_t *pool, uint8_t *plane, int32_t *tokst)
        __attribute__((always_inline)) {
        const int pos0 = lo + j * kMacro + w * kSub;
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(plane + w * C::BLOCK));
        // the stage being refilled was read by this wave's previous step
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        if (two_slot) {
            const int sa = divp(pos0, dm);
            const int ua = pos0 - sa * ps;
            const int na = min(kSub, ps - ua);            // rows in the first slot
            const int2v ea = slots[min(max(sa - slot0, 0), kSlots - 1)];
            const int2v eb = slots[min(max(sa + 1 - slot0, 0), kSlots - 1)];
            const int phys_a = __builtin_amdgcn_readfirstlane(ea.x);
            const int tb_a = __builtin_amdgcn_readfirstlane(ea.y);
            const int phys_b = __builtin_amdgcn_readfirstlane(eb.x);
            const int tb_b = __builtin_amdgcn_readfirstlane(eb.y);
            const int hip = hi - pos0;
            // valid rows: [0, end_a) in the first slot, [na, end_b) in the second
            int end_a = min(na, hip), end_b = hip;
            if (SPARSE) {
                end_a = phys_a >= 0 ? min(end_a, lmax - (tb_a + ua)) : 0;
                end_b = phys_b >= 0 ? min(end_b, na + lmax - tb_b) : 0;
            }
            const int64_t base_a = (int64_t)phys_a * a.page_stride + (int64_t)ua * a.token_stride + head_off;
            if (na == kSub && end_a == kSub) {
                // the whole block is valid and inside one page: SGPR base + lane offset
                const uint8_t *sb = pool + base_a;
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
                        tokst[w * kSub + r] = tb_a + ua + r;
                    }
                }
            } else {
                const int64_t base_b = (int64_t)phys_b * a.page_stride - (int64_t)na * a.token_stride + head_off;
#pragma unroll
                for (int i = 0; i < C::DMA; ++i) {
                    const int r = i * C::ROWS_PER_DMA + lane / C::LANES_PER_ROW;
                    const bool in_b = r >= na;
                    const bool ok = in_b ? (r < end_b) : (r < end_a);
                    const int64_t src = ok ? (in_b ? base_b : base_a) + loff[i] : 0;
                    dma16(pool + src, dst + i * 1024);
                    if (SPARSE && tokst != nullptr && cp == 0)
                        tokst[w * kSub + r] = ok ? (in_b ? tb_b - na + r : tb_a + ua + r) : INT32_MAX;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::DMA; ++i) {
                const int row = i * C::ROWS_PER_DMA + lane / C::LANES_PER_ROW;
                int64_t off;
                int t;
                const bool ok = resolve(pos0 + row, off, t);
                const int64_t src = ok ? off + 16 * (cp ^ swz<D>(row)) : 0;
                dma16(pool + src, dst + i * 1024);
                if (SPARSE && tokst != nullptr && cp == 0)
                    tokst[w * kSub + row] = ok ? t : INT32_MAX;
            }
        }
    };

    // ---- state -------------------------------------------------------------
    f32x4 acc[kRowBlocks][C::DBW];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
        for (int d = 0; d < C::DBW; ++d)
            acc[rb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_true[kRowBlocks], m_ref[kRowBlocks], l_part[kRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        m_true[rb] = -INFINITY;
        m_ref[rb] = -INFINITY;
        l_part[rb] = 0.0f;
    }
    const float c = a.logit_scale;

    // One macro-step on the stage pair (kst, vst).  Every step issues K(j+2)
    // after its QK and V(j+1) after its step-max barrier; past the end of the
    // split these are dummy loads (every position invalid) into stages that are
    // not read again, so the wait counts below are the same for every step:
    //  * before QK(j), the groups issued after K(j) are V(j-1), K(j+1), V(j);
    //    V(j-1) is complete already (P.V of step j-1 waited for it), so leaving
    //    two groups in flight means K(j) has landed (steps 0 and 1 have exactly
    //    two later groups: V(0), K(1) and K(2), V(1));
    //  * before the P.V barrier, the groups issued after V(j) are K(j+2) and
    //    V(j+1) (step 0 also has K(1), so it waits a little longer).
    auto step = [&](int j, uint8_t *kst, uint8_t *vst, uint8_t *kst_next2, uint8_t *vst_next1,
                    int32_t *tok_cur, int32_t *tok_next1) __attribute__((always_inline)) {
        const int pos0 = lo + j * kMacro;
        wait_vmcnt<2 * C::DMA>();

        // ---- S^T = K Q^T on this wave's 32 tokens --------------------------
        f32x4 s[kRowBlocks][2];
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
            s[rb][0] = s[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint8_t *kblk = kst + w * C::BLOCK;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            // MFMA row m of block bb is token 8(m/4) + 4bb + m%4
            const int krow = 8 * (n >> 2) + 4 * bb + (n & 3);
            const uint8_t *kr = kblk + krow * D + ((g & 1) << 3);
            const int sw = swz<D>(krow);
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) {
                const int2v raw = *(const int2v *)(kr + (((2 * kb + (g >> 1)) ^ sw) << 4));
                QFrag kf;
                if (SPARSE)
                    kf = __builtin_bit_cast(QFrag, dec_bf16(raw));
                else
                    kf = __builtin_bit_cast(QFrag, dec_f16(raw));
#pragma unroll
                for (int rb = 0; rb < kRowBlocks; ++rb)
                    s[rb][bb] = mfma_qk(kf, qf[rb][kb], s[rb][bb]);
            }
        }
        issue_plane(j + 2, a.k_pool, kst_next2, nullptr);

        // ---- visibility of this lane's 8 scores (tokens 32w + 8g + jj) ---------
        // vis[rb] bit jj: row 16rb + n sees token jj.  Row blocks that see the
        // whole block skip the selects; blocks that see none of it skip P.
        int tok[8];
        if (SPARSE) {
            const int4v t0 = *(const int4v *)&tok_cur[w * kSub + 8 * g];
            const int4v t1 = *(const int4v *)&tok_cur[w * kSub + 8 * g + 4];
            tok[0] = t0.x; tok[1] = t0.y; tok[2] = t0.z; tok[3] = t0.w;
            tok[4] = t1.x; tok[5] = t1.y; tok[6] = t1.z; tok[7] = t1.w;
        }
        const int tfirst = pos0 + w * kSub + 8 * g;
        uint32_t vis[kRowBlocks];
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
            if (!SPARSE) {
                const int nv = min(max(min(lrow[rb], hi) - tfirst, 0), 8);
                vis[rb] = (1u << nv) - 1u;
            } else {
                uint32_t m = 0;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    m |= (tok[jj] < lrow[rb]) ? (1u << jj) : 0u;   // invalid tok = INT32_MAX
                vis[rb] = m;
            }
            // c > 0, so the largest logit comes from the largest raw score
            float mloc = -INFINITY;
            if (__all(vis[rb] == 0xFFu)) {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    mloc = fmaxf(mloc, s[rb][jj >> 2][jj & 3]);
            } else if (!__all(vis[rb] == 0u)) {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    mloc = fmaxf(mloc, ((vis[rb] >> jj) & 1u) ? s[rb][jj >> 2][jj & 3] : -INFINITY);
            }
            mloc = max_over_groups(mloc) * c;
            if (g == 0)
                xmax[w][rb * 16 + n] = mloc;
        }
        barrier_lds();   // step maxima published; every wave is past P.V of step j-1
        issue_plane(j + 1, a.v_pool, vst_next1, tok_next1);

        // ---- online softmax with the shared reference max --------------------
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
            float mstep = xmax[0][rb * 16 + n];
#pragma unroll
            for (int v = 1; v < kWaves; ++v)
                mstep = fmaxf(mstep, xmax[v][rb * 16 + n]);
            const float mt = fmaxf(m_true[rb], mstep);
            m_true[rb] = mt;
            // identical inputs in every wave, so every wave takes the same branch
            if (__any(mt > m_ref[rb] + kLazy)) {
                const float alpha = (mt == -INFINITY) ? 1.0f : exp2f(m_ref[rb] - mt);
                l_part[rb] *= alpha;
#pragma unroll
                for (int d = 0; d < C::DBW; ++d)
                    acc[rb][d] *= alpha;
                m_ref[rb] = mt;
            }
            // p = 2^(logit - m_ref + 6) = exp2(fma(s, c, 6 - m_ref)): P carries 2^6
            const float bias = kPLog2 - ((m_ref[rb] == -INFINITY) ? 0.0f : m_ref[rb]);
            half8 ph = {}, pl = {};
            if (!__all(vis[rb] == 0u)) {
                const bool full = __all(vis[rb] == 0xFFu);
                float lsum = 0.0f;
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2) {
                    float a0 = __builtin_fmaf(s[rb][jj >> 2][jj & 3], c, bias);
                    float a1 = __builtin_fmaf(s[rb][(jj + 1) >> 2][(jj + 1) & 3], c, bias);
                    if (!full) {
                        a0 = ((vis[rb] >> jj) & 1u) ? a0 : -INFINITY;
                        a1 = ((vis[rb] >> (jj + 1)) & 1u) ? a1 : -INFINITY;
                    }
                    const float s0 = exp2f(a0), s1 = exp2f(a1);
                    lsum += s0 + s1;
                    const float h0 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, s0) & 0xFFFFE000u);
                    const float h1 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, s1) & 0xFFFFE000u);
                    const half2v hh = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(h0, h1));
                    const half2v ll = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(s0 - h0, s1 - h1));
                    ph[jj] = hh.x;
                    ph[jj + 1] = hh.y;
                    pl[jj] = ll.x;
                    pl[jj + 1] = ll.y;
                }
                l_part[rb] += lsum;
            }
            p_s[w][rb][0][lane] = __builtin_bit_cast(int4v, ph);
            p_s[w][rb][1][lane] = __builtin_bit_cast(int4v, pl);
        }
        wait_vmcnt<2 * C::DMA>();   // V(j) landed; K(j+2), V(j+1) may fly
        barrier_lds();   // P^T of all four token blocks and V(j) are in LDS

        // ---- O^T[d-quarter w] += V^T P^T over the 128 tokens ------------------
#pragma unroll
        for (int kk = 0; kk < kWaves; ++kk) {
            half8 ph[kRowBlocks], pl[kRowBlocks];
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; ++rb) {
                ph[rb] = __builtin_bit_cast(half8, p_s[kk][rb][0][lane]);
                pl[rb] = __builtin_bit_cast(half8, p_s[kk][rb][1][lane]);
            }
            // V rows of token block kk that no row may see are zeroed (select)
            uint32_t vm_lo = 0xFFFFFFFFu, vm_hi = 0xFFFFFFFFu;
            const int tbase = pos0 + kk * kSub + 8 * g;
            if (!SPARSE) {
                if (pos0 + kMacro > hi) {
                    vm_lo = 0;
                    vm_hi = 0;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        vm_lo |= (tbase + jj < hi) ? (0xFFu << (8 * jj)) : 0u;
                        vm_hi |= (tbase + 4 + jj < hi) ? (0xFFu << (8 * jj)) : 0u;
                    }
                }
            } else {
                vm_lo = 0;
                vm_hi = 0;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    vm_lo |= (tok_cur[kk * kSub + 8 * g + jj] != INT32_MAX) ? (0xFFu << (8 * jj)) : 0u;
                    vm_hi |= (tok_cur[kk * kSub + 8 * g + 4 + jj] != INT32_MAX) ? (0xFFu << (8 * jj)) : 0u;
                }
            }
            // supplier lane (n, g) of the transposing read points at row 8g + n/2,
            // half n%2 of the 16-byte chunk of d-block db
            const int vrow = 8 * g + (n >> 1);
            const uint8_t *vr = vst + kk * C::BLOCK + vrow * D + ((n & 1) << 3);
            const int vsw = swz<D>(vrow);
#pragma unroll
            for (int d = 0; d < C::DBW; ++d) {
                const int db = w * C::DBW + d;
                int2v raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) int2v *)(vr + ((db ^ vsw) << 4)));
                raw.x &= (int)vm_lo;
                raw.y &= (int)vm_hi;
                const half8 vf = dec_f16(raw);
#pragma unroll
                for (int rb = 0; rb < kRowBlocks; ++rb) {
                    acc[rb][d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph[rb], acc[rb][d], 0, 0, 0);
                    acc[rb][d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl[rb], acc[rb][d], 0, 0, 0);
                }
            }
        }
    };

    // ---- pipeline ------------------------------------------------------------
    if (nms > 0) {
        issue_plane(0, a.k_pool, k_s0, nullptr);
        issue_plane(0, a.v_pool, v_s0, &tok_s[0][0]);
        issue_plane(1, a.k_pool, k_s1, nullptr);
    }
    for (int j = 0; j < nms; j += 2) {
        step(j, k_s0, v_s0, k_s0, v_s1, &tok_s[0][0], &tok_s[1][0]);
        if (j + 1 < nms)
            step(j + 1, k_s1, v_s1, k_s1, v_s0, &tok_s[1][0], &tok_s[0][0]);
    }

    // ---- finish: exact max, summed l, this wave's d-quarter ----------------------
    wait_vmcnt<0>();   // the trailing dummy loads
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        l_part[rb] = sum_over_groups(l_part[rb]);
        if (g == 0)
            xl[w][rb * 16 + n] = l_part[rb];
    }
    __syncthreads();
    const int64_t ws_base = (int64_t)split * a.total_rows;
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        const int r = rb * 16 + n;
        if (r < R) {
            // acc and l are relative to m_ref and both carry the 2^6 of P
            const float sc = (m_ref[rb] == -INFINITY) ? 0.0f : exp2f(m_ref[rb] - m_true[rb]);
            const float sa = sc * kPUnscale;
            const int i = r / G, h = kvh * G + (r - i * G);
            const int64_t orow = ((int64_t)b * a.q_rows + i) * a.num_heads + h;
            float *dst = a.ws_acc + (ws_base + orow) * D;
            // lane (n, g) of d-block db holds d = 16 db + 4 g + k
#pragma unroll
            for (int d = 0; d < C::DBW; ++d)
                *(f32x4 *)(dst + 16 * (w * C::DBW + d) + 4 * g) = acc[rb][d] * sa;
            if (w == 0 && g == 0) {
                float L = 0.0f;
#pragma unroll
                for (int v = 0; v < kWaves; ++v)
                    L += xl[v][r];
                a.ws_max[ws_base + orow] = m_true[rb];
                a.ws_sum[ws_base + orow] = L * sa;
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

template <int D, bool SPARSE>
hipError_t launch_t(const VerifyArgs &a, hipStream_t stream)
{
    // every split's page slots must fit the LDS slot cache
    const int64_t slots = (int64_t)(a.tokens_per_split - 1) / a.page_size + 2;
    if (slots > max_slots<D>())
        return hipErrorNotSupported;
    dim3 grid(a.num_splits, a.batch * a.num_kv_heads);
    hipLaunchKernelGGL((verify_mfma_kernel<D, SPARSE>), grid, dim3(kThreads), 0, stream, a,
                       make_magic(a.page_size));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_mfma(const VerifyArgs &a, int head_dim, bool sparse, hipStream_t stream)
{
    if (a.rows > 16 * kRowBlocks)
        return hipErrorNotSupported;
    if (head_dim == 256)
        return sparse ? launch_t<256, true>(a, stream) : launch_t<256, false>(a, stream);
    if (head_dim == 128)
        return sparse ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return hipErrorNotSupported;
}

}  // namespace pa
