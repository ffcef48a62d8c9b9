// Top-k selection of key positions from bf16 indexer logits and their remap to cache rows (gfx950):
// the index lists the top-k sparse decode reads.
//
// What it computes (vLLM API pages, cited by title and section):
//   vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.topk_exchange, push_local_topk and
//   the merge's radix select: a row's candidates are its non-NaN bf16 logits at columns
//   [0, min(row_end, N)); each is ranked by a 16-bit order key of its bits; the threshold v is the
//   K-th largest key; the columns above v are all selected and the lowest-numbered columns equal
//   to v fill the remaining places; the output lists the columns above v in increasing column
//   order, then those equal to v in increasing column order. A row with fewer than K candidates
//   selects all of them, in column order.
//   vllm.model_executor.kernels.attention.dsa.sparse_mqa_logits, the remap: selected columns
//   become positions, and places without a valid position hold -1. Here position j of request b
//   is cache row table[b, j / page_size] * page_size + j % page_size (the dense decode's rule).
// The order key (a reading: the pages do not print it) is the monotone map of the sign-magnitude
// pattern to an unsigned integer: positive bits | 0x8000, negative ~bits.
//
// One 1024-thread workgroup per row. The row is taken in spans of 32768 columns; in a span thread
// t owns the 32 consecutive columns 32 t .. 32 t + 31 (four 16-byte loads), whose ranks (the order
// key less 0x7E, 0 for NaN and past the row end, formed two at a time by packed 16-bit arithmetic)
// it keeps packed two to a register, so a row of at most 32768 columns is read from memory once
// for all three passes. The threshold comes from two radix histograms in LDS. The first covers the
// ranks from a lower bound to the row's largest in 4096 bins of 2^sb ranks, sb as small as fits:
// for a row held in registers the bound is the least m-th largest rank of the threads' 32
// (m = ceil(K / 1024)), and for N(0, 1) logits every rank then gets a bin of its own (sb = 0),
// which finds the threshold exactly and skips the second histogram; otherwise that one resolves
// the chosen bin's 2^sb ranks. The ordered output: per thread two 32-bit masks (columns above /
// equal to the threshold, one compare and one add-with-carry per bit), one workgroup prefix sum
// per span of both popcounts packed in one word (wave prefix by DPP row shifts and the rows'
// totals, then the 16 wave totals through LDS) and the set bits in ascending order: thread order
// is column order, so the lists come out in column order without a sort. Lists of up to 8192
// entries are built in LDS and remapped from there.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_decode.h"

namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_VEC = 4;                         // 16-byte loads (8 columns each) per thread
constexpr int TK_OWN = 8 * TK_VEC;                // columns per thread per span
constexpr int TK_SPAN = TK_THREADS * TK_OWN;      // 32768 columns

typedef int v4i_t __attribute__((ext_vector_type(4)));

constexpr int TK_HI_BITS = 12;                    // the first histogram: 4096 bins
constexpr int TK_LO_BITS = 16 - TK_HI_BITS;       // bins of at most 2^4 ranks, the second's 16 bins
constexpr int TK_BINS = 1 << TK_HI_BITS;
constexpr int TK_BPT = TK_BINS / TK_THREADS;      // bins per thread in the threshold search (4)

constexpr int TK_LDS_K = 8192;   // lists of up to this many entries are built in LDS

struct TkShared {
    alignas(16) uint32_t hist[TK_BINS + 64];   // the bins (read and cleared 16 bytes at a time),
                                               // then a spare counter per lane, never read
    alignas(16) uint32_t hist2[1 << TK_LO_BITS];   // the second pass (cleared with the first)
    uint32_t wave_min[TK_WAVES];
    uint32_t wave_max[TK_WAVES];
    int wave_tot[TK_WAVES];
    int sel[2];   // the first histogram's chosen bin, ranks above it
};

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

template <bool STAGE>
struct TkList {   // the selected columns: in LDS (K <= TK_LDS_K), else in the output row itself
    int32_t col[STAGE ? TK_LDS_K : 1];
};

typedef short s16x2_t __attribute__((ext_vector_type(2)));

// The ranks of two bf16 patterns (one per 16-bit half): the order key minus 0x7E, or 0 for NaN.
// The order key is b ^ 0xFFFF (= ~b) for a set sign bit, b ^ 0x8000 (= b | 0x8000) for a clear
// one: -inf maps to 0x7F, +inf to 0xFF80, the negative NaNs below 0x7F and the positive ones
// above 0xFF80. Three packed 16-bit steps, two columns per instruction: + 0x7E saturating (the
// positive NaNs, and only they, reach 0xFFFF), + 1 wrapping (they become 0), - 0xFD saturating
// (the negative NaNs, at most 0xFC by then, become 0). Numbers come out at 1 .. 0xFF02 in the
// keys' order, so every comparison of ranks is one of keys.
__device__ inline uint32_t tk_rank2(uint32_t w)
{
    const s16x2_t sgn = __builtin_bit_cast(s16x2_t, w) >> (s16x2_t){15, 15};   // 0xFFFF where negative
    const u16x2_t key = __builtin_bit_cast(u16x2_t, w ^ (__builtin_bit_cast(uint32_t, sgn) | 0x80008000u));
    const u16x2_t a = __builtin_elementwise_add_sat(key, (u16x2_t){0x7E, 0x7E}) + (u16x2_t){1, 1};
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(a, (u16x2_t){0xFD, 0xFD}));
}

// Inclusive prefix sum over the wave's lanes: within each row of 16 lanes by DPP row shifts of 1,
// 2, 4 and 8 (a lane whose source lies before its row adds 0), then the rows' totals (lanes 15, 31
// and 47, read into scalars) added to the rows after them. No LDS round trips.
__device__ inline int tk_wave_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Minimum over the wave's lanes (the same in every lane): within each row of 16 lanes by quad swaps
// and the half-row and row mirrors, then across the four rows by readlane.
__device__ inline uint32_t tk_wave_min(uint32_t v)
{
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return min(min(a, b), min(c, d));
}

// Exclusive prefix sum over the workgroup's threads in thread order (and the total). One barrier:
// the caller puts another between this scan's reads of wave_tot and the next scan's writes.
__device__ inline int tk_scan(int x, TkShared& sh, int& total)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int v = tk_wave_scan(x);
    if (lane == 63)
        sh.wave_tot[wave] = v;
    __syncthreads();
    // the 16 wave totals in lanes 0..15 (each row of 16 lanes holds a copy), scanned inside the
    // row by DPP shifts; this wave's offset and the total are read out as scalars
    static_assert(TK_WAVES == 16, "one DPP row of wave totals");
    int wt = sh.wave_tot[lane & 15];
    wt += __builtin_amdgcn_update_dpp(0, wt, 0x111, 0xF, 0xF, true);   // row_shr:1
    wt += __builtin_amdgcn_update_dpp(0, wt, 0x112, 0xF, 0xF, true);   // row_shr:2
    wt += __builtin_amdgcn_update_dpp(0, wt, 0x114, 0xF, 0xF, true);   // row_shr:4
    wt += __builtin_amdgcn_update_dpp(0, wt, 0x118, 0xF, 0xF, true);   // row_shr:8
    total = __builtin_amdgcn_readlane(wt, TK_WAVES - 1);
    const int off = wave > 0 ? __builtin_amdgcn_readlane(wt, wave > 0 ? wave - 1 : 0) : 0;
    return off + v - x;
}

constexpr int TK_KW = TK_OWN / 2;                 // rank registers per thread (two ranks each)

// This thread's 32 columns of the span starting at s0 as raw bf16 vectors (1 <= lim <= N and
// N % 8 == 0: a 16-byte vector that starts before lim lies wholly in the row). A vector starting
// at or past column lim is read from the last vector that starts before lim instead (its keys are
// masked later as past the row end), so that all four loads go out together without branches.
__device__ inline void tk_load(const uint16_t* row, int lim, int s0, v4i_t (&raw)[TK_VEC])
{
    const int c = s0 + TK_OWN * (int)threadIdx.x;
    const int last = (lim - 1) & ~7;
#pragma unroll
    for (int m = 0; m < TK_VEC; m++) {
        const int cm = c + 8 * m < lim ? c + 8 * m : last;
        raw[m] = *reinterpret_cast<const v4i_t*>(row + cm);
    }
}

// Their ranks: kw[i] holds column 2 i in its low half and column 2 i + 1 in its high half (0 at
// and past the row end n, which only the threads holding columns at or past n mask).
__device__ inline void tk_form(const v4i_t (&raw)[TK_VEC], int n, int s0, uint32_t (&kw)[TK_KW])
{
    const int c = s0 + TK_OWN * (int)threadIdx.x;
#pragma unroll
    for (int i = 0; i < TK_KW; i++)
        kw[i] = tk_rank2((uint32_t)raw[i >> 2][i & 3]);
    if (c + TK_OWN > n) {
#pragma unroll
        for (int i = 0; i < TK_KW; i++) {
            const int col = c + 2 * i;
            // 0xFFFF where the column lies before n (the sign of col - n), else 0
            const uint32_t mlo = ((uint32_t)(col - n) >> 31) * 0xFFFFu;
            const uint32_t mhi = ((uint32_t)(col + 1 - n) >> 31) * 0xFFFF0000u;
            kw[i] &= mlo | mhi;
        }
    }
}

// Two more columns into the threshold masks: the rank pair w (column 2 i in the low half, 2 i + 1
// in the high half), taken from the last column down, so that column e ends at bit e. Per column one
// compare of the selected 16-bit half with v into VCC and one add-with-carry m = m + m + VCC.
__device__ inline void tk_mask_step(uint32_t w, uint32_t v, uint32_t& gm, uint32_t& em)
{
    asm("v_cmp_gt_u32_sdwa vcc, %2, %3 src0_sel:WORD_1 src1_sel:DWORD\n\t"
        "v_addc_co_u32 %0, vcc, %0, %0, vcc\n\t"
        "v_cmp_eq_u32_sdwa vcc, %2, %3 src0_sel:WORD_1 src1_sel:DWORD\n\t"
        "v_addc_co_u32 %1, vcc, %1, %1, vcc\n\t"
        "v_cmp_gt_u32_sdwa vcc, %2, %3 src0_sel:WORD_0 src1_sel:DWORD\n\t"
        "v_addc_co_u32 %0, vcc, %0, %0, vcc\n\t"
        "v_cmp_eq_u32_sdwa vcc, %2, %3 src0_sel:WORD_0 src1_sel:DWORD\n\t"
        "v_addc_co_u32 %1, vcc, %1, %1, vcc"
        : "+v"(gm), "+v"(em)
        : "v"(w), "v"(v)
        : "vcc");
}

// The ranks of this thread's 32 columns of the span starting at s0 (0 past the row end n).
__device__ inline void tk_keys(const uint16_t* row, int n, int s0, uint32_t (&kw)[TK_KW])
{
    v4i_t raw[TK_VEC];
    tk_load(row, n, s0, raw);
    tk_form(raw, n, s0, kw);
}

// Of the TK_BINS bins of the first histogram (counts in sh.hist), the highest bin b whose count together with
// the bins above it reaches need: sh.sel[0] = b, sh.sel[1] = the count above b (left at -1 and 0,
// as cleared, if there is none). Thread t looks at the four bins 4 (1023 - t) + 3 .. 4 (1023 - t),
// from the top; the bin is found by the one thread whose share crosses need.
__device__ inline void tk_pick_bin(TkShared& sh, int need)
{
    const int t = threadIdx.x;
    const int b0 = TK_BINS - TK_BPT * (t + 1);
    static_assert(TK_BPT == 4, "one 16-byte LDS read per thread");
    const v4i_t h = *reinterpret_cast<const v4i_t*>(&sh.hist[b0]);
    int total;
    int excl = tk_scan(h[0] + h[1] + h[2] + h[3], sh, total);
#pragma unroll
    for (int i = TK_BPT - 1; i >= 0; i--) {
        if (h[i] > 0 && excl < need && excl + h[i] >= need) {
            sh.sel[0] = b0 + i;
            sh.sel[1] = excl;
        }
        excl += h[i];
    }
    __syncthreads();
}

// Division of a 32-bit unsigned n by an invariant d (1 <= d < 2^31): with l = ceil(log2 d),
// magic = floor(2^32 (2^l - d) / d) + 1, t = umulhi(n, magic), n / d = (t + ((n - t) >> s1)) >> s2,
// s1 = min(l, 1), s2 = max(l - 1, 0) (Granlund and Montgomery, "Division by invariant integers
// using multiplication", 1994, Figure 4.1). A few instructions instead of a division routine.
struct TkDiv {
    uint32_t magic;
    int s1, s2;
};

TkDiv tk_division(int d)
{
    int l = 0;
    while ((1ll << l) < d)
        l++;
    TkDiv v;
    v.magic = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - (uint64_t)d)) / (uint64_t)d + 1);
    v.s1 = l < 1 ? l : 1;
    v.s2 = l - 1 > 0 ? l - 1 : 0;
    return v;
}

__device__ inline uint32_t tk_div(const TkDiv& v, uint32_t n)
{
    const uint32_t t = __umulhi(n, v.magic);
    return (t + ((n - t) >> v.s1)) >> v.s2;
}

// What the selected columns become: with `si` set, sparse logit columns -> request-local
// positions (column j * sbk + o of row r scores position (si[r, j] - floor(ks[r] / sbk)) * sbk + o);
// then, with `table` set, positions -> cache rows through request r / Q's page table.
struct TkRemap {
    const int32_t* si;      // [R, S] sparse block ids backing the logit columns, or null
    int S, sbk;
    TkDiv sdiv;             // division by sbk
    const int32_t* ks;      // [R] K range starts (the sparse ids' anchor)
    const int32_t* table;   // [R / Q, max_pages] page ids, or null
    int max_pages, page_size, Q;
    TkDiv pdiv;             // division by page_size
    int64_t num_rows;
};

__device__ inline int64_t tk_floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// A row's share of the remap, looked up once per row: its sparse block ids and their anchor
// floor(ks[r] / sbk), and its request's page table row.
struct TkRowMap {
    const int32_t* si_row;
    int64_t anchor;
    const int32_t* table_row;
};

__device__ inline TkRowMap tk_row_map(const TkRemap& m, int r)
{
    TkRowMap rm{nullptr, 0, nullptr};
    if (m.si) {
        rm.si_row = m.si + (int64_t)r * m.S;
        rm.anchor = tk_floor_div(m.ks[r], m.sbk);
    }
    if (m.table)
        rm.table_row = m.table + (int64_t)(r / m.Q) * m.max_pages;
    return rm;
}

// One selected column -> the list entry (-1 where the position or its page or row is invalid).
// The column (in [0, N), N < 2^31) and the position (checked to lie in [0, 2^31)) divide as 32-bit
// unsigned values.
__device__ inline int32_t tk_remap(const TkRemap& m, const TkRowMap& rm, int col)
{
    int64_t j = col;
    if (m.si) {
        const uint32_t q = tk_div(m.sdiv, (uint32_t)col);
        const int64_t blk = rm.si_row[q];
        j = (blk - rm.anchor) * m.sbk + (int64_t)((uint32_t)col - q * (uint32_t)m.sbk);
        if (j < 0 || j > 0x7FFFFFFF)
            return -1;
    }
    if (!m.table)
        return (int32_t)j;
    const uint32_t pgi = tk_div(m.pdiv, (uint32_t)j);
    if ((int64_t)pgi >= m.max_pages)
        return -1;
    const int64_t page = rm.table_row[pgi];
    const int64_t cr = page * m.page_size + (int64_t)((uint32_t)j - pgi * (uint32_t)m.page_size);
    return (page >= 0 && cr < m.num_rows) ? (int32_t)cr : -1;
}

// ONE: every row fits one span (N <= 32768), so the ranks stay in registers for all passes
// and the span loops run once (a separate instantiation keeps the other case's code out).
template <bool STAGE, bool ONE>
__global__ __launch_bounds__(TK_THREADS) void mla_topk_kernel(
    const uint16_t* __restrict__ logits, const int32_t* __restrict__ row_ends, int N, int K,
    const TkRemap remap, int32_t* __restrict__ rows_out, int32_t* __restrict__ valid_out)
{
    __shared__ TkShared sh;
    __shared__ TkList<STAGE> lst;
    const int r = blockIdx.x;
    const int t = threadIdx.x;
    const uint16_t* row = logits + (int64_t)r * N;
    // the first span's columns are requested together with the row end (bounded by the row's
    // width, not its end), so the two loads share one round trip
    v4i_t raw0[TK_VEC];
    tk_load(row, N < TK_SPAN ? N : TK_SPAN, 0, raw0);
    int n = row_ends[r];
    n = n < 0 ? 0 : (n > N ? N : n);
    int32_t* out = rows_out + (int64_t)r * K;
    int32_t* list = STAGE ? lst.col : out;   // the ordered columns before the remap
    // a row of one span stays in registers for all three passes
    const bool resident = ONE || n <= TK_SPAN;
    const int s_end = ONE ? (n > 0 ? 1 : 0) : n;   // the span loops: s0 < s_end
    uint32_t kw[TK_KW];
    // The first histogram covers ranks base .. M in 4096 bins (k - base) >> sb, with the least sb
    // (0 .. 4) that fits; ranks below base go to per-lane spare counters (no branch, no shared
    // counter). Without more knowledge base = 1 (every candidate) and sb = 4. A row held in
    // registers gives more: with m = ceil(K / 1024) <= 2, every thread holding at least m
    // candidates has m ranks >= its m-th largest, so if these threads number F with m F >= K, at
    // least K ranks are >= the least of their m-th largest, L, and so is the threshold: base = L.
    // M = the row's largest rank. For N(0, 1) logits this leaves about a quarter of the ranks in
    // range, and M - base < 4096: sb = 0, every rank has its own bin and the threshold is found
    // without a second pass.
    uint32_t base = 1u;
    int sb = TK_LO_BITS;
    const int m = K / TK_THREADS + (K % TK_THREADS != 0 ? 1 : 0);   // ceil, without overflow
    bool any = true;   // this lane holds a rank >= base (resident rows)
    uint32_t m1 = 0u;
    if (resident) {
        tk_form(raw0, n, 0, kw);
        // the largest and second-largest rank of the even and the odd columns, two lanes at once
        u16x2_t a1 = {0, 0}, a2 = {0, 0};
#pragma unroll
        for (int i = 0; i < TK_KW; i++) {
            const u16x2_t k = __builtin_bit_cast(u16x2_t, kw[i]);
            a2 = __builtin_elementwise_max(a2, __builtin_elementwise_min(a1, k));
            a1 = __builtin_elementwise_max(a1, k);
        }
        m1 = a1[0] > a1[1] ? a1[0] : a1[1];
        const uint32_t lo1 = a1[0] > a1[1] ? a1[1] : a1[0];
        const uint32_t hi2 = a2[0] > a2[1] ? a2[0] : a2[1];
        const uint32_t m2 = lo1 > hi2 ? lo1 : hi2;
        const uint32_t mth = m == 1 ? m1 : m2;   // 0: fewer than m candidates
        const bool full = m <= 2 && mth != 0u;
        const uint32_t wmin = tk_wave_min(full ? mth : 0xFFFFu);
        const uint32_t wmax = 0xFFFFu - tk_wave_min(0xFFFFu - m1);
        const int wfull = __builtin_popcountll(__ballot(full));
        if ((t & 63) == 0) {
            sh.wave_min[t >> 6] = wmin;
            sh.wave_max[t >> 6] = wmax;
            sh.wave_tot[t >> 6] = wfull;
        }
    }

    // pass 1: the first histogram
    *reinterpret_cast<v4i_t*>(&sh.hist[TK_BPT * t]) = v4i_t{0, 0, 0, 0};
    if (t < (1 << TK_LO_BITS))
        sh.hist2[t] = 0u;
    if (t == 0) {
        sh.sel[0] = -1;
        sh.sel[1] = 0;
    }
    __syncthreads();
    if (resident) {
        uint32_t L = 0xFFFFu, M = 0u;
        int F = 0;
#pragma unroll
        for (int w = 0; w < TK_WAVES; w++) {
            L = min(L, sh.wave_min[w]);
            M = max(M, sh.wave_max[w]);
            F += sh.wave_tot[w];
        }
        if (m * F >= K)
            base = L;   // >= 1: a qualifying thread's m-th largest rank is a candidate's
        sb = 0;
        while (M >= base && ((M - base) >> sb) >= (uint32_t)TK_BINS)
            sb++;   // at most 4: ranks are below 2^16
        any = m1 >= base;
    }
    const uint32_t spare = TK_BINS + (t & 63);
    if (__ballot(any) != 0ull) {   // a wave with no rank in range has nothing to count
        for (int s0 = 0; s0 < s_end; s0 += TK_SPAN) {
            if (!resident)
                tk_keys(row, n, s0, kw);
#pragma unroll
            for (int e = 0; e < TK_OWN; e++) {
                const uint32_t k = (kw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                atomicAdd(&sh.hist[k >= base ? (k - base) >> sb : spare], 1u);
            }
        }
    }
    __syncthreads();
    // the threshold: v = 0 selects every candidate (fewer than K of them)
    uint32_t v = 0u;
    int c_gt = 0;
    tk_pick_bin(sh, K);   // ends with a barrier: wave_tot is free again
    const int b1 = sh.sel[0];
    if (b1 >= 0) {
        const int above = sh.sel[1];
        const uint32_t lo = base + ((uint32_t)b1 << sb);   // bin b1: ranks lo .. lo + 2^sb - 1
        v = lo;
        c_gt = above;
        if (sb > 0) {
            // pass 2: histogram of the ranks in bin b1 by their offset from lo (hist2 was
            // cleared with hist; a rank below lo wraps to a large offset)
            const uint32_t width = 1u << sb;
            for (int s0 = 0; s0 < s_end; s0 += TK_SPAN) {
                if (!resident)
                    tk_keys(row, n, s0, kw);
#pragma unroll
                for (int e = 0; e < TK_OWN; e++) {
                    const uint32_t k = (kw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    if (k - lo < width)
                        atomicAdd(&sh.hist2[k - lo], 1u);
                }
            }
            __syncthreads();
            // every thread finds the offset itself from the counts: the highest offset d whose
            // count together with those above it reaches K - above (bin b1's counts reach it)
            const int need = K - above;
            int cum = 0, d = 0, cum_d = 0;
#pragma unroll
            for (int q = (1 << TK_LO_BITS) / 4 - 1; q >= 0; q--) {
                const v4i_t h = *reinterpret_cast<const v4i_t*>(&sh.hist2[4 * q]);
#pragma unroll
                for (int i = 3; i >= 0; i--) {
                    const int c = __builtin_amdgcn_readfirstlane(h[i]);   // the same in every lane
                    if (cum < need && cum + c >= need) {
                        d = 4 * q + i;
                        cum_d = cum;
                    }
                    cum += c;
                }
            }
            v = lo + (uint32_t)d;
            c_gt = above + cum_d;
        }
    }
    // pass 3: the selected columns in order, remapped to cache rows
    int gt_run = 0, eq_run = 0;
    const int eq_room = K - c_gt;
    for (int s0 = 0; s0 < s_end; s0 += TK_SPAN) {
        if (!resident)
            tk_keys(row, n, s0, kw);
        // bit e of the masks: column e of this thread's part is above / equal to the threshold
        // (a rank equal to v is never 0: v = 0 only when every candidate is taken)
        static_assert(TK_OWN == 32, "one 32-bit mask per thread");
        uint32_t gm = 0u, em = 0u;
#pragma unroll
        for (int i = TK_KW - 1; i >= 0; i--)
            tk_mask_step(kw[i], v, gm, em);
        em = v != 0u ? em : 0u;
        // both prefix sums in one: the counts above the threshold in the low 16 bits, those equal
        // to it in the high 16 (each at most 32768 per span, so neither carries into the other)
        int tot;
        const int pre = tk_scan(__builtin_popcount(gm) | (__builtin_popcount(em) << 16), sh, tot);
        int pg = gt_run + (pre & 0xFFFF);
        int pe = eq_run + (pre >> 16);
        const int cbase = s0 + TK_OWN * t;
        for (uint32_t g = gm; g; g &= g - 1)   // in column order
            list[pg++] = cbase + __builtin_ctz(g);
        for (uint32_t q = em; q && pe < eq_room; q &= q - 1)
            list[c_gt + pe++] = cbase + __builtin_ctz(q);
        gt_run += tot & 0xFFFF;
        eq_run += tot >> 16;
        if (s0 + TK_SPAN < s_end)
            __syncthreads();   // the next span's scan rewrites wave_tot
    }
    const int count = b1 >= 0 ? K : gt_run;
    // the columns -> positions -> cache rows, each thread a strided share of the list (its writes
    // are the workgroup's, visible after the barrier)
    __syncthreads();
    // two entries per thread and round, both looked up before either is stored (the stores could
    // alias the tables for all the compiler knows, which would serialize the lookups)
    const TkRowMap rm = tk_row_map(remap, r);
    for (int i = t; i < K; i += 2 * TK_THREADS) {
        const int i2 = i + TK_THREADS;
        const int32_t a = i < count ? tk_remap(remap, rm, list[i]) : -1;
        const int32_t b = i2 < count ? tk_remap(remap, rm, list[i2]) : -1;
        out[i] = a;
        if (i2 < K)
            out[i2] = b;
    }
    if (t == 0)
        valid_out[r] = count;
}

// ---- candidate blocks -> sparse block ids --------------------------------------------------------
// vllm.model_executor.kernels.attention.dsa.sparse_mqa_logits, _expand_candidates_kernel and
// candidate_blocks_to_sparse_indices: per row, candidate c (in units of candidate_block_size
// positions) stands for sparse blocks c (ratio 1) or 2c, 2c + 1 (ratio 2, in that order); the blocks
// inside the row's K range [ks, ke) (0 <= b < ceil(max(ke - ks, 0) / sbk)) come out ascending and
// anchored at floor(ks / sbk), the rest of the row repeats the last one (or holds the anchor when
// none is valid); end = the valid sparse-token columns, every valid block full but the last, which
// holds min(max(ke - (last * sbk + ks), 1), sbk).
//
// One workgroup per row: the row's K * ratio block ids, invalid ones as INT32_MAX, sorted
// ascending by a bitonic sort in LDS (padded to a power of two, at most EX_MAX), then written out.
constexpr int EX_THREADS = 256;
constexpr int EX_MAX = 16384;   // 64 KB of LDS

__global__ __launch_bounds__(EX_THREADS) void mla_expand_kernel(
    const int32_t* __restrict__ cand, int K, int ratio, const int32_t* __restrict__ row_ks,
    const int32_t* __restrict__ row_ke, int sbk, int npad, int32_t* __restrict__ si,
    int32_t* __restrict__ end)
{
    extern __shared__ int32_t ex_v[];
    __shared__ int ex_valid;
    const int r = blockIdx.x, t = threadIdx.x;
    const int64_t ks = row_ks[r], ke = row_ke[r];
    const int64_t kv_len = ke - ks > 0 ? ke - ks : 0;
    const int64_t max_block = (kv_len + sbk - 1) / sbk;
    const int S = K * ratio;
    if (t == 0)
        ex_valid = 0;
    __syncthreads();
    int nv = 0;
    for (int i = t; i < npad; i += EX_THREADS) {
        int32_t v = 0x7FFFFFFF;
        if (i < S) {
            const int64_t c = cand[(int64_t)r * K + i / ratio];
            const int64_t b = ratio == 2 ? 2 * c + (i & 1) : c;
            if (b >= 0 && b < max_block) {
                v = (int32_t)b;
                nv++;
            }
        }
        ex_v[i] = v;
    }
    atomicAdd(&ex_valid, nv);
    // bitonic sort, ascending: stage (k, j) compares element i with i ^ j
    for (int k = 2; k <= npad; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            __syncthreads();
            for (int i = t; i < npad; i += EX_THREADS) {
                const int p = i ^ j;
                if (p > i) {
                    const int32_t a = ex_v[i], b = ex_v[p];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        ex_v[i] = b;
                        ex_v[p] = a;
                    }
                }
            }
        }
    }
    __syncthreads();
    const int n = ex_valid;
    const int64_t base = tk_floor_div(ks, sbk);
    const int64_t last = n > 0 ? ex_v[n - 1] : -1;
    const int32_t pad = (int32_t)(n > 0 ? last + base : base);
    for (int i = t; i < S; i += EX_THREADS)
        si[(int64_t)r * S + i] = i < n ? (int32_t)(ex_v[i] + base) : pad;
    if (t == 0) {
        int64_t e = 0;
        if (n > 0) {
            const int64_t fill = ke - (last * sbk + ks);
            e = (int64_t)(n - 1) * sbk + (fill < 1 ? 1 : (fill > sbk ? sbk : fill));
        }
        end[r] = (int32_t)e;
    }
}

bool tk_aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

mla_status_t mla_topk_rows(const void* logits, const int32_t* row_ends, int R, int N, int K,
                           const int32_t* block_table, int max_pages, int page_size, int Q,
                           int64_t num_rows, int32_t* rows_out, int32_t* valid_out, void* stream)
{
    return mla_topk_sparse_rows(logits, row_ends, R, N, K, nullptr, block_table, max_pages,
                                page_size, Q, num_rows, rows_out, valid_out, stream);
}

mla_status_t mla_topk_sparse_rows(const void* logits, const int32_t* end, int R, int N, int K,
                                  const mla_sparse_cols_t* cols, const int32_t* block_table,
                                  int max_pages, int page_size, int Q, int64_t num_rows,
                                  int32_t* rows_out, int32_t* valid_out, void* stream)
{
    // N below 2^31 - 32768: column arithmetic of the last span stays inside int
    if (R < 0 || N < 8 || N % 8 != 0 || N > 0x7FFFFFFF - TK_SPAN || K < 1 || Q < 1)
        return MLA_ERR_SHAPE;
    if (block_table && (max_pages < 1 || page_size < 1 || num_rows < 0 ||
                        (int64_t)max_pages * page_size > 0x7FFFFFFF))
        return MLA_ERR_SHAPE;
    if (cols && (cols->sparse_block_kv < 1 || cols->S < 1 ||
                 (int64_t)cols->S * cols->sparse_block_kv < N))
        return MLA_ERR_SHAPE;
    if (R == 0)
        return MLA_OK;
    if (!logits || !end || !rows_out || !valid_out || (cols && (!cols->sparse_indices || !cols->row_ks)))
        return MLA_ERR_NULL;
    if (!tk_aligned(logits, 16) || !tk_aligned(end, 4) || !tk_aligned(rows_out, 4) ||
        !tk_aligned(valid_out, 4) || !tk_aligned(block_table, 4) ||
        (cols && (!tk_aligned(cols->sparse_indices, 4) || !tk_aligned(cols->row_ks, 4))))
        return MLA_ERR_ALIGN;
    TkRemap m{};
    if (cols) {
        m.si = cols->sparse_indices;
        m.S = cols->S;
        m.sbk = cols->sparse_block_kv;
        m.sdiv = tk_division(m.sbk);
        m.ks = cols->row_ks;
    }
    m.table = block_table;
    m.max_pages = max_pages;
    m.page_size = page_size;
    if (block_table)
        m.pdiv = tk_division(page_size);
    m.Q = Q;
    m.num_rows = num_rows;
    auto kern = K <= TK_LDS_K ? (N <= TK_SPAN ? mla_topk_kernel<true, true> : mla_topk_kernel<true, false>)
                              : (N <= TK_SPAN ? mla_topk_kernel<false, true> : mla_topk_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)R), dim3(TK_THREADS), 0, (hipStream_t)stream,
                       (const uint16_t*)logits, end, N, K, m, rows_out, valid_out);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status_t mla_expand_candidates(const int32_t* candidate_blocks, int rows, int K,
                                   const int32_t* row_ks, const int32_t* row_ke,
                                   int candidate_block_size, int sparse_block_kv,
                                   int32_t* sparse_indices, int32_t* end, void* stream)
{
    if (rows < 0 || K < 1 || sparse_block_kv < 1 || candidate_block_size < 1)
        return MLA_ERR_SHAPE;
    const int ratio = candidate_block_size / sparse_block_kv;
    if ((ratio != 1 && ratio != 2) || ratio * sparse_block_kv != candidate_block_size ||
        (int64_t)K * ratio > EX_MAX)
        return MLA_ERR_SHAPE;
    if (rows == 0)
        return MLA_OK;
    if (!candidate_blocks || !row_ks || !row_ke || !sparse_indices || !end)
        return MLA_ERR_NULL;
    if (!tk_aligned(candidate_blocks, 4) || !tk_aligned(row_ks, 4) || !tk_aligned(row_ke, 4) ||
        !tk_aligned(sparse_indices, 4) || !tk_aligned(end, 4))
        return MLA_ERR_ALIGN;
    const int S = K * ratio;
    int npad = 64;
    while (npad < S)
        npad *= 2;
    hipLaunchKernelGGL(mla_expand_kernel, dim3((unsigned)rows), dim3(EX_THREADS),
                       (size_t)npad * sizeof(int32_t), (hipStream_t)stream, candidate_blocks, K,
                       ratio, row_ks, row_ke, sparse_block_kv, npad, sparse_indices, end);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

}  // extern "C"
