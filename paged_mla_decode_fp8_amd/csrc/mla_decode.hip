// mla_decode.hip -- MLA decode attention over an FP8 E4M3 latent cache for MI355X (gfx950).
//
// One kernel serves the dense (paged block table) and the sparse (top-k row list) forms. The
// arithmetic follows the vLLM API pages:
//   * vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.attn_sparse, module docstring and
//     SparseDcpDecode.kernel / .merge: key split per = ceil(n / S); per chunk the running maximum in
//     log2 units, P = 448 * exp2(x - max) rounded to E4M3 (round to nearest even, saturating), row sums
//     of the unrounded P, rescaling of O and l when the maximum rises; the FP32 merge of the splits in
//     split order; o = BF16(O * k_scale / l), LSE = (max - log2 448 + log2 l) * ln 2; empty rows give
//     o = 0, LSE = -inf.
//   * vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_attn, module docstring and its
//     helper index (q_split, lds_dma, sig, tr_read, mfma_f8): the causal bound of verify rows; the
//     bf16 query split into exact E4M3 hi + lo of q * 2^k; K rows moved into LDS by global_load_lds
//     one block ahead into one of two slots; S^T = K Q^T by 16x16x128 FP8 MFMAs with the K order
//     permuted alike in both operands; V^T read by ds_read_b64_tr_b8; a split's workgroups kept on
//     one XCD.
//   * vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.attention.attn2, module docstring: a
//     cross-workgroup merge through a global workspace with a per-row arrival counter (the last
//     arriver merges in a fixed order and resets the counter), so results do not depend on timing.
//
// Workgroup = (key group, split, set of T 16-row tiles), 512 threads = 8 waves, two per SIMD,
// specialised as on the AMD page (QK waves and PV waves). Wave i runs on SIMD i % 4:
//   QK waves 0..3: wave w owns key half w % 2 (64 of the block's 128 keys) of tile pair w / 2.
//          Per 128-key block: S^T of its 64 keys x 16 rows of both tiles by 9 16x16x128 MFMAs per
//          16-key subtile and tile (4 latent steps x {hi, lo} + 1 rope step packing rope hi | rope lo
//          against rope | rope), each K fragment streamed from LDS through a register ring and used
//          for both tiles; then the softmax inside the wave: block maximum (exchanged with the
//          other key half through LDS), running max, P = 448 exp2(x - max) -> E4M3 into LDS, row
//          sums of the unrounded P in a fixed order, rescale factor to LDS; then, in the time the
//          PV waves still need before the next barrier, the row pointers and presence bits of
//          block i + 2 for PV wave 4 + w (its 32 keys of the block), into that block's table.
//   PV waves 4..7: wave 4 + c owns latent columns 128c..128c+127 of every tile. They run one block
//          behind: after issuing the gather of block i + 1 (raw indices DMA'd into LDS three blocks
//          ahead, row pointers from the block's LDS table, 18 row DMAs per wave into the other LDS
//          slot) they take O^T += V^T P^T of block i - 1, whose MFMAs share each SIMD's
//          matrix pipe with the QK wave's MFMAs of block i; then they copy block i's V^T
//          (ds_read_b64_tr_b8) into registers while its slot is valid, so two slots suffice.
// Two barriers per block: B1 "block i landed; P and the rescale factors of block i - 1 published",
// B2 "both key halves' maxima of block i published; the PV waves hold P of block i - 1" (the QK
// waves then run the softmax of block i and write its P, the PV waves copy V^T of block i).
//
// LDS slot layout (73728 B = 8 subtiles x 9216 B). Within a 16-key subtile, the 16-byte unit of
// key k and latent chunk c (c < 32) sits at unit 32 k + (c ^ k), and rope chunk c (32..35) at
// unit 512 + 16 (c - 32) + k. A latent DMA instruction then moves two keys x 512 contiguous bytes
// (whole cache lines), and the XOR keeps both the QK operand read (16 keys x one chunk) and the
// transposed V read (8 keys x 16 columns) free of bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mla_decode.h"

namespace {

constexpr int ROW = 576;
constexpr int LATENT = 512;
constexpr int BLK = 128;             // keys per block
constexpr int NSUB = 8;              // 16-key subtiles per block
constexpr int WAVES = 8;
constexpr int THREADS = 512;
constexpr int SLOT = BLK * ROW;      // 73728
constexpr int SUBB = 16 * ROW;       // 9216
constexpr int PPITCH = 144;          // bytes per P row in LDS (128 keys + 16 pad)
constexpr int PTILE = 16 * PPITCH;   // 2304
constexpr float ANCHOR = 448.0f;
constexpr float LOG2_ANCHOR = 8.807354922057604f;  // log2(448)
constexpr float LN2 = 0.6931471805599453f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v2i lds_v2i;

struct Params {
    const uint16_t* q;
    const uint8_t* kv;
    int64_t num_rows;
    int page_size;
    uint32_t pg_magic;   // n / page_size = (t + ((n - t) >> pg_s1)) >> pg_s2, t = umulhi(n, pg_magic)
    int pg_s1, pg_s2;
    const int32_t* table;
    int max_pages;
    const int32_t* seq_lens;
    const int32_t* rows;
    int K;
    const int32_t* valid;
    float scale_log2;   // scale * k_scale * log2(e)
    float k_scale;
    int Q, H;
    int S;               // uniform plan: splits per key group; balanced plan: pieces
    int balanced;
    int groups;          // dense: B, sparse: B * Q
    int rows_per_group;  // dense: Q * H, sparse: H
    int tilesets;        // (rows_per_group / 16) / T
    int units;           // uniform: groups * S (group, split) pairs; balanced: S pieces
    uint16_t* o;
    float* lse;
    float* ws_o;         // [partial slot][T * 16 rows][512]
    float* ws_ml;        // [partial slot][T * 16 rows][2]
    uint32_t* ws_cnt;    // [groups * tilesets]
};

// Source of the absent keys' DMA: 576 zero bytes (V rows of absent keys must be 0, not garbage,
// since 0 * NaN would poison the PV sum).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[ROW];

template <int T, bool PS = false>
struct Smem {
    static constexpr int OFF_KV = 0;
    static constexpr int OFF_P = 2 * SLOT;                     // E4M3 P [T][16][PPITCH]
    static constexpr int OFF_ALPHA = OFF_P + T * PTILE;        // float [T*16]
    static constexpr int OFF_FM = OFF_ALPHA + T * 16 * 4;      // float [T*16]
    static constexpr int OFF_FL = OFF_FM + T * 16 * 4;         // float [4][T*16] (32-key parts)
    static constexpr int OFF_XMAX = OFF_FL + 4 * T * 16 * 4;   // float [4][T*16] block maxima per QK wave
    static constexpr int OFF_KMASK = OFF_XMAX + 4 * T * 16 * 4; // uint32 [4][4] key presence bits
    static constexpr int OFF_IDX = OFF_KMASK + 4 * 16;         // int32 [2][BLK] raw key indices
    static constexpr int OFF_PTAB = OFF_IDX + 2 * BLK * 4;     // uint64 [2 block parities][4 waves][32] key pointers
    static constexpr int OFF_MISC = OFF_PTAB + 2 * 4 * 32 * 8; // int [4]
    // E4M3 P lo [T][16][PPITCH] when P goes to PV as hi + lo (after everything else, so that the
    // other offsets do not depend on it)
    static constexpr int OFF_PLO = (OFF_MISC + 16 + 15) / 16 * 16;
    static constexpr int BYTES = PS ? OFF_PLO + T * PTILE : OFF_MISC + 16;
};
static_assert(Smem<4>::BYTES <= 163840, "LDS budget");
static_assert(Smem<2, true>::BYTES <= 163840, "LDS budget (P hi + lo, at most two tiles)");
static_assert(Smem<4, true>::BYTES > 163840, "four tiles with P hi + lo would fit: allow them");

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Two floats -> two BF16 codes (a in the low half), round to nearest even: gfx950's packed
// conversion, one instruction for both (checked on MI355X against (u + 0x7FFF + lsb) >> 16 on every
// non-NaN FP32 bit pattern, denormals and infinities included: no difference).
__device__ inline uint32_t pack_bf16(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

// Four floats (|x| <= 448 after the clamp) -> one dword of four E4M3 codes, RNE, saturating.
__device__ inline uint32_t pack_e4m3(float a, float b, float c, float d)
{
    a = fminf(fmaxf(a, -ANCHOR), ANCHOR);
    b = fminf(fmaxf(b, -ANCHOR), ANCHOR);
    c = fminf(fmaxf(c, -ANCHOR), ANCHOR);
    d = fminf(fmaxf(d, -ANCHOR), ANCHOR);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// x unchanged, but opaque to the optimizer: values derived from it at a use site are computed
// there instead of being hoisted out of loops and kept live (or spilled) across them.
__device__ inline int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// This lane's index in the wave, computed afresh (mbcnt) where it is used. In the gather loop any
// scratch reload would wait (vmcnt is in order) for the row DMAs issued before it, so lane-derived
// values there are recomputed rather than held live where the compiler might spill them.
__device__ inline int lane_now()
{
    return opaque((int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
}

// x / y from r = 1 / y (rounded): the product x r, then one correction with its exactly computed
// residual x - q y (fma). Exact whenever x / y is representable (a single key's O / l = v), and
// within an ulp otherwise; three operations instead of a full division per element.
__device__ inline float div_by(float x, float y, float r)
{
    const float q = x * r;
    return fmaf(fmaf(-q, y, x), r, q);
}

__device__ inline v8i cat(v4i a, v4i b) { return v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}; }

__device__ inline v4i lds_read16(const uint8_t* smem, int off)
{
    return *reinterpret_cast<const v4i*>(smem + off);
}

__device__ inline v4f mfma(v8i a, v8i b, v4f c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Workgroup barrier for this wave's LDS reads and writes only. __syncthreads() (and an LDS fence)
// would also wait for the outstanding global_load_lds of the next block, which must stay in flight
// across the barriers of the current block; the caller waits for it explicitly (vmcnt) when it
// needs the data. The memory clobber keeps the compiler from moving memory accesses across.
__device__ inline void lds_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one MFMA row / column held in the four
// k-groups), with gfx950's row-swap permutes: after a 32-lane swap each half holds the other
// half's value, after a 16-lane swap each 16-lane row the neighbouring row's. Every lane ends with
// the same value, combined in the same order.
__device__ inline float wave_max16(float v)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline float wave_sum16(float v)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The 32-bit LDS address of a pointer into __shared__ memory (wave-uniform by construction).
__device__ inline uint32_t lds_addr(const uint8_t* ptr)
{
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ptr);
}

// One global_load_lds_dwordx4: 16 bytes at this lane's gsrc -> LDS byte lds_base + 16 * lane.
// Written in asm so that the compiler's wait-count pass does not treat every later LDS read as
// depending on this DMA (it would wait for the next block's DMA before reading the current one);
// the kernel waits for its DMAs itself (vmcnt(0)) before the barrier that publishes a block. M0
// is saved and restored.
__device__ inline void dma16(const uint8_t* gsrc, uint32_t lds_base)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(gsrc)
        : "memory");
}

// Nine row DMAs into consecutive 1 KB LDS pieces: instruction i moves 16 bytes at this lane's
// src[i] to LDS byte lds_base + 1024 i + 16 lane. One asm block steps M0 itself, so all nine
// sources are computed before the first DMA issues and the DMAs go out back to back.
__device__ inline void dma9(const uint8_t* const (&src)[9], uint32_t lds_base)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %5, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %6, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %7, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %8, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %9, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %10, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(src[0]), "v"(src[1]), "v"(src[2]), "v"(src[3]), "v"(src[4]),
          "v"(src[5]), "v"(src[6]), "v"(src[7]), "v"(src[8])
        : "memory", "scc");
}

// One global_load_lds_dword: 4 bytes at this lane's gsrc -> LDS byte lds_base + 4 * lane (asm
// for the same reasons as dma16).
__device__ inline void dma4(const void* gsrc, uint32_t lds_base)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(gsrc)
        : "memory");
}

// n / page_size for n < 2^32 by a multiply with the divisor's precomputed magic number
// (Granlund and Montgomery, "Division by invariant integers using multiplication", 1994, the
// unsigned N-bit form of their Figure 4.1).
__device__ inline uint32_t page_div(const Params& p, uint32_t n)
{
    const uint32_t t = __umulhi(n, p.pg_magic);
    return (t + ((n - t) >> p.pg_s1)) >> p.pg_s2;
}

template <bool DENSE>
__device__ inline const int32_t* index_ptr(const Params& p, int g, int64_t jabs)
{
    if (DENSE)
        return p.table + (int64_t)g * p.max_pages + page_div(p, (uint32_t)jabs);
    return p.rows + (int64_t)g * p.K + jabs;
}

// The cache row of a key (or -1 when absent) from its raw index (page id or row id).
template <bool DENSE>
__device__ inline int64_t key_row(const Params& p, int64_t jabs, bool inrange, int32_t idx)
{
    int64_t row = -1;
    if (inrange) {
        if (DENSE) {
            if (idx >= 0)
                row = (int64_t)idx * p.page_size +
                      (int64_t)((uint32_t)jabs - page_div(p, (uint32_t)jabs) * (uint32_t)p.page_size);
        } else {
            row = idx;
        }
    }
    return (row >= 0 && row < p.num_rows) ? row : -1;
}

// One work item of a workgroup: tile set ts of key group g, the group's keys
// [first, first + mine) of n_grp, in nblk blocks of 128. The group's keys are divided among
// `count` items (one per split); count == 1 finishes the rows directly, otherwise the item leaves a
// partial in workspace slot `slot` and the last of the group's items to arrive merges them.
struct Work {
    int g, ts, nblk;
    int count;   // items (splits) of the group
    int slot;    // partial slot of this item (tile set folded in)
    int fp;      // balanced plan: the group's first piece
    int64_t n_grp, first, mine, row_base;
};

template <bool DENSE>
__device__ inline int64_t group_keys(const Params& p, int g)
{
    if (DENSE) {
        const int64_t cap = (int64_t)p.max_pages * p.page_size;
        const int64_t sl = p.seq_lens[g];
        return sl < 0 ? 0 : (sl > cap ? cap : sl);
    }
    const int64_t v = p.valid[g];
    return v < 0 ? 0 : (v > p.K ? p.K : v);
}

__device__ inline int64_t nblocks(int64_t n) { return (n + BLK - 1) / BLK; }

// Uniform plan (the pages' rule): unit = (split s, group g); the split holds keys
// [s per, min(n, (s + 1) per)) with per = ceil(n / S). n_known: the group's key count when the
// caller has already loaded it (else -1).
template <bool DENSE>
__device__ inline void decode_uniform(const Params& p, int unit, int ts, Work& w, int64_t n_known = -1)
{
    const int s = unit / p.groups;
    w.g = unit % p.groups;
    w.ts = ts;
    w.n_grp = n_known >= 0 ? n_known : group_keys<DENSE>(p, w.g);
    const int64_t per = (w.n_grp + p.S - 1) / p.S;
    w.first = (int64_t)s * per < w.n_grp ? (int64_t)s * per : w.n_grp;
    w.mine = (w.n_grp - w.first) < per ? (w.n_grp - w.first) : per;
    w.nblk = (int)nblocks(w.mine);
    w.count = p.S;
    w.fp = 0;
    w.slot = (w.g * p.S + s) * p.tilesets + ts;
    w.row_base = (int64_t)w.g * p.rows_per_group;
}

// Raw indices of the first two blocks and the group's key count, requested together: for split 0
// of a uniform plan the keys start at 0, so lanes 0..31 of PV wave pw load those of keys 32 pw + lane
// and 128 + 32 pw + lane that lie within the list's capacity (their count mask comes later). The
// parameters these loads need (and the first parameter line, which the gather reads next) are read
// in one batch, so that the loads wait for one round trip to the parameters instead of several.
struct FirstIdx {
    int32_t i0, i1;
    bool ok;
    int64_t n;   // the group's key count (clamped as group_keys does), or -1
};

template <bool DENSE>
__device__ inline FirstIdx first_indices(const Params& p, int unit, int pw)
{
    FirstIdx f{-1, -1, false, -1};
    const int bal = p.balanced, groups = p.groups;
    const int64_t cap = DENSE ? (int64_t)p.max_pages * p.page_size : (int64_t)p.K;
    const int32_t* cnt = DENSE ? p.seq_lens : p.valid;
    const int32_t* ibase = DENSE ? p.table : p.rows;
    const uint8_t* kv = p.kv;
    asm volatile("" ::"s"(bal), "s"(groups), "s"(cap), "s"(cnt), "s"(ibase), "s"(kv));
    if (bal || unit >= groups)
        return f;
    f.ok = true;
    const int g = unit;
    const int ln = lane_now();
    const int kk = 32 * pw + ln;
    if (ln < 32 && kk < cap)
        f.i0 = *index_ptr<DENSE>(p, g, kk);
    if (ln < 32 && BLK + kk < cap)
        f.i1 = *index_ptr<DENSE>(p, g, BLK + kk);
    const int64_t n = cnt[g];   // after the index loads, so that its wait covers them too
    f.n = n < 0 ? 0 : (n > cap ? cap : n);
    return f;
}

// Balanced plan: every group is a run of ITEM_BLOCKS + (its 128-key blocks) virtual blocks, the
// leading ITEM_BLOCKS standing for the fixed cost of a work item (query staging and conversion,
// pipeline fill, output); the runs, concatenated in group order (V virtual blocks), are cut into
// S pieces of equal size (piece q = [floor(q V / S), floor((q + 1) V / S))), one per workgroup
// (and tile set). A group's real blocks go to the pieces their virtual positions fall in, so a
// group is split where piece boundaries fall among its blocks. A piece walks the groups it overlaps
// from the last to the first: its part of the group it starts then comes in early, and the last
// part of a split group to finish more often finds every other part counted in before its epilogue
// (it then merges from LDS without storing its own partial). An empty group belongs to the piece
// holding the start of its run.
constexpr int ITEM_BLOCKS = 6;

struct Span {
    int g_lo, g_hi;   // the piece's groups
    int64_t pre_hi;   // virtual blocks before group g_hi (0 when the piece holds no group)
    int64_t V;        // virtual blocks of all groups
};

__device__ inline int piece_of(int64_t v, int64_t V, int np) { return (int)(((v + 1) * np - 1) / V); }

// The pieces holding the first and the last real block of a group whose run starts at virtual
// block pre (nb real blocks); an empty group: the piece holding the start of its run.
__device__ inline int first_piece(int64_t pre, int64_t nb, int64_t V, int np)
{
    return piece_of(nb > 0 ? pre + ITEM_BLOCKS : pre, V, np);
}

__device__ inline int last_piece(int64_t pre, int64_t nb, int64_t V, int np)
{
    return piece_of(nb > 0 ? pre + ITEM_BLOCKS + nb - 1 : pre, V, np);
}

__device__ inline int wave_sum_i32(int v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    return v;
}

// The piece's groups, by the whole workgroup: a block-wide prefix sum of the groups' run lengths
// into the (still unused) KV slots, then counts of the groups wholly before the piece and of the
// groups starting at or before it. The host bounds V below 2^31 and the groups by the slots' size.
// Contains workgroup barriers; every thread returns the same span.
template <bool DENSE>
__device__ Span piece_span(const Params& p, uint8_t* smem, int piece, int tid, int lane)
{
    const int G = p.groups;
    const int np = p.S;
    const int wave = tid >> 6;
    int32_t* pre = reinterpret_cast<int32_t*>(smem);                 // [G + 1]
    int32_t* red = reinterpret_cast<int32_t*>(smem + 2 * SLOT);      // [8] wave sums, [2] counts
    int carry = 0;
    for (int base = 0; base < G; base += THREADS) {
        const int g = base + tid;
        const int len = g < G ? ITEM_BLOCKS + (int)nblocks(group_keys<DENSE>(p, g)) : 0;
        int incl = len;   // inclusive prefix within the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d);
            if (lane >= d)
                incl += t;
        }
        if (lane == 63)
            red[wave] = incl;
        __syncthreads();
        int before = carry, chunk = 0;
#pragma unroll
        for (int k = 0; k < WAVES; k++) {
            const int v = red[k];
            before += k < wave ? v : 0;
            chunk += v;
        }
        if (g < G)
            pre[g] = before + incl - len;
        carry += chunk;
        __syncthreads();   // the wave sums are reused by the next chunk
    }
    const int V = carry;
    if (tid == 0) {
        pre[G] = V;
        red[8] = 0;
        red[9] = 0;
    }
    __syncthreads();
    int lo = 0, hi = 0;
    for (int g = tid; g < G; g += THREADS) {
        const int pg = pre[g];
        const int nb = pre[g + 1] - pg - ITEM_BLOCKS;
        lo += last_piece(pg, nb, V, np) < piece ? 1 : 0;
        hi += first_piece(pg, nb, V, np) <= piece ? 1 : 0;
    }
    lo = wave_sum_i32(lo);
    hi = wave_sum_i32(hi);
    if (lane == 0) {
        atomicAdd(&red[8], lo);
        atomicAdd(&red[9], hi);
    }
    __syncthreads();
    Span sp;
    sp.g_lo = __builtin_amdgcn_readfirstlane(red[8]);
    sp.g_hi = __builtin_amdgcn_readfirstlane(red[9]) - 1;
    sp.pre_hi = sp.g_hi >= sp.g_lo ? __builtin_amdgcn_readfirstlane(pre[sp.g_hi]) : 0;
    sp.V = V;
    __syncthreads();   // every wave has read the span before the slots fill
    return sp;
}

// Item of group g (whose run starts at virtual block pre) in piece `piece`.
template <bool DENSE>
__device__ inline void balanced_item(const Params& p, int piece, int ts, int g, int64_t pre,
                                     const Span& sp, Work& w)
{
    const int np = p.S;
    w.g = g;
    w.ts = ts;
    w.n_grp = group_keys<DENSE>(p, g);
    const int64_t nb = nblocks(w.n_grp);
    const int fp = first_piece(pre, nb, sp.V, np);
    const int lp = last_piece(pre, nb, sp.V, np);
    int64_t lo = 0, hi = 0;
    if (nb > 0) {
        const int64_t b0 = pre + ITEM_BLOCKS;   // virtual position of the group's first block
        const int64_t a0 = (int64_t)piece * sp.V / np, a1 = (int64_t)(piece + 1) * sp.V / np;
        lo = (a0 > b0 ? a0 : b0) - b0;
        hi = (a1 < b0 + nb ? a1 : b0 + nb) - b0;
        if (lo > nb)
            lo = nb;
        if (hi < lo)
            hi = lo;
    }
    w.first = lo * BLK;
    const int64_t end = hi * BLK < w.n_grp ? hi * BLK : w.n_grp;
    w.mine = end > w.first ? end - w.first : 0;
    w.nblk = (int)(hi - lo);
    w.count = lp - fp + 1;
    w.fp = fp;
    w.slot = (2 * piece + (piece == fp ? 1 : 0)) * p.tilesets + ts;
    w.row_base = (int64_t)g * p.rows_per_group;
}

// Partial slot of the c-th item (split) of the work item's group.
__device__ inline int contributor_slot(const Params& p, const Work& w, int c)
{
    const int unit = p.balanced ? 2 * (w.fp + c) + (c == 0 ? 1 : 0) : w.g * p.S + c;
    return unit * p.tilesets + w.ts;
}

// A slot's partial O (T * 16 rows x 512 columns, FP32) is kept in the PV accumulators' own order,
// [column quarter pw][tile t][column block c][lane][4]: element (row 16 t + lane % 16, column
// 128 pw + 16 c + 4 (lane / 16) + e). Each store of a PV wave and each load of the merge then
// moves 1 KB of contiguous memory. Offset in floats.
template <int T>
__device__ inline int64_t partial_o_offset(int slot, int pw, int t, int c, int lane)
{
    return ((((int64_t)slot * 4 + pw) * T + t) * 8 + c) * 256 + 4 * lane;
}

// Where an item found last before its epilogue keeps its own (m, l) rows in LDS: right after its O
// partial (both in the KV slots, free once the block loop is done). Offset in floats.
template <int T>
__device__ constexpr int own_ml_offset() { return 4 * T * 8 * 256; }
static_assert((own_ml_offset<4>() + 4 * 16 * 2) * 4 <= 2 * SLOT, "own partial fits the KV slots");

// Q staging: the tile set's T * 16 query rows (bf16, 1152 B each, from row row0 of q) are DMA'd by
// the QK waves into KV slot 1, which stays free until iteration 0 issues the DMA of block 1. LDS
// unit (16 bytes) 72 r + c of row r holds the row's unit c ^ s(r) for the latent units c < 64,
// s(r) = (r / 2) % 4, and unit c for the rope units 64..71.
template <int T>
__device__ inline void stage_q(const Params& p, uint8_t* smem, int64_t row0, int qw, int lane)
{
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(p.q + row0 * ROW);
    for (int i = qw; i < T * 18; i += 4) {   // 64 units per instruction, T * 16 * 72 units
        const int u = 64 * i + lane;
        const int r = u / 72, c = u - 72 * r;
        const int src = c < 64 ? (c ^ ((r >> 1) & 3)) : c;
        dma16(qbase + (int64_t)r * (2 * ROW) + 16 * src, lds_addr(smem + SLOT + 1024 * i));
    }
}

// The power of two of a query row: the largest k with max|q| 2^k <= 448 (0 for a zero row), at most
// 126 so that 2^-k stays a normal float (a row whose entries are all below 2^-117 keeps fewer bits).
__device__ inline int row_shift(float amax)
{
    if (!(amax > 0.f))
        return 0;
    int e;
    const float mm = frexpf(amax, &e);   // amax = mm * 2^e, mm in [0.5, 1)
    const int k = (2.f * mm <= 1.75f) ? (9 - e) : (8 - e);
    return k < 126 ? k : 126;
}

// Maximum over each aligned group of N lanes (N = 4, 8, 16 or 32; every lane of a group gets it):
// quad swaps (4), the half-row mirror (8), the row mirror (16), the 16-lane row swap (32).
template <int N>
__device__ inline float group_max(float v)
{
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true)));
    if (N >= 8)
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true)));
    if (N >= 16)
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true)));
    if (N >= 32) {
        auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
    }
    return v;
}

// The exact E4M3 split of one 16-byte unit (8 bf16 query values) of a row whose power of two is
// 2^k (sinv = 2^-k): hi = E4M3(q 2^k), lo = E4M3(q 2^k - hi) (|q 2^k| <= 448 and |q 2^k - hi| <=
// 16, so neither rounding saturates), as {hi of values 0..3, hi of 4..7, lo of 0..3, lo of 4..7}.
// gfx950's scaled conversions: bf16 / f32 -> E4M3 computes RNE(x / s) and E4M3 -> f32 computes
// v * s (both exact for a power of two s; checked bit for bit against the plain conversions of
// x / s and v * s on MI355X): hi, its value in q units hi 2^-k, the exact remainder
// d = q - hi 2^-k and lo = E4M3(d 2^k). QE: the E4M3 query, lo = 0.
template <bool QE>
__device__ __forceinline__ v4i split_unit(const v4i raw, float sinv)
{
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint32_t qa = (uint32_t)raw[2 * h], qb = (uint32_t)raw[2 * h + 1];   // q 4h .. 4h + 3
        v2s hw = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v2s{0, 0}, __builtin_bit_cast(v2bf, qa), sinv, false);
        hw = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw, __builtin_bit_cast(v2bf, qb), sinv, true);
        hi[h] = __builtin_bit_cast(uint32_t, hw);
        const v2f b01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)hi[h], sinv, false);
        const v2f b23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)hi[h], sinv, true);
        const float d0 = bf16_to_f32(qa & 0xFFFF) - b01.x, d1 = bf16_to_f32(qa >> 16) - b01.y;
        const float d2 = bf16_to_f32(qb & 0xFFFF) - b23.x, d3 = bf16_to_f32(qb >> 16) - b23.y;
        v2s lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, d0, d1, sinv, false);
        lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw, d2, d3, sinv, true);
        lo[h] = QE ? 0u : __builtin_bit_cast(uint32_t, lw);
    }
    return v4i{(int)hi[0], (int)hi[1], (int)lo[0], (int)lo[1]};
}

// Unit c (values 8 c .. 8 c + 7) of tile-set row r, split, into the QK waves' MFMA B operands at
// qop: [tile][operand][lane][32 B], operands 0..3 the hi steps, 4..7 the lo steps, 8 the rope
// step (k-groups 0, 1 carry hi, 2, 3 lo).
__device__ __forceinline__ void store_unit(uint8_t* qop, int r, int c, const v4i hl)
{
    const int t = r >> 4, n16 = r & 15;
    const int v0 = 8 * c;
    int op_hi, op_lo, lane_hi, lane_lo, wi;
    if (v0 < LATENT) {   // latent step st, k-group g: byte v0 % 32 of that lane's operand
        const int st = v0 >> 7, g = (v0 >> 5) & 3;
        op_hi = st;
        op_lo = 4 + st;
        lane_hi = lane_lo = n16 + 16 * g;
        wi = v0 & 31;
    } else {             // rope half: hi in k-group half, lo in k-group 2 + half
        const int half = (v0 - LATENT) >> 5;
        op_hi = op_lo = 8;
        lane_hi = n16 + 16 * half;
        lane_lo = n16 + 16 * (2 + half);
        wi = (v0 - LATENT) & 31;
    }
    *reinterpret_cast<v2i*>(qop + ((t * 9 + op_hi) * 64 + lane_hi) * 32 + wi) = v2i{hl[0], hl[1]};
    *reinterpret_cast<v2i*>(qop + ((t * 9 + op_lo) * 64 + lane_lo) * 32 + wi) = v2i{hl[2], hl[3]};
}

// The staged query rows -> the QK waves' MFMA B operands, by all 512 threads: per row the power
// of two 2^k with max |q 2^k| <= 448 (k the largest such integer, 0 for a zero row), then the
// exact E4M3 split hi = E4M3(q 2^k), lo = E4M3(q 2^k - hi) (|q 2^k| <= 448 and |q 2^k - hi| <= 16,
// so neither rounding saturates). LPR = 32 / T consecutive lanes (inside one wave) share a row:
// lane li of the group takes the row's 16-byte units li, li + LPR, .. (8 bf16 each), so the row
// maximum is a reduction inside the lane group. The operands replace the rows in slot 1:
// [tile][operand][lane][32 B], operands 0..3 the hi steps, 4..7 the lo steps, 8 the rope step
// (k-groups 0, 1 carry hi, 2, 3 lo); the row maxima go to the P area (free until the first P) for
// the row scales. Two workgroup barriers. QE: the E4M3 query, hi alone (lo = 0).
template <int T, bool QE>
__device__ __forceinline__ void convert_q(uint8_t* smem, int tid)
{
    using L = Smem<T>;
    constexpr int LPR = 32 / T;                  // lanes per row
    constexpr int UPL = (72 + LPR - 1) / LPR;    // units per lane
    const int r = tid / LPR, li = tid % LPR;     // row of the tile set, lane in the row's group
    const int sw = (r >> 1) & 3;                 // the staged row's unit swizzle
    v4i raw[UPL];
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < UPL; k++) {
        const int c = li + LPR * k;
        raw[k] = v4i{0, 0, 0, 0};
        if (c < 72) {
            raw[k] = *reinterpret_cast<const v4i*>(smem + SLOT + 16 * (72 * r + (c < 64 ? c ^ sw : c)));
#pragma unroll
            for (int d = 0; d < 4; d++) {
                m = fmaxf(m, fabsf(bf16_to_f32((uint32_t)raw[k][d] & 0xFFFF)));
                m = fmaxf(m, fabsf(bf16_to_f32((uint32_t)raw[k][d] >> 16)));
            }
        }
    }
    m = group_max<LPR>(m);
    if (li == 0)
        reinterpret_cast<float*>(smem + L::OFF_P)[r] = m;
    // gfx950's scaled conversions: bf16 / f32 -> E4M3 computes RNE(x / s) and E4M3 -> f32 computes
    // v * s (both exact for a power of two s; checked bit for bit against the plain conversions of
    // x / s and v * s on MI355X). With s = 2^-k: hi = E4M3(q 2^k), its value in q units hi 2^-k,
    // the exact remainder d = q - hi 2^-k and lo = E4M3(d 2^k).
    const float sinv = ldexpf(1.f, -row_shift(m));
#pragma unroll
    for (int k = 0; k < UPL; k++) {
        uint32_t hi[2], lo[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const uint32_t qa = (uint32_t)raw[k][2 * h], qb = (uint32_t)raw[k][2 * h + 1];   // q 4h .. 4h + 3
            v2s hw = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v2s{0, 0}, __builtin_bit_cast(v2bf, qa), sinv, false);
            hw = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw, __builtin_bit_cast(v2bf, qb), sinv, true);
            hi[h] = __builtin_bit_cast(uint32_t, hw);
            const v2f b01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)hi[h], sinv, false);
            const v2f b23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)hi[h], sinv, true);
            const float d0 = bf16_to_f32(qa & 0xFFFF) - b01.x, d1 = bf16_to_f32(qa >> 16) - b01.y;
            const float d2 = bf16_to_f32(qb & 0xFFFF) - b23.x, d3 = bf16_to_f32(qb >> 16) - b23.y;
            v2s lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, d0, d1, sinv, false);
            lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw, d2, d3, sinv, true);
            lo[h] = QE ? 0u : __builtin_bit_cast(uint32_t, lw);
        }
        raw[k] = v4i{(int)hi[0], (int)hi[1], (int)lo[0], (int)lo[1]};
    }
    __syncthreads();   // every raw read of slot 1 has been made (the operands overwrite the rows)
    uint8_t* qop = smem + SLOT;
    const int t = r >> 4, n16 = r & 15;
#pragma unroll
    for (int k = 0; k < UPL; k++) {
        const int c = li + LPR * k;
        if (c >= 72)
            continue;
        // values 8 c .. 8 c + 7 of row r: tile t, row n16 of the tile
        const int v0 = 8 * c;
        int op_hi, op_lo, lane_hi, lane_lo, wi;
        if (v0 < LATENT) {   // latent step st, k-group g: byte v0 % 32 of that lane's operand
            const int st = v0 >> 7, g = (v0 >> 5) & 3;
            op_hi = st;
            op_lo = 4 + st;
            lane_hi = lane_lo = n16 + 16 * g;
            wi = v0 & 31;
        } else {             // rope half: hi in k-group half, lo in k-group 2 + half
            const int half = (v0 - LATENT) >> 5;
            op_hi = op_lo = 8;
            lane_hi = n16 + 16 * half;
            lane_lo = n16 + 16 * (2 + half);
            wi = (v0 - LATENT) & 31;
        }
        *reinterpret_cast<v2i*>(qop + ((t * 9 + op_hi) * 64 + lane_hi) * 32 + wi) = v2i{raw[k][0], raw[k][1]};
        *reinterpret_cast<v2i*>(qop + ((t * 9 + op_lo) * 64 + lane_lo) * 32 + wi) = v2i{raw[k][2], raw[k][3]};
    }
    __syncthreads();   // the operands and the row maxima are in LDS
}

// Each QK wave stages and converts a quarter of the tile set's rows itself, right as they land,
// while the PV waves issue block 0's row DMAs, with no workgroup barrier: QK wave qw owns rows
// RW qw .. RW qw + RW - 1 (RW = 4 T), staged at slot 1 + 1152 RW qw, unit c of its row rl at
// 16 (72 rl + c). With one or two tiles a wave's rows feed operands spread over the tile, so the
// operands go to slot 1 + 18432 T, after every staged row. With four tiles a wave's rows are tile
// qw, whose operands take exactly the bytes its rows were staged in: the wave reads all of them
// before it writes any, so it converts in place. Not for the dense four-tile kernel: there the
// 512-thread conversion after Q0 measured faster (its block loop's register allocation moves).
template <int T, bool DENSE>
constexpr bool OWN_Q = T <= 2 || !DENSE;
template <int T>
constexpr int OPBASE = T == 4 ? 0 : 18432 * T;   // the operands' offset in slot 1

template <int T>
__device__ inline void stage_q_own(const Params& p, uint8_t* smem, int64_t row0, int qw, int lane)
{
    constexpr int RW = 4 * T;
    constexpr int NU = RW * 72;                       // 16-byte units of the wave's rows
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(p.q + (row0 + RW * qw) * ROW);
    uint8_t* dst = smem + SLOT + 1152 * RW * qw;
#pragma unroll
    for (int i = 0; i < (NU + 63) / 64; i++) {        // 64 units per instruction (the last may be half)
        const int u = 64 * i + lane;
        if (u < NU) {
            const int rl = u / 72, c = u - 72 * rl;
            dma16(qbase + (int64_t)rl * (2 * ROW) + 16 * c, lds_addr(dst + 1024 * i));
        }
    }
}

template <int T, bool QE>
__device__ __forceinline__ void convert_q_own(uint8_t* smem, int qw, int lane)
{
    using L = Smem<T>;
    constexpr int RW = 4 * T;
    constexpr int LPR = 64 / RW;                      // lanes per row: 16, 8, 4 (one, two, four tiles)
    constexpr int UPL = (72 + LPR - 1) / LPR;         // units per lane: 5, 9, 18
    const int rl = lane / LPR, li = lane % LPR;
    const int r = RW * qw + rl;                       // row of the tile set
    const uint8_t* src = smem + SLOT + 1152 * r;      // the wave's rows follow one another
    v4i raw[UPL];
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < UPL; k++) {
        const int c = li + LPR * k;
        raw[k] = v4i{0, 0, 0, 0};
        if (c < 72) {
            raw[k] = *reinterpret_cast<const v4i*>(src + 16 * c);
#pragma unroll
            for (int d = 0; d < 4; d++) {
                m = fmaxf(m, fabsf(bf16_to_f32((uint32_t)raw[k][d] & 0xFFFF)));
                m = fmaxf(m, fabsf(bf16_to_f32((uint32_t)raw[k][d] >> 16)));
            }
        }
    }
    m = group_max<LPR>(m);
    if (li == 0)
        reinterpret_cast<float*>(smem + L::OFF_P)[r] = m;
    const float sinv = ldexpf(1.f, -row_shift(m));
#pragma unroll
    for (int k = 0; k < UPL; k++) {
        const int c = li + LPR * k;
        if (c < 72)
            store_unit(smem + SLOT + OPBASE<T>, r, c, split_unit<QE>(raw[k], sinv));
    }
}

// The nine row DMA sources of subtile 2 pw + h of a block, from PV wave pw's pointer table (entry
// 16 (k % 2) + 8 (k / 16) + (k % 16) / 2 holds key k of the wave's 32). Latent instruction i moves
// keys 16 h + 2 i (lanes 0..31) and 16 h + 2 i + 1 (lanes 32..63), chunk (lane % 32) ^ key; the
// rope instruction: key 16 h + lane % 16, chunk 32 + lane / 16.
__device__ inline void subtile_sources(const uint64_t* tab, int h, const uint8_t* (&src)[9])
{
    const int ln = lane_now();
    const int hb = ln >> 5;
    const uint32_t boff = 16u * (uint32_t)((ln & 31) ^ hb);   // 16 ((lane % 32) ^ key) ^ 32 i
    const uint64_t* row8 = tab + 16 * hb + 8 * h;             // the 8 keys of this lane's half
    uint64_t kp[8];
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const v4i two = *reinterpret_cast<const v4i*>(row8 + 2 * m);
        kp[2 * m] = ((uint64_t)(uint32_t)two.y << 32) | (uint32_t)two.x;
        kp[2 * m + 1] = ((uint64_t)(uint32_t)two.w << 32) | (uint32_t)two.z;
    }
    const int rk = ln & 15;   // rope key 16 h + rk
    const uint64_t rp = tab[16 * (rk & 1) + 8 * h + (rk >> 1)];
#pragma unroll
    for (int i = 0; i < 8; i++)
        src[i] = reinterpret_cast<const uint8_t*>(kp[i] + (boff ^ (32u * i)));
    src[8] = reinterpret_cast<const uint8_t*>(rp + 512 + 16 * (ln >> 4));
}

__device__ inline void issue_subtile(uint8_t* smem, const uint8_t* const (&src)[9], int blk, int pw, int h)
{
    dma9(src, lds_addr(smem + (blk & 1) * SLOT + (2 * pw + h) * SUBB));
}

// ---- QK waves: Q stage, S^T = K (hi + lo)^T, softmax; P and the rescale factors to LDS ----
// The QK waves share a tile pair's keys: T <= 2 (one pair of TW = T tiles): wave qw owns subtiles
// 2 qw, 2 qw + 1 of every block; T = 4 (two pairs): wave qw owns subtiles 4 (qw % 2) .. + 3 of
// pair qw / 2. Each K fragment read from LDS feeds the MFMAs of the pair's tiles. The waves of a
// pair exchange their block maxima through LDS (all then hold the same running maximum) and keep
// a row sum per 32-key part (subtiles 2 p, 2 p + 1), added in part order at the end, so results
// do not depend on T. QE: the E4M3 query (the hi operands alone; no lo MFMAs).
template <int T, bool DENSE, bool QE, bool PS>
__device__ __forceinline__ void qk_role(const Params& p, uint8_t* smem, const Work& w, int qw,
                                        int lane)
{
    using L = Smem<T>;
    constexpr int TW = T >= 2 ? 2 : 1;   // tiles per QK wave
    constexpr int KW = T >= 4 ? 2 : 4;    // QK waves per tile pair
    constexpr int KS = NSUB / KW;         // subtiles per QK wave
    constexpr int PPW = KS / 2;           // 32-key parts per QK wave
    const int n16 = lane & 15;   // MFMA row / column within 16
    const int grp = lane >> 4;   // MFMA k-group 0..3
    const int kq = qw % KW;      // key range: subtiles sub0 .. sub0 + KS - 1 of every block
    const int sub0 = KS * kq;
    const int qt0 = (qw / KW) * TW;   // first tile of the pair within the tile set
    const bool active = true;
    int lim[TW];   // keys [first, first + lim) of the item are visible to tile j (lim may be < 0)
#pragma unroll
    for (int j = 0; j < TW; j++) {
        int64_t c = w.n_grp;
        if (DENSE) {
            const int pos = (16 * (w.ts * T + qt0 + j)) / p.H;
            c = w.n_grp - p.Q + pos + 1;
            c = c < 0 ? 0 : (c > w.n_grp ? w.n_grp : c);
        }
        lim[j] = (int)(c - w.first);   // |c - first| <= n_grp < 2^31
    }

    __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0): this wave's staged Q rows landed
    if (OWN_Q<T, DENSE> && w.nblk > 0)
        convert_q_own<T, QE>(smem, qw, lane);
    lds_sync();                          // Q0: every staged row (or every operand) is in LDS
    if (!OWN_Q<T, DENSE> && w.nblk > 0)
        convert_q<T, QE>(smem, qw * 64 + lane);

    // ---- the tiles' B operands (exact E4M3 hi + lo of q * 2^k) and row scales from LDS ----
    v8i qhi[TW][4], qlo[TW][4], qrope[TW];
    float row_scale[TW];  // scale_log2 * 2^-k for row n16
#pragma unroll
    for (int j = 0; j < TW; j++) {
        row_scale[j] = 0.f;
        if (w.nblk > 0 && active) {
            const int t = qt0 + j;
            auto op = [&](int o) {
                const int off = SLOT + (OWN_Q<T, DENSE> ? OPBASE<T> : 0) + ((t * 9 + o) * 64 + lane) * 32;
                return cat(lds_read16(smem, off), lds_read16(smem, off + 16));
            };
#pragma unroll
            for (int st = 0; st < 4; st++) {
                qhi[j][st] = op(st);
                if (!QE)
                    qlo[j][st] = op(4 + st);
            }
            qrope[j] = op(8);
            const float am = __uint_as_float(reinterpret_cast<const uint32_t*>(smem + L::OFF_P)[16 * t + n16]);
            row_scale[j] = ldexpf(p.scale_log2, -row_shift(am));
        }
    }

    // This lane's LDS byte offset within a key half of a slot for its operand read of step st,
    // half h, subtile u: u * SUBB + koff. For the latent steps koff = 16 (32 n16 + ((8 st + 2 grp
    // + h) ^ n16)) = ka_h ^ (128 st), with ka_h = 512 n16 + 128 (n16 >> 3) + 16 ((2 grp + h) ^
    // (n16 & 7)) (the bits of 128 st meet only the 128 (n16 >> 3) term). Rope: 8192 + 256 (2 (grp
    // & 1) + h) + 16 n16.
    const float neg_inf = -INFINITY;
    float m_run[TW], l_run[TW][PPW];   // running max (log2 units), running sum per part, row n16
#pragma unroll
    for (int j = 0; j < TW; j++) {
        m_run[j] = neg_inf;
#pragma unroll
        for (int pp = 0; pp < PPW; pp++) l_run[j][pp] = 0.f;
    }
    float* xalpha = reinterpret_cast<float*>(smem + L::OFF_ALPHA);
    float* xmax = reinterpret_cast<float*>(smem + L::OFF_XMAX);   // [4 waves][T * 16] block maxima
    // The gather's pointer table of PV wave qw (keys 32 qw .. 32 qw + 31 of every block), built here
    // two blocks ahead: the row pointer of each key (the zero row when absent) and the presence word.
    const int32_t* idx_lds = reinterpret_cast<const int32_t*>(smem + L::OFF_IDX);
    uint64_t* ptabs = reinterpret_cast<uint64_t*>(smem + L::OFF_PTAB) + 32 * qw;   // block parity b: + 128 b
    uint64_t kv_base = (uint64_t)(uintptr_t)p.kv, zero_row = (uint64_t)(uintptr_t)g_zero_row;
    uint64_t ibase = (uint64_t)(uintptr_t)(DENSE ? p.table + (int64_t)w.g * p.max_pages : p.rows + (int64_t)w.g * p.K);
    int64_t nrows = p.num_rows;
    uint32_t psz = (uint32_t)p.page_size, pmag = p.pg_magic;
    int ps1 = p.pg_s1, ps2 = p.pg_s2;
    asm volatile("" : "+s"(kv_base), "+s"(zero_row), "+s"(ibase), "+s"(nrows), "+s"(psz), "+s"(pmag), "+s"(ps1), "+s"(ps2));
    auto pdiv = [&](uint32_t n) {
        const uint32_t t = __umulhi(n, pmag);
        return (t + ((n - t) >> ps1)) >> ps2;
    };
    auto key_ptrs_all = [&](int blk, int32_t idx) {
        const int ln = lane_now();
        const int kk = 32 * qw + (ln & 31);
        const int64_t left = w.mine - (int64_t)blk * BLK;
        const int64_t j = w.first + (int64_t)blk * BLK + kk;
        const int64_t rd = DENSE ? (int64_t)idx * psz + (int64_t)((uint32_t)j - pdiv((uint32_t)j) * psz) : (int64_t)idx;
        const bool ok = kk < left && idx >= 0 && rd < nrows;
        const uint32_t word = (uint32_t)__ballot(ok);
        *reinterpret_cast<uint32_t*>(smem + L::OFF_KMASK + (blk & 3) * 16 + 4 * qw) = word;
        ptabs[128 * (blk & 1) + 16 * (ln & 1) + 8 * ((ln >> 4) & 1) + ((ln & 15) >> 1)] = ok ? kv_base + (uint64_t)rd * ROW : zero_row;
    };

    // iteration i: QK and softmax of block i (the PV waves work on block i - 1)
    for (int i = 0; i <= w.nblk; i++) {
        const int slot = i & 1;
        lds_sync();   // B1: block i landed; P and the rescale factors of block i - 1 published
        const bool work = active && i < w.nblk;
        v4f acc[TW][KS];
        float bmax[TW];
        if (work) {
            // presence bits of the block's keys, read before the MFMAs so that the LDS latency
            // hides behind them; this lane's keys: bit 4u + jj <-> key 16 (sub0 + u) + 4 grp + jj
            const v4i mw = *reinterpret_cast<const v4i*>(smem + L::OFF_KMASK + (i & 3) * 16);
            const uint8_t* kslot = smem;
            // the lane's bases for this slot and key half, recomputed from the lane id here rather
            // than held in registers across the loop
            const int ln = lane_now(), r16 = ln & 15, g4 = ln >> 4;
            int kb0 = 512 * r16 + 128 * (r16 >> 3) + 16 * ((2 * g4) ^ (r16 & 7));
            int kb1 = 512 * r16 + 128 * (r16 >> 3) + 16 * ((2 * g4 + 1) ^ (r16 & 7));
            int kbr = 8192 + 256 * (2 * (g4 & 1)) + 16 * r16;
            const int soff = slot * SLOT + sub0 * SUBB;
            kb0 += soff;
            kb1 += soff;
            kbr += soff;
#pragma unroll
            for (int j = 0; j < TW; j++)
#pragma unroll
                for (int u = 0; u < KS; u++) acc[j][u] = v4f{0.f, 0.f, 0.f, 0.f};
            // Fragment f: step f / KS, subtile f % KS of this half. Step f issues the hi MFMAs of
            // fragment f (or its packed rope MFMAs) and the lo MFMAs of fragment f - 1, so no MFMA
            // waits on the one just issued; a fragment stays in the ring until its lo MFMAs.
            constexpr int NFRAG = 5 * KS;
            constexpr int AHEAD = 1, RING = AHEAD + 2;
            v8i kf[RING];
            auto load_frag = [&](int f) {
                const int st = f / KS, sub = f % KS;
                if (st < 4)
                    return cat(lds_read16(kslot, (kb0 ^ (128 * st)) + sub * SUBB),
                               lds_read16(kslot, (kb1 ^ (128 * st)) + sub * SUBB));
                return cat(lds_read16(kslot, kbr + sub * SUBB), lds_read16(kslot, kbr + 256 + sub * SUBB));
            };
#pragma unroll
            for (int f = 0; f < AHEAD; f++) kf[f % RING] = load_frag(f);
#pragma unroll
            for (int f = 0; f <= NFRAG; f++) {
                if (f + AHEAD < NFRAG)
                    kf[(f + AHEAD) % RING] = load_frag(f + AHEAD);
                if (f < NFRAG) {
                    const int st = f / KS, sub = f % KS;
#pragma unroll
                    for (int j = 0; j < TW; j++)
                        acc[j][sub] = mfma(kf[f % RING], st < 4 ? qhi[j][st] : qrope[j], acc[j][sub]);
                }
                if (!QE && f >= 1 && f - 1 < 4 * KS) {
                    const int st = (f - 1) / KS, sub = (f - 1) % KS;
#pragma unroll
                    for (int j = 0; j < TW; j++)
                        acc[j][sub] = mfma(kf[(f - 1) % RING], qlo[j][st], acc[j][sub]);
                }
            }
            // all of this wave's keys present (the words are the same in every lane; word k holds
            // subtiles 2 k, 2 k + 1) and the block wholly before the tiles' bounds: nothing to mask
            uint32_t all_in = ~0u;
#pragma unroll
            for (int k = 0; k < KS / 2; k++)
                all_in &= (uint32_t)__builtin_amdgcn_readfirstlane(mw[sub0 / 2 + k]);
            // ---- mask, this half's block maxima (in-lane, then across the 4 k-groups), to LDS.
            // The row scale is positive, so max(s * scale) = scale * max(s) exactly. ----
#pragma unroll
            for (int j = 0; j < TW; j++) {
                const int lr = lim[j] - i * BLK;      // keys of the block before the tile's bound
                if (!(all_in == 0xFFFFFFFFu && lr >= BLK)) {
                    uint32_t vis = 0;
#pragma unroll
                    for (int u = 0; u < KS; u++) {
                        // subtile sub0 + u: word (sub0 + u) / 2 of the block, half u % 2
                        vis |= (((uint32_t)mw[(sub0 + u) >> 1] >> (16 * (u & 1) + 4 * grp)) & 0xFu) << (4 * u);
                    }
                    const int lim_rel = lr < 0 ? 0 : (lr > BLK ? BLK : (int)lr);
#pragma unroll
                    for (int u = 0; u < KS; u++) {
                        const int keep = lim_rel - (16 * (sub0 + u) + 4 * grp);   // of the 4 in bound
                        const uint32_t nib = keep >= 4 ? 0xFu : (keep <= 0 ? 0u : ((1u << keep) - 1u));
                        vis &= ~(0xFu << (4 * u)) | (nib << (4 * u));
                    }
#pragma unroll
                    for (int u = 0; u < KS; u++)
#pragma unroll
                        for (int jj = 0; jj < 4; jj++)
                            acc[j][u][jj] = ((vis >> (4 * u + jj)) & 1u) ? acc[j][u][jj] : neg_inf;
                }
                float bm = neg_inf;
#pragma unroll
                for (int u = 0; u < KS; u++)
                    bm = fmaxf(bm, fmaxf(fmaxf(acc[j][u][0], acc[j][u][1]), fmaxf(acc[j][u][2], acc[j][u][3])));
                bmax[j] = wave_max16(bm);
                if (grp == 0)
                    xmax[qw * (T * 16) + (qt0 + j) * 16 + (opaque(lane) & 15)] = bmax[j];
            }
        }
        lds_sync();   // B2: the pair's maxima are published; the PV waves hold P of block i - 1
        uint32_t pk[TW][KS];   // E4M3 P of this lane's 4 keys of each subtile
        uint32_t pkl[TW][KS];  // with PS: E4M3 lo = E4M3(P - hi) of the same keys
        float alpha[TW];
        if (work) {
#pragma unroll
            for (int j = 0; j < TW; j++) {
                // the pair's waves combine the same maxima (fmaxf is exact and symmetric)
                float bmx = bmax[j];
#pragma unroll
                for (int k = 1; k < KW; k++)
                    bmx = fmaxf(bmx, xmax[(qw / KW * KW + (kq + k) % KW) * (T * 16) + (qt0 + j) * 16 + (opaque(lane) & 15)]);
                const float bm = bmx * row_scale[j];
                const float m_new = fmaxf(m_run[j], bm);
                alpha[j] = (m_run[j] == neg_inf) ? 1.f : __builtin_amdgcn_exp2f(m_run[j] - m_new);
                const float m_use = (m_new == neg_inf) ? 0.f : m_new;   // exp2(-inf - m_use) = 0
                // ---- P = 448 exp2(s * scale - m) -> E4M3 (P <= 448: no clamp); each part's row
                // sum of the unrounded P in a fixed order ----
                float bsum[PPW];
#pragma unroll
                for (int pp = 0; pp < PPW; pp++) bsum[pp] = 0.f;
#pragma unroll
                for (int u = 0; u < KS; u++) {
                    float pr[4];
#pragma unroll
                    for (int jj = 0; jj < 4; jj++)
                        pr[jj] = ANCHOR * __builtin_amdgcn_exp2f(fmaf(acc[j][u][jj], row_scale[j], -m_use));
                    int wp = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], 0, false);
                    pk[j][u] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], wp, true);
                    if (PS) {
                        // P - hi is exact in FP32 (hi is within a factor of two of P, or 0)
                        const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pk[j][u], false);
                        const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pk[j][u], true);
                        int wl = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0] - h01.x, pr[1] - h01.y, 0, false);
                        pkl[j][u] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(pr[2] - h23.x, pr[3] - h23.y, wl, true);
                    }
                    bsum[u >> 1] = bsum[u >> 1] + (((pr[0] + pr[1]) + pr[2]) + pr[3]);
                }
#pragma unroll
                for (int pp = 0; pp < PPW; pp++) l_run[j][pp] = l_run[j][pp] * alpha[j] + wave_sum16(bsum[pp]);
                m_run[j] = m_new;
            }
        }
        // P of block i may overwrite P of block i - 1: the PV waves took that before B2
        if (work) {
            const int lo = opaque(lane);
#pragma unroll
            for (int j = 0; j < TW; j++) {
#pragma unroll
                for (int u = 0; u < KS; u++)
                    *reinterpret_cast<uint32_t*>(smem + L::OFF_P + (qt0 + j) * PTILE + (lo & 15) * PPITCH +
                                                 16 * (sub0 + u) + 4 * (lo >> 4)) = pk[j][u];
                if (PS) {
#pragma unroll
                    for (int u = 0; u < KS; u++)
                        *reinterpret_cast<uint32_t*>(smem + L::OFF_PLO + (qt0 + j) * PTILE + (lo & 15) * PPITCH +
                                                     16 * (sub0 + u) + 4 * (lo >> 4)) = pkl[j][u];
                }
                if (grp == 0 && kq == 0)
                    xalpha[(qt0 + j) * 16 + (lo & 15)] = alpha[j];
            }
        }
        // the pointers and presence word of block i + 2 (its indices landed before B1; the PV wave
        // reads the other parity's table, block i + 1's, in this iteration)
        key_ptrs_all(i + 2, idx_lds[(i & 1) * BLK + 32 * qw + (lane_now() & 31)]);
    }

    // ---- epilogue: m and the parts' sums to LDS; the row sum is ((p0 + p1) + p2) + p3 ----
    float* fm = reinterpret_cast<float*>(smem + L::OFF_FM);
    float* fl = reinterpret_cast<float*>(smem + L::OFF_FL);   // [4 parts][T * 16]
    if (grp == 0) {
#pragma unroll
        for (int j = 0; j < TW; j++) {
            if (kq == 0)
                fm[(qt0 + j) * 16 + n16] = m_run[j];
#pragma unroll
            for (int pp = 0; pp < PPW; pp++)
                fl[(sub0 / 2 + pp) * (T * 16) + (qt0 + j) * 16 + n16] = l_run[j][pp];
        }
    }
    int* misc = reinterpret_cast<int*>(smem + L::OFF_MISC);
    if (w.count > 1 && qw == 0 && lane == 0) {
        // A split item that finds every other item of its (group, tile set) counted in is the
        // last: it keeps its partial in LDS and merges at once (no store, release or count).
        const uint32_t seen = __hip_atomic_load(p.ws_cnt + (int64_t)w.g * p.tilesets + w.ts,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = seen == (uint32_t)(w.count - 1);
        if (last)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the others' released partials
        misc[1] = last ? 1 : 0;
    }
    __syncthreads();   // E1
    if (!(grp == 0 && kq == 0))
        return;
#pragma unroll
    for (int j = 0; j < TW; j++) {
        const int r = (qt0 + j) * 16 + n16;
        const float l = ((fl[r] + fl[T * 16 + r]) + fl[2 * T * 16 + r]) + fl[3 * T * 16 + r];
        const int64_t orow = w.row_base + 16 * (w.ts * T + qt0 + j) + n16;
        if (w.count == 1) {
            p.lse[orow] = (l > 0.f) ? (m_run[j] - LOG2_ANCHOR + log2f(l)) * LN2 : neg_inf;
        } else {
            float* dst = misc[1] == 0 ? p.ws_ml + ((int64_t)w.slot * (T * 16) + r) * 2
                                      : reinterpret_cast<float*>(smem) + own_ml_offset<T>() + r * 2;
            dst[0] = m_run[j];
            dst[1] = l;
        }
    }
}

// ---- PV waves: the gather, and O^T += V^T P^T for 128 latent columns of every tile ----
template <int T, bool DENSE, bool QE, bool PS>
__device__ __forceinline__ void pv_role(const Params& p, uint8_t* smem, const Work& w, int pw,
                                        int lane, const FirstIdx& fi, v4f (&O)[T][8])
{
    using L = Smem<T>;
    const int n16 = lane & 15;
    const int grp = lane >> 4;

    // Gather: this wave moves keys 32 pw .. 32 pw + 31 (subtiles 2 pw, 2 pw + 1) of every block.
    // The raw indices (page ids or row ids) of block b arrive in LDS slot b % 2 by DMA three blocks
    // ahead; two blocks ahead QK wave pw turns them into row pointers (the zero row when absent),
    // which go to this wave's pointer table of block parity b % 2, and a presence word (this wave
    // does it itself for blocks 0 and 1); one block ahead the wave issues the block's 18 row DMAs
    // with each lane's source read from the table.
    uint64_t* ptabs = reinterpret_cast<uint64_t*>(smem + L::OFF_PTAB) + 32 * pw;   // the wave's tables (+ 128 per block parity)
    // The gather's scalars (the same arithmetic as index_ptr and key_row), made opaque so that the
    // loop keeps them in scalar registers instead of reloading them from the kernel arguments
    uint64_t kv_base = (uint64_t)(uintptr_t)p.kv, zero_row = (uint64_t)(uintptr_t)g_zero_row;
    uint64_t ibase = (uint64_t)(uintptr_t)(DENSE ? p.table + (int64_t)w.g * p.max_pages : p.rows + (int64_t)w.g * p.K);
    int64_t nrows = p.num_rows;
    uint32_t psz = (uint32_t)p.page_size, pmag = p.pg_magic;
    int ps1 = p.pg_s1, ps2 = p.pg_s2;
    asm volatile("" : "+s"(kv_base), "+s"(zero_row), "+s"(ibase), "+s"(nrows), "+s"(psz), "+s"(pmag), "+s"(ps1), "+s"(ps2));
    auto pdiv = [&](uint32_t n) {
        const uint32_t t = __umulhi(n, pmag);
        return (t + ((n - t) >> ps1)) >> ps2;
    };
    auto dma_indices = [&](int blk) {  // raw indices of block blk -> idx slot blk % 2
        const int ln = lane_now();
        const int kk = 32 * pw + ln;
        const int64_t left = w.mine - (int64_t)blk * BLK;
        if (ln < 32 && kk < left) {
            const int64_t j = w.first + (int64_t)blk * BLK + kk;
            const int32_t* ip = reinterpret_cast<const int32_t*>(ibase) + (DENSE ? (int64_t)pdiv((uint32_t)j) : j);
            dma4(ip, lds_addr(smem + L::OFF_IDX + (blk & 1) * BLK * 4 + 32 * pw * 4));
        }
    };
    // Lane k < 32: the pointer of key 32 pw + k of block blk (idx: its raw index) into table entry
    // 16 (k % 2) + 8 (k / 16) + (k % 16) / 2, i.e. the keys of latent DMA i of subtile h (keys
    // 16 h + 2 i and 16 h + 2 i + 1 of the wave) sit at entries 8 h + i and 16 + 8 h + i. The
    // presence word of the wave's 32 keys goes to LDS for the QK waves.
    auto key_ptrs = [&](int blk, int32_t idx) {
        const int ln = lane_now();
        const int kk = 32 * pw + ln;
        const int64_t left = w.mine - (int64_t)blk * BLK;
        const bool in = ln < 32 && kk < left;
        const int64_t j = w.first + (int64_t)blk * BLK + kk;
        int64_t row = -1;
        if (in) {
            if (DENSE) {
                if (idx >= 0)
                    row = (int64_t)idx * psz + (int64_t)((uint32_t)j - pdiv((uint32_t)j) * psz);
            } else {
                row = idx;
            }
        }
        row = (row >= 0 && row < nrows) ? row : -1;
        const uint32_t word = (uint32_t)__ballot(row >= 0);   // lanes 0..31: keys 32 pw + lane
        if (ln == 0)
            *reinterpret_cast<uint32_t*>(smem + L::OFF_KMASK + (blk & 3) * 16 + 4 * pw) = word;
        const uint64_t ptr = row >= 0 ? kv_base + (uint64_t)row * ROW : zero_row;
        if (ln < 32)
            ptabs[128 * (blk & 1) + 16 * (ln & 1) + 8 * (ln >> 4) + ((ln & 15) >> 1)] = ptr;
    };
    auto issue_half = [&](int blk, int h) {   // one subtile's 9 row DMAs, pointers from the table
        const uint8_t* src[9];
        subtile_sources(ptabs + 128 * (blk & 1), h, src);
        issue_subtile(smem, src, blk, pw, h);
    };
    // Sparse lists with four tiles issue a block's second subtile after B2 (the scattered rows'
    // DMAs then spread over both phases; measured faster there, slower for paged KV)
    constexpr bool SPLIT_ISSUE = !DENSE && T == 4;
    if (w.nblk > 0) {
        const int kk = 32 * pw + lane;
        int32_t idx0 = fi.i0, idx1 = fi.i1;
        if (!fi.ok) {
            if (lane < 32 && kk < w.mine)
                idx0 = *index_ptr<DENSE>(p, w.g, w.first + kk);
            if (lane < 32 && BLK + kk < w.mine)
                idx1 = *index_ptr<DENSE>(p, w.g, w.first + BLK + kk);
        }
        if (w.nblk > 2)
            dma_indices(2);
        key_ptrs(0, idx0);
        issue_half(0, 0);
        issue_half(0, 1);
        if (w.nblk > 1)
            key_ptrs(1, idx1);   // the table's reads for block 0 precede these writes (one wave)
    }
    lds_sync();   // Q0: the QK waves' staged query rows landed
    if (!OWN_Q<T, DENSE> && w.nblk > 0)
        convert_q<T, QE>(smem, 256 + pw * 64 + lane);

    // This lane's transposed V read of column chunk 8 pw + c, key half rb of subtile 2 grp + sp:
    // LDS unit 32 kk + (cc ^ kk) of the subtile, kk = 8 rb + m, cc = 8 pw + c, m = n16 / 2, plus
    // 8 bytes for odd n16. Its byte offset in the slot is (vb + 128 (pw ^ rb)) ^ 16 c plus
    // sp SUBB + 4096 rb, with vb = 2 grp SUBB + 528 m + 8 (n16 % 2): 16 (c ^ m) = 16 c ^ 16 m, and
    // no other term has bits 4..8 set.
    auto vbase = [](int ln) { return 2 * (ln >> 4) * SUBB + 528 * ((ln & 15) >> 1) + 8 * (ln & 1); };
    auto load_vt = [&](int slot, int c, int vb0, int vb1) {
        v2i tr[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int off = ((r & 1 ? vb1 : vb0) ^ (16 * c)) + (r >> 1) * SUBB + 4096 * (r & 1);
            tr[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(smem + off));
        }
        return v8i{tr[0].x, tr[0].y, tr[1].x, tr[1].y, tr[2].x, tr[2].y, tr[3].x, tr[3].y};
    };
    const float* xalpha = reinterpret_cast<const float*>(smem + L::OFF_ALPHA);
    v8i vt[8];   // V^T of the block the next iteration multiplies (copied while its slot is valid)

    // iteration i, before B2: P and the rescale factors of block i - 1 (published before B1) and
    // the row DMAs of block i + 1 (its slot's last readers finished before B1); after B2, in one
    // stretch of code: the PV of block i - 1 (its V^T is in registers), each V^T chunk replaced by
    // block i's once its MFMAs are issued (the slot is refilled only after the next B1); then the
    // indices of block i + 3. Meanwhile the QK waves write the pointers and presence words of block
    // i + 2 (the other parity's table; presence words and index slots alternate by block, away from
    // the readers of the current ones). With four tiles every iteration runs the whole stretch (the first
    // multiplies zeros, the last reads an unused slot: registers are too few for a second copy of
    // the code); otherwise the first and last iterations take the same steps one by one.
    if (T == 4) {
#pragma unroll
        for (int c = 0; c < 8; c++) vt[c] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
    for (int i = 0; i <= w.nblk; i++) {
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's DMAs of block i (and indices)
        lds_sync();   // B1: block i landed; P of block i - 1 published
        // block i + 2's indices (landed with this iteration's vmcnt wait; any block's slot is
        // readable)
        float alpha[T];
        v8i pb[T];
        v8i pl[T];   // with PS: P lo
        if (T == 4) {
#pragma unroll
            for (int t = 0; t < T; t++) pb[t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
        if (i >= 1) {
#pragma unroll
            for (int t = 0; t < T; t++) {
                const int lo = lane_now();
                alpha[t] = xalpha[t * 16 + (lo & 15)];
                const int off = L::OFF_P + t * PTILE + (lo & 15) * PPITCH + 32 * (lo >> 4);
                pb[t] = cat(lds_read16(smem, off), lds_read16(smem, off + 16));
                if (PS) {
                    const int offl = off - L::OFF_P + L::OFF_PLO;
                    pl[t] = cat(lds_read16(smem, offl), lds_read16(smem, offl + 16));
                }
            }
        }
        if (i + 1 < w.nblk) {
            issue_half(i + 1, 0);
            if (!SPLIT_ISSUE)
                issue_half(i + 1, 1);
        }
        if (i >= 1) {
#pragma unroll
            for (int t = 0; t < T; t++) {
                const float a = alpha[t];
                if (!__all(a == 1.f)) {
#pragma unroll
                    for (int c = 0; c < 8; c++) O[t][c] *= a;
                }
            }
        }
        lds_sync();   // B2: the PV waves hold P of block i - 1; the QK waves' maxima are published
        // the lane's V^T base for block i's slot (recomputed here, not held across the loop)
        const int b = (i & 1) * SLOT + vbase(lane_now());
        if (SPLIT_ISSUE && i + 1 < w.nblk)
            issue_half(i + 1, 1);
        if (T == 4 || (i >= 1 && i < w.nblk)) {
#pragma unroll
            for (int c = 0; c < 8; c++) {
#pragma unroll
                for (int t = 0; t < T; t++) {
                    O[t][c] = mfma(vt[c], pb[t], O[t][c]);
                    if (PS)
                        O[t][c] = mfma(vt[c], pl[t], O[t][c]);
                }
                vt[c] = load_vt(i & 1, c, b + 128 * pw, b + 128 * (pw ^ 1));
            }
        } else {
            if (i >= 1) {
#pragma unroll
                for (int c = 0; c < 8; c++)
#pragma unroll
                    for (int t = 0; t < T; t++) {
                        O[t][c] = mfma(vt[c], pb[t], O[t][c]);
                        if (PS)
                            O[t][c] = mfma(vt[c], pl[t], O[t][c]);
                    }
            }
            if (i < w.nblk) {
#pragma unroll
                for (int c = 0; c < 8; c++) vt[c] = load_vt(i & 1, c, b + 128 * pw, b + 128 * (pw ^ 1));
            }
        }
        if (i + 3 < w.nblk)
            dma_indices(i + 3);
    }

    // ---- epilogue ----
    __syncthreads();   // E1: (m, l) of every row in LDS
    const float* fl = reinterpret_cast<const float*>(smem + L::OFF_FL);
    if (w.count == 1) {
        // o = BF16(O / l * k_scale); the single-split merge (weight exp2(0) = 1) is this exactly
#pragma unroll
        for (int t = 0; t < T; t++) {
            const int r = t * 16 + n16;
            const float lt = ((fl[r] + fl[T * 16 + r]) + fl[2 * T * 16 + r]) + fl[3 * T * 16 + r];
            const float rl = 1.f / lt;   // one division per row
            const int64_t orow = w.row_base + 16 * (w.ts * T + t) + n16;
            // Column blocks c and c + 1 in pairs: lane (n16, grp) holds columns 4 grp .. 4 grp + 3 of
            // both. One 16-lane row swap (odd rows of the first operand with even rows of the
            // second) leaves an even-grp lane with columns 8 (grp / 2) .. + 7 of block c (its own
            // four, then its neighbour's) and an odd-grp lane with the same columns of block c + 1,
            // so that every lane writes 16 contiguous bytes: half the store instructions.
#pragma unroll
            for (int c = 0; c < 8; c += 2) {
                uint32_t a01 = 0, a23 = 0, b01 = 0, b23 = 0;
                if (lt > 0.f) {
                    a01 = pack_bf16(div_by(O[t][c][0], lt, rl) * p.k_scale, div_by(O[t][c][1], lt, rl) * p.k_scale);
                    a23 = pack_bf16(div_by(O[t][c][2], lt, rl) * p.k_scale, div_by(O[t][c][3], lt, rl) * p.k_scale);
                    b01 = pack_bf16(div_by(O[t][c + 1][0], lt, rl) * p.k_scale, div_by(O[t][c + 1][1], lt, rl) * p.k_scale);
                    b23 = pack_bf16(div_by(O[t][c + 1][2], lt, rl) * p.k_scale, div_by(O[t][c + 1][3], lt, rl) * p.k_scale);
                }
                const auto x01 = __builtin_amdgcn_permlane16_swap(a01, b01, false, false);
                const auto x23 = __builtin_amdgcn_permlane16_swap(a23, b23, false, false);
                const int col = 128 * pw + 16 * (c + (grp & 1)) + 8 * (grp >> 1);
                *reinterpret_cast<v4i*>(p.o + orow * LATENT + col) =
                    v4i{(int)x01[0], (int)x23[0], (int)x01[1], (int)x23[1]};
            }
        }
        return;
    }
    // a split item: the partial to the workspace, or, for the item found last before E1, to the
    // KV slots (free now, 128 KB for four tiles) for its own merge
    const bool last = reinterpret_cast<const int*>(smem + L::OFF_MISC)[1] != 0;
#pragma unroll
    for (int t = 0; t < T; t++)
#pragma unroll
        for (int c = 0; c < 8; c++) {
            if (last)
                *reinterpret_cast<v4f*>(smem + 4 * partial_o_offset<T>(0, pw, t, c, lane)) = O[t][c];
            else
                *reinterpret_cast<v4f*>(p.ws_o + partial_o_offset<T>(w.slot, pw, t, c, lane)) = O[t][c];
        }
}

// The last arriving item of a (group, tile set) merges the group's FP32 partials in split order.
// Thread (wave c, lane) owns the four adjacent column blocks 4 (c % 2) .. + 3 of column quarter
// c / 2 of every tile, for rows 16 t + lane % 16: per contributor it weighs T rows and issues 4 T
// contiguous loads at once; adjacent blocks pair up for 16-byte output stores.
// own_lds: this item's own partial is in LDS, in the workspace's layout at the start of the KV
// slots (O, then (m, l) at own_ml_offset<T>()), rather than in the workspace; the loads go through
// generic pointers so that one code path reads both.
template <int T>
__device__ void merge_splits(const Params& p, const Work& w, int tid, const uint8_t* smem, bool own_lds)
{
    const float neg_inf = -INFINITY;
    const int lane = tid & 63, c = tid >> 6;
    const int n16 = lane & 15, grp = lane >> 4;
    auto o_base = [&](int slot) -> const float* {
        return (own_lds && slot == w.slot) ? reinterpret_cast<const float*>(smem)
                                           : p.ws_o + partial_o_offset<T>(slot, 0, 0, 0, 0);
    };
    auto ml_base = [&](int slot) -> const float* {
        return (own_lds && slot == w.slot) ? reinterpret_cast<const float*>(smem) + own_ml_offset<T>()
                                           : p.ws_ml + (int64_t)slot * (T * 16) * 2;
    };
    // per contributor: its (m, l) for the T rows and its 4 T partial loads
    struct Part {
        v2f ml[T];
        v4f x[4][T];
    };
    auto load_part = [&](int q, Part& pt) {
        const int slot = contributor_slot(p, w, q);
        const float* mlb = ml_base(slot);
        const float* ob = o_base(slot);
#pragma unroll
        for (int t = 0; t < T; t++)
            pt.ml[t] = *reinterpret_cast<const v2f*>(mlb + (16 * t + n16) * 2);
#pragma unroll
        for (int k = 0; k < 4; k++)
#pragma unroll
            for (int t = 0; t < T; t++)
                pt.x[k][t] = *reinterpret_cast<const v4f*>(ob + partial_o_offset<T>(0, c >> 1, t, 4 * (c & 1) + k, lane));
    };
    // One round trip for the common case: the first two contributors' partials and every
    // contributor's maximum are requested before any of them is used.
    Part a, b;
    load_part(0, a);
    if (w.count > 1)
        load_part(1, b);
    float top[T], total[T];
#pragma unroll
    for (int t = 0; t < T; t++) {
        top[t] = a.ml[t][0];
        total[t] = 0.f;
    }
    for (int q = 2; q < w.count; q++) {
        const float* mlb = ml_base(contributor_slot(p, w, q));
#pragma unroll
        for (int t = 0; t < T; t++) top[t] = fmaxf(top[t], mlb[(16 * t + n16) * 2]);
    }
    if (w.count > 1) {
#pragma unroll
        for (int t = 0; t < T; t++) top[t] = fmaxf(top[t], b.ml[t][0]);
    }
    v4f acc[4][T];
#pragma unroll
    for (int pw = 0; pw < 4; pw++)
#pragma unroll
        for (int t = 0; t < T; t++) acc[pw][t] = v4f{0.f, 0.f, 0.f, 0.f};
    auto add_part = [&](const Part& pt) {
#pragma unroll
        for (int t = 0; t < T; t++) {
            if (pt.ml[t][0] == neg_inf)
                continue;   // an empty split (and a row with no key at all)
            const float wq = exp2f(pt.ml[t][0] - top[t]);
            total[t] = total[t] + wq * pt.ml[t][1];
#pragma unroll
            for (int pw = 0; pw < 4; pw++) acc[pw][t] = acc[pw][t] + wq * pt.x[pw][t];
        }
    };
    // in split order; two contributors in flight at a time
    add_part(a);
    if (w.count > 1)
        add_part(b);
    int q = 2;
    for (; q + 1 < w.count; q += 2) {
        load_part(q, a);
        load_part(q + 1, b);
        add_part(a);
        add_part(b);
    }
    if (q < w.count) {
        load_part(q, a);
        add_part(a);
    }
#pragma unroll
    for (int t = 0; t < T; t++) {
        const int64_t orow = w.row_base + 16 * (w.ts * T + t) + n16;
        // blocks k and k + 1: the same 16-lane row swap as the single-split epilogue leaves each lane
        // 8 contiguous columns (even grp: block k, odd grp: block k + 1)
#pragma unroll
        for (int k = 0; k < 4; k += 2) {
            uint32_t w[2][2] = {{0, 0}, {0, 0}};
            if (total[t] > 0.f) {
                const float rt = 1.f / total[t];
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) v[e] = div_by(acc[k + h][t][e], total[t], rt) * p.k_scale;
                    w[h][0] = pack_bf16(v[0], v[1]);
                    w[h][1] = pack_bf16(v[2], v[3]);
                }
            }
            const auto x01 = __builtin_amdgcn_permlane16_swap(w[0][0], w[1][0], false, false);
            const auto x23 = __builtin_amdgcn_permlane16_swap(w[0][1], w[1][1], false, false);
            const int col = 128 * (c >> 1) + 16 * (4 * (c & 1) + k + (grp & 1)) + 8 * (grp >> 1);
            *reinterpret_cast<v4i*>(p.o + orow * LATENT + col) = v4i{(int)x01[0], (int)x23[0], (int)x01[1], (int)x23[1]};
        }
        if (c == 0 && grp == 0)
            p.lse[orow] = total[t] > 0.f ? (top[t] - LOG2_ANCHOR + log2f(total[t])) * LN2 : neg_inf;
    }
}

// After a work item (all threads): for a split item, the arrival count and, by the last of the
// group's items to arrive, the merge.
template <int T>
__device__ __forceinline__ void finish_item(const Params& p, uint8_t* smem, const Work& w, int tid)
{
    using L = Smem<T>;
    if (w.count == 1)
        return;
    int* misc = reinterpret_cast<int*>(smem + L::OFF_MISC);
    uint32_t* cnt = p.ws_cnt + (int64_t)w.g * p.tilesets + w.ts;
    if (misc[1] != 0) {
        // found last before E1 (its acquire made there): the partial is in LDS; merge now
        __syncthreads();   // E2: the PV waves' LDS copies of O
        merge_splits<T>(p, w, tid, smem, true);
        if (tid == 0)
            __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    // a split item: every thread's partial stores completed (vmcnt(0)) before the barrier; one
    // thread then releases them at agent scope and counts this item in; the last arriver merges.
    __builtin_amdgcn_s_waitcnt(0xF70);
    __syncthreads();   // E2
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == (uint32_t)(w.count - 1);
        if (last)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the others' released partials
        misc[0] = last ? 1 : 0;
    }
    __syncthreads();   // E3
    if (misc[0] == 0)
        return;
    merge_splits<T>(p, w, tid, smem, false);
    if (tid == 0)
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef const __attribute__((address_space(4))) Params kernarg_params;

// The kernel's parameters read anew: the pointer to them (the first kernel argument) passes
// through an empty asm, so the compiler cannot prove loads through it invariant across work items
// and does not keep every value derived from them live across the item loop (it would run out
// of scalar registers and spill).
__device__ inline const Params& fresh_params()
{
    kernarg_params* k = (kernarg_params*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(k));
    return *(const Params*)k;   // loads through it stay scalar (address-space inference)
}

template <int T, bool DENSE, bool QE, bool PS>
__global__ __launch_bounds__(THREADS) void mla_decode_kernel(const Params p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<T, PS>::BYTES];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    // a unit's tile sets share one XCD (blockIdx % 8). With at most two tile sets, consecutive
    // units do too (XCD x runs units x ceil(units / 8) ..): the pieces a split group spans mostly
    // share one L2, which then holds the partials their merge reads (measured faster there, and
    // no better with more tile sets, where the units go round the XCDs)
    const int bid = blockIdx.x;
    const int slotid = bid >> 3;
    {
        // both 64-byte lines of parameters the first steps read, fetched in one round trip
        const void* line0 = p.kv;
        const int line1 = p.tilesets;
        asm volatile("" ::"s"(line0), "s"(line1));
    }
    const int ts = slotid % p.tilesets;
    const int unit = p.tilesets <= 2 ? (bid & 7) * (int)(((int64_t)p.units + 7) / 8) + slotid / p.tilesets
                                     : (slotid / p.tilesets) * 8 + (bid & 7);
    if (unit >= p.units)
        return;
    // uniform plan: the one item (group unit % groups); balanced plan: the piece's groups, last first
    Span sp{unit % p.groups, unit % p.groups, 0, 0};
    if (p.balanced)
        sp = piece_span<DENSE>(p, smem, unit, tid, lane);
    auto item = [&](const Params& pi, int g, int64_t pre, Work& w, int64_t n_known = -1) {
        if (pi.balanced)
            balanced_item<DENSE>(pi, unit, ts, g, pre, sp, w);
        else
            decode_uniform<DENSE>(pi, unit, ts, w, n_known);
    };
    // waves 0..3: QK (tile = wave); waves 4..7: gather + PV (columns 128 (wave - 4) ..); wave i runs
    // on SIMD i % 4, so each SIMD pairs one QK wave with one PV wave. Each role walks the items
    // itself (same items, same barriers), so neither keeps the other's values live.
    if (wave < 4) {
        int64_t pre = sp.pre_hi;
        for (int g = sp.g_hi; g >= sp.g_lo; g--) {
            const Params& pi = fresh_params();
            int li = lane;   // lane-derived offsets are recomputed per item, not kept live
            asm volatile("" : "+v"(li));
            // the query rows go out before the key counts are read (they depend on g and ts only)
            if (OWN_Q<T, DENSE>)
                stage_q_own<T>(pi, smem, (int64_t)g * pi.rows_per_group + 16 * ts * T, wave, li);
            else
                stage_q<T>(pi, smem, (int64_t)g * pi.rows_per_group + 16 * ts * T, wave, li);
            Work w;
            item(pi, g, pre, w);
            if (g > sp.g_lo)
                pre -= ITEM_BLOCKS + nblocks(group_keys<DENSE>(pi, g - 1));
            qk_role<T, DENSE, QE, PS>(pi, smem, w, wave, li);
            finish_item<T>(pi, smem, w, tid);
            __syncthreads();   // the next item reuses every LDS area
        }
    } else {
        int64_t pre = sp.pre_hi;
        for (int g = sp.g_hi; g >= sp.g_lo; g--) {
            const Params& pi = fresh_params();
            const FirstIdx fi = first_indices<DENSE>(pi, unit, wave - 4);
            Work w;
            item(pi, g, pre, w, fi.n);
            if (g > sp.g_lo)
                pre -= ITEM_BLOCKS + nblocks(group_keys<DENSE>(pi, g - 1));
            v4f O[T][8];
#pragma unroll
            for (int t = 0; t < T; t++)
#pragma unroll
                for (int c = 0; c < 8; c++) O[t][c] = v4f{0.f, 0.f, 0.f, 0.f};
            int li = lane;
            asm volatile("" : "+v"(li));
            pv_role<T, DENSE, QE, PS>(pi, smem, w, wave - 4, li, fi, O);
            finish_item<T>(pi, smem, w, tid);
            __syncthreads();
        }
    }
}

// ---- host side ------------------------------------------------------------------------------

constexpr size_t ALIGN_WS = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: [arrival counters | (m, l) partials | O partials]. The counters come first so that
// their offset does not depend on the shape: a workspace whose leading counter bytes are zero can
// serve any call, and every call leaves its counters zero again.
struct WsLayout {
    size_t cnt_bytes, ml_bytes, o_bytes, total;
};

// Partial rows: a uniform plan with S > 1 leaves every row once per split; a balanced plan with
// more than one piece leaves at most two partials (of a tile set's rows) per piece and tile set.
WsLayout ws_layout(int dense, int B, int Q, int H, const mla_plan_t& pl)
{
    WsLayout w{};
    if (pl.splits <= 1)
        return w;
    const size_t rows = (size_t)B * Q * H;
    const size_t rows_per_group = dense ? (size_t)Q * H : (size_t)H;
    const size_t prows = pl.mode == MLA_SPLIT_BALANCED ? 2 * (size_t)pl.splits * rows_per_group
                                                       : rows * (size_t)pl.splits;
    w.cnt_bytes = round_up(rows / 16 * sizeof(uint32_t), ALIGN_WS);
    w.ml_bytes = round_up(prows * 2 * sizeof(float), ALIGN_WS);
    w.o_bytes = round_up(prows * LATENT * sizeof(float), ALIGN_WS);
    w.total = w.cnt_bytes + w.ml_bytes + w.o_bytes;
    return w;
}

// Group count a balanced plan supports: the prefix sums of the groups' block counts (G + 1 int32)
// are staged in the two LDS slots.
constexpr int MAX_BALANCED_GROUPS = 2 * SLOT / 4 - 1;

int choose_tiles(int tiles_per_group)
{
    if (tiles_per_group % 4 == 0)
        return 4;
    if (tiles_per_group % 2 == 0)
        return 2;
    return 1;
}

// A plan from shapes only. One workgroup fills a CU's LDS, so 256 workgroups cover the chip once.
// Groups of at most two 128-key blocks: one workgroup per group and tile set (uniform, S = 1).
// Longer groups: either one workgroup per group and tile set (S = 1, no partials to merge) or a
// balanced plan of 256 / tilesets pieces, which evens out ragged key counts but adds work items
// and merges. The cost of each is estimated in 128-key blocks per CU, every group at its maximum
// key count and every work item costing ITEM_BLOCKS more; a balanced piece also pays for the
// group it continues and for the FP32 partials and their merge, about two items (measured on
// MI355X). For more groups than a balanced plan stages, uniform splits up to one workgroup per
// CU.
mla_plan_t choose_plan(int groups, int tiles_per_group, int64_t max_keys)
{
    mla_plan_t pl{};
    pl.tiles = choose_tiles(tiles_per_group);
    const int tilesets = tiles_per_group / pl.tiles;
    const int64_t mb = (max_keys + BLK - 1) / BLK;
    pl.splits = 1;
    pl.mode = MLA_SPLIT_UNIFORM;
    if (max_keys <= 2 * BLK)
        return pl;
    if (groups <= MAX_BALANCED_GROUPS && (int64_t)groups * (mb + ITEM_BLOCKS) < INT32_MAX) {
        const int64_t wgs = (int64_t)groups * tilesets;
        const int64_t whole = (wgs + 255) / 256 * (mb + ITEM_BLOCKS);   // S = 1: rounds of workgroups
        const int64_t balanced = (wgs * (mb + ITEM_BLOCKS) + 255) / 256 + 2 * ITEM_BLOCKS;
        if (balanced < whole) {
            pl.splits = 256 / tilesets > 1 ? 256 / tilesets : 1;
            pl.mode = MLA_SPLIT_BALANCED;
        }
        return pl;
    }
    int64_t s = 256 / ((int64_t)groups * tilesets);
    const int64_t cap = max_keys / (2 * BLK);
    s = s > cap ? cap : s;
    pl.splits = (int)(s < 1 ? 1 : (s > 64 ? 64 : s));
    return pl;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// The magic number and shifts of division by d (1 <= d < 2^31) for 32-bit dividends: with
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, s1 = min(l, 1), s2 = max(l - 1, 0)
// (Granlund and Montgomery 1994, Figure 4.1).
void set_page_division(Params& p, int d)
{
    int l = 0;
    while ((1ll << l) < d)
        l++;
    p.pg_magic = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - (uint64_t)d)) / (uint64_t)d + 1);
    p.pg_s1 = l < 1 ? l : 1;
    p.pg_s2 = l - 1 > 0 ? l - 1 : 0;
}

template <int T, bool DENSE, bool QE, bool PS>
hipError_t launch_t(const Params& p, hipStream_t stream)
{
    const int64_t gs_pad = ((int64_t)p.units + 7) / 8 * 8;
    const int64_t grid = gs_pad * p.tilesets;
    hipLaunchKernelGGL((mla_decode_kernel<T, DENSE, QE, PS>), dim3((unsigned)grid), dim3(THREADS), 0,
                       stream, p);
    return hipGetLastError();
}

template <bool DENSE, bool QE>
hipError_t launch_q(int T, bool ps, const Params& p, hipStream_t stream)
{
    if (ps)   // at most two tiles (the entry points cap the plan)
        return T == 1 ? launch_t<1, DENSE, QE, true>(p, stream) : launch_t<2, DENSE, QE, true>(p, stream);
    switch (T) {
    case 1: return launch_t<1, DENSE, QE, false>(p, stream);
    case 2: return launch_t<2, DENSE, QE, false>(p, stream);
    default: return launch_t<4, DENSE, QE, false>(p, stream);
    }
}

template <bool DENSE>
hipError_t launch(int T, int precision, const Params& p, hipStream_t stream)
{
    const bool ps = (precision & MLA_P_SPLIT) != 0;
    return (precision & MLA_Q_E4M3) ? launch_q<DENSE, true>(T, ps, p, stream)
                                    : launch_q<DENSE, false>(T, ps, p, stream);
}

// The precision flags the entry points take.
bool precision_ok(int precision) { return (precision & ~(MLA_Q_E4M3 | MLA_P_SPLIT)) == 0; }

mla_status_t common_checks(const void* q, const mla_kv_t* kv, int B, int Q, int H, void* o,
                           float* lse)
{
    if (!kv)
        return MLA_ERR_NULL;
    if (B < 0 || Q < 1 || H < 16 || H % 16 != 0)
        return MLA_ERR_SHAPE;
    if (B == 0)
        return MLA_OK;
    if (!q || !kv->data || !o || !lse)
        return MLA_ERR_NULL;
    if (kv->num_rows < 0)
        return MLA_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(kv->data, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return MLA_ERR_ALIGN;
    return MLA_OK;
}

// The plan a call runs (the caller's, or the chooser's) if the kernels implement it.
mla_status_t check_plan(const mla_plan_t* in, mla_plan_t chosen, int groups, int tiles_per_group,
                        int64_t max_keys, mla_plan_t* out)
{
    mla_plan_t pl = in ? *in : chosen;
    if (pl.splits < 1 || pl.splits > 4096)
        return MLA_ERR_UNSUPPORTED;
    if (!(pl.tiles == 1 || pl.tiles == 2 || pl.tiles == 4) || tiles_per_group % pl.tiles != 0)
        return MLA_ERR_UNSUPPORTED;
    if (pl.mode != MLA_SPLIT_UNIFORM && pl.mode != MLA_SPLIT_BALANCED)
        return MLA_ERR_UNSUPPORTED;
    if (pl.mode == MLA_SPLIT_BALANCED &&
        (groups > MAX_BALANCED_GROUPS ||
         (int64_t)groups * ((max_keys + BLK - 1) / BLK + ITEM_BLOCKS) >= INT32_MAX))
        return MLA_ERR_UNSUPPORTED;
    *out = pl;
    return MLA_OK;
}

mla_status_t finish_plan(const mla_plan_t* in, mla_plan_t chosen, int dense, int groups,
                         int tiles_per_group, int64_t max_keys, int B, int Q, int H, void* ws,
                         size_t ws_bytes, mla_plan_t* out)
{
    mla_plan_t pl;
    const mla_status_t st = check_plan(in, chosen, groups, tiles_per_group, max_keys, &pl);
    if (st != MLA_OK)
        return st;
    if (pl.splits > 1) {
        const WsLayout w = ws_layout(dense, B, Q, H, pl);
        if (!ws || ws_bytes < w.total)
            return MLA_ERR_WORKSPACE;
        if (!aligned(ws, ALIGN_WS))
            return MLA_ERR_ALIGN;
    }
    *out = pl;
    return MLA_OK;
}

void fill_workspace(Params& p, int dense, int B, int Q, int H, const mla_plan_t& pl, void* ws)
{
    const WsLayout w = ws_layout(dense, B, Q, H, pl);
    uint8_t* base = (uint8_t*)ws;
    p.ws_cnt = p.S > 1 ? (uint32_t*)base : nullptr;
    p.ws_ml = p.S > 1 ? (float*)(base + w.cnt_bytes) : nullptr;
    p.ws_o = p.S > 1 ? (float*)(base + w.cnt_bytes + w.ml_bytes) : nullptr;
}

// The checks, plan and kernel parameters of a dense call (the workspace pointers stay null). A call
// with B == 0 returns MLA_OK after the argument checks; there is nothing to launch.
mla_status_t dense_setup(const void* q, const mla_kv_t* kv, const int32_t* block_table, int max_pages,
                         const int32_t* seq_lens, float scale, int B, int Q, int H,
                         const mla_plan_t* plan, int precision, void* o, float* lse, Params& p,
                         mla_plan_t& pl)
{
    if (!precision_ok(precision) || ((precision & MLA_P_SPLIT) && plan && plan->tiles == 4))
        return MLA_ERR_UNSUPPORTED;
    mla_status_t st = common_checks(q, kv, B, Q, H, o, lse);
    if (st != MLA_OK || B == 0)
        return st;
    if (max_pages < 1 || kv->page_size < 1 || (int64_t)max_pages * kv->page_size > INT32_MAX)
        return MLA_ERR_SHAPE;
    if (!block_table || !seq_lens)
        return MLA_ERR_NULL;
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
        return MLA_ERR_ALIGN;
    mla_plan_t chosen;
    mla_plan_dense(B, Q, H, max_pages, kv->page_size, &chosen);
    if ((precision & MLA_P_SPLIT) && chosen.tiles == 4)
        chosen.tiles = 2;
    st = check_plan(plan, chosen, B, Q * H / 16, (int64_t)max_pages * kv->page_size, &pl);
    if (st != MLA_OK)
        return st;
    p.q = (const uint16_t*)q;
    p.kv = (const uint8_t*)kv->data;
    p.num_rows = kv->num_rows;
    p.page_size = kv->page_size;
    set_page_division(p, kv->page_size);
    p.table = block_table;
    p.max_pages = max_pages;
    p.seq_lens = seq_lens;
    p.scale_log2 = (float)((double)scale * (double)kv->k_scale * 1.4426950408889634);
    p.k_scale = kv->k_scale;
    p.Q = Q;
    p.H = H;
    p.S = pl.splits;
    p.balanced = pl.mode == MLA_SPLIT_BALANCED;
    p.groups = B;
    p.rows_per_group = Q * H;
    p.tilesets = Q * H / 16 / pl.tiles;
    p.units = p.balanced ? pl.splits : B * pl.splits;
    p.o = (uint16_t*)o;
    p.lse = lse;
    return MLA_OK;
}

// ---- the scratch of mla_decode_dense_q_noalloc -------------------------------------------------
// One array per device, held until the process ends: the arrival counters in a fixed leading
// region (no call's partials ever land there, and every call leaves its counters zero: the last
// arriving workgroup of each tile resets its counter), then the FP32 partials of the call.
constexpr size_t STATIC_BYTES = MLA_NOALLOC_SCRATCH_BYTES;
constexpr size_t STATIC_CNT_BYTES = 64 << 10;   // 16384 counters: calls of up to 262144 query rows
static_assert(STATIC_CNT_BYTES % ALIGN_WS == 0, "partials stay 256-byte aligned");

static __device__ __align__(256) uint8_t scratch[STATIC_BYTES];

constexpr int MAX_DEVICES = 64;

struct StaticScratch {
    std::mutex mu;
    uint8_t* ptr[MAX_DEVICES] = {};    // the array's device address, per device
    bool cleared[MAX_DEVICES] = {};    // its counter region zeroed by a completed launch order
};
StaticScratch g_static;

__global__ void zero_words(uint32_t* __restrict__ p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

// This device's scratch address (looked up once per device, with that device current) and, until
// a launch outside graph capture has done it, a fill kernel that zeroes the counter region, on the
// caller's stream ahead of the decode (a fill kernel rather than hipMemsetAsync, so that a
// captured graph replays it correctly).
mla_status_t static_scratch(hipStream_t stream, uint8_t** out)
{
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess)
        return MLA_ERR_LAUNCH;
    int dev = cur;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess)
        return MLA_ERR_LAUNCH;
    if (dev < 0 || dev >= MAX_DEVICES)
        return MLA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_static.mu);
    if (!g_static.ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess)
            return MLA_ERR_LAUNCH;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess)
            return MLA_ERR_LAUNCH;
        if (e != hipSuccess || !ptr)
            return MLA_ERR_LAUNCH;
        g_static.ptr[dev] = (uint8_t*)ptr;
    }
    if (!g_static.cleared[dev]) {
        constexpr int words = (int)(STATIC_CNT_BYTES / 4);
        hipLaunchKernelGGL(zero_words, dim3(words / 256), dim3(256), 0, stream,
                           (uint32_t*)g_static.ptr[dev], words);
        if (hipGetLastError() != hipSuccess)
            return MLA_ERR_LAUNCH;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
            g_static.cleared[dev] = true;
    }
    *out = g_static.ptr[dev];
    return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status_t status)
{
    switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "null pointer";
    case MLA_ERR_SHAPE: return "bad shape";
    case MLA_ERR_ALIGN: return "misaligned pointer";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_UNSUPPORTED: return "unsupported plan";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

size_t mla_workspace_bytes(int dense, int B, int Q, int H, const mla_plan_t* plan)
{
    if (B <= 0 || Q <= 0 || H <= 0 || !plan)
        return 0;
    return ws_layout(dense, B, Q, H, *plan).total;
}

size_t mla_workspace_zero_bytes(int dense, int B, int Q, int H, const mla_plan_t* plan)
{
    if (B <= 0 || Q <= 0 || H <= 0 || !plan)
        return 0;
    return ws_layout(dense, B, Q, H, *plan).cnt_bytes;
}

mla_status_t mla_plan_dense(int B, int Q, int H, int max_pages, int page_size, mla_plan_t* plan)
{
    if (!plan)
        return MLA_ERR_NULL;
    if (B < 0 || Q < 1 || H < 16 || H % 16 != 0 || max_pages < 1 || page_size < 1 ||
        (int64_t)max_pages * page_size > INT32_MAX)
        return MLA_ERR_SHAPE;
    *plan = choose_plan(B > 0 ? B : 1, Q * H / 16, (int64_t)max_pages * page_size);
    return MLA_OK;
}

mla_status_t mla_plan_sparse(int B, int Q, int H, int K, mla_plan_t* plan)
{
    if (!plan)
        return MLA_ERR_NULL;
    if (B < 0 || Q < 1 || H < 16 || H % 16 != 0 || K < 1)
        return MLA_ERR_SHAPE;
    *plan = choose_plan(B > 0 ? B * Q : 1, H / 16, K);
    return MLA_OK;
}

mla_status_t mla_decode_dense_q(const void* q, const mla_kv_t* kv, const int32_t* block_table,
                                int max_pages, const int32_t* seq_lens, float scale, int B, int Q,
                                int H, const mla_plan_t* plan, int precision, void* o, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    Params p{};
    mla_plan_t pl;
    mla_status_t st = dense_setup(q, kv, block_table, max_pages, seq_lens, scale, B, Q, H, plan,
                                  precision, o, lse, p, pl);
    if (st != MLA_OK || B == 0)
        return st;
    if (pl.splits > 1) {
        const WsLayout w = ws_layout(1, B, Q, H, pl);
        if (!workspace || workspace_bytes < w.total)
            return MLA_ERR_WORKSPACE;
        if (!aligned(workspace, ALIGN_WS))
            return MLA_ERR_ALIGN;
    }
    fill_workspace(p, 1, B, Q, H, pl, workspace);
    if (launch<true>(pl.tiles, precision, p, (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_LAUNCH;
    return MLA_OK;
}

mla_status_t mla_decode_dense_q_noalloc(const void* q, const mla_kv_t* kv,
                                        const int32_t* block_table, int max_pages,
                                        const int32_t* seq_lens, float scale, int B, int Q, int H,
                                        const mla_plan_t* plan, int precision, void* o, float* lse,
                                        void* stream)
{
    Params p{};
    mla_plan_t pl;
    mla_status_t st = dense_setup(q, kv, block_table, max_pages, seq_lens, scale, B, Q, H, plan,
                                  precision, o, lse, p, pl);
    if (st != MLA_OK || B == 0)
        return st;
    if (pl.splits > 1) {
        // the counters in the scratch's fixed counter region, the partials after it
        const WsLayout w = ws_layout(1, B, Q, H, pl);
        if (w.cnt_bytes > STATIC_CNT_BYTES || STATIC_CNT_BYTES + w.ml_bytes + w.o_bytes > STATIC_BYTES)
            return MLA_ERR_WORKSPACE;
        uint8_t* base = nullptr;
        st = static_scratch((hipStream_t)stream, &base);
        if (st != MLA_OK)
            return st;
        p.ws_cnt = (uint32_t*)base;
        p.ws_ml = (float*)(base + STATIC_CNT_BYTES);
        p.ws_o = (float*)(base + STATIC_CNT_BYTES + w.ml_bytes);
    }
    if (launch<true>(pl.tiles, precision, p, (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_LAUNCH;
    return MLA_OK;
}

mla_status_t mla_decode_sparse_q(const void* q, const mla_kv_t* kv, const int32_t* rows, int K,
                                 const int32_t* valid, float scale, int B, int Q, int H,
                                 const mla_plan_t* plan, int precision, void* o, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream)
{
    if (!precision_ok(precision) || ((precision & MLA_P_SPLIT) && plan && plan->tiles == 4))
        return MLA_ERR_UNSUPPORTED;
    mla_status_t st = common_checks(q, kv, B, Q, H, o, lse);
    if (st != MLA_OK || B == 0)
        return st;
    if (K < 1)
        return MLA_ERR_SHAPE;
    if (!rows || !valid)
        return MLA_ERR_NULL;
    if (!aligned(rows, 4) || !aligned(valid, 4))
        return MLA_ERR_ALIGN;
    mla_plan_t chosen;
    mla_plan_sparse(B, Q, H, K, &chosen);
    if ((precision & MLA_P_SPLIT) && chosen.tiles == 4)
        chosen.tiles = 2;
    mla_plan_t pl;
    st = finish_plan(plan, chosen, 0, B * Q, H / 16, K, B, Q, H, workspace, workspace_bytes, &pl);
    if (st != MLA_OK)
        return st;
    Params p{};
    p.q = (const uint16_t*)q;
    p.kv = (const uint8_t*)kv->data;
    p.num_rows = kv->num_rows;
    p.page_size = 1;
    set_page_division(p, 1);
    p.rows = rows;
    p.K = K;
    p.valid = valid;
    p.scale_log2 = (float)((double)scale * (double)kv->k_scale * 1.4426950408889634);
    p.k_scale = kv->k_scale;
    p.Q = Q;
    p.H = H;
    p.S = pl.splits;
    p.balanced = pl.mode == MLA_SPLIT_BALANCED;
    p.groups = B * Q;
    p.rows_per_group = H;
    p.tilesets = H / 16 / pl.tiles;
    p.units = p.balanced ? pl.splits : B * Q * pl.splits;
    p.o = (uint16_t*)o;
    p.lse = lse;
    fill_workspace(p, 0, B, Q, H, pl, workspace);
    if (launch<false>(pl.tiles, precision, p, (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_LAUNCH;
    return MLA_OK;
}

mla_status_t mla_decode_dense(const void* q, const mla_kv_t* kv, const int32_t* block_table,
                              int max_pages, const int32_t* seq_lens, float scale, int B, int Q,
                              int H, const mla_plan_t* plan, void* o, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    return mla_decode_dense_q(q, kv, block_table, max_pages, seq_lens, scale, B, Q, H, plan,
                              MLA_Q_SPLIT, o, lse, workspace, workspace_bytes, stream);
}

mla_status_t mla_decode_sparse(const void* q, const mla_kv_t* kv, const int32_t* rows, int K,
                               const int32_t* valid, float scale, int B, int Q, int H,
                               const mla_plan_t* plan, void* o, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream)
{
    return mla_decode_sparse_q(q, kv, rows, K, valid, scale, B, Q, H, plan, MLA_Q_SPLIT, o, lse,
                               workspace, workspace_bytes, stream);
}

}  // extern "C"
