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
//   QK waves 0..3: wave t owns tile t. Per 128-key block: S^T of all 128 keys x 16 rows by 9
//          16x16x128 MFMAs per 16-key subtile (4 latent steps x {hi, lo} + 1 rope step packing
//          rope hi | rope lo against rope | rope), K fragments streamed from LDS through a register
//          ring; then the whole softmax inside the wave: row max, running max, P = 448 exp2(x - max)
//          -> E4M3 into LDS, row sums of the unrounded P in a fixed order, rescale factor to LDS.
//   PV waves 4..7: wave 4 + c owns latent columns 128c..128c+127 of every tile. They run one block
//          behind: O^T += V^T P^T of block i - 1 while the QK waves work on block i, so on each
//          SIMD one wave's softmax VALU overlaps the other's MFMAs. They also do the gather: raw
//          indices DMA'd into LDS two blocks ahead, row pointers, 18 row DMAs per wave one block
//          ahead into the other LDS slot, and they copy each block's V^T (ds_read_b64_tr_b8) into
//          registers while its slot is valid, so two slots suffice.
// Three barriers per block: B1 "block i landed, P of block i - 1 published", B2 "the QK waves have
// issued the MFMAs of block i" (the PV waves' MFMAs of block i - 1 then overlap the QK waves'
// softmax) and B3 "the PV waves hold P of block i - 1 and V^T of block i in registers" (the QK
// waves then write P of block i).
//
// LDS slot layout (73728 B = 8 subtiles x 9216 B). Within a 16-key subtile, the 16-byte unit of
// key k and latent chunk c (c < 32) sits at unit 32 k + (c ^ k), and rope chunk c (32..35) at
// unit 512 + 16 (c - 32) + k. A latent DMA instruction then moves two keys x 512 contiguous bytes
// (whole cache lines), and the XOR keeps both the QK operand read (16 keys x one chunk) and the
// transposed V read (8 keys x 16 columns) free of bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v2i lds_v2i;

struct Params {
    const uint16_t* q;
    const uint8_t* kv;
    int64_t num_rows;
    int page_size;
    const int32_t* table;
    int max_pages;
    const int32_t* seq_lens;
    const int32_t* rows;
    int K;
    const int32_t* valid;
    float scale_log2;   // scale * k_scale * log2(e)
    float k_scale;
    int Q, H;
    int S;
    int groups;          // dense: B, sparse: B * Q
    int rows_per_group;  // dense: Q * H, sparse: H
    int tilesets;        // (rows_per_group / 16) / T
    int gs_count;        // groups * S
    uint16_t* o;
    float* lse;
    float* ws_o;         // [B*Q*H][S][512]
    float* ws_ml;        // [B*Q*H][S][2]
    uint32_t* ws_cnt;    // [groups * tilesets]
};

// Source of the absent keys' DMA: 576 zero bytes (V rows of absent keys must be 0, not garbage,
// since 0 * NaN would poison the PV sum).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[ROW];

template <int T>
struct Smem {
    static constexpr int OFF_KV = 0;
    static constexpr int OFF_P = 2 * SLOT;                     // E4M3 P [T][16][PPITCH]
    static constexpr int OFF_ALPHA = OFF_P + T * PTILE;        // float [T*16]
    static constexpr int OFF_FM = OFF_ALPHA + T * 16 * 4;      // float [T*16]
    static constexpr int OFF_FL = OFF_FM + T * 16 * 4;         // float [T*16]
    static constexpr int OFF_KMASK = OFF_FL + T * 16 * 4;      // uint32 [2][4] key presence bits
    static constexpr int OFF_IDX = OFF_KMASK + 2 * 16;         // int32 [2][BLK] raw key indices
    static constexpr int OFF_RP = OFF_IDX + 2 * BLK * 4;       // uint64 [2][BLK] key row pointers
    static constexpr int OFF_MISC = OFF_RP + 2 * BLK * 8;      // int [4]
    static constexpr int BYTES = OFF_MISC + 16;
};
static_assert(Smem<4>::BYTES <= 163840, "LDS budget");

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ inline uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
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

template <bool DENSE>
__device__ inline const int32_t* index_ptr(const Params& p, int g, int64_t jabs)
{
    if (DENSE)
        return p.table + (int64_t)g * p.max_pages + (uint32_t)jabs / (uint32_t)p.page_size;
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
                row = (int64_t)idx * p.page_size + (int64_t)((uint32_t)jabs % (uint32_t)p.page_size);
        } else {
            row = idx;
        }
    }
    return (row >= 0 && row < p.num_rows) ? row : -1;
}

// Source address of DMA instruction i (0..8) of a subtile for this lane, from the row pointers of
// the subtile's 16 keys (rp: 16 x u64 in LDS). Latent instruction i: key 2i + lane / 32, chunk
// (lane % 32) ^ key; rope instruction 8: key lane % 16, chunk 32 + lane / 16.
__device__ inline const uint8_t* dma_src(const uint64_t* rp, int i, int lane)
{
    if (i < 8) {
        const int k = 2 * i + (lane >> 5);
        return reinterpret_cast<const uint8_t*>(rp[k]) + 16 * ((lane & 31) ^ k);
    }
    return reinterpret_cast<const uint8_t*>(rp[lane & 15]) + 512 + 16 * (lane >> 4);
}

// The work of one workgroup: key group g, split s of S, tile set ts; the split's keys
// [first, first + mine) of the group's n_grp, in nblk blocks of 128.
struct Work {
    int g, s, ts, nblk;
    int64_t n_grp, first, mine, row_base;
};

template <bool DENSE>
__device__ inline bool decode_work(const Params& p, Work& w)
{
    // a split's tile sets share one XCD (blockIdx % 8)
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int slotid = bid >> 3;
    w.ts = slotid % p.tilesets;
    const int gs = (slotid / p.tilesets) * 8 + xcd;
    if (gs >= p.gs_count)
        return false;
    w.s = gs / p.groups;
    w.g = gs % p.groups;
    if (DENSE) {
        const int64_t cap = (int64_t)p.max_pages * p.page_size;
        const int64_t sl = p.seq_lens[w.g];
        w.n_grp = sl < 0 ? 0 : (sl > cap ? cap : sl);
    } else {
        const int64_t v = p.valid[w.g];
        w.n_grp = v < 0 ? 0 : (v > p.K ? p.K : v);
    }
    // the pages' per / first / mine
    const int64_t per = (w.n_grp + p.S - 1) / p.S;
    w.first = (int64_t)w.s * per < w.n_grp ? (int64_t)w.s * per : w.n_grp;
    w.mine = (w.n_grp - w.first) < per ? (w.n_grp - w.first) : per;
    w.nblk = (int)((w.mine + BLK - 1) / BLK);
    w.row_base = (int64_t)w.g * p.rows_per_group;
    return true;
}

// ---- QK waves: Q stage, S^T = K (hi + lo)^T, softmax; P and the rescale factors to LDS ----
template <int T, bool DENSE>
__device__ __forceinline__ void qk_role(const Params& p, uint8_t* smem, const Work& w, int qw,
                                        int lane)
{
    using L = Smem<T>;
    const int n16 = lane & 15;   // MFMA row / column within 16
    const int grp = lane >> 4;   // MFMA k-group 0..3
    const bool active = qw < T;
    const int qt = active ? qw : 0;
    const int tile = w.ts * T + qt;
    int64_t lim;   // keys [0, lim) of the group are visible to this tile
    if (DENSE) {
        const int pos = (16 * tile) / p.H;
        const int64_t c = w.n_grp - p.Q + pos + 1;
        lim = c < 0 ? 0 : (c > w.n_grp ? w.n_grp : c);
    } else {
        lim = w.n_grp;
    }

    // ---- Q of this tile -> exact E4M3 hi + lo of q * 2^k (B operands) ----
    v8i qhi[4], qlo[4], qrope;
    float row_scale = 0.f;  // scale_log2 * 2^-k for row n16
    if (w.nblk > 0 && active) {
        const uint16_t* qrow = p.q + (w.row_base + 16 * tile + n16) * ROW;
        // 32 bf16 per operand step st: values q[128 st + 32 grp + 0..31] (rope: 512 + 32 (grp & 1))
        v4i raw[10], rawb[10];
#pragma unroll
        for (int st = 0; st < 5; st++) {
            const uint16_t* src = st < 4 ? qrow + 128 * st + 32 * grp : qrow + 512 + 32 * (grp & 1);
            raw[2 * st] = *reinterpret_cast<const v4i*>(src);
            raw[2 * st + 1] = *reinterpret_cast<const v4i*>(src + 8);
            rawb[2 * st] = *reinterpret_cast<const v4i*>(src + 16);
            rawb[2 * st + 1] = *reinterpret_cast<const v4i*>(src + 24);
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 10; i++) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t wa = (uint32_t)raw[i][e], wb = (uint32_t)rawb[i][e];
                amax = fmaxf(amax, fabsf(bf16_to_f32(wa & 0xFFFF)));
                amax = fmaxf(amax, fabsf(bf16_to_f32(wa >> 16)));
                amax = fmaxf(amax, fabsf(bf16_to_f32(wb & 0xFFFF)));
                amax = fmaxf(amax, fabsf(bf16_to_f32(wb >> 16)));
            }
        }
        amax = wave_max16(amax);
        // k: the largest integer with amax * 2^k <= 448 (0 for a zero row)
        int k = 0;
        if (amax > 0.f) {
            int e;
            const float m = frexpf(amax, &e);  // amax = m * 2^e, m in [0.5, 1)
            k = (2.f * m <= 1.75f) ? (9 - e) : (8 - e);
        }
        row_scale = ldexpf(p.scale_log2, -k);
        auto split4 = [&](uint32_t w0, uint32_t w1, uint32_t& hi, uint32_t& lo) {
            const float x0 = ldexpf(bf16_to_f32(w0 & 0xFFFF), k);
            const float x1 = ldexpf(bf16_to_f32(w0 >> 16), k);
            const float x2 = ldexpf(bf16_to_f32(w1 & 0xFFFF), k);
            const float x3 = ldexpf(bf16_to_f32(w1 >> 16), k);
            hi = pack_e4m3(x0, x1, x2, x3);
            const float h0 = __builtin_amdgcn_cvt_f32_fp8((int)hi, 0);
            const float h1 = __builtin_amdgcn_cvt_f32_fp8((int)hi, 1);
            const float h2 = __builtin_amdgcn_cvt_f32_fp8((int)hi, 2);
            const float h3 = __builtin_amdgcn_cvt_f32_fp8((int)hi, 3);
            lo = pack_e4m3(x0 - h0, x1 - h1, x2 - h2, x3 - h3);
        };
#pragma unroll
        for (int st = 0; st < 5; st++) {
            // dword e of the operand holds values 4e..4e+3
            const uint32_t wd[16] = {
                (uint32_t)raw[2 * st][0], (uint32_t)raw[2 * st][1], (uint32_t)raw[2 * st][2],
                (uint32_t)raw[2 * st][3], (uint32_t)raw[2 * st + 1][0], (uint32_t)raw[2 * st + 1][1],
                (uint32_t)raw[2 * st + 1][2], (uint32_t)raw[2 * st + 1][3], (uint32_t)rawb[2 * st][0],
                (uint32_t)rawb[2 * st][1], (uint32_t)rawb[2 * st][2], (uint32_t)rawb[2 * st][3],
                (uint32_t)rawb[2 * st + 1][0], (uint32_t)rawb[2 * st + 1][1],
                (uint32_t)rawb[2 * st + 1][2], (uint32_t)rawb[2 * st + 1][3]};
            v8i vh, vl;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                uint32_t h, l;
                split4(wd[2 * e], wd[2 * e + 1], h, l);
                vh[e] = (int)h;
                vl[e] = (int)l;
            }
            if (st < 4) {
                qhi[st] = vh;
                qlo[st] = vl;
            } else {
                qrope = grp < 2 ? vh : vl;  // rope step: k-groups 0,1 carry hi, 2,3 carry lo
            }
        }
    }

    // this lane's LDS byte offset within a subtile of its operand read (step st, half h)
    auto koff = [&](int st, int h) {
        return st < 4 ? 16 * (32 * n16 + ((8 * st + 2 * grp + h) ^ n16))
                      : 16 * (512 + 16 * (2 * (grp & 1) + h) + n16);
    };
    const float neg_inf = -INFINITY;
    float m_run = neg_inf;   // running max (log2 units) of row n16
    float l_run = 0.f;       // running sum of the unrounded P of that row
    float* xalpha = reinterpret_cast<float*>(smem + L::OFF_ALPHA);

    // iteration i: QK and softmax of block i (the PV waves work on block i - 1)
    for (int i = 0; i <= w.nblk; i++) {
        const int slot = i & 1;
        lds_sync();   // B1: block i landed; P of block i - 1 published
        const bool work = active && i < w.nblk;
        v4f acc[NSUB];
        if (work) {
            const uint8_t* kslot = smem + slot * SLOT;
#pragma unroll
            for (int u = 0; u < NSUB; u++) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
            // Fragment f: step f / 8, subtile f % 8. Step f issues the hi MFMA of fragment f (or its
            // packed rope MFMA) and the lo MFMA of fragment f - 1, so no MFMA waits on the one just
            // issued; a fragment stays in the ring until its lo MFMA.
            constexpr int NFRAG = 5 * NSUB;
            constexpr int AHEAD = 2, RING = AHEAD + 2;
            v8i kf[RING];
            auto load_frag = [&](int f) {
                const int st = f / NSUB, sub = f % NSUB;
                return cat(lds_read16(kslot, sub * SUBB + koff(st, 0)),
                           lds_read16(kslot, sub * SUBB + koff(st, 1)));
            };
#pragma unroll
            for (int f = 0; f < AHEAD; f++) kf[f % RING] = load_frag(f);
#pragma unroll
            for (int f = 0; f <= NFRAG; f++) {
                if (f + AHEAD < NFRAG)
                    kf[(f + AHEAD) % RING] = load_frag(f + AHEAD);
                if (f < NFRAG) {
                    const int st = f / NSUB, sub = f % NSUB;
                    acc[sub] = mfma(kf[f % RING], st < 4 ? qhi[st] : qrope, acc[sub]);
                }
                if (f >= 1 && f - 1 < 4 * NSUB) {
                    const int st = (f - 1) / NSUB, sub = (f - 1) % NSUB;
                    acc[sub] = mfma(kf[(f - 1) % RING], qlo[st], acc[sub]);
                }
            }
        }
        lds_sync();   // B2: the PV waves start on block i - 1
        uint32_t pk[NSUB];   // E4M3 P of this lane's 4 keys of each subtile
        float alpha = 1.f;
        if (work) {
            // ---- visibility of this lane's 32 keys: bit 4u + j <-> key 16u + 4 grp + j ----
            const int64_t kbase = w.first + (int64_t)i * BLK;
            const int64_t lr = lim - kbase;      // keys of the block before the tile's bound
            const int lim_rel = lr < 0 ? 0 : (lr > BLK ? BLK : (int)lr);
            const v4i mw = lds_read16(smem, L::OFF_KMASK + slot * 16);
            uint32_t vis = 0;
#pragma unroll
            for (int u = 0; u < NSUB; u++) {
                uint32_t nib = ((uint32_t)mw[u >> 1] >> (16 * (u & 1) + 4 * grp)) & 0xFu;
                const int keep = lim_rel - (16 * u + 4 * grp);   // how many of the 4 are in bound
                nib &= keep >= 4 ? 0xFu : (keep <= 0 ? 0u : ((1u << keep) - 1u));
                vis |= nib << (4 * u);
            }
            // ---- mask, row max over the block (in-lane, then across the 4 k-groups). The row
            // scale is positive, so max(s * scale) = scale * max(s) exactly. ----
            float bmax = neg_inf;
            if (!__all(vis == 0xFFFFFFFFu)) {
#pragma unroll
                for (int u = 0; u < NSUB; u++)
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        acc[u][j] = ((vis >> (4 * u + j)) & 1u) ? acc[u][j] : neg_inf;
            }
#pragma unroll
            for (int u = 0; u < NSUB; u++)
                bmax = fmaxf(bmax, fmaxf(fmaxf(acc[u][0], acc[u][1]), fmaxf(acc[u][2], acc[u][3])));
            bmax = wave_max16(bmax) * row_scale;
            const float m_new = fmaxf(m_run, bmax);
            alpha = (m_run == neg_inf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            const float m_use = (m_new == neg_inf) ? 0.f : m_new;   // exp2(-inf - m_use) = 0
            // ---- P = 448 exp2(s * scale - m) -> E4M3 (P <= 448: no clamp); row sum of the
            // unrounded P in a fixed order ----
            float bsum = 0.f;
#pragma unroll
            for (int u = 0; u < NSUB; u++) {
                float pr[4];
#pragma unroll
                for (int j = 0; j < 4; j++)
                    pr[j] = ANCHOR * __builtin_amdgcn_exp2f(fmaf(acc[u][j], row_scale, -m_use));
                int wp = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], 0, false);
                pk[u] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], wp, true);
                bsum = bsum + (((pr[0] + pr[1]) + pr[2]) + pr[3]);
            }
            bsum = wave_sum16(bsum);
            l_run = l_run * alpha + bsum;
            m_run = m_new;
        }
        lds_sync();   // B3: the PV waves have taken P of block i - 1 into registers
        if (work) {
#pragma unroll
            for (int u = 0; u < NSUB; u++)
                *reinterpret_cast<uint32_t*>(smem + L::OFF_P + qt * PTILE + n16 * PPITCH + 16 * u +
                                             4 * grp) = pk[u];
            if (grp == 0)
                xalpha[qt * 16 + n16] = alpha;
        }
    }

    // ---- epilogue: (m, l) to the column owners, LSE ----
    float* fm = reinterpret_cast<float*>(smem + L::OFF_FM);
    float* fl = reinterpret_cast<float*>(smem + L::OFF_FL);
    if (active && grp == 0) {
        fm[qt * 16 + n16] = m_run;
        fl[qt * 16 + n16] = l_run;
    }
    __syncthreads();   // E1
    const int64_t orow = w.row_base + 16 * tile + n16;
    if (p.S == 1) {
        if (active && grp == 0)
            p.lse[orow] = (l_run > 0.f) ? (m_run - LOG2_ANCHOR + log2f(l_run)) * LN2 : neg_inf;
        return;
    }
    if (active && grp == 0) {
        p.ws_ml[(orow * p.S + w.s) * 2 + 0] = m_run;
        p.ws_ml[(orow * p.S + w.s) * 2 + 1] = l_run;
    }
}

// ---- PV waves: the gather, and O^T += V^T P^T for 128 latent columns of every tile ----
template <int T, bool DENSE>
__device__ __forceinline__ void pv_role(const Params& p, uint8_t* smem, const Work& w, int pw,
                                        int lane, v4f (&O)[T][8])
{
    using L = Smem<T>;
    const int n16 = lane & 15;
    const int grp = lane >> 4;

    // Gather: this wave moves keys 32 pw .. 32 pw + 31 (subtiles 2 pw, 2 pw + 1) of every block.
    // Per block: the raw indices (page ids or row ids) arrive in an LDS slot by DMA one block
    // earlier; lanes 0..31 turn them into row pointers (the zero row when absent) and a presence
    // word; the wave then issues its 18 row DMAs.
    int32_t* idx_lds = reinterpret_cast<int32_t*>(smem + L::OFF_IDX);
    uint64_t* rpt = reinterpret_cast<uint64_t*>(smem + L::OFF_RP);
    auto dma_indices = [&](int blk) {  // raw indices of block blk -> idx slot blk % 2
        const int kk = 32 * pw + lane;
        const int64_t left = w.mine - (int64_t)blk * BLK;
        if (lane < 32 && kk < left)
            dma4(index_ptr<DENSE>(p, w.g, w.first + (int64_t)blk * BLK + kk),
                 lds_addr(smem + L::OFF_IDX + (blk & 1) * BLK * 4 + 32 * pw * 4));
    };
    auto prepare_rows = [&](int blk, int32_t idx) {  // idx: raw index of key 32 pw + lane
        const int kk = 32 * pw + lane;
        const int64_t left = w.mine - (int64_t)blk * BLK;
        const bool in = lane < 32 && kk < left;
        const int64_t row = key_row<DENSE>(p, w.first + (int64_t)blk * BLK + kk, in, idx);
        const uint64_t ptr = row >= 0 ? (uint64_t)(uintptr_t)(p.kv + row * ROW)
                                      : (uint64_t)(uintptr_t)g_zero_row;
        if (lane < 32)
            rpt[(blk & 1) * BLK + kk] = ptr;
        const uint32_t word = (uint32_t)__ballot(row >= 0);   // lanes 0..31: keys 32 pw + lane
        if (lane == 0)
            *reinterpret_cast<uint32_t*>(smem + L::OFF_KMASK + (blk & 1) * 16 + 4 * pw) = word;
    };
    auto issue_block = [&](int blk) {   // this wave's 18 row DMAs of block blk
#pragma unroll
        for (int i = 0; i < 18; i++) {
            const int sub = 2 * pw + i / 9;
            const uint8_t* src = dma_src(rpt + (blk & 1) * BLK + 16 * sub, i % 9, lane);
            dma16(src, lds_addr(smem + (blk & 1) * SLOT + sub * SUBB + 1024 * (i % 9)));
        }
    };
    if (w.nblk > 0) {
        int32_t idx0 = -1;
        if (lane < 32 && 32 * pw + lane < w.mine)
            idx0 = *index_ptr<DENSE>(p, w.g, w.first + 32 * pw + lane);
        prepare_rows(0, idx0);
        issue_block(0);
        if (w.nblk > 1)
            dma_indices(1);
    }

    // this lane's LDS byte offset within a subtile of its transposed V read (column chunk
    // 8 pw + c, key half rb)
    auto voff = [&](int c, int rb) {
        const int kk = 8 * rb + (n16 >> 1), cc = 8 * pw + c;
        return 2 * grp * SUBB + 16 * (32 * kk + (cc ^ kk)) + 8 * (n16 & 1);
    };
    auto load_vt = [&](int slot, int c) {
        v2i tr[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int off = slot * SLOT + (r >> 1) * SUBB + voff(c, r & 1);
            tr[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(smem + off));
        }
        return v8i{tr[0].x, tr[0].y, tr[1].x, tr[1].y, tr[2].x, tr[2].y, tr[3].x, tr[3].y};
    };
    const float* xalpha = reinterpret_cast<const float*>(smem + L::OFF_ALPHA);
    v8i vt[8];   // V^T of the block the next iteration multiplies (copied while its slot is valid)

    // iteration i: gather of block i + 1; PV of block i - 1; V^T of block i into registers
    for (int i = 0; i <= w.nblk; i++) {
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's DMAs of block i (and indices)
        lds_sync();   // B1: block i landed; P of block i - 1 published
        if (i + 1 < w.nblk) {
            prepare_rows(i + 1, lane < 32 ? idx_lds[((i + 1) & 1) * BLK + 32 * pw + lane] : -1);
            issue_block(i + 1);
        }
        if (i + 2 < w.nblk)
            dma_indices(i + 2);
        if (i >= 1) {   // rescale O for block i - 1 while the QK waves issue their MFMAs
#pragma unroll
            for (int t = 0; t < T; t++) {
                const float a = xalpha[t * 16 + n16];
                if (!__all(a == 1.f)) {
#pragma unroll
                    for (int c = 0; c < 8; c++) O[t][c] *= a;
                }
            }
        }
        lds_sync();   // B2: the QK waves have issued their MFMAs of block i
        if (i >= 1) {
#pragma unroll
            for (int t = 0; t < T; t++) {
                const int off = L::OFF_P + t * PTILE + n16 * PPITCH + 32 * grp;
                const v8i pb = cat(lds_read16(smem, off), lds_read16(smem, off + 16));
#pragma unroll
                for (int c = 0; c < 8; c++) O[t][c] = mfma(vt[c], pb, O[t][c]);
            }
        }
        if (i < w.nblk) {
#pragma unroll
            for (int c = 0; c < 8; c++) vt[c] = load_vt(i & 1, c);
        }
        lds_sync();   // B3: P of block i - 1 and V^T of block i are in registers
    }

    // ---- epilogue ----
    __syncthreads();   // E1: (m, l) of every row in LDS
    const float* fl = reinterpret_cast<const float*>(smem + L::OFF_FL);
    if (p.S == 1) {
        // o = BF16(O / l * k_scale); the single-split merge (weight exp2(0) = 1) is this exactly
#pragma unroll
        for (int t = 0; t < T; t++) {
            const float lt = fl[t * 16 + n16];
            const int64_t orow = w.row_base + 16 * (w.ts * T + t) + n16;
#pragma unroll
            for (int c = 0; c < 8; c++) {
                const int col = 128 * pw + 16 * c + 4 * grp;
                uint32_t b0 = 0, b1 = 0, b2 = 0, b3 = 0;
                if (lt > 0.f) {
                    b0 = f32_to_bf16_rne(O[t][c][0] / lt * p.k_scale);
                    b1 = f32_to_bf16_rne(O[t][c][1] / lt * p.k_scale);
                    b2 = f32_to_bf16_rne(O[t][c][2] / lt * p.k_scale);
                    b3 = f32_to_bf16_rne(O[t][c][3] / lt * p.k_scale);
                }
                v2i wv = v2i{(int)(b0 | (b1 << 16)), (int)(b2 | (b3 << 16))};
                *reinterpret_cast<v2i*>(p.o + orow * LATENT + col) = wv;
            }
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < T; t++) {
        const int64_t orow = w.row_base + 16 * (w.ts * T + t) + n16;
#pragma unroll
        for (int c = 0; c < 8; c++) {
            const int col = 128 * pw + 16 * c + 4 * grp;
            *reinterpret_cast<v4f*>(p.ws_o + (orow * p.S + w.s) * LATENT + col) = O[t][c];
        }
    }
}

// The last arriving split of a (group, tile set) merges the FP32 partials in split order.
template <int T>
__device__ void merge_splits(const Params& p, const Work& w, int tid)
{
    const float neg_inf = -INFINITY;
    for (int item = tid; item < T * 16 * 32; item += THREADS) {
        const int r = item >> 5;
        const int c0 = (item & 31) * 16;
        const int64_t orow = w.row_base + 16 * w.ts * T + r;
        const float* ml = p.ws_ml + orow * p.S * 2;
        float top = neg_inf;
        for (int q = 0; q < p.S; q++) top = fmaxf(top, ml[2 * q]);
        float total = 0.f;
        float acc[16];
#pragma unroll
        for (int e = 0; e < 16; e++) acc[e] = 0.f;
        if (top != neg_inf) {
            for (int q = 0; q < p.S; q++) {
                const float mq = ml[2 * q];
                if (mq == neg_inf)
                    continue;
                const float wq = exp2f(mq - top);
                total = total + wq * ml[2 * q + 1];
                const v4f* src = reinterpret_cast<const v4f*>(p.ws_o + (orow * p.S + q) * LATENT + c0);
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const v4f x4 = src[v];
#pragma unroll
                    for (int e = 0; e < 4; e++) acc[4 * v + e] = acc[4 * v + e] + wq * x4[e];
                }
            }
        }
        uint32_t bits[16];
#pragma unroll
        for (int e = 0; e < 16; e++) bits[e] = total > 0.f ? f32_to_bf16_rne(acc[e] / total * p.k_scale) : 0u;
        v4i w0 = v4i{(int)(bits[0] | (bits[1] << 16)), (int)(bits[2] | (bits[3] << 16)),
                     (int)(bits[4] | (bits[5] << 16)), (int)(bits[6] | (bits[7] << 16))};
        v4i w1 = v4i{(int)(bits[8] | (bits[9] << 16)), (int)(bits[10] | (bits[11] << 16)),
                     (int)(bits[12] | (bits[13] << 16)), (int)(bits[14] | (bits[15] << 16))};
        *reinterpret_cast<v4i*>(p.o + orow * LATENT + c0) = w0;
        *reinterpret_cast<v4i*>(p.o + orow * LATENT + c0 + 8) = w1;
        if ((item & 31) == 0)
            p.lse[orow] = total > 0.f ? (top - LOG2_ANCHOR + log2f(total)) * LN2 : neg_inf;
    }
}

template <int T, bool DENSE>
__global__ __launch_bounds__(THREADS) void mla_decode_kernel(const Params p)
{
    using L = Smem<T>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[L::BYTES];
    Work w;
    if (!decode_work<DENSE>(p, w))
        return;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    // waves 0..3: QK (tile = wave); waves 4..7: gather + PV (columns 128 (wave - 4) ..); wave i runs
    // on SIMD i % 4, so each SIMD pairs one QK wave with one PV wave
    if (wave < 4) {
        qk_role<T, DENSE>(p, smem, w, wave, lane);
    } else {
        v4f O[T][8];
#pragma unroll
        for (int t = 0; t < T; t++)
#pragma unroll
            for (int c = 0; c < 8; c++) O[t][c] = v4f{0.f, 0.f, 0.f, 0.f};
        pv_role<T, DENSE>(p, smem, w, wave - 4, lane, O);
    }
    if (p.S == 1)
        return;
    // S > 1: every thread's partial stores completed (vmcnt(0)) before the barrier; one thread then
    // releases them at agent scope and counts this split in; the last arriver merges.
    __builtin_amdgcn_s_waitcnt(0xF70);
    __syncthreads();   // E2
    int* misc = reinterpret_cast<int*>(smem + L::OFF_MISC);
    uint32_t* cnt = p.ws_cnt + (int64_t)w.g * p.tilesets + w.ts;
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        misc[0] = (old == (uint32_t)(p.S - 1)) ? 1 : 0;
    }
    __syncthreads();   // E3
    if (misc[0] == 0)
        return;
    merge_splits<T>(p, w, tid);
    if (tid == 0)
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

WsLayout ws_layout(int B, int Q, int H, int S)
{
    WsLayout w{};
    if (S <= 1)
        return w;
    const size_t rows = (size_t)B * Q * H;
    w.cnt_bytes = round_up(rows / 16 * sizeof(uint32_t), ALIGN_WS);
    w.ml_bytes = round_up(rows * S * 2 * sizeof(float), ALIGN_WS);
    w.o_bytes = round_up(rows * S * LATENT * sizeof(float), ALIGN_WS);
    w.total = w.cnt_bytes + w.ml_bytes + w.o_bytes;
    return w;
}

int choose_tiles(int tiles_per_group)
{
    if (tiles_per_group % 4 == 0)
        return 4;
    if (tiles_per_group % 2 == 0)
        return 2;
    return 1;
}

// Splits from shapes only: enough workgroups to cover the 256 CUs once (one workgroup fills a CU's
// LDS), each with at least two 128-key blocks of its group's key capacity; every extra split adds
// a partial per row and a merge.
int choose_splits(int groups, int tilesets, int64_t max_keys)
{
    const int64_t wgs = (int64_t)groups * tilesets;
    int64_t s = 256 / wgs;
    const int64_t cap = max_keys / (2 * BLK);
    if (s > cap)
        s = cap;
    if (s < 1)
        s = 1;
    if (s > 64)
        s = 64;
    return (int)s;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

template <int T, bool DENSE>
hipError_t launch_t(const Params& p, hipStream_t stream)
{
    const int64_t gs_pad = ((int64_t)p.gs_count + 7) / 8 * 8;
    const int64_t grid = gs_pad * p.tilesets;
    hipLaunchKernelGGL((mla_decode_kernel<T, DENSE>), dim3((unsigned)grid), dim3(THREADS), 0, stream,
                       p);
    return hipGetLastError();
}

template <bool DENSE>
hipError_t launch(int T, const Params& p, hipStream_t stream)
{
    switch (T) {
    case 1: return launch_t<1, DENSE>(p, stream);
    case 2: return launch_t<2, DENSE>(p, stream);
    default: return launch_t<4, DENSE>(p, stream);
    }
}

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
    if (!aligned(q, 16) || !aligned(kv->data, 16) || !aligned(o, 8) || !aligned(lse, 4))
        return MLA_ERR_ALIGN;
    return MLA_OK;
}

mla_status_t finish_plan(const mla_plan_t* in, mla_plan_t chosen, int tiles_per_group, int B, int Q,
                         int H, void* ws, size_t ws_bytes, mla_plan_t* out)
{
    mla_plan_t pl = in ? *in : chosen;
    if (pl.splits < 1 || pl.splits > 4096)
        return MLA_ERR_UNSUPPORTED;
    if (!(pl.tiles == 1 || pl.tiles == 2 || pl.tiles == 4) || tiles_per_group % pl.tiles != 0)
        return MLA_ERR_UNSUPPORTED;
    if (pl.splits > 1) {
        const WsLayout w = ws_layout(B, Q, H, pl.splits);
        if (!ws || ws_bytes < w.total)
            return MLA_ERR_WORKSPACE;
        if (!aligned(ws, ALIGN_WS))
            return MLA_ERR_ALIGN;
    }
    *out = pl;
    return MLA_OK;
}

void fill_workspace(Params& p, int B, int Q, int H, void* ws)
{
    const WsLayout w = ws_layout(B, Q, H, p.S);
    uint8_t* base = (uint8_t*)ws;
    p.ws_cnt = p.S > 1 ? (uint32_t*)base : nullptr;
    p.ws_ml = p.S > 1 ? (float*)(base + w.cnt_bytes) : nullptr;
    p.ws_o = p.S > 1 ? (float*)(base + w.cnt_bytes + w.ml_bytes) : nullptr;
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

size_t mla_workspace_bytes(int B, int Q, int H, int splits)
{
    if (B <= 0 || Q <= 0 || H <= 0)
        return 0;
    return ws_layout(B, Q, H, splits).total;
}

size_t mla_workspace_zero_bytes(int B, int Q, int H, int splits)
{
    if (B <= 0 || Q <= 0 || H <= 0)
        return 0;
    return ws_layout(B, Q, H, splits).cnt_bytes;
}

mla_status_t mla_plan_dense(int B, int Q, int H, int max_pages, int page_size, mla_plan_t* plan)
{
    if (!plan)
        return MLA_ERR_NULL;
    if (B < 0 || Q < 1 || H < 16 || H % 16 != 0 || max_pages < 1 || page_size < 1)
        return MLA_ERR_SHAPE;
    const int tpg = Q * H / 16;
    plan->tiles = choose_tiles(tpg);
    plan->splits = choose_splits(B > 0 ? B : 1, tpg / plan->tiles, (int64_t)max_pages * page_size);
    return MLA_OK;
}

mla_status_t mla_plan_sparse(int B, int Q, int H, int K, mla_plan_t* plan)
{
    if (!plan)
        return MLA_ERR_NULL;
    if (B < 0 || Q < 1 || H < 16 || H % 16 != 0 || K < 1)
        return MLA_ERR_SHAPE;
    const int tpg = H / 16;
    plan->tiles = choose_tiles(tpg);
    plan->splits = choose_splits(B > 0 ? B * Q : 1, tpg / plan->tiles, K);
    return MLA_OK;
}

mla_status_t mla_decode_dense(const void* q, const mla_kv_t* kv, const int32_t* block_table,
                              int max_pages, const int32_t* seq_lens, float scale, int B, int Q,
                              int H, const mla_plan_t* plan, void* o, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    mla_status_t st = common_checks(q, kv, B, Q, H, o, lse);
    if (st != MLA_OK || B == 0)
        return st;
    if (max_pages < 1 || kv->page_size < 1)
        return MLA_ERR_SHAPE;
    if (!block_table || !seq_lens)
        return MLA_ERR_NULL;
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
        return MLA_ERR_ALIGN;
    mla_plan_t chosen;
    mla_plan_dense(B, Q, H, max_pages, kv->page_size, &chosen);
    mla_plan_t pl;
    st = finish_plan(plan, chosen, Q * H / 16, B, Q, H, workspace, workspace_bytes, &pl);
    if (st != MLA_OK)
        return st;
    Params p{};
    p.q = (const uint16_t*)q;
    p.kv = (const uint8_t*)kv->data;
    p.num_rows = kv->num_rows;
    p.page_size = kv->page_size;
    p.table = block_table;
    p.max_pages = max_pages;
    p.seq_lens = seq_lens;
    p.scale_log2 = (float)((double)scale * (double)kv->k_scale * 1.4426950408889634);
    p.k_scale = kv->k_scale;
    p.Q = Q;
    p.H = H;
    p.S = pl.splits;
    p.groups = B;
    p.rows_per_group = Q * H;
    p.tilesets = Q * H / 16 / pl.tiles;
    p.gs_count = B * pl.splits;
    p.o = (uint16_t*)o;
    p.lse = lse;
    fill_workspace(p, B, Q, H, workspace);
    if (launch<true>(pl.tiles, p, (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_LAUNCH;
    return MLA_OK;
}

mla_status_t mla_decode_sparse(const void* q, const mla_kv_t* kv, const int32_t* rows, int K,
                               const int32_t* valid, float scale, int B, int Q, int H,
                               const mla_plan_t* plan, void* o, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream)
{
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
    mla_plan_t pl;
    st = finish_plan(plan, chosen, H / 16, B, Q, H, workspace, workspace_bytes, &pl);
    if (st != MLA_OK)
        return st;
    Params p{};
    p.q = (const uint16_t*)q;
    p.kv = (const uint8_t*)kv->data;
    p.num_rows = kv->num_rows;
    p.page_size = 1;
    p.rows = rows;
    p.K = K;
    p.valid = valid;
    p.scale_log2 = (float)((double)scale * (double)kv->k_scale * 1.4426950408889634);
    p.k_scale = kv->k_scale;
    p.Q = Q;
    p.H = H;
    p.S = pl.splits;
    p.groups = B * Q;
    p.rows_per_group = H;
    p.tilesets = H / 16 / pl.tiles;
    p.gs_count = B * Q * pl.splits;
    p.o = (uint16_t*)o;
    p.lse = lse;
    fill_workspace(p, B, Q, H, workspace);
    if (launch<false>(pl.tiles, p, (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_LAUNCH;
    return MLA_OK;
}

}  // extern "C"
