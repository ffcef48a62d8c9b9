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
// Workgroup = (key group, split, set of T 16-row tiles), 512 threads = 8 waves. Per 128-key block:
//   DMA    wave w gathers keys 16w..16w+15 of the next block into the other LDS slot (9 x 1 KB
//          global_load_lds_dwordx4); absent keys read a zero row.
//   QK     wave w: tile w % T, key subtiles (w / T) * T .. + T - 1; 9 MFMAs per subtile (4 latent steps
//          x {hi, lo} + 1 rope step packing rope hi | rope lo against rope | rope).
//   softmax  row max over the 8 subtiles through LDS; P -> E4M3 into LDS; per-subtile row sums
//          through LDS, added in subtile order 0..7 (so the result does not depend on T).
//   PV     wave w: latent columns 64w..64w+63 of every tile; O^T += V^T P^T, 4 MFMAs per tile.
//
// LDS slot layout (73728 B = 8 subtiles x 9216 B): within a 16-key subtile the 16-byte unit
// (chunk c of the 36 in a row, key k) sits at (c * 16 + k) * 16. Consecutive lanes of a DMA
// instruction then fill consecutive units (lane l: key l % 16, chunk 4i + l / 16), the QK operand
// read of 16 keys x one chunk is 256 contiguous bytes, and the transposed V reads of 8 keys x 16
// columns are 128 contiguous bytes.
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
    static constexpr int OFF_P = 2 * SLOT;
    static constexpr int OFF_XM = OFF_P + T * PTILE;           // float [NSUB][T*16]
    static constexpr int OFF_XS = OFF_XM + NSUB * T * 16 * 4;  // float [NSUB][T*16]
    static constexpr int OFF_ALPHA = OFF_XS + NSUB * T * 16 * 4;  // float [T*16]
    static constexpr int OFF_FM = OFF_ALPHA + T * 16 * 4;      // float [T*16]
    static constexpr int OFF_FL = OFF_FM + T * 16 * 4;         // float [T*16]
    static constexpr int OFF_FLAG = OFF_FL + T * 16 * 4;       // uint8 [2][BLK]
    static constexpr int OFF_MISC = OFF_FLAG + 2 * BLK;        // int [4]
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

__device__ inline float wave_max16(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ inline float wave_sum16(float v)
{
    v = v + __shfl_xor(v, 16);
    v = v + __shfl_xor(v, 32);
    return v;
}

// The 32-bit LDS address of a pointer into __shared__ memory (wave-uniform by construction).
__device__ inline uint32_t lds_addr(const uint8_t* ptr)
{
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ptr);
}

// One global_load_lds_dwordx4: 16 bytes at this lane's gsrc -> LDS byte lds_base + 16 * lane.
// Written in asm so that the compiler's wait-count pass does not treat every later LDS read as
// depending on this DMA (it would wait for the next block's DMA before reading the current one);
// the kernel waits for the DMA itself (vmcnt(0)) before the barrier that publishes a block. M0 is
// saved and restored around the instruction.
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

template <bool DENSE>
__device__ inline int32_t fetch_index(const Params& p, int g, int64_t jabs, bool inrange)
{
    if (!inrange)
        return -1;
    if (DENSE)
        return __builtin_nontemporal_load(p.table + (int64_t)g * p.max_pages + jabs / p.page_size);
    return __builtin_nontemporal_load(p.rows + (int64_t)g * p.K + jabs);
}

// Issue the 9 DMAs of this wave's 16 keys of a block into LDS slot `slot` and record each key's
// presence flag. `idx` is the raw index fetched for this lane's key (-1 past the block's count).
template <bool DENSE>
__device__ inline void issue_block(const Params& p, uint8_t* smem, int slot, int wave, int lane,
                                   int64_t jabs, bool inrange, int32_t idx, int flag_off)
{
    int64_t row = -1;
    if (inrange) {
        if (DENSE) {
            if (idx >= 0)
                row = (int64_t)idx * p.page_size + jabs % p.page_size;
        } else {
            row = idx;
        }
    }
    const bool ok = row >= 0 && row < p.num_rows;
    const uint8_t* src = ok ? p.kv + row * ROW : g_zero_row;
    src += 16 * (lane >> 4);
    const uint32_t dst = lds_addr(smem + slot * SLOT + wave * SUBB);
#pragma unroll
    for (int i = 0; i < 9; i++)
        dma16(src + 64 * i, dst + 1024 * i);
    if ((lane >> 4) == 0)
        smem[flag_off + slot * BLK + wave * 16 + (lane & 15)] = ok ? 1 : 0;
}

template <int T, bool DENSE>
__global__ __launch_bounds__(THREADS) void mla_decode_kernel(const Params p)
{
    using L = Smem<T>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[L::BYTES];

    // ---- which (key group, split, tile set): a split's tile sets share one XCD (blockIdx % 8) ----
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int slotid = bid >> 3;
    const int ts = slotid % p.tilesets;
    const int gs = (slotid / p.tilesets) * 8 + xcd;
    if (gs >= p.gs_count)
        return;
    const int s = gs / p.groups;
    const int g = gs % p.groups;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n16 = lane & 15;   // MFMA row / column within 16
    const int grp = lane >> 4;   // MFMA k-group 0..3

    // ---- key range of this split (the pages' per / first / mine) ----
    int64_t n_grp;
    if (DENSE) {
        const int64_t cap = (int64_t)p.max_pages * p.page_size;
        const int64_t sl = p.seq_lens[g];
        n_grp = sl < 0 ? 0 : (sl > cap ? cap : sl);
    } else {
        const int64_t v = p.valid[g];
        n_grp = v < 0 ? 0 : (v > p.K ? p.K : v);
    }
    const int64_t per = (n_grp + p.S - 1) / p.S;
    const int64_t first = (int64_t)s * per < n_grp ? (int64_t)s * per : n_grp;
    const int64_t mine = (n_grp - first) < per ? (n_grp - first) : per;
    const int nblk = (int)((mine + BLK - 1) / BLK);

    // ---- this wave's QK tile and keys ----
    const int qt = wave % T;              // tile within the set
    const int kw = wave / T;              // which T-subtile slice of the block
    const int tile = ts * T + qt;         // tile within the key group
    int64_t lim;                          // keys [0, lim) of the group are visible to this tile
    if (DENSE) {
        const int pos = (16 * tile) / p.H;
        int64_t c = n_grp - p.Q + pos + 1;
        lim = c < 0 ? 0 : (c > n_grp ? n_grp : c);
    } else {
        lim = n_grp;
    }
    const int64_t row_base = (int64_t)g * p.rows_per_group;  // first output row of the group

    // ---- the DMA prologue: block 0 now, block 1's index in flight ----
    const int dkey = 16 * wave + n16;
    int32_t idx_next = -1;
    if (nblk > 0) {
        const int64_t j0 = first + dkey;
        const bool in0 = dkey < mine;
        const int32_t i0 = fetch_index<DENSE>(p, g, j0, in0);
        issue_block<DENSE>(p, smem, 0, wave, lane, j0, in0, i0, L::OFF_FLAG);
        if (nblk > 1) {
            const int64_t j1 = first + BLK + dkey;
            idx_next = fetch_index<DENSE>(p, g, j1, dkey < mine - BLK);
        }
    }

    // ---- Q of this wave's tile -> exact E4M3 hi + lo of q * 2^k (B operands) ----
    v8i qhi[4], qlo[4], qrope;
    float row_scale = 0.f;  // scale_log2 * 2^-k for row n16 of tile qt
    if (nblk > 0) {
        const uint16_t* qrow = p.q + (row_base + 16 * tile + n16) * ROW;
        v4i raw[10];  // 8 bf16 per v4i: [p*2 + h] latent step p half h; [8], [9] rope
#pragma unroll
        for (int st = 0; st < 4; st++) {
            raw[2 * st] = *reinterpret_cast<const v4i*>(qrow + 128 * st + 32 * grp);
            raw[2 * st + 1] = *reinterpret_cast<const v4i*>(qrow + 128 * st + 32 * grp + 8);
        }
        // (32 bf16 per step = 4 x v4i; loaded in two passes below to bound registers)
        float amax = 0.f;
        v4i rawb[10];
#pragma unroll
        for (int st = 0; st < 4; st++) {
            rawb[2 * st] = *reinterpret_cast<const v4i*>(qrow + 128 * st + 32 * grp + 16);
            rawb[2 * st + 1] = *reinterpret_cast<const v4i*>(qrow + 128 * st + 32 * grp + 24);
        }
        raw[8] = *reinterpret_cast<const v4i*>(qrow + 512 + 32 * (grp & 1));
        raw[9] = *reinterpret_cast<const v4i*>(qrow + 512 + 32 * (grp & 1) + 8);
        rawb[8] = *reinterpret_cast<const v4i*>(qrow + 512 + 32 * (grp & 1) + 16);
        rawb[9] = *reinterpret_cast<const v4i*>(qrow + 512 + 32 * (grp & 1) + 24);
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
            // amax = (2m) 2^(e-1); (2m) 2^(e-1+k) <= 1.75 * 2^8
            k = (2.f * m <= 1.75f) ? (8 - (e - 1)) : (7 - (e - 1));
        }
        row_scale = ldexpf(p.scale_log2, -k);
        auto split8 = [&](v4i a, v4i b, int word, uint32_t& hi, uint32_t& lo) {
            // word 0..3 of the 8-dword operand: a holds dwords 0..3 (bf16 0..7), b dwords 4..7
            const uint32_t w0 = (uint32_t)(word < 2 ? a[2 * word] : b[2 * (word - 2)]);
            const uint32_t w1 = (uint32_t)(word < 2 ? a[2 * word + 1] : b[2 * (word - 2) + 1]);
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
        // operand step st: 32 bytes = 32 values q[128 st + 32 grp + 0..31]; raw[2st] holds values
        // 0..7, raw[2st+1] 8..15, rawb[2st] 16..23, rawb[2st+1] 24..31
#pragma unroll
        for (int st = 0; st < 5; st++) {
            const v4i r0 = raw[2 * st], r1 = raw[2 * st + 1], r2 = rawb[2 * st], r3 = rawb[2 * st + 1];
            uint32_t h[8], l[8];
            split8(r0, r1, 0, h[0], l[0]);
            split8(r0, r1, 1, h[1], l[1]);
            split8(r0, r1, 2, h[2], l[2]);
            split8(r0, r1, 3, h[3], l[3]);
            split8(r2, r3, 0, h[4], l[4]);
            split8(r2, r3, 1, h[5], l[5]);
            split8(r2, r3, 2, h[6], l[6]);
            split8(r2, r3, 3, h[7], l[7]);
            v8i vh, vl;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                vh[e] = (int)h[e];
                vl[e] = (int)l[e];
            }
            if (st < 4) {
                qhi[st] = vh;
                qlo[st] = vl;
            } else {
                qrope = grp < 2 ? vh : vl;  // rope step: k-groups 0,1 carry hi, 2,3 carry lo
            }
        }
    }

    // ---- the block loop ----
    float m_run = -INFINITY;   // running max (log2 units) of row n16 of tile qt
    float l_run = 0.f;         // running sum (leader waves kw == 0 only)
    v4f O[T][4];
#pragma unroll
    for (int t = 0; t < T; t++)
#pragma unroll
        for (int c = 0; c < 4; c++) O[t][c] = v4f{0.f, 0.f, 0.f, 0.f};

    const float neg_inf = -INFINITY;
    float* xm = reinterpret_cast<float*>(smem + L::OFF_XM);
    float* xs = reinterpret_cast<float*>(smem + L::OFF_XS);
    float* xalpha = reinterpret_cast<float*>(smem + L::OFF_ALPHA);

    for (int b = 0; b < nblk; b++) {
        const int slot = b & 1;
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's DMA of block b (and index) landed
        lds_sync();                          // every wave's DMA landed; slot ^ 1 is free
        if (b + 1 < nblk) {
            const int64_t j = first + (int64_t)(b + 1) * BLK + dkey;
            const bool in = dkey < mine - (int64_t)(b + 1) * BLK;
            issue_block<DENSE>(p, smem, slot ^ 1, wave, lane, j, in, idx_next, L::OFF_FLAG);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (b + 2 < nblk) {
            const int64_t j = first + (int64_t)(b + 2) * BLK + dkey;
            idx_next = fetch_index<DENSE>(p, g, j, dkey < mine - (int64_t)(b + 2) * BLK);
        }

        // ---- QK: S^T of this wave's T subtiles ----
        const uint8_t* kslot = smem + slot * SLOT;
        v4f acc[T];
#pragma unroll
        for (int u = 0; u < T; u++) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 5; st++) {
            const int c0 = st < 4 ? 8 * st + 2 * grp : 32 + 2 * (grp & 1);
#pragma unroll
            for (int u = 0; u < T; u++) {
                const int sub = kw * T + u;
                const int off = sub * SUBB + (c0 * 16 + n16) * 16;
                const v8i a = cat(lds_read16(kslot, off), lds_read16(kslot, off + 256));
                if (st < 4) {
                    acc[u] = mfma(a, qhi[st], acc[u]);
                    acc[u] = mfma(a, qlo[st], acc[u]);
                } else {
                    acc[u] = mfma(a, qrope, acc[u]);
                }
            }
        }

        // ---- scale, mask, row max over this wave's keys ----
        const int64_t kbase = first + (int64_t)b * BLK;
        float x[T][4];
        float wmax = neg_inf;
#pragma unroll
        for (int u = 0; u < T; u++) {
            const int sub = kw * T + u;
            const int kin = 16 * sub + 4 * grp;  // first of this lane's 4 keys in the block
            const uint32_t fl = *reinterpret_cast<const uint32_t*>(smem + L::OFF_FLAG + slot * BLK + kin);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const bool vis = ((fl >> (8 * j)) & 0xFF) && (kbase + kin + j < lim);
                x[u][j] = vis ? acc[u][j] * row_scale : neg_inf;
                wmax = fmaxf(wmax, x[u][j]);
            }
        }
        wmax = wave_max16(wmax);
        if (grp == 0)
            xm[kw * T * 16 + qt * 16 + n16] = wmax;
        lds_sync();

        // ---- running max, P (E4M3 at 448), per-subtile row sums ----
        float bmax = neg_inf;
#pragma unroll
        for (int w = 0; w < WAVES / T; w++) bmax = fmaxf(bmax, xm[w * T * 16 + qt * 16 + n16]);
        const float m_new = fmaxf(m_run, bmax);
        const float alpha = (m_run == neg_inf) ? 1.f : exp2f(m_run - m_new);
#pragma unroll
        for (int u = 0; u < T; u++) {
            const int sub = kw * T + u;
            float pr[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                pr[j] = (x[u][j] == neg_inf) ? 0.f : ANCHOR * exp2f(x[u][j] - m_new);
            const uint32_t packed = pack_e4m3(pr[0], pr[1], pr[2], pr[3]);
            *reinterpret_cast<uint32_t*>(smem + L::OFF_P + qt * PTILE + n16 * PPITCH + 16 * sub +
                                         4 * grp) = packed;
            float ssum = ((pr[0] + pr[1]) + pr[2]) + pr[3];
            ssum = wave_sum16(ssum);
            if (grp == 0)
                xs[sub * T * 16 + qt * 16 + n16] = ssum;
        }
        if (kw == 0 && grp == 0)
            xalpha[qt * 16 + n16] = alpha;
        m_run = m_new;
        lds_sync();

        // ---- l update (leader waves): block sum in subtile order ----
        if (kw == 0) {
            float bsum = 0.f;
#pragma unroll
            for (int sub = 0; sub < NSUB; sub++) bsum = bsum + xs[sub * T * 16 + qt * 16 + n16];
            l_run = l_run * alpha + bsum;
        }

        // ---- PV: O^T[64 columns of this wave] += V^T P^T for every tile ----
        v8i pb[T];
#pragma unroll
        for (int t = 0; t < T; t++) {
            const float a = xalpha[t * 16 + n16];
#pragma unroll
            for (int c = 0; c < 4; c++) O[t][c] *= a;
            const int off = L::OFF_P + t * PTILE + n16 * PPITCH + 32 * grp;
            pb[t] = cat(lds_read16(smem, off), lds_read16(smem, off + 16));
        }
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int chunk = 4 * wave + c;
            v2i tr[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int off = slot * SLOT + (2 * grp + (r >> 1)) * SUBB +
                                (chunk * 16 + 8 * (r & 1) + (n16 >> 1)) * 16 + 8 * (n16 & 1);
                tr[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(smem + off));
            }
            const v8i va = v8i{tr[0].x, tr[0].y, tr[1].x, tr[1].y, tr[2].x, tr[2].y, tr[3].x, tr[3].y};
#pragma unroll
            for (int t = 0; t < T; t++) O[t][c] = mfma(va, pb[t], O[t][c]);
        }
    }

    // ---- per-row (m, l) to LDS for the column owners ----
    float* fm = reinterpret_cast<float*>(smem + L::OFF_FM);
    float* fl = reinterpret_cast<float*>(smem + L::OFF_FL);
    if (kw == 0 && grp == 0) {
        fm[qt * 16 + n16] = m_run;
        fl[qt * 16 + n16] = l_run;
    }
    __syncthreads();

    if (p.S == 1) {
        // o = BF16(O / l * k_scale); the single-split merge (weight exp2(0) = 1) is this exactly
#pragma unroll
        for (int t = 0; t < T; t++) {
            const float lt = fl[t * 16 + n16];
            const int64_t orow = row_base + 16 * (ts * T + t) + n16;
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int col = 64 * wave + 16 * c + 4 * grp;
                uint32_t b0 = 0, b1 = 0, b2 = 0, b3 = 0;
                if (lt > 0.f) {
                    b0 = f32_to_bf16_rne(O[t][c][0] / lt * p.k_scale);
                    b1 = f32_to_bf16_rne(O[t][c][1] / lt * p.k_scale);
                    b2 = f32_to_bf16_rne(O[t][c][2] / lt * p.k_scale);
                    b3 = f32_to_bf16_rne(O[t][c][3] / lt * p.k_scale);
                }
                v2i w = v2i{(int)(b0 | (b1 << 16)), (int)(b2 | (b3 << 16))};
                *reinterpret_cast<v2i*>(p.o + orow * LATENT + col) = w;
            }
        }
        if (kw == 0 && grp == 0) {
            const int64_t orow = row_base + 16 * tile + n16;
            p.lse[orow] = (l_run > 0.f) ? (m_run - LOG2_ANCHOR + log2f(l_run)) * LN2 : neg_inf;
        }
        return;
    }

    // ---- S > 1: emit this split's FP32 partial, then the last arriver merges ----
#pragma unroll
    for (int t = 0; t < T; t++) {
        const int64_t orow = row_base + 16 * (ts * T + t) + n16;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int col = 64 * wave + 16 * c + 4 * grp;
            *reinterpret_cast<v4f*>(p.ws_o + (orow * p.S + s) * LATENT + col) = O[t][c];
        }
    }
    if (kw == 0 && grp == 0) {
        const int64_t orow = row_base + 16 * tile + n16;
        p.ws_ml[(orow * p.S + s) * 2 + 0] = m_run;
        p.ws_ml[(orow * p.S + s) * 2 + 1] = l_run;
    }
    __threadfence();   // release this thread's partial at agent scope
    __syncthreads();
    int* misc = reinterpret_cast<int*>(smem + L::OFF_MISC);
    uint32_t* cnt = p.ws_cnt + (int64_t)g * p.tilesets + ts;
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        misc[0] = (old == (uint32_t)(p.S - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (misc[0] == 0)
        return;
    __threadfence();   // acquire the other splits' partials

    // merge: T*16 rows x 32 column chunks of 16; thread -> (row, chunk) items
    for (int item = tid; item < T * 16 * 32; item += THREADS) {
        const int r = item >> 5;
        const int c0 = (item & 31) * 16;
        const int64_t orow = row_base + 16 * ts * T + r;
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
                const float w = exp2f(mq - top);
                total = total + w * ml[2 * q + 1];
                const v4f* src = reinterpret_cast<const v4f*>(p.ws_o + (orow * p.S + q) * LATENT + c0);
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const v4f x4 = src[v];
#pragma unroll
                    for (int e = 0; e < 4; e++) acc[4 * v + e] = acc[4 * v + e] + w * x4[e];
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

// Splits from shapes only: enough workgroups to cover the 256 CUs about twice, each with at least
// two 128-key blocks of its group's key capacity.
int choose_splits(int groups, int tilesets, int64_t max_keys)
{
    const int64_t wgs = (int64_t)groups * tilesets;
    int64_t s = (512 + wgs - 1) / wgs;
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
