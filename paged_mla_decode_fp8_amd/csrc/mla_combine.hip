// Combine of R partial decodes of the same query rows (decode-context parallelism, gfx950).
//
// With decode-context parallelism each of R ranks decodes its share of every row's keys and sends
// the row's result (o, LSE) to the row's owner, which merges them the way the split partials of one
// decode are merged (vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.attn_sparse,
// module docstring: the merge weights each partial by the exponential of its maximum minus the
// largest one and divides by the weighted total; "push" sends a rank's merged rows to the owners,
// and a row with no key sends only its LSE). Here, with natural-log LSEs, in rank order, FP32:
//   M = max_r lse_r;  w_r = exp(lse_r - M) (a rank with lse_r = -inf is skipped: its o row may hold
//   anything and never enters the sums);
//   L = sum_r w_r;  o = BF16_RNE(sum_r w_r o_r / L);  lse = M + ln L;
// a row that no rank holds a key of gets o = +0 and lse = -inf.
//
// One wave per row: lane l owns latent columns 8 l .. 8 l + 7 (16 bytes of bf16 per rank). The
// row's R LSEs are wave-uniform loads; the o rows and LSEs of the first eight ranks are all
// requested before any is waited for (one memory round trip for R <= 8), later ranks eight at a
// time. HBM-bound for large
// row counts (each partial byte is read once), latency-bound for the small ones. The partials are
// read and the outputs written with the non-temporal hint: neither is read again by this kernel
// (measured 2-8 % faster, outputs identical).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "mla_decode.h"

namespace {

constexpr int CB_ROWS = 4;                  // rows (waves) per workgroup
constexpr int CB_THREADS = 64 * CB_ROWS;
constexpr int CB_UNROLL = 8;                // o rows requested together

typedef int v4i_c __attribute__((ext_vector_type(4)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef float v2f_c __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_c __attribute__((ext_vector_type(2)));

// Two floats -> two BF16 codes (a in the low half), round to nearest even, with gfx950's packed
// conversion (identical to (u + 0x7FFF + lsb) >> 16 on every non-NaN FP32 bit pattern, as checked
// on MI355X).
__device__ inline uint32_t pack_bf16_c(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f_c{a, b}, v2bf_c));
}

__global__ __launch_bounds__(CB_THREADS) void mla_combine_kernel(const uint16_t* __restrict__ o_parts,
                                                                 const float* __restrict__ lse_parts,
                                                                 int R, int64_t rows,
                                                                 uint16_t* __restrict__ o,
                                                                 float* __restrict__ lse)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * CB_ROWS + wave;
    if (row >= rows)
        return;
    // the first eight ranks' o rows and LSEs, all requested before any of them is waited for: the
    // rank index is clamped to R - 1 so that every load is in bounds and none sits behind a branch
    // (ranks >= R are masked afterwards; rows of ranks without keys are read but never used)
    v4i_c part[CB_UNROLL];
    float lv[CB_UNROLL];
#pragma unroll
    for (int u = 0; u < CB_UNROLL; u++) {
        const int64_t r = u < R ? u : R - 1;
        part[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i_c*>(o_parts + (r * rows + row) * 512 + 8 * lane));
        lv[u] = lse_parts[r * rows + row];
    }
    // the largest LSE of the row (wave-uniform)
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < CB_UNROLL; u++)
        M = u < R ? fmaxf(M, lv[u]) : M;
    for (int r = CB_UNROLL; r < R; r++)
        M = fmaxf(M, lse_parts[(int64_t)r * rows + row]);
    uint16_t* orow = o + row * 512 + 8 * lane;
    if (M == -INFINITY) {
        *reinterpret_cast<v4i_c*>(orow) = v4i_c{0, 0, 0, 0};
        if (lane == 0)
            lse[row] = -INFINITY;
        return;
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    for (int r0 = 0; r0 < R; r0 += CB_UNROLL) {
        float w[CB_UNROLL];
#pragma unroll
        for (int u = 0; u < CB_UNROLL; u++) {
            const int r = r0 + u;
            if (r0 > 0) {
                const int64_t rr = r < R ? r : R - 1;
                part[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i_c*>(o_parts + (rr * rows + row) * 512 + 8 * lane));
                lv[u] = lse_parts[rr * rows + row];
            }
            const float l = r < R ? lv[u] : -INFINITY;
            w[u] = l == -INFINITY ? 0.f : expf(l - M);
        }
#pragma unroll
        for (int u = 0; u < CB_UNROLL; u++) {
            if (w[u] == 0.f)
                continue;
            L += w[u];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t d = (uint32_t)part[u][k];
                acc[2 * k] = fmaf(w[u], bf16_lo(d), acc[2 * k]);
                acc[2 * k + 1] = fmaf(w[u], bf16_hi(d), acc[2 * k + 1]);
            }
        }
    }
    uint32_t outw[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
        outw[k] = pack_bf16_c(acc[2 * k] / L, acc[2 * k + 1] / L);
    __builtin_nontemporal_store(v4i_c{(int)outw[0], (int)outw[1], (int)outw[2], (int)outw[3]}, reinterpret_cast<v4i_c*>(orow));
    if (lane == 0)
        lse[row] = M + logf(L);
}

bool aligned_c(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

mla_status_t mla_combine(const void* o_parts, const float* lse_parts, int R, int64_t rows, void* o,
                         float* lse, void* stream)
{
    if (R < 1 || rows < 0 || rows > (int64_t)CB_ROWS * 0x7FFFFFFF)
        return MLA_ERR_SHAPE;
    if (rows == 0)
        return MLA_OK;
    if (!o_parts || !lse_parts || !o || !lse)
        return MLA_ERR_NULL;
    if (!aligned_c(o_parts, 16) || !aligned_c(o, 16) || !aligned_c(lse_parts, 4) || !aligned_c(lse, 4))
        return MLA_ERR_ALIGN;
    const int64_t grid = (rows + CB_ROWS - 1) / CB_ROWS;
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)grid), dim3(CB_THREADS), 0,
                       (hipStream_t)stream, (const uint16_t*)o_parts, lse_parts, R, rows,
                       (uint16_t*)o, lse);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

}  // extern "C"
