/*
 * mla_decode.h -- C ABI of an MI355X (gfx950) MLA decode attention library over an FP8 E4M3 latent
 * KV cache.
 *
 * The operation (vLLM API pages, cited by title and section):
 *   - vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.attn_sparse, module docstring: every
 *     query head attends a list of 576-byte E4M3 cache rows (bytes [0,512) are the latent, which is
 *     V and the first 512 columns of K; bytes [512,576) are the rope part of K), with one per-tensor
 *     k_scale; a row's keys are split into partials, each an online softmax in base 2 with P taken
 *     at 448 of the running maximum and rounded to E4M3, the partials merged in FP32 into a BF16
 *     latent output and a natural-log LSE; rows with no key give o = 0 and LSE = -inf.
 *   - the same page, SparseDcpDecode.kernel / run_sparse: the top-k form reads keys through a list
 *     of flat cache row ids and a per-row count clamped to [0, K].
 *   - vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_attn, module docstring: the dense
 *     form reads a request's paged KV; position i of the request's Q query rows sees keys
 *     0 .. seq_len - Q + i.
 *
 * All pointers named "device" are HIP device pointers; the caller owns every buffer (inputs,
 * outputs, workspace). The library allocates nothing on the decode path and keeps no per-call
 * state. Calls are asynchronous on the given HIP stream (a hipStream_t passed as void*, NULL is the
 * default stream) and never synchronize. Errors found on the host return a status and launch
 * nothing; no exception crosses the ABI.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_NULL = 1,        /* a required pointer is NULL */
    MLA_ERR_SHAPE = 2,       /* B, Q, H, K, max_pages or page_size out of range (H % 16 != 0,
                                max_pages * page_size above 2^31 - 1 ...) */
    MLA_ERR_ALIGN = 3,       /* a pointer is not aligned as documented */
    MLA_ERR_WORKSPACE = 4,   /* the workspace is missing or smaller than mla_workspace_bytes() */
    MLA_ERR_UNSUPPORTED = 5, /* a plan the kernels do not implement (tiles not 1/2/4 or not
                                dividing the row tiles, splits outside [1, 4096], an unknown mode,
                                a balanced plan over more than 36863 groups or 2^31 virtual
                                blocks) */
    MLA_ERR_LAUNCH = 6       /* the kernel launch failed (HIP error) */
} mla_status_t;

/* The E4M3 cache. data: device, num_rows rows of 576 bytes each (OCP E4M3FN codes), 16-byte
 * aligned. Dense: row r = page * page_size + slot. Sparse: page_size is ignored. k_scale: the
 * per-tensor dequantization scale of K and V (value = k_scale * E4M3 value). */
typedef struct {
    const void* data;
    int64_t num_rows;
    int32_t page_size;
    float k_scale;
} mla_kv_t;

/* How a key group's keys are split among workgroups. A key group is a request b (dense; all its Q*H
 * query rows) or a list (b, i) (sparse; its H rows); n is its key count and its keys form
 * ceil(n / 128) blocks of 128.
 *   MLA_SPLIT_UNIFORM   the pages' rule: every group in `splits` = S parts, part s holding keys
 *                       [s*per, min(n, (s+1)*per)), per = ceil(n / S).
 *   MLA_SPLIT_BALANCED  every group counts as a run of 6 + (its blocks) virtual blocks, the 6
 *                       standing for the fixed cost of one work item; the runs, concatenated in
 *                       group order (V virtual blocks), are cut into `splits` = P pieces of equal
 *                       size: piece p holds virtual blocks [floor(p*V/P), floor((p+1)*V/P)), and
 *                       block j of a group whose run starts at virtual block r sits at r + 6 + j.
 *                       A group is split where a piece boundary falls among its blocks (so split
 *                       boundaries are multiples of 128 keys) and each piece goes to one
 *                       workgroup per tile set, which evens out ragged key counts. A group's
 *                       result then depends on the key counts of the whole call (still
 *                       bit-identical for identical inputs). At most 36863 groups, and fewer than
 *                       2^31 virtual blocks in total (counted at each group's maximum key count). */
enum { MLA_SPLIT_UNIFORM = 0, MLA_SPLIT_BALANCED = 1 };

/* A launch plan. splits: S >= 1 (see mode); tiles: 16-row query tiles per workgroup (1, 2 or 4),
 * which must divide the row tiles of a key group (dense: Q*H/16, sparse: H/16). The result depends
 * on where the splits fall (where P is anchored and rounded; within the tolerance of the
 * definition) but is bit-identical for any tiles. */
typedef struct {
    int32_t splits;
    int32_t tiles;
    int32_t mode;   /* MLA_SPLIT_UNIFORM or MLA_SPLIT_BALANCED */
} mla_plan_t;

/* A plan chosen from shapes only (never from device data): fills *plan. Returns MLA_ERR_NULL or
 * MLA_ERR_SHAPE for bad arguments. Dense: max_keys = max_pages * page_size; sparse: max_keys = K. */
mla_status_t mla_plan_dense(int B, int Q, int H, int max_pages, int page_size, mla_plan_t* plan);
mla_status_t mla_plan_sparse(int B, int Q, int H, int K, mla_plan_t* plan);

/* Workspace bytes a call of these shapes (dense = 1 for mla_decode_dense, 0 for
 * mla_decode_sparse) and plan needs: 0 when splits == 1, else one arrival counter per 16-row tile
 * (first), then FP32 split partials of 514 floats per row: B*Q*H*S rows for a uniform plan, at most
 * 2*P*(rows of a group) for a balanced one. */
size_t mla_workspace_bytes(int dense, int B, int Q, int H, const mla_plan_t* plan);

/* The leading bytes of the workspace that must be zero when a call starts (its arrival counters);
 * the call leaves them zero again (the last arriving workgroup of each tile resets its counter) and
 * leaves the rest of the workspace undefined. A workspace that served a call whose zero prefix was
 * at least as long can serve the next call as is; otherwise zero the longer prefix first. Calls that
 * share a workspace must be ordered on one stream. */
size_t mla_workspace_zero_bytes(int dense, int B, int Q, int H, const mla_plan_t* plan);

/*
 * Dense paged decode.
 *   q            device bf16 [B, Q, H, 576], row-major, 16-byte aligned: query rows of position i of
 *                request b, head h.
 *   kv           the cache (see mla_kv_t); page_size >= 1.
 *   block_table  device int32 [B, max_pages]: page ids of request b's keys; key j is cache row
 *                block_table[b, j / page_size] * page_size + j % page_size. The whole [B,
 *                max_pages] table must be allocated: entries covering keys < seq_len are used;
 *                others may be read (the kernel fetches the first blocks' entries before it
 *                knows seq_len) but never change the result. A page id whose row falls outside
 *                [0, num_rows) makes its keys absent (they contribute nothing and are not read).
 *   seq_lens     device int32 [B]: keys of request b, clamped to [0, max_pages * page_size].
 *   scale        softmax scale multiplying q . K (k_scale is applied on top).
 *   plan         NULL for mla_plan_dense()'s choice.
 *   o            device bf16 [B, Q, H, 512] (16-byte aligned): softmax-weighted latent, RNE.
 *   lse          device float [B, Q, H]: natural-log sum of exp(scale * q . K) over the row's keys.
 *   Position i sees keys j < seq_len - Q + i + 1; a row with none gets o = +0 and lse = -inf.
 *   workspace    device, >= mla_workspace_bytes(1, B, Q, H, plan) bytes, 256-byte aligned (may
 *                be NULL when splits == 1).
 */
mla_status_t mla_decode_dense(const void* q, const mla_kv_t* kv, const int32_t* block_table,
                              int max_pages, const int32_t* seq_lens, float scale, int B, int Q,
                              int H, const mla_plan_t* plan, void* o, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Top-k sparse decode.
 *   rows   device int32 [B, Q, K]: flat cache rows of the keys of position i of request b; the
 *          first valid[b, i] entries are used (in order); an entry outside [0, num_rows) is an
 *          absent key (contributes nothing, is not read). Duplicate entries count once each. The
 *          whole [B, Q, K] array must be allocated: entries past valid[b, i] may be read but
 *          never change the result.
 *   valid  device int32 [B, Q]: the count of each list, clamped to [0, K].
 *   Other arguments as for mla_decode_dense; all H heads of (b, i) share the list.
 */
mla_status_t mla_decode_sparse(const void* q, const mla_kv_t* kv, const int32_t* rows, int K,
                               const int32_t* valid, float scale, int B, int Q, int H,
                               const mla_plan_t* plan, void* o, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Precision flags of the _q entry points (the argument precision: one query flag plus one P flag).
 * Query precision of the QK product:
 *   MLA_Q_SPLIT  the AMD page's exact query split (mono.attention.mla_attn, module docstring): per
 *                query row the power of two 2^k, k the largest integer with max |q| 2^k <= 448 (at
 *                most 126; 0 for an all-zero row), and q 2^k = hi + lo with hi = E4M3(q 2^k),
 *                lo = E4M3(q 2^k - hi); the logits see the bf16 query exactly wherever q 2^k - hi
 *                is an E4M3 value (always for |q 2^k| >= 2^-2). Two FP8 MFMAs per latent step.
 *   MLA_Q_E4M3   the E4M3 query of the sparse page's Precision paragraph (FlashInfer's precision):
 *                the logits use E4M3(q 2^k) 2^-k (round to nearest even, same k) in place of q.
 *                Half the QK MFMAs of MLA_Q_SPLIT; |q - query used| <= 2^-4 |q| per value where
 *                |q 2^k| >= 2^-6.
 * Precision of P = 448 exp2(x - m) in the PV product (the row sums always take P unrounded, FP32):
 *   MLA_P_E4M3   E4M3(P), round to nearest even (the sparse page's module docstring).
 *   MLA_P_SPLIT  E4M3 hi + lo with hi = E4M3(P), lo = E4M3(P - hi) (the AMD page's module docstring
 *                and fp8_split4): V meets both, two FP8 MFMAs per PV step; |P - (hi + lo)| <=
 *                max(2^-8 P, 2^-10) against 2^-4 P for MLA_P_E4M3. The P lo tile takes LDS that
 *                four tiles per workgroup leave no room for: a plan with tiles = 4 returns
 *                MLA_ERR_UNSUPPORTED, and with plan = NULL the planner's choice runs with tiles =
 *                min(tiles, 2) (size the workspace for that plan).
 */
enum { MLA_Q_SPLIT = 0, MLA_Q_E4M3 = 1, MLA_P_E4M3 = 0, MLA_P_SPLIT = 2 };

/*
 * mla_decode_dense and mla_decode_sparse with the precision as an argument (they are these with
 * MLA_Q_SPLIT | MLA_P_E4M3). A precision with bits other than MLA_Q_E4M3 and MLA_P_SPLIT, or
 * MLA_P_SPLIT with a plan of four tiles, returns MLA_ERR_UNSUPPORTED before anything else is
 * checked. Other arguments, layouts and errors as for the plain entry points.
 */
mla_status_t mla_decode_dense_q(const void* q, const mla_kv_t* kv, const int32_t* block_table,
                                int max_pages, const int32_t* seq_lens, float scale, int B, int Q,
                                int H, const mla_plan_t* plan, int precision, void* o, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);
mla_status_t mla_decode_sparse_q(const void* q, const mla_kv_t* kv, const int32_t* rows, int K,
                                 const int32_t* valid, float scale, int B, int Q, int H,
                                 const mla_plan_t* plan, int precision, void* o, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_dense_q for callers that cannot allocate device memory or own a workspace (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same decode, with
 * the split partials and arrival counters in a file-scope device array of
 * MLA_NOALLOC_SCRATCH_BYTES held by each GPU the library runs on until the process ends (a fixed
 * 64 KiB counter region, then the partials). The call allocates nothing. Arguments, plan, results
 * and errors as for mla_decode_dense_q without the workspace; a plan whose workspace would exceed
 * the array (more than 262144 query rows, or partials beyond MLA_NOALLOC_SCRATCH_BYTES - 64 KiB)
 * returns MLA_ERR_WORKSPACE before anything is launched. Results are bit-identical to
 * mla_decode_dense_q with the same plan. The first call on a device looks up the array's address
 * (hipGetSymbolAddress, so make it outside graph capture) and zeroes the counter region with a
 * fill kernel on `stream`; calls leave the counters zero again. Every call on a GPU shares that
 * GPU's array: calls that overlap in time on one GPU (other streams, other threads) race and must
 * be ordered by the caller.
 */
enum { MLA_NOALLOC_SCRATCH_BYTES = 80 << 20 };
mla_status_t mla_decode_dense_q_noalloc(const void* q, const mla_kv_t* kv,
                                        const int32_t* block_table, int max_pages,
                                        const int32_t* seq_lens, float scale, int B, int Q, int H,
                                        const mla_plan_t* plan, int precision, void* o, float* lse,
                                        void* stream);

/*
 * Combine of R partial decodes of the same query rows over disjoint parts of their keys: the
 * decode-context-parallel merge at a row's owner (vllm.models.kimi_k3.nvidia.specialized_decode.
 * cutedsl.dsa.attn_sparse, module docstring and "push": each rank decodes its share of the keys and
 * sends the row's (o, LSE); the owner merges them as the split partials are merged). In rank order,
 * FP32: M = max_r lse_r, w_r = exp(lse_r - M), o = BF16_RNE(sum_r w_r o_r / sum_r w_r),
 * lse = M + ln(sum_r w_r). A partial with lse_r = -inf (a rank holding none of the row's keys) is
 * skipped: its o row may hold anything (NaN included) and never enters the sums; a row that no
 * rank holds a key of gets o = +0 and lse = -inf.
 *   o_parts    device bf16 [R, rows, 512] (rank-major; each rank's rows as mla_decode_* writes o,
 *              flattened), 16-byte aligned.
 *   lse_parts  device float [R, rows]: natural-log LSEs as mla_decode_* writes them.
 *   o, lse     device bf16 [rows, 512] (16-byte aligned) and float [rows].
 * R >= 1; rows >= 0 (0: nothing launched). Errors: MLA_ERR_SHAPE (R < 1, rows < 0 or above
 * 4 * (2^31 - 1)), MLA_ERR_NULL, MLA_ERR_ALIGN, MLA_ERR_LAUNCH. Asynchronous on `stream`; no
 * workspace.
 */
mla_status_t mla_combine(const void* o_parts, const float* lse_parts, int R, int64_t rows, void* o,
                         float* lse, void* stream);

/*
 * Top-k selection of key positions from bf16 indexer logits, remapped to cache rows: the index
 * lists (rows, valid) mla_decode_sparse reads. (vllm.models.kimi_k3.nvidia.specialized_decode.
 * cutedsl.dsa.topk_exchange, push_local_topk and the merge's radix select; vllm.model_executor.
 * kernels.attention.dsa.sparse_mqa_logits, the remap.) For logits row r (request b = r / Q):
 *   - candidates: the non-NaN values at columns [0, min(row_ends[r], N)), ranked by the 16-bit
 *     order key of their bits (positive: bits | 0x8000, negative: ~bits; -0 just below +0);
 *   - fewer than K candidates: all of them, in column order; otherwise the threshold key v is the
 *     K-th largest, and the list is every column above v in column order, then the lowest columns
 *     equal to v, in column order, up to K in all;
 *   - each selected column j becomes cache row block_table[b, j / page_size] * page_size +
 *     j % page_size (-1 when its page index is >= max_pages, its page id is negative or its row is
 *     >= num_rows); with block_table NULL the column itself;
 *   - rows_out[r, 0 .. count) holds the list, rows_out[r, count .. K) holds -1, valid_out[r] =
 *     count (min(K, candidates)).
 *   logits     device bf16 [R, N], 16-byte aligned; N a multiple of 8.
 *   row_ends   device int32 [R]; block_table device int32 [ceil(R / Q), max_pages] or NULL.
 *   rows_out   device int32 [R, K]; valid_out device int32 [R].
 * Errors: MLA_ERR_SHAPE (R < 0, N < 8, not a multiple of 8 or above 2^31 - 32769, K < 1, Q < 1,
 * or with a table max_pages < 1, page_size < 1, num_rows < 0 or max_pages * page_size above
 * 2^31 - 1),
 * MLA_ERR_NULL, MLA_ERR_ALIGN, MLA_ERR_LAUNCH. R = 0 launches nothing. Asynchronous on `stream`.
 */
mla_status_t mla_topk_rows(const void* logits, const int32_t* row_ends, int R, int N, int K,
                           const int32_t* block_table, int max_pages, int page_size, int Q,
                           int64_t num_rows, int32_t* rows_out, int32_t* valid_out, void* stream);

/*
 * The indexer's candidate blocks -> sparse block ids and valid column counts
 * (vllm.model_executor.kernels.attention.dsa.sparse_mqa_logits, candidate_blocks_to_sparse_indices
 * and _expand_candidates_kernel). ratio = candidate_block_size / sparse_block_kv must be 1 or 2.
 * For row r with K range [ks, ke) = [row_ks[r], row_ke[r]) (kv_len = max(ke - ks, 0)):
 *   - candidate c (request-local, in units of candidate_block_size positions; -1 padding) stands
 *     for sparse blocks c (ratio 1) or 2c, 2c + 1 (ratio 2); a block b is valid when
 *     0 <= b < ceil(kv_len / sparse_block_kv);
 *   - sparse_indices[r, 0 .. n) = the n valid blocks in ascending order plus floor(ks /
 *     sparse_block_kv) (repeats kept, each counting), sparse_indices[r, n .. K * ratio) = the last
 *     of them (the anchor floor(ks / sparse_block_kv) alone when n = 0);
 *   - end[r] = (n - 1) * sparse_block_kv + min(max(ke - (last * sparse_block_kv + ks), 1),
 *     sparse_block_kv) with last the largest valid block (0 when n = 0): the valid sparse-token
 *     columns, which form a prefix of the row.
 *   candidate_blocks  device int32 [rows, K]; row_ks, row_ke device int32 [rows];
 *   sparse_indices    device int32 [rows, K * ratio]; end device int32 [rows].
 * Errors: MLA_ERR_SHAPE (rows < 0, K < 1, a ratio other than 1 or 2, K * ratio > 16384),
 * MLA_ERR_NULL, MLA_ERR_ALIGN, MLA_ERR_LAUNCH. rows = 0 launches nothing. Asynchronous on `stream`.
 */
mla_status_t mla_expand_candidates(const int32_t* candidate_blocks, int rows, int K,
                                   const int32_t* row_ks, const int32_t* row_ke,
                                   int candidate_block_size, int sparse_block_kv,
                                   int32_t* sparse_indices, int32_t* end, void* stream);

/* The sparse logit columns of mla_topk_sparse_rows: column j * sparse_block_kv + o of logits row r
 * scores request-local position (sparse_indices[r, j] - floor(row_ks[r] / sparse_block_kv)) *
 * sparse_block_kv + o. S * sparse_block_kv must cover the logits' N columns. */
typedef struct {
    const int32_t* sparse_indices;   /* device int32 [R, S] (mla_expand_candidates' output) */
    int32_t S;
    int32_t sparse_block_kv;
    const int32_t* row_ks;           /* device int32 [R]: the K range starts */
} mla_sparse_cols_t;

/*
 * Top-k over sparse logits, remapped to positions, then (with a block table) to cache rows
 * (vllm.model_executor.kernels.attention.dsa.sparse_mqa_logits, sparse_topk_remap and
 * _sparse_topk_remap_kernel): the select of mla_topk_rows over columns [0, min(end[r], N)) of
 * logits row r, then every selected column becomes its position by `cols` (-1 for a position
 * outside [0, 2^31)), then, when block_table is not NULL, the cache row of that position as in
 * mla_topk_rows. cols NULL: the columns are the positions (mla_topk_rows is this with cols NULL).
 * Arguments and errors otherwise as for mla_topk_rows; MLA_ERR_SHAPE also for S < 1,
 * sparse_block_kv < 1 or S * sparse_block_kv < N.
 */
mla_status_t mla_topk_sparse_rows(const void* logits, const int32_t* end, int R, int N, int K,
                                  const mla_sparse_cols_t* cols, const int32_t* block_table,
                                  int max_pages, int page_size, int Q, int64_t num_rows,
                                  int32_t* rows_out, int32_t* valid_out, void* stream);

/* A static, human-readable name of a status. */
const char* mla_status_string(mla_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
