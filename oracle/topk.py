"""Top-k selection of key positions from bf16 indexer logits, and their remap to cache rows: the
step that produces the top-k sparse decode's index lists.

TEST INFRASTRUCTURE (see the package docstring): only the tests, the smoke entry point and the
benchmark's CPU baseline may use it; it shares no code with the HIP library.

What it computes (vLLM API pages, cited by title and section):

* ``vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.topk_exchange`` -- the local top-k
  select of ``push_local_topk`` and the merge's ``_make_radix_select``: a row's logits are the
  bf16 values at columns ``[0, min(row_end, N))``; NaNs take no part; each value is ranked by a
  16-bit order key of its bits; the threshold key ``v`` is the K-th largest key of the row; every
  column whose key is above ``v`` is selected, and of the columns whose key equals ``v`` the
  lowest-numbered ones fill the remaining places (the tie rule). The selected columns come out in
  that order: the columns above the threshold in increasing column order, then the threshold
  columns in increasing column order. A row with fewer than K candidates selects all of them, in
  column order (the threshold is found only once K candidates are reached).
* ``vllm.model_executor.kernels.attention.dsa.sparse_mqa_logits`` -- the remap of selected
  columns to positions and the -1 padding of the lists (columns outside the row's range become
  -1). Here the positions are a request's key positions, turned into cache rows through the
  request's page table as the dense decode does.

Readings taken here (also in the design notes): the 16-bit order key is the usual monotone map of
an IEEE sign-magnitude pattern to an unsigned integer (positive: bits | 0x8000; negative:
~bits & 0xFFFF), so the key order is the numeric order of the values with -0 just below +0 and
+-inf at the ends; a list holds K places, the unfilled ones -1, and its count is the number of
filled places.
"""
from __future__ import annotations

import numpy as np


def order_key(bits: np.ndarray) -> np.ndarray:
    """The 16-bit order key of bf16 bit patterns (uint16 -> int64): the monotone map above."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    return np.where(b & 0x8000, (~b) & 0xFFFF, b | 0x8000)


def is_nan(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.int64)
    return (b & 0x7FFF) > 0x7F80


def select_row(bits_row: np.ndarray, row_end: int, k: int) -> np.ndarray:
    """The selected columns of one row, in the pages' output order (length <= k)."""
    n = max(0, min(int(row_end), bits_row.shape[0]))
    cols = np.arange(n)
    cols = cols[~is_nan(bits_row[:n])]
    keys = order_key(bits_row[:n])[cols]
    if cols.size < k:
        return cols.copy()
    # rank by (key descending, column ascending); the k-th is the threshold
    order = np.lexsort((cols, -keys))
    chosen = cols[order[:k]]
    v = keys[order[k - 1]]
    ck = order_key(bits_row[chosen])
    above = np.sort(chosen[ck > v])
    at = np.sort(chosen[ck == v])
    return np.concatenate([above, at])


def select(logits_bits: np.ndarray, row_ends: np.ndarray, k: int):
    """Per row of ``logits_bits`` (uint16 bf16 bits [R, N]) and ``row_ends`` [R]: the selected
    columns [R, k] (-1 padded, int32) and the counts [R] (int32)."""
    bits = np.asarray(logits_bits, np.uint16)
    R = bits.shape[0]
    out = np.full((R, k), -1, np.int32)
    cnt = np.zeros(R, np.int32)
    for r in range(R):
        s = select_row(bits[r], int(row_ends[r]), k)
        out[r, :s.size] = s
        cnt[r] = s.size
    return out, cnt


def remap(cols: np.ndarray, block_table: np.ndarray, page_size: int, q_per_request: int,
          num_rows: int) -> np.ndarray:
    """Selected key positions -> cache rows: row r of ``cols`` belongs to request
    r // q_per_request, and position j is cache row table[b, j // page_size] * page_size +
    j % page_size; -1 stays -1, and so does a position whose page or row lies outside the table
    or the cache."""
    cols = np.asarray(cols, np.int64)
    table = np.asarray(block_table, np.int64)
    out = np.full(cols.shape, -1, np.int32)
    for r in range(cols.shape[0]):
        b = r // q_per_request
        for t in range(cols.shape[1]):
            j = cols[r, t]
            if j < 0:
                continue
            pg = j // page_size
            if pg >= table.shape[1]:
                continue
            page = table[b, pg]
            row = page * page_size + j % page_size
            if page >= 0 and 0 <= row < num_rows:
                out[r, t] = row
    return out


# ---- candidate blocks -> sparse block ids, and sparse logit columns -> positions --------------------
#
# vllm.model_executor.kernels.attention.dsa.sparse_mqa_logits: the indexer names candidate blocks of
# a row's context; they are expanded into sparse blocks (candidate_blocks_to_sparse_indices and
# _expand_candidates_kernel), the logits are scored over the sparse blocks' columns, the top-k runs
# over those columns (bounded by the row's valid column count), and the chosen columns are mapped
# back to request-local positions (sparse_topk_remap and _sparse_topk_remap_kernel).

def expand_candidates(candidate_blocks, row_ks, row_ke, candidate_block_size: int,
                      sparse_block_kv: int):
    """Candidate blocks -> (sparse block ids [rows, K * ratio], valid column counts [rows]).

    ratio = candidate_block_size / sparse_block_kv (1 or 2); with ratio 2 candidate c stands for
    sparse blocks 2c and 2c + 1, in that order. A row's K range is [ks, ke) (kv_len = max(ke - ks,
    0) positions); a sparse block b is valid when 0 <= b < ceil(kv_len / sparse_block_kv). The
    valid blocks come out in ascending order, offset by ks // sparse_block_kv (the row's anchor),
    and the rest of the row repeats the last (largest) valid one, or holds the anchor when none is
    valid. The count of valid sparse-token columns: every valid block is full except the last,
    which holds the positions from its start to kv_len (at least one, at most a block)."""
    cand = np.asarray(candidate_blocks, np.int64)
    ks = np.asarray(row_ks, np.int64).reshape(-1)
    ke = np.asarray(row_ke, np.int64).reshape(-1)
    sbk = int(sparse_block_kv)
    ratio = int(candidate_block_size) // sbk
    assert ratio * sbk == candidate_block_size and ratio in (1, 2)
    rows, K = cand.shape
    S = K * ratio
    si = np.zeros((rows, S), np.int32)
    end = np.zeros(rows, np.int32)
    for r in range(rows):
        blocks = []
        for c in cand[r].tolist():
            blocks += [c] if ratio == 1 else [2 * c, 2 * c + 1]
        kv_len = max(int(ke[r] - ks[r]), 0)
        max_block = -(-kv_len // sbk)
        valid = sorted(b for b in blocks if 0 <= b < max_block)
        base = int(ks[r]) // sbk
        pad = valid[-1] + base if valid else base
        si[r] = [b + base for b in valid] + [pad] * (S - len(valid))
        if valid:
            last_start = valid[-1] * sbk + int(ks[r])
            end[r] = (len(valid) - 1) * sbk + min(max(int(ke[r]) - last_start, 1), sbk)
    return si, end


def sparse_cols_to_positions(cols, sparse_indices, row_ks, sparse_block_kv: int, width: int):
    """Selected sparse logit columns [rows, k] -> request-local positions: column j * sbk + o of a
    row scores position (sparse_indices[row, j] - ks // sbk) * sbk + o; a column outside
    [0, width) (an unfilled place, -1) becomes -1, and so does a position outside [0, 2^31) (only
    sparse ids below the row's anchor give one: read as an absent key, like the -1 places)."""
    cols = np.asarray(cols, np.int64)
    si = np.asarray(sparse_indices, np.int64)
    ks = np.asarray(row_ks, np.int64).reshape(-1)
    sbk = int(sparse_block_kv)
    out = np.full(cols.shape, -1, np.int32)
    for r in range(cols.shape[0]):
        for t in range(cols.shape[1]):
            c = int(cols[r, t])
            if 0 <= c < width:
                pos = (si[r, c // sbk] - int(ks[r]) // sbk) * sbk + c % sbk
                out[r, t] = pos if 0 <= pos < 2**31 else -1
    return out


def sparse_topk(logits_bits, end, k: int, sparse_indices, row_ks, sparse_block_kv: int):
    """The top-k over sparse logits [rows, width] bounded by each row's valid column count
    ``end``, remapped to request-local positions: (positions [rows, k], -1 padded; counts)."""
    bits = np.asarray(logits_bits, np.uint16)
    cols, cnt = select(bits, np.asarray(end), k)
    return sparse_cols_to_positions(cols, sparse_indices, row_ks, sparse_block_kv,
                                    bits.shape[1]), cnt
