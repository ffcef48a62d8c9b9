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
