"""Pins of the oracle's top-k select and remap against brute force and library routines: the order
key against torch's bf16 values for every bit pattern, the select against a plain Python sort of
the values on small rows full of ties, NaNs, infinities and signed zeros, and the remap against
the dense decode's key-to-row rule."""
import numpy as np
import pytest
import torch

from oracle import topk

ALL = np.arange(65536, dtype=np.uint16)
VALS = torch.from_numpy(ALL.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def test_order_key_follows_the_values_for_every_bf16_pattern():
    keep = ~np.isnan(VALS)
    bits, vals = ALL[keep], VALS[keep]
    keys = topk.order_key(bits)
    assert np.array_equal(np.isnan(VALS), topk.is_nan(ALL))
    order = np.argsort(keys, kind="stable")
    v = vals[order]
    assert np.all(np.diff(v) >= 0)                       # keys sort the values
    assert len(np.unique(keys)) == len(keys)             # one key per pattern
    # equal values (only +0 and -0) sit next to each other, -0 first
    assert topk.order_key(np.array([0x0000], np.uint16))[0] == topk.order_key(np.array([0x8000], np.uint16))[0] + 1
    assert keys.min() == topk.order_key(np.array([0xFF80], np.uint16))[0]     # -inf
    assert keys.max() == topk.order_key(np.array([0x7F80], np.uint16))[0]     # +inf


def _brute(bits_row, row_end, k):
    """Plain Python: candidates are the non-NaN columns below the row end; fewer than k: all, in
    column order; else the k best by (value descending, then -0 below +0, column ascending),
    output as those strictly above the k-th one's (value, sign) in column order, then those tied
    with it in column order."""
    n = max(0, min(row_end, len(bits_row)))
    def rank(c):
        val = VALS[bits_row[c]]
        neg_zero = val == 0 and bits_row[c] == 0x8000
        return (val, 0 if neg_zero else 1)
    cand = [c for c in range(n) if not np.isnan(VALS[bits_row[c]])]
    if len(cand) < k:
        return cand
    best = sorted(cand, key=lambda c: (tuple(-x for x in rank(c)), c))[:k]
    thr = rank(best[-1])
    return sorted(c for c in best if rank(c) > thr) + sorted(c for c in best if rank(c) == thr)


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_a_plain_sort_on_rows_full_of_ties(seed):
    rng = np.random.default_rng(seed)
    palette = np.array([0x3F80, 0x3F80, 0x4000, 0xBF80, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0,
                        0x3F81, 0x4040, 0xC000], np.uint16)       # 1, 2, -1, +-0, +-inf, NaN, ...
    for _ in range(25):
        n = int(rng.integers(1, 60))
        row = palette[rng.integers(0, len(palette), size=n)]
        end = int(rng.integers(0, n + 5))
        k = int(rng.integers(1, 20))
        got = topk.select_row(row, end, k)
        assert list(got) == _brute(row, end, k), (row, end, k)


def test_select_on_random_values_and_the_padded_lists():
    rng = np.random.default_rng(9)
    R, N, K = 5, 300, 64
    vals = torch.from_numpy(rng.standard_normal((R, N)).astype(np.float32)).to(torch.bfloat16)
    bits = vals.view(torch.int16).numpy().view(np.uint16).copy()
    bits[1, ::7] = 0x7FC0                                   # NaNs are never chosen
    ends = np.array([300, 250, 40, 0, 1000], np.int32)
    cols, cnt = topk.select(bits, ends, K)
    for r in range(R):
        ref = _brute(bits[r], int(ends[r]), K)
        assert cnt[r] == len(ref)
        assert list(cols[r, :cnt[r]]) == ref
        assert np.all(cols[r, cnt[r]:] == -1)
    assert cnt[2] == 40 and list(cols[2, :40]) == list(range(40))   # fewer candidates than K
    assert cnt[3] == 0


def test_exactly_k_candidates_come_out_in_threshold_order():
    # 1.0, 2.0, 1.0, 3.0 with k = 4: the threshold is 1.0; above it columns 1, 3, then 0, 2
    bits = np.array([0x3F80, 0x4000, 0x3F80, 0x4040], np.uint16)
    assert list(topk.select_row(bits, 4, 4)) == [1, 3, 0, 2]
    assert list(topk.select_row(bits, 4, 5)) == [0, 1, 2, 3]   # fewer than k: column order


def test_remap_follows_the_page_table():
    rng = np.random.default_rng(3)
    B, Q, page, pages = 2, 3, 16, 5
    table = rng.permutation(B * pages).astype(np.int32).reshape(B, pages)
    table[1, 4] = 2 ** 31 - 1                               # an unused entry
    num_rows = B * pages * page
    cols = rng.integers(-1, pages * page, size=(B * Q, 12)).astype(np.int32)
    cols[4, 0] = 4 * page + 3                               # request 1, unused page -> -1
    out = topk.remap(cols, table, page, Q, num_rows)
    for r in range(B * Q):
        b = r // Q
        for t in range(12):
            j = cols[r, t]
            if j < 0 or (b == 1 and j // page == 4):
                assert out[r, t] == -1
            else:
                assert out[r, t] == table[b, j // page] * page + j % page
