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


def test_remap_through_an_identity_table_is_the_closed_form():
    """table[b, p] = b * P + p lays request b's positions out contiguously from row b * P * page:
    position j must become row b * P * page + j, whatever the page size."""
    for page, P, Q in ((1, 40, 1), (16, 5, 3), (64, 3, 2), (7, 11, 4)):
        B = 3
        table = (np.arange(B)[:, None] * P + np.arange(P)[None, :]).astype(np.int32)
        cols = np.stack([np.arange(P * page) for _ in range(B * Q)]).astype(np.int32)
        out = topk.remap(cols, table, page, Q, B * P * page)
        b = np.arange(B * Q)[:, None] // Q
        assert np.array_equal(out, b * P * page + cols), (page, P, Q)
        # past the table (page index P) and past the cache: -1
        assert np.all(topk.remap(np.full((B * Q, 1), P * page), table, page, Q, B * P * page) == -1)
        assert np.all(topk.remap(cols, table, page, Q, B * P * page - 1)[-Q:, -1] == -1)


@pytest.mark.parametrize("seed", range(3))
def test_sparse_decode_over_remapped_positions_equals_the_dense_decode(seed):
    """The remap is the dense decode's key -> row rule: a sparse list of positions 0 .. n_i - 1
    (n_i = seq_len - Q + i + 1, the causal bound of row i) remapped through the page table gives,
    in the oracle's sparse front end, bit for bit what its dense front end computes from the table
    itself (one split, 128-key chunks, so both walk the same keys in the same chunks)."""
    import oracle
    import workloads as wl
    rng = np.random.default_rng(seed)
    B, Q, H, page = 3, 3, 2, int(rng.choice([1, 16, 64]))
    seq = rng.integers(1, 300, size=B)
    seq[0] = 1                                    # row 0 before its causal bound: no key
    x = wl.dense_case(B, Q, H, seq, page_size=page, seed=40 + seed, extra_pages=5)
    n_i = np.clip(x.seq_lens[:, None] - Q + np.arange(Q)[None, :] + 1, 0, None)   # [B, Q]
    K = int(x.seq_lens.max())
    cols = np.full((B * Q, K), -1, np.int32)
    for r in range(B * Q):
        cols[r, :n_i.reshape(-1)[r]] = np.arange(n_i.reshape(-1)[r])
    rows = topk.remap(cols, x.block_table, page, Q, x.kv.shape[0]).reshape(B, Q, K)
    for mode in (oracle.EXACT, oracle.METHOD):
        od, ld = oracle.dense(x.q_bits, x.kv, page, x.k_scale, x.block_table, x.seq_lens, x.scale,
                              mode=mode, splits=1, chunk=128)
        os_, ls = oracle.sparse(x.q_bits, x.kv, x.k_scale, rows, n_i.astype(np.int32), x.scale,
                                mode=mode, splits=1, chunk=128)
        assert np.array_equal(od, os_) and np.array_equal(ld, ls), mode
    assert np.all(np.isneginf(ld[0, :Q - 1]))


# ---- candidate blocks -> sparse blocks -> positions -------------------------------------------------

def _brute_positions(cands, ks, ke, cbs):
    """Plain sets: the request-local positions the valid candidate blocks cover inside the row's
    K range, ascending (candidate c covers positions [c * cbs, (c + 1) * cbs))."""
    kv_len = max(ke - ks, 0)
    cover = set()
    for c in cands:
        if c >= 0:
            cover.update(p for p in range(c * cbs, (c + 1) * cbs) if p < kv_len)
    return sorted(cover)


@pytest.mark.parametrize("cbs,sbk", [(16, 16), (8, 8), (32, 16), (16, 8)])
def test_expanded_columns_map_back_to_the_candidates_positions(cbs, sbk):
    """For unique candidates, the sparse columns [0, end) map back (through the sparse block ids)
    to exactly the positions the valid candidate blocks cover below kv_len, ascending -- whatever
    the K range's start ks (the ids are anchored at ks // sbk, positions are request-local)."""
    rng = np.random.default_rng(cbs * 100 + sbk)
    rows, K = 40, 16
    cand = np.full((rows, K), -1, np.int64)
    ks = rng.integers(0, 500, rows)
    ke = ks + rng.integers(0, 400, rows)
    ke[3] = ks[3] - 5                          # an empty range
    for r in range(rows):
        n = int(rng.integers(0, K + 1))
        cand[r, :n] = rng.permutation(40)[:n]  # unique, some past the range
    si, end = topk.expand_candidates(cand.astype(np.int32), ks, ke, cbs, sbk)
    width = si.shape[1] * sbk
    assert si.shape == (rows, K * cbs // sbk)
    for r in range(rows):
        want = _brute_positions(cand[r].tolist(), int(ks[r]), int(ke[r]), cbs)
        assert end[r] == len(want), r
        got = topk.sparse_cols_to_positions(np.arange(end[r])[None, :], si[r:r + 1], ks[r:r + 1],
                                            sbk, width)[0]
        assert got.tolist() == want, r
    assert end[3] == 0 and np.all(si[3] == ks[3] // sbk)


def test_expanded_blocks_are_sorted_then_padded_with_the_last():
    """The docstring's layout: the valid blocks ascending (anchored at ks // sbk), then the last
    valid block repeated; ratio 2 makes candidate c into sparse blocks 2c and 2c + 1; candidates
    outside the range (or -1) are dropped; repeats are kept (each copy counts)."""
    cand = np.array([[5, 1, -1, 3], [2, 2, 0, -1], [9, -1, -1, -1]], np.int32)
    si, end = topk.expand_candidates(cand, [0, 0, 0], [64, 64, 64], 8, 8)
    # row 0: blocks 5, 1, 3 valid (max_block 8): 1 3 5 then 5
    assert si[0].tolist() == [1, 3, 5, 5] and end[0] == 24
    assert si[1].tolist() == [0, 2, 2, 2] and end[1] == 24      # the repeat counts
    assert si[2].tolist() == [0, 0, 0, 0] and end[2] == 0       # 9 >= 8: nothing valid
    si, end = topk.expand_candidates(cand[:1], [17], [17 + 40], 16, 8)
    # ratio 2: 10, 11, 2, 3, 6, 7 (max_block 5, anchor 17 // 8 = 2): 2 3 then 4 4 ... anchored
    assert si[0].tolist() == [4, 5, 5, 5, 5, 5, 5, 5]
    assert end[0] == 8 + 8                                        # block 3 holds positions 24..31 < 40


def test_sparse_columns_outside_the_logits_width_become_minus_one():
    si = np.array([[4, 9, 2]], np.int32)
    cols = np.array([[0, 7, 8, 23, 24, -1, 100]])
    pos = topk.sparse_cols_to_positions(cols, si, [16], 8, width=24)
    # ks // 8 = 2: block 4 -> positions 16..23, block 9 -> 56..63, block 2 -> 0..7
    assert pos[0].tolist() == [16, 23, 56, 7, -1, -1, -1]
