"""Pins of the oracle's combine of partial decodes (the decode-context-parallel merge of per-rank
(o, LSE) rows), independent of its code: the split identity against the oracle's unsplit exact
decode, closed forms (one rank, equal LSEs, a single non-empty rank, all ranks empty) and the bf16
front end against library decoding."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def _slices(n, R, rng):
    """R consecutive key slices of [0, n) (some possibly empty)."""
    cuts = np.sort(rng.integers(0, n + 1, size=R - 1))
    edges = np.concatenate([[0], cuts, [n]])
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:])]


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("R", [1, 2, 3, 8])
def test_combine_of_key_slices_equals_the_unsplit_decode(seed, R):
    """Each rank decodes a slice of every row's key list (EXACT mode, FP64); the combine of the
    ranks' (o, LSE) equals the decode over the whole list (the split-merge identity)."""
    rng = np.random.default_rng(seed)
    B, Q, H, K = 2, 2, 16, 150
    valid = rng.integers(0, K + 1, size=(B, Q))
    x = wl.sparse_case(B, Q, H, K, valid.tolist(), 1000, seed=300 + seed)
    o_full, lse_full = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale,
                                     mode=oracle.EXACT)
    o_parts = np.zeros((R, B, Q, H, 512))
    lse_parts = np.zeros((R, B, Q, H))
    # every (b, i) list cut into R slices; rank r decodes slice r of each list
    sl = {(b, i): _slices(int(x.valid[b, i]), R, rng) for b in range(B) for i in range(Q)}
    for r in range(R):
        rows = np.zeros_like(x.rows)
        valid_r = np.zeros_like(x.valid)
        for b in range(B):
            for i in range(Q):
                a, e = sl[(b, i)][r]
                rows[b, i, :e - a] = x.rows[b, i, a:e]
                valid_r[b, i] = e - a
        o_parts[r], lse_parts[r] = oracle.sparse(x.q_bits, x.kv, x.k_scale, rows, valid_r, x.scale,
                                                 mode=oracle.EXACT)
    o, lse = oracle.combine(o_parts, lse_parts)
    empty = np.isneginf(lse_full)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(o[empty] == 0)
    np.testing.assert_allclose(lse[~empty], lse_full[~empty], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[~empty], o_full[~empty], rtol=0, atol=1e-12)


def test_one_rank_is_the_identity():
    rng = np.random.default_rng(1)
    o1 = rng.standard_normal((1, 7, 512))
    l1 = rng.standard_normal((1, 7)) * 5
    o, lse = oracle.combine(o1, l1)
    np.testing.assert_allclose(o, o1[0], rtol=1e-15, atol=0)
    assert np.array_equal(lse, l1[0])


def test_equal_lses_give_the_mean_and_plus_log_r():
    rng = np.random.default_rng(2)
    R = 5
    op = rng.standard_normal((R, 3, 512))
    lp = np.broadcast_to(np.array([0.5, -3.0, 40.0]), (R, 3)).copy()
    o, lse = oracle.combine(op, lp)
    np.testing.assert_allclose(o, op.mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lp[0] + np.log(R), rtol=0, atol=1e-14)


def test_empty_ranks_contribute_nothing():
    rng = np.random.default_rng(3)
    R = 4
    op = rng.standard_normal((R, 2, 512))
    lp = np.full((R, 2), -np.inf)
    lp[2, 0] = 1.25                      # row 0: one rank holds keys; row 1: none does
    op[:, 1] = np.nan                     # never read for a row without keys
    op[[0, 1, 3], 0] = np.nan             # nor the empty ranks' rows of row 0
    o, lse = oracle.combine(op, lp)
    assert np.array_equal(o[0], op[2, 0]) and lse[0] == 1.25
    assert np.all(o[1] == 0) and not np.signbit(o[1]).any() and np.isneginf(lse[1])


def test_bf16_front_end_decodes_exactly():
    rng = np.random.default_rng(4)
    R, rows = 3, 6
    vals = torch.from_numpy(rng.standard_normal((R, rows, 512)).astype(np.float32)).to(torch.bfloat16)
    bits = vals.view(torch.int16).numpy().view(np.uint16)
    lp = rng.standard_normal((R, rows)).astype(np.float32)
    a = oracle.combine(bits, lp)
    b = oracle.combine(vals.to(torch.float64).numpy(), lp.astype(np.float64))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
