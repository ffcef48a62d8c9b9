"""Pins of the oracle's E4M3 query (the FlashInfer precision of the sparse page's Precision
paragraph, with the per-row power-of-two scale of the AMD page's query split), independent of the
oracle's code: the scale exponent against its definition, brute-force nearest E4M3 values over the
codes torch decodes, queries already on the E4M3 grid (the E4M3 query is then the query itself),
and the textbook softmax of the rounded query on tiny inputs."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle
import workloads as wl

# every finite E4M3 value, decoded by torch (a library routine)
_CODES = np.arange(256, dtype=np.uint8)
_VALS = torch.from_numpy(_CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
_FINITE = np.isfinite(_VALS)
_GRID = _VALS[_FINITE]
_GRID_CODES = _CODES[_FINITE]


def _bf16_bits(x):
    """float -> bf16 bits, round to nearest even (torch's cast)."""
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _dec(q_bits):
    t = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _nearest_e4m3(v):
    """Brute force: the finite E4M3 values nearest to v; ties to the even code (mantissa bit 0
    clear), saturating at +-448."""
    v = min(max(v, -448.0), 448.0)
    d = np.abs(_GRID - v)
    cand = np.flatnonzero(d == d.min())
    vals = {float(_GRID[c]) for c in cand}
    if len(vals) == 1:
        return vals.pop()
    even = [c for c in cand if (_GRID_CODES[c] & 1) == 0]
    return float(_GRID[even[0]])


def _rows(seed, n, scale_exp=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 576)) * np.exp2(rng.integers(-3, 4, size=(n, 1)) + scale_exp)
    return _bf16_bits(x)


@pytest.mark.parametrize("seed", range(3))
def test_scale_exponent_is_the_largest_that_keeps_the_row_within_448(seed):
    for q in _rows(seed, 20):
        qd = _dec(q)
        _, k = oracle.q_e4m3_row(q)
        amax = np.abs(qd).max()
        assert amax * 2.0 ** k <= 448.0
        assert amax * 2.0 ** (k + 1) > 448.0


def test_scale_exponent_special_rows():
    z = np.zeros(576, np.uint16)
    qe, k = oracle.q_e4m3_row(z)
    assert k == 0 and np.all(qe == 0)
    # max exactly 448 * 2^-3: k = 3; a hair above: k = 2
    q = _bf16_bits(np.full(576, 0.25))
    q[7] = _bf16_bits([56.0])[0]
    assert oracle.q_e4m3_row(q)[1] == 3
    q[7] = _bf16_bits([56.25])[0]
    assert oracle.q_e4m3_row(q)[1] == 2
    # a tiny row: the exponent stops at 126
    tiny = np.full(576, 0x0001, np.uint16)   # the smallest positive bf16 subnormal, 2^-133
    assert oracle.q_e4m3_row(tiny)[1] == 126


@pytest.mark.parametrize("seed", range(2))
def test_each_value_is_the_nearest_e4m3_value_at_the_row_scale(seed):
    for q in _rows(seed, 4):
        qd = _dec(q)
        qe, k = oracle.q_e4m3_row(q)
        for c in range(576):
            ref = _nearest_e4m3(qd[c] * 2.0 ** k) * 2.0 ** -k
            assert qe[c] == ref, (c, qd[c], qe[c], ref)


def test_ties_round_to_even_codes():
    # at scale 2^0 (row max 448): 1.0625 lies between 1.0 (code 0x38, even) and 1.125 (0x39)
    q = np.zeros(576, np.uint16)
    q[0] = _bf16_bits([448.0])[0]
    q[1] = _bf16_bits([1.0625])[0]
    q[2] = _bf16_bits([1.1875])[0]    # between 1.125 (0x39) and 1.25 (0x3A, even)
    qe, k = oracle.q_e4m3_row(q)
    assert k == 0
    assert qe[1] == 1.0 and qe[2] == 1.25


def test_grid_queries_are_unchanged_and_give_the_bf16_results():
    """A query whose scaled values are E4M3 values is its own E4M3 query, so both oracle modes agree
    exactly on it."""
    rng = np.random.default_rng(7)
    B, Q, H, n = 1, 1, 16, 40
    x = wl.sparse_case(B, Q, H, n, [[n]], 96, seed=11, distinct=False)
    k = rng.integers(0, 5, size=(H, 1))
    vals = _GRID[rng.integers(0, len(_GRID), size=(H, 576))] * np.exp2(-k)
    vals[:, 0] = 448.0 * np.exp2(-k[:, 0])    # pin the row scale to 2^k
    q_bits = _bf16_bits(vals).reshape(B, Q, H, 576)
    assert np.array_equal(_dec(q_bits).reshape(H, 576), vals)   # exact in bf16
    for h in range(H):
        qe, kk = oracle.q_e4m3_row(q_bits[0, 0, h])
        assert kk == k[h, 0] and np.array_equal(qe, vals[h])
    for mode in (oracle.EXACT, oracle.METHOD):
        a = oracle.sparse(q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=mode, splits=2)
        b = oracle.sparse(q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=mode, splits=2,
                          q_e4m3=True)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("seed", range(4))
def test_e4m3_query_softmax_matches_scipy_on_tiny_inputs(seed):
    """Exact mode with the E4M3 query: scipy's softmax of the logits formed from the brute-force
    rounded query."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    x = wl.sparse_case(1, 1, 16, n, [[n]], 64, seed=200 + seed, distinct=False)
    o, lse = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=oracle.EXACT,
                           q_e4m3=True)
    kvd = torch.from_numpy(np.ascontiguousarray(x.kv[x.rows[0, 0]])).view(torch.float8_e4m3fn)
    K = x.k_scale * kvd.to(torch.float64).numpy()
    qd = _dec(x.q_bits[0, 0])
    qe = np.empty_like(qd)
    for h in range(16):
        amax = np.abs(qd[h]).max()
        k = 0
        while amax * 2.0 ** (k + 1) <= 448.0 and k < 126:
            k += 1
        while amax * 2.0 ** k > 448.0:
            k -= 1
        qe[h] = [_nearest_e4m3(v * 2.0 ** k) * 2.0 ** -k for v in qd[h]]
    logits = x.scale * (qe @ K.T)
    np.testing.assert_allclose(lse[0, 0], logsumexp(logits, axis=1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, 0], softmax(logits, axis=1) @ K[:, :512], rtol=0, atol=1e-12)


def test_e4m3_query_moves_the_logits_by_at_most_half_an_e4m3_step():
    """|qe - q| <= 2^-4 |q| per value (E4M3 keeps 3 fraction bits) for normal E4M3 magnitudes,
    so the E4M3 query changes LSE by at most scale * sum |q - qe| |K|."""
    x = wl.sparse_case(2, 1, 16, 50, [[50], [31]], 128, seed=5, distinct=True)
    a = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=oracle.EXACT)
    b = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=oracle.EXACT,
                      q_e4m3=True)
    kvd = torch.from_numpy(np.ascontiguousarray(x.kv)).view(torch.float8_e4m3fn)
    kabs = x.k_scale * np.abs(kvd.to(torch.float64).numpy())
    for bb in range(2):
        for h in range(16):
            qd = _dec(x.q_bits[bb, 0, h])
            qe, k = oracle.q_e4m3_row(x.q_bits[bb, 0, h])
            big = np.abs(qd * 2.0 ** k) >= 2.0 ** -6
            assert np.all(np.abs(qe - qd)[big] <= 2.0 ** -4 * np.abs(qd)[big])
            rows = x.rows[bb, 0, :x.valid[bb, 0]]
            bound = x.scale * (np.abs(qe - qd) @ kabs[rows].T).max()
            assert abs(a[1][bb, 0, h] - b[1][bb, 0, h]) <= bound + 1e-12
