"""Pins of the FP64 oracle against what the pages and the mathematics fix, independent of the
oracle's own code: closed forms (single key, identical keys, empty rows), hand-derived worked
examples, the split-merge identity, the E4M3 error bound, library softmax on tiny inputs, and
structural invariances (causal bound, sparse == dense, page permutation, absent keys)."""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _dec_kv(kv_bytes):
    """Dequantize E4M3 bytes with torch (a library routine, independent of the oracle)."""
    t = torch.from_numpy(np.ascontiguousarray(kv_bytes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _dec_q(q_bits):
    t = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _sparse_single_list(q_bits, kv, idx, k_scale=wl.K_SCALE, scale=wl.SCALE, **kw):
    """One request, one position; key list ``idx``."""
    B, Q = 1, 1
    rows = np.asarray(idx, np.int32).reshape(1, 1, -1)
    valid = np.array([[rows.shape[2]]], np.int32)
    return oracle.sparse(q_bits.reshape(B, Q, -1, 576), kv, k_scale, rows, valid, scale, **kw)


ALL_MODES = [oracle.EXACT, oracle.ONLINE, oracle.METHOD]


# ---- closed forms ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ALL_MODES)
def test_count_zero_rows_give_plus_zero_and_minus_inf(mode):
    x = wl.tiny_sparse()
    o, lse = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=mode)
    assert np.all(o[1] == 0) and not np.any(np.signbit(o[1]))
    assert np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(lse[0]))
    # dense: a request shorter than its verify rows leaves the early rows with no key
    d = wl.dense_case(2, 4, 16, [2, 0], page_size=4, seed=3)
    o, lse = oracle.dense(d.q_bits, d.kv, d.page_size, d.k_scale, d.block_table, d.seq_lens,
                          d.scale, mode=mode, splits=2, chunk=4)
    # request 0 (seq_len 2, qlen 4): rows 0 and 1 see seq_len-4+i+1 <= 0 keys; request 1 none
    assert np.all(np.isneginf(lse[0, :2])) and np.all(np.isfinite(lse[0, 2:]))
    assert np.all(np.isneginf(lse[1]))
    assert np.all(o[0, :2] == 0) and np.all(o[1] == 0) and not np.any(np.signbit(o[1]))


@pytest.mark.parametrize("mode", ALL_MODES)
def test_single_key_returns_its_v_row_and_logit(mode):
    x = wl.sparse_case(1, 1, 16, 1, [[1]], 32, seed=11)
    o, lse = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=mode)
    r = x.rows[0, 0, 0]
    kd = _dec_kv(x.kv[r])
    v = x.k_scale * kd[:512]
    qd = _dec_q(x.q_bits[0, 0])
    logit = x.scale * (qd @ (x.k_scale * kd))
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v, (16, 512)), rtol=1e-14, atol=0)
    np.testing.assert_allclose(lse[0, 0], logit, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ALL_MODES)
@pytest.mark.parametrize("n", [2, 7, 300])
def test_identical_keys_give_v_and_logit_plus_log_n(mode, n):
    kv = wl.e4m3_cache(4, wl._gen(5))
    q = wl.bf16_query(1, 1, 16, wl._gen(6))
    o, lse = _sparse_single_list(q, kv, [2] * n, mode=mode, splits=3, chunk=16)
    kd = _dec_kv(kv[2])
    logit = wl.SCALE * (_dec_q(q[0, 0]) @ (wl.K_SCALE * kd))
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(wl.K_SCALE * kd[:512], (16, 512)),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], logit + math.log(n), rtol=1e-12, atol=1e-12)


# ---- worked examples (hand-derived; tests/golden/worked_examples.json) -----------------------

def _worked_inputs(ex):
    n = len(ex["logits"])
    kv = np.zeros((n, 576), np.uint8)
    for j in range(n):
        kv[j, :512] = ex["v_codes"][j]
        kv[j, 512] = ex["logit_codes"][j]
    q = np.zeros((1, 1, 16, 576), np.uint16)
    q[..., 512] = 0x3F80  # bf16 1.0
    return q, kv


@pytest.mark.parametrize("name", [e["name"] for e in json.load(open(GOLDEN))["examples"]])
def test_worked_examples(name):
    data = json.load(open(GOLDEN))
    ex = next(e for e in data["examples"] if e["name"] == name)
    q, kv = _worked_inputs(ex)
    idx = list(range(len(ex["logits"])))
    for mode, key in ((oracle.METHOD, "o_method"), (oracle.EXACT, "o_exact"),
                      (oracle.ONLINE, "o_exact")):
        o, lse = _sparse_single_list(q, kv, idx, k_scale=data["k_scale"], scale=data["scale"],
                                     mode=mode, splits=1, chunk=128)
        np.testing.assert_allclose(o[0, 0], ex[key], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse[0, 0], ex["lse"], rtol=1e-13, atol=1e-15)


# ---- split-merge identity, LSE invariance, E4M3 error bound -----------------------------------

def _cases():
    yield "sparse", wl.sparse_case(2, 3, 16, 300, [[300, 17, 0], [129, 128, 1]], 4096, seed=21)
    yield "dense", wl.dense_case(3, 4, 16, [700, 3, 129], page_size=16, seed=22, extra_pages=5)
    yield "dense_p1", wl.dense_case(1, 2, 16, [77], page_size=1, seed=23)


def _run(name, x, **kw):
    if x.kind == "dense":
        return oracle.dense(x.q_bits, x.kv, x.page_size, x.k_scale, x.block_table, x.seq_lens,
                            x.scale, **kw)
    return oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, **kw)


@pytest.mark.parametrize("splits,chunk", [(1, 128), (1, 1), (2, 16), (3, 128), (5, 7), (16, 32),
                                          (400, 3)])
def test_online_softmax_and_merge_equal_the_definition(splits, chunk):
    for name, x in _cases():
        o0, l0 = _run(name, x, mode=oracle.EXACT)
        o1, l1 = _run(name, x, mode=oracle.ONLINE, splits=splits, chunk=chunk)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12, err_msg=name)
        np.testing.assert_array_equal(np.isneginf(l1), np.isneginf(l0))
        fin = np.isfinite(l0)
        np.testing.assert_allclose(l1[fin], l0[fin], rtol=0, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("splits,chunk", [(1, 128), (3, 16), (7, 128)])
def test_method_lse_is_the_definition_and_o_within_e4m3_bound(splits, chunk):
    for name, x in _cases():
        o0, l0 = _run(name, x, mode=oracle.EXACT)
        o2, l2 = _run(name, x, mode=oracle.METHOD, splits=splits, chunk=chunk)
        fin = np.isfinite(l0)
        np.testing.assert_allclose(l2[fin], l0[fin], rtol=0, atol=1e-12)
        # |P_hat - P| <= 2^-4 P (normal) or 2^-10 (subnormal), the merged total is >= 448 and the
        # weights are <= 1, so |o_method - o_exact| <= k_scale max|v| (2^-4 + 2^-10 n / 448)
        vmax = x.k_scale * 448.0
        n = x.kv_rows_read() + 1
        bound = vmax * (2.0 ** -4 + 2.0 ** -10 * n / 448)
        assert np.max(np.abs(o2 - o0)) <= bound
        # and it is not identical: the rounding of P is really applied
        assert np.max(np.abs(o2 - o0)) > 1e-6


def _groups_keys(x):
    """Key count of each key group (dense: request b; sparse: list (b, i))."""
    if x.kind == "dense":
        cap = x.block_table.shape[1] * x.page_size
        return np.clip(x.seq_lens.astype(np.int64), 0, cap)
    return np.clip(x.valid.reshape(-1).astype(np.int64), 0, x.rows.shape[2])


@pytest.mark.parametrize("seed", range(4))
def test_online_merge_equals_the_definition_for_any_split_boundaries(seed):
    """The merge identity does not depend on where the splits fall: random consecutive splits per
    group (empty ones included, boundaries off the chunk grid) reproduce the definition."""
    rng = np.random.default_rng(seed)
    for name, x in _cases():
        cuts = []
        for n in _groups_keys(x):
            k = int(rng.integers(0, 5))
            inner = np.sort(rng.integers(0, n + 1, size=k)) if n > 0 else np.zeros(k, np.int64)
            cuts.append(np.concatenate([[0], inner]))
        o0, l0 = _run(name, x, mode=oracle.EXACT)
        o1, l1 = _run(name, x, mode=oracle.ONLINE, cuts=cuts, chunk=16)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12, err_msg=name)
        np.testing.assert_array_equal(np.isneginf(l1), np.isneginf(l0))
        fin = np.isfinite(l0)
        np.testing.assert_allclose(l1[fin], l0[fin], rtol=0, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_cuts_at_the_uniform_boundaries_equal_the_uniform_plan(splits):
    for name, x in _cases():
        cuts = []
        for n in _groups_keys(x):
            per = -(-int(n) // splits)
            cuts.append([min(s * per, int(n)) for s in range(splits)])
        a = _run(name, x, mode=oracle.METHOD, splits=splits, chunk=32)
        b = _run(name, x, mode=oracle.METHOD, cuts=cuts, chunk=32)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def test_cuts_that_do_not_cover_the_keys_are_rejected():
    x = wl.sparse_case(1, 2, 16, 40, [[40, 10]], 100, seed=5)
    for bad in ([[0], [5]], [[0, 30, 20], [0]], [[0, 41], [0]], [[], [0]]):
        with pytest.raises(ValueError):
            _run("sparse", x, mode=oracle.METHOD, cuts=bad)


# ---- rounding allowance ------------------------------------------------------------------------

def test_allowance_is_zero_where_rounding_is_unambiguous():
    x = wl.sparse_case(2, 2, 16, 40, [[1, 1], [0, 1]], 64, seed=31)
    for mode in (oracle.EXACT, oracle.ONLINE):
        assert not _run("s", x, mode=mode, allowance=True)[2].any()
    # one key: P = 448 exactly, far from any midpoint
    o, lse, amb = _run("s", x, mode=oracle.METHOD, allowance=True)
    assert not amb.any()


def test_allowance_equals_the_effect_of_flipping_each_ambiguous_rounding():
    """Brute force with torch's E4M3 codec (a library routine): every key whose FP32 P lies within
    its error bound of an E4M3 rounding midpoint, rounded the other way, moves o by at most the
    allowance, and the allowance is the sum of those moves (one split, one chunk). The key's bound
    is the logit bound d(x) = logit_bound + 2^-23 (|x| + |x - m|), plus d(m) (the largest of the
    keys' d), as relative error exp2(d(x) + d(m)) - 1 + 2^-22."""
    x = wl.sparse_case(1, 1, 16, 3000, [[3000]], 3000, seed=32, distinct=True)
    o, lse, amb = _run("s", x, mode=oracle.METHOD, allowance=True, splits=1, chunk=4096)
    q = _dec_q(x.q_bits)[0, 0]                       # [16, 576]
    keys = x.rows[0, 0]
    kd = _dec_kv(x.kv[keys])                          # [3000, 576] E4M3 values
    x2 = (q @ kd.T) * x.scale * x.k_scale / math.log(2)   # logits in log2 units, [16, 3000]
    m = x2.max(axis=1, keepdims=True)
    p = 448.0 * np.exp2(x2 - m)

    def e4m3(v):
        t = torch.from_numpy(np.clip(v.astype(np.float32), -448, 448))
        return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()

    bound = np.array([[oracle.logit_bound(x.q_bits[0, 0, h], x.kv[j], x.scale, x.k_scale)
                       for j in keys] for h in range(16)])
    dx = bound + np.abs(x2) * 2.0 ** -23
    dm = dx.max(axis=1, keepdims=True)
    eps = np.exp2(dx + np.abs(x2 - m) * 2.0 ** -23 + dm) - 1 + 2.0 ** -22
    pf = p.astype(np.float32).astype(np.float64)     # the decision is taken on P in FP32
    ph = e4m3(pf)
    alt_lo, alt_hi = e4m3(pf * (1 - eps)), e4m3(pf * (1 + eps))
    d = np.maximum(np.abs(alt_lo - ph), np.abs(alt_hi - ph))
    L = p.sum(axis=1, keepdims=True)
    v = kd[:, :512]
    amb_py = (d @ np.abs(v)) * x.k_scale / L
    np.testing.assert_allclose(amb[0, 0], amb_py, rtol=1e-9, atol=1e-15)
    n_amb = 0
    for h, j in zip(*np.nonzero(d)):
        n_amb += 1
        alt = alt_lo[h, j] if alt_lo[h, j] != ph[h, j] else alt_hi[h, j]
        moved = np.abs((alt - ph[h, j]) * v[j] * x.k_scale / L[h, 0])
        assert np.all(moved <= amb[0, 0, h] * (1 + 1e-12))
    assert n_amb > 0, "the case must contain ambiguous roundings"


# ---- library softmax on tiny inputs -----------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_exact_mode_matches_scipy_softmax_on_tiny_inputs(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    x = wl.sparse_case(1, 1, 16, n, [[n]], 64, seed=100 + seed, distinct=False)
    o, lse = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=oracle.EXACT)
    K = x.k_scale * _dec_kv(x.kv[x.rows[0, 0]])          # [n, 576]
    qd = _dec_q(x.q_bits[0, 0])                          # [16, 576]
    logits = x.scale * (qd @ K.T)                        # [16, n]
    ref_lse = logsumexp(logits, axis=1)
    ref_o = softmax(logits, axis=1) @ K[:, :512]
    np.testing.assert_allclose(lse[0, 0], ref_lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, 0], ref_o, rtol=0, atol=1e-12)
    # the exact definition does not depend on the order of the key list
    perm = rng.permutation(n)
    o2, lse2 = _sparse_single_list(x.q_bits, x.kv, x.rows[0, 0][perm], k_scale=x.k_scale,
                                   mode=oracle.EXACT)
    np.testing.assert_allclose(o2[0, 0], o[0, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2[0, 0], lse[0, 0], rtol=0, atol=1e-13)


# ---- structure: causal bound, sparse vs dense, pages, absent keys, clamping ----------------

@pytest.mark.parametrize("mode", [oracle.EXACT, oracle.ONLINE])
def test_causal_row_equals_shorter_single_row_request(mode):
    Q = 4
    d = wl.dense_case(1, Q, 16, [203], page_size=16, seed=31)
    o, lse = oracle.dense(d.q_bits, d.kv, 16, d.k_scale, d.block_table, d.seq_lens, d.scale,
                          mode=mode, splits=3, chunk=32)
    for i in range(Q):
        seq_i = np.array([203 - Q + i + 1], np.int32)
        oi, li = oracle.dense(d.q_bits[:, i:i + 1], d.kv, 16, d.k_scale, d.block_table, seq_i,
                              d.scale, mode=mode, splits=2, chunk=16)
        np.testing.assert_allclose(o[0, i], oi[0, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, i], li[0, 0], rtol=0, atol=1e-12)
        # and it equals a sparse list of exactly keys 0 .. seq_len - qlen + i (no causal logic there)
        n_i = 203 - Q + i + 1
        keys = [d.block_table[0, j // 16] * 16 + j % 16 for j in range(n_i)]
        os_, ls = _sparse_single_list(d.q_bits[:, i:i + 1], d.kv, keys, mode=oracle.EXACT)
        np.testing.assert_allclose(o[0, i], os_[0, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, i], ls[0, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ALL_MODES)
def test_sparse_over_all_keys_equals_dense(mode):
    d = wl.dense_case(2, 1, 32, [300, 129], page_size=64, seed=41, extra_pages=3)
    od, ld = oracle.dense(d.q_bits, d.kv, 64, d.k_scale, d.block_table, d.seq_lens, d.scale,
                          mode=mode, splits=3, chunk=64)
    K = 300
    rows = np.zeros((2, 1, K), np.int32)
    for b in range(2):
        for j in range(d.seq_lens[b]):
            rows[b, 0, j] = d.block_table[b, j // 64] * 64 + j % 64
    os_, ls = oracle.sparse(d.q_bits, d.kv, d.k_scale, rows, d.seq_lens.reshape(2, 1), d.scale,
                            mode=mode, splits=3, chunk=64)
    np.testing.assert_array_equal(os_, od)
    np.testing.assert_array_equal(ls, ld)


def test_page_permutation_invariance():
    d = wl.dense_case(2, 2, 16, [190, 64], page_size=16, seed=51, extra_pages=4)
    ref = oracle.dense(d.q_bits, d.kv, 16, d.k_scale, d.block_table, d.seq_lens, d.scale,
                       mode=oracle.METHOD, splits=2, chunk=32)
    pool = d.kv.shape[0] // 16
    perm = np.random.default_rng(0).permutation(pool)         # new page id of old page p
    kv2 = np.empty_like(d.kv).reshape(pool, 16, 576)
    kv2[perm] = d.kv.reshape(pool, 16, 576)
    t2 = d.block_table.copy()
    used = t2 != wl.INT32_MAX
    t2[used] = perm[t2[used]]
    got = oracle.dense(d.q_bits, kv2.reshape(-1, 576), 16, d.k_scale, t2, d.seq_lens, d.scale,
                       mode=oracle.METHOD, splits=2, chunk=32)
    np.testing.assert_array_equal(got[0], ref[0])
    np.testing.assert_array_equal(got[1], ref[1])


def test_absent_keys_are_dropped_and_counts_clamped():
    x = wl.sparse_case(1, 1, 16, 40, [[40]], 100, seed=61)
    idx = x.rows[0, 0].copy()
    o0, l0 = _sparse_single_list(x.q_bits, x.kv, idx, mode=oracle.EXACT)
    bad = idx.copy()
    bad[[3, 17, 39]] = [-1, 100, 2**31 - 1]
    o1, l1 = _sparse_single_list(x.q_bits, x.kv, bad, mode=oracle.EXACT)
    keep = np.delete(idx, [3, 17, 39])
    o2, l2 = _sparse_single_list(x.q_bits, x.kv, keep, mode=oracle.EXACT)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    assert not np.array_equal(o0, o1)
    # valid above K behaves as K, below 0 as 0
    rows = idx.reshape(1, 1, -1)
    for v, ref_n in ((10**6, 40), (-5, 0)):
        o, lse = oracle.sparse(x.q_bits, x.kv, x.k_scale, rows, np.array([[v]], np.int32),
                               x.scale, mode=oracle.EXACT)
        if ref_n == 0:
            assert np.all(o == 0) and np.all(np.isneginf(lse))
        else:
            np.testing.assert_array_equal(o, o0)


def test_unused_pages_out_of_pool_are_absent():
    d = wl.dense_case(1, 1, 16, [100], page_size=16, seed=71)
    ref = oracle.dense(d.q_bits, d.kv, 16, d.k_scale, d.block_table, d.seq_lens, d.scale,
                       mode=oracle.EXACT)
    # point page 2 (keys 32..47) outside the pool: those keys drop out
    t = d.block_table.copy()
    t[0, 2] = wl.INT32_MAX
    got = oracle.dense(d.q_bits, d.kv, 16, d.k_scale, t, d.seq_lens, d.scale, mode=oracle.EXACT)
    rows = [d.block_table[0, j // 16] * 16 + j % 16 for j in range(100) if not 32 <= j < 48]
    exp = _sparse_single_list(d.q_bits, d.kv, rows, mode=oracle.EXACT)
    np.testing.assert_array_equal(got[0], exp[0])
    assert not np.array_equal(got[0], ref[0])


# ---- the logit error bound against the measured MFMA accumulation --------------------------------

def _e4m3_np(v):
    t = torch.from_numpy(np.clip(np.asarray(v, np.float64), -448, 448).astype(np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _mfma_emulated_sum(hi, lo, kd, rng):
    """A logit's sum as MI355X's FP8 MFMA was measured to form it: 9 instructions of 128 products
    (latent steps of hi and lo, 128 columns each, and one rope step of 64 hi then 64 lo columns);
    in each, groups of 8 consecutive products cut toward zero to a multiple of 2^(e - 13) (e the
    floor log2 of the group's largest |product|), then the group sums added to an FP32 accumulator
    with round to nearest even, in a random order."""
    steps = [(hi, slice(128 * s, 128 * s + 128)) for s in range(4)] + \
            [(lo, slice(128 * s, 128 * s + 128)) for s in range(4)]
    acc = np.float32(0.0)
    chains = [np.concatenate([hi[512:] * kd[512:], lo[512:] * kd[512:]])]
    chains = [op[sl] * kd[sl] for op, sl in steps] + chains
    for prods in [chains[i] for i in rng.permutation(len(chains))]:
        groups = prods.reshape(16, 8)
        sums = []
        for g in groups:
            mx = np.abs(g).max()
            if mx == 0:
                sums.append(0.0)
                continue
            w = 2.0 ** (math.floor(math.log2(mx)) - 13)
            sums.append(float(np.sum(np.trunc(g / w) * w)))   # exact in FP64 (a few dozen bits)
        for v in [sums[i] for i in rng.permutation(16)]:
            acc = np.float32(np.float64(acc) + v)             # one FP32 rounding per addition
    return float(acc)


@pytest.mark.parametrize("seed", range(3))
def test_logit_bound_covers_the_measured_mfma_accumulation(seed):
    """The sum part of the per-key bound holds for an emulation of the measured MFMA arithmetic
    (group truncation, FP32 adds in random orders) on random rows and on rows built to lose the most
    (groups of one large product and seven just below the cut), and is not vacuous: within a few
    hundred times the error typical rows actually make."""
    rng = np.random.default_rng(seed)
    scale, k_scale = wl.SCALE, wl.K_SCALE
    errs, bounds = [], []
    for trial in range(60):
        q = torch.randn(576, dtype=torch.float32).to(torch.bfloat16)
        kraw = rng.standard_normal(576) / k_scale
        if trial % 3 == 2:                       # adversarial: per group one big, seven small
            kraw = np.where(np.arange(576) % 8 == 0, 400.0, 400.0 * 2.0 ** -13.9)
            q = torch.full((576,), 1.0).to(torch.bfloat16)
        kbytes = torch.from_numpy(kraw.astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
        kd = kbytes.to(torch.float64).numpy()
        qd = q.to(torch.float64).numpy()
        k = int(np.floor(np.log2(448.0 / np.abs(qd).max())))
        y = qd * 2.0 ** k
        hi = _e4m3_np(y)
        lo = _e4m3_np(y - hi)
        got = _mfma_emulated_sum(hi, lo, kd, rng)
        exact = float(np.sum(y * kd))                   # the bf16 query's sum (q 2^k units)
        rs = scale * k_scale / math.log(2) * 2.0 ** -k
        b = oracle.logit_bound(q.view(torch.int16).numpy().view(np.uint16), kbytes.view(torch.uint8).numpy(),
                               scale, k_scale)
        errs.append(abs(got - exact) * rs)
        bounds.append(b)
        assert abs(got - exact) * rs <= b, (trial, abs(got - exact) * rs, b)
    errs, bounds = np.array(errs), np.array(bounds)
    adv = np.arange(60) % 3 == 2
    assert np.all(errs[adv] >= 0.25 * bounds[adv])      # the adversarial rows come near the bound
    assert np.median(bounds[~adv] / np.maximum(errs[~adv], 1e-30)) < 1000
