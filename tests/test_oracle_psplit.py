"""Pins of the oracle's P as E4M3 hi + lo (the AMD mla_attn page: module docstring and fp8_split4;
P meets V as two E4M3 values whose sum approximates it), independent of the oracle's code: the
pair against torch's float8_e4m3fn conversion, its monotonicity (on which the rounding allowance
rests) and error bound, a two-key decode whose closed form tells hi + lo from hi alone and from an
unrounded lo, and the decode-level bound against the textbook softmax."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
import workloads as wl


def _torch_pair(p):
    """hi = E4M3(p), lo = E4M3(p - hi) with torch's conversion (FP32 in, RNE)."""
    pf = torch.tensor(p, dtype=torch.float32)
    hi = pf.to(torch.float8_e4m3fn).to(torch.float32)
    lo = (pf - hi).to(torch.float8_e4m3fn).to(torch.float32)
    return hi.double().numpy(), lo.double().numpy(), pf.double().numpy()


def _grid():
    rng = np.random.default_rng(0)
    # every binade of (0, 448], log-uniform, plus the E4M3 values and their midpoints
    g = np.exp2(rng.uniform(-14, math.log2(448), 20000))
    codes = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    mids = (codes[1:] + codes[:-1]) / 2
    return np.concatenate([g, codes[1:], mids, [448.0]])


def test_pair_matches_torch_conversion():
    g = _grid()
    hi, lo, pf = _torch_pair(g)
    got = np.array([oracle.p_used(x, True) for x in g])
    single = np.array([oracle.p_used(x, False) for x in g])
    assert np.array_equal(got, hi + lo)
    assert np.array_equal(single, hi)


def test_pair_is_monotone_and_within_its_bound():
    g = np.sort(_grid())
    got = np.array([oracle.p_used(x, True) for x in g])
    assert np.all(np.diff(got) >= 0)
    pf = g.astype(np.float32).astype(np.float64)
    # |P - (hi + lo)| <= half an E4M3 step of lo: <= 2^-8 P while lo is normal, else <= 2^-10
    assert np.all(np.abs(got - pf) <= np.maximum(pf * 2.0 ** -8, 2.0 ** -10))
    # and the single E4M3 value is off by up to 2^-4 P: the pair is the finer one
    single = np.array([oracle.p_used(x, False) for x in g])
    assert np.max(np.abs(single - pf) / pf) > 2.0 ** -5


def _two_keys(p2):
    """One query row (q = 1 at column 0) and two keys whose column-0 bytes are 1 and 0: logits
    scale k_scale and 0, so with the anchor at the larger one P = (448, 448 exp(-scale k_scale)).
    The scale is chosen so that the second P is p2 (up to FP32 rounding of the scale)."""
    rng = np.random.default_rng(5)
    H = 16
    q = np.zeros((1, 1, H, 576), np.uint16)
    q[..., 0] = 0x3F80                                    # bf16 1.0
    kv = rng.integers(0, 0x7F, size=(2, 576), dtype=np.uint8)
    kv[kv == 0x7F] = 0
    kv[:, 512:] = 0                                       # rope bytes: no part in the logit
    kv[0, 0] = 0x38                                       # E4M3 1.0
    kv[1, 0] = 0x00
    ks = np.float32(wl.K_SCALE)
    scale = np.float32(math.log(448.0 / p2) / float(ks))
    p2_exact = 448.0 * math.exp(-float(scale) * float(ks))
    rows = np.array([[[0, 1]]], np.int32)
    valid = np.array([[2]], np.int32)
    v = torch.from_numpy(kv[:, :512].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return q, kv, ks, rows, valid, scale, p2_exact, v


@pytest.mark.parametrize("p2,used_split,used_single", [(301.3, 301.0, 288.0), (300.0, 300.0, 288.0),
                                                      (17.2, 17.1875, 18.0)])
def test_two_key_decode_closed_form(p2, used_split, used_single):
    # 301.3: E4M3 steps are 32 in [256, 448) -> hi = 288; 13.3 in [8, 16) (steps of 1) -> lo = 13.
    # 17.2: steps of 2 in [16, 32) -> hi = 18; -0.8 in [0.5, 1) (steps of 1/16) -> lo = -0.8125.
    q, kv, ks, rows, valid, scale, p2e, v = _two_keys(p2)
    lse_ref = math.log(math.exp(float(scale) * float(ks)) + 1.0)
    for split, used in ((True, used_split), (False, used_single)):
        o, lse = oracle.sparse(q, kv, ks, rows, valid, scale, mode=oracle.METHOD, p_split=split)
        ref = float(ks) * (448.0 * v[0] + used * v[1]) / (448.0 + p2e)
        np.testing.assert_allclose(o[0, 0], np.broadcast_to(ref, o[0, 0].shape), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse[0, 0], lse_ref, rtol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_decode_within_the_pair_bound_of_the_textbook_softmax(seed):
    """One split, one chunk (one anchor, the row maximum): each P used is within
    max(2^-8 P, 2^-10) (+ FP32 rounding of P) of the exact 448 exp(x - max), so
    |o - o_exact| <= k_scale sum_j (2^-8 w_j + 2^-10 / l + 2^-23 w_j) |V_j| with w the softmax
    weights and l = sum_j 448 exp(x_j - max)."""
    n, H = 200, 16
    x = wl.sparse_case(1, 1, H, n, [[n]], 600, seed=700 + seed)
    q = torch.from_numpy(x.q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    kvd = torch.from_numpy(x.kv.reshape(-1, 576)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ks = float(np.float32(x.k_scale))
    K = ks * kvd[x.rows[0, 0, :n]]
    V = ks * kvd[x.rows[0, 0, :n], :512]
    o_ps, _ = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale,
                            mode=oracle.METHOD, p_split=True, chunk=4096)
    o_1, _ = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale,
                           mode=oracle.METHOD, chunk=4096)
    worst_single = 0.0
    for h in range(H):
        logits = float(np.float32(x.scale)) * (K @ q[0, 0, h])
        w = np.exp(logits - logsumexp(logits))
        o_ex = w @ V
        l = 448.0 * np.exp(logits - logits.max()).sum()
        bound = (2.0 ** -8 + 2.0 ** -23) * (w @ np.abs(V)) + 2.0 ** -10 / l * np.abs(V).sum(axis=0)
        assert np.all(np.abs(o_ps[0, 0, h] - o_ex) <= bound * (1 + 1e-9) + 1e-15)
        worst_single = max(worst_single, float(np.max(np.abs(o_1[0, 0, h] - o_ex) / bound)))
    assert worst_single > 1.0      # the bound would catch a dropped lo


def test_p_split_needs_method_mode():
    x = wl.sparse_case(1, 1, 16, 8, [[8]], 50, seed=1)
    with pytest.raises(ValueError):
        oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=oracle.ONLINE,
                      p_split=True)
