"""GPU parity of the decode-context-parallel combine (C ABI mla_combine) against the oracle's FP64
combine of the same bf16 / FP32 partials, and end to end: every row's keys cut into R rank
shares, each share decoded on the GPU, the shares combined on the GPU, against the oracle's decode
with the same cuts (the split identity)."""
import numpy as np
import pytest
import torch

import oracle
import paged_mla_decode_fp8_amd as mla
import workloads as wl
from gpu_util import assert_parity, bits, say, upload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _partials(R, rows, seed, empty_frac=0.2, scale=3.0):
    rng = np.random.default_rng(seed)
    o = torch.from_numpy((rng.standard_normal((R, rows, 512)) * scale).astype(np.float32)).to(torch.bfloat16)
    lse = (rng.standard_normal((R, rows)) * 4).astype(np.float32)
    lse[rng.random((R, rows)) < empty_frac] = -np.inf
    o_np = o.view(torch.int16).numpy().view(np.uint16).copy()
    # rows of ranks without keys hold garbage (NaN bits): they must not be read
    o_np[np.isneginf(lse)] = 0x7FC0
    return o_np, lse


def _check(o_gpu, lse_gpu, o_ref, lse_ref, o_parts_bits, what):
    og = o_gpu.float().cpu().numpy().astype(np.float64).reshape(-1, 512)
    lg = lse_gpu.cpu().numpy().astype(np.float64).reshape(-1)
    o_ref = o_ref.reshape(-1, 512)
    lse_ref = lse_ref.reshape(-1)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty), what
    assert np.all(bits(o_gpu).reshape(-1, 512)[empty] == 0), what
    # FP32 accumulation then one bf16 rounding: within 2^-8 |o| plus FP32-level cancellation
    parts = torch.from_numpy(o_parts_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    big = np.nan_to_num(np.abs(parts), nan=0.0).max(axis=0).reshape(-1, 512).max(axis=1, keepdims=True)
    err = np.abs(og[~empty] - o_ref[~empty])
    tol = (2.0 ** -8 * np.abs(o_ref) + 1e-6 * big)[~empty]
    assert np.all(err <= tol), f"{what}: max o err {err.max():.3g}"
    lerr = np.abs(lg[~empty] - lse_ref[~empty])   # masked first: -inf - -inf is NaN
    assert lerr.size == 0 or lerr.max() <= 1e-5 * np.maximum(1.0, np.abs(lse_ref[~empty])).max(), what


@pytest.mark.parametrize("R,rows", [(1, 5), (2, 33), (8, 320), (3, 1001), (17, 64), (8, 10240)])
def test_combine_matches_the_oracle(R, rows):
    say("combine", R, rows)
    o_np, lse_np = _partials(R, rows, seed=R * 1000 + rows)
    o_parts = torch.from_numpy(o_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    lse_parts = torch.from_numpy(lse_np).to(DEV)
    o, lse = mla.combine(o_parts, lse_parts)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.combine(o_np, lse_np)
    _check(o, lse, o_ref, lse_ref, o_np, f"combine R={R} rows={rows}")
    o2, lse2 = mla.combine(o_parts, lse_parts)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o2)) and np.array_equal(lse.cpu().numpy(), lse2.cpu().numpy())


def test_combine_all_ranks_empty_and_one_rank():
    R, rows = 4, 9
    o_np, lse_np = _partials(R, rows, seed=7, empty_frac=0.0)
    lse_np[:, :3] = -np.inf                        # rows 0..2: no rank holds a key
    lse_np[1:, 3:6] = -np.inf                      # rows 3..5: only rank 0 does
    o_np[np.isneginf(lse_np)] = 0x7FC0
    o_parts = torch.from_numpy(o_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    o, lse = mla.combine(o_parts, torch.from_numpy(lse_np).to(DEV))
    torch.cuda.synchronize()
    ob = bits(o)
    assert np.all(ob[:3] == 0) and np.all(np.isneginf(lse[:3].cpu().numpy()))
    # one rank: w = 1, o_r / 1 rounds back to the same bf16 bits
    assert np.array_equal(ob[3:6], o_np[0, 3:6])
    assert np.array_equal(lse[3:6].cpu().numpy(), lse_np[0, 3:6])


def _rank_shares(x, R, rng):
    """Cut every (b, i) key list into R consecutive shares; returns per-rank (rows, valid) and the
    share starts per list (the oracle's cuts)."""
    B, Q, K = x.rows.shape
    shares = [(np.zeros_like(x.rows), np.zeros_like(x.valid)) for _ in range(R)]
    cuts = []
    for b in range(B):
        for i in range(Q):
            n = int(np.clip(x.valid[b, i], 0, K))
            edges = np.concatenate([[0], np.sort(rng.integers(0, n + 1, size=R - 1)), [n]])
            cuts.append([int(e) for e in edges[:-1]])
            for r in range(R):
                a, e = int(edges[r]), int(edges[r + 1])
                shares[r][0][b, i, :e - a] = x.rows[b, i, a:e]
                shares[r][1][b, i] = e - a
    return shares, cuts


@pytest.mark.parametrize("R", [2, 8])
def test_dcp_decode_then_combine_equals_the_whole_decode(R):
    """The latency checkpoint's rows with their keys spread over R ranks: each rank's share decoded
    by mla.sparse, the shares merged by mla.combine, against the oracle's decode of the whole lists
    cut at the same places."""
    x = wl.latency_sparse()
    rng = np.random.default_rng(R)
    shares, cuts = _rank_shares(x, R, rng)
    dev = upload(x)
    o_parts = torch.empty((R, x.B, x.Q, x.H, 512), dtype=torch.bfloat16, device=DEV)
    lse_parts = torch.empty((R, x.B, x.Q, x.H), dtype=torch.float32, device=DEV)
    for r, (rows_r, valid_r) in enumerate(shares):
        say("rank", r, "keys", int(valid_r.sum()))
        mla.sparse(dev["q"], dev["kv"], torch.from_numpy(rows_r).to(DEV),
                   torch.from_numpy(valid_r).to(DEV), x.scale, x.k_scale, plan=(1, 1),
                   o=o_parts[r], lse=lse_parts[r])
    o, lse = mla.combine(o_parts, lse_parts)
    torch.cuda.synchronize()
    o_ref, lse_ref, amb = oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale,
                                        mode=oracle.METHOD, chunk=128, cuts=cuts, allowance=True)
    # each rank's o is rounded to bf16 before the merge: 2^-9 of its magnitude on top of the
    # decode's tolerance
    assert_parity(o, lse, o_ref, lse_ref, amb + 2.0 ** -9 * np.abs(o_ref) + 1e-6,
                  what=f"DCP{R} decode + combine")
