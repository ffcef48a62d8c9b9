"""GPU parity against the oracle (METHOD mode, the same split plan) on seeded random shapes and
plans: dense and sparse, uniform and balanced splits, tiles per workgroup, ragged and empty
rows, empty groups, page sizes that are not powers of two, counts outside [0, K]. The named
cases elsewhere pick their shapes by hand; these draw combinations nobody chose. Every case is
bounded in size so that the FP64 oracle finishes in about a second."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import BALANCED, UNIFORM, assert_parity, run_gpu, run_oracle, say, upload

pytestmark = pytest.mark.gpu

WORK = 1_000_000   # bound on sum over query rows of their key counts


def _tiles(tiles_per_group, r):
    return int(r.choice([t for t in (1, 2, 4) if tiles_per_group % t == 0]))


def _plan(r, tiles):
    if r.random() < 0.5:
        return (int(r.integers(1, 13)), tiles, BALANCED)
    return (int(r.integers(1, 5)), tiles, UNIFORM)


def _dense(seed):
    r = np.random.default_rng(seed)
    B, Q = int(r.integers(1, 5)), int(r.integers(1, 5))
    H = int(r.choice([16, 32, 64, 128]))
    page = int(r.choice([1, 7, 16, 64, 100]))
    seq = r.integers(0, 2600, B)
    seq[r.random(B) < 0.2] = 0
    seq[r.random(B) < 0.2] = r.integers(1, 20)
    scale = WORK / max(1, Q * H * int(seq.sum()))
    if scale < 1:
        seq = (seq * scale).astype(np.int64)
    x = wl.dense_case(B, Q, H, [int(s) for s in seq], page_size=page, seed=seed,
                      extra_pages=int(r.integers(0, 5)))
    return x, _plan(r, _tiles(Q * H // 16, r))


def _sparse(seed):
    r = np.random.default_rng(seed)
    B, Q = int(r.integers(1, 4)), int(r.integers(1, 5))
    H = int(r.choice([16, 32, 48, 64]))
    K = int(r.integers(1, 700))
    K = max(1, min(K, WORK // (B * Q * H)))
    valid = r.integers(-3, K + 6, (B, Q)).astype(np.int32)
    valid[r.random((B, Q)) < 0.15] = 0
    N = int(r.integers(max(K, 64), 4000))
    x = wl.sparse_case(B, Q, H, K, valid, N, seed=seed)
    return x, _plan(r, _tiles(H // 16, r))


@pytest.mark.parametrize("seed", range(7000, 7012))
def test_random_dense_shapes_match_the_oracle(seed):
    x, plan = _dense(seed)
    say("random dense", seed, "seq", list(x.seq_lens), "page", x.page_size)
    dev = upload(x)
    o, lse = run_gpu(x, dev, plan)
    o_ref, lse_ref, amb = run_oracle(x, plan)
    assert_parity(o, lse, o_ref, lse_ref, amb, what=f"random dense {seed} plan {plan}")


@pytest.mark.parametrize("seed", range(7100, 7112))
def test_random_sparse_shapes_match_the_oracle(seed):
    x, plan = _sparse(seed)
    say("random sparse", seed, "K", x.rows.shape[-1], "valid", x.valid.reshape(-1).tolist())
    dev = upload(x)
    o, lse = run_gpu(x, dev, plan)
    o_ref, lse_ref, amb = run_oracle(x, plan)
    assert_parity(o, lse, o_ref, lse_ref, amb, what=f"random sparse {seed} plan {plan}")
