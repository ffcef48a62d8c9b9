"""GPU parity of the E4M3-query precision (C ABI mla_decode_dense_q / mla_decode_sparse_q with
MLA_Q_E4M3) against the oracle's E4M3 query in METHOD mode under the same split plan, with the
same tolerance as the default precision, plus its bit-level properties: determinism, tiles
invariance, and equality with the default precision on queries already on the E4M3 grid (there the
split's lo part is zero)."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import (BALANCED, assert_parity, bits, run_gpu, run_oracle, sample_rows, say,
                      upload)

pytestmark = pytest.mark.gpu

E4M3 = "e4m3"


def _parity(x, plan, what, sel=None):
    say(what, "(E4M3 query)", x.kind, "B,Q,H =", x.B, x.Q, x.H, "plan", plan)
    dev = upload(x)
    o, lse = run_gpu(x, dev, plan, q_precision=E4M3)
    o_ref, lse_ref, amb = run_oracle(x, plan, sel=sel, q_e4m3=True)
    return assert_parity(o, lse, o_ref, lse_ref, amb, sel=sel, what=what), o, lse


@pytest.mark.parametrize("splits", [1, 2])
def test_tiny_and_latency_sparse(splits):
    _parity(wl.tiny_sparse(), (splits, 1), f"tiny_sparse S={splits}")
    _parity(wl.latency_sparse(), (splits, 1), f"latency_sparse S={splits}")


SPARSE_CASES = [
    (1, 1, 16, 1, [[1]], 64, (1, 1)),
    (2, 3, 16, 33, [[0, 1, 15], [16, 17, 33]], 200, (1, 1)),
    (2, 2, 32, 129, [[127, 128], [129, 31]], 500, (2, 2)),
    (3, 2, 64, 300, [[300, 257, 0], [1, 2, 255]], 4096, (3, 4)),
    (2, 1, 128, 1000, [[1000], [999]], 8000, (4, 4)),
    (2, 2, 64, 1500, [[1500, 700], [1, 1200]], 9000, (9, 4, BALANCED)),
]


@pytest.mark.parametrize("case", range(len(SPARSE_CASES)))
def test_sparse_cases(case):
    B, Q, H, K, valid, rows, plan = SPARSE_CASES[case]
    x = wl.sparse_case(B, Q, H, K, valid, rows, seed=700 + case)
    _parity(x, plan, f"sparse case {case}")


DENSE_CASES = [
    (1, 1, 16, [1], 64, (1, 1)),
    (2, 4, 16, [130, 3], 16, (2, 2)),
    (3, 2, 32, [500, 64, 1], 64, (3, 4)),
    (2, 3, 64, [0, 700], 32, (2, 4)),
    (1, 2, 128, [2100], 64, (5, 4)),
    (3, 4, 32, [2000, 5, 900], 16, (11, 4, BALANCED)),
]


@pytest.mark.parametrize("case", range(len(DENSE_CASES)))
def test_dense_cases(case):
    B, Q, H, seq, page, plan = DENSE_CASES[case]
    x = wl.dense_case(B, Q, H, seq, page, seed=800 + case)
    _parity(x, plan, f"dense case {case}")


def test_determinism_and_tiles_invariance():
    x = wl.dense_case(2, 2, 64, [700, 333], 64, seed=901)
    dev = upload(x)
    ref = run_gpu(x, dev, (3, 4), q_precision=E4M3)
    for plan in ((3, 4), (3, 2), (3, 1)):
        o, lse = run_gpu(x, dev, plan, q_precision=E4M3)
        assert np.array_equal(bits(o), bits(ref[0]))
        assert np.array_equal(lse.cpu().numpy(), ref[1].cpu().numpy())


def test_grid_queries_give_the_default_precision_bits():
    """Query rows whose values times the row's 2^k are E4M3 values: the split's lo part is zero, so
    both precisions multiply the same operands."""
    rng = np.random.default_rng(17)
    x = wl.sparse_case(2, 2, 32, 300, [[300, 129], [1, 257]], 2000, seed=905)
    codes = np.arange(256, dtype=np.uint8)
    grid = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    grid = grid[np.isfinite(grid)]
    k = rng.integers(0, 6, size=(x.B, x.Q, x.H, 1))
    vals = grid[rng.integers(0, len(grid), size=(x.B, x.Q, x.H, 576))] * np.exp2(-k)
    vals[..., 0] = 448.0 * np.exp2(-k[..., 0])
    q = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(q.to(torch.float64).numpy(), vals)
    x.q_bits = q.view(torch.int16).numpy().view(np.uint16)
    dev = upload(x)
    for plan in ((1, 2), (3, 1)):
        a = run_gpu(x, dev, plan)
        b = run_gpu(x, dev, plan, q_precision=E4M3)
        assert np.array_equal(bits(a[0]), bits(b[0]))
        assert np.array_equal(a[1].cpu().numpy(), b[1].cpu().numpy())


@pytest.mark.timeout(900)   # the FP64 oracle over 256+ rows of 131072 keys takes about a minute
@pytest.mark.parametrize("name", ["dense_paged", "topk_sparse", "long_dense"])
def test_full_size_workloads_sampled(name):
    w = wl.WORKLOADS[name]
    x = w.make()
    sel = sample_rows(x, 256, seed=5)
    assert len(sel) >= 256
    _parity(x, w.plan, f"{name} sampled", sel=sel)
