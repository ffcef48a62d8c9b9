"""GPU parity of the top-k producer (C ABI mla_topk_rows) against the oracle's select and remap,
bit-exact (index work), and end to end: logits -> top-k rows -> mla_decode_sparse against the
oracle's decode over the oracle's lists."""
import numpy as np
import pytest
import torch

import oracle
import paged_mla_decode_fp8_amd as mla
import workloads as wl
from gpu_util import assert_parity, run_oracle, say, upload
from oracle import topk as otopk

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _logits(R, N, seed, tie_levels=None, nan_frac=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, N)).astype(np.float32)
    if tie_levels:
        x = np.round(x * tie_levels) / tie_levels
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if nan_frac:
        bits[rng.random((R, N)) < nan_frac] = 0x7FC0
    return bits


def _run(bits, ends, k, **kw):
    lg = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    re = torch.from_numpy(np.asarray(ends, np.int32)).to(DEV)
    rows, valid = mla.topk_rows(lg, re, k, **kw)
    torch.cuda.synchronize()
    return rows.cpu().numpy(), valid.cpu().numpy()


CASES = [
    # R, N, K, ends, ties, nan
    (3, 8, 1, [8, 3, 0], None, 0.0),
    (4, 64, 7, [64, 7, 6, 100], 4, 0.1),
    (5, 4096, 64, [4096, 4095, 64, 63, 1], None, 0.0),
    (3, 4104, 100, [4104, 4097, 4100], 2, 0.05),
    (4, 32768, 2048, [32768, 32764, 2048, 20000], None, 0.01),
    (2, 32768, 2048, [32768, 32768], 1, 0.0),          # massive ties: values in {-3..3}
    (2, 512, 1000, [512, 300], None, 0.0),             # K > N
    # rows longer than one 32768-column span: the keys are reloaded per span and the output runs
    # carry over from span to span
    (3, 40000, 2048, [32769, 40000, 35000], None, 0.0),   # ends just past, well past the first span
    (2, 65536, 2048, [65536, 50000], 2, 0.05),             # ties at the threshold in both spans
    (1, 131072, 2048, [131072], None, 0.01),               # four spans
    (2, 65544, 4096, [65544, 40001], 8, 0.0),              # K above 2048, a ragged last span
    # K above the 8192 entries the kernel lists in LDS: the list is built in the output row
    (3, 40000, 9000, [40000, 9000, 5000], 4, 0.02),
    (2, 16384, 10000, [16384, 12000], 2, 0.05),        # the same with the row in one span
    (2, 32768, 8192, [32768, 30000], None, 0.0),       # the largest list built in LDS
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_topk_select_is_bit_exact(case):
    R, N, K, ends, ties, nan = CASES[case]
    say("topk", R, N, K, ends)
    bits = _logits(R, N, seed=40 + case, tie_levels=ties, nan_frac=nan)
    # poison: +inf past each row's end must never be chosen
    for r, e in enumerate(ends):
        if e < N:
            bits[r, max(e, 0):] = 0x7F80
    rows, valid = _run(bits, ends, K)
    ref, cnt = otopk.select(bits, np.asarray(ends), K)
    assert np.array_equal(valid, cnt)
    assert np.array_equal(rows, ref)


@pytest.mark.parametrize("page", [64, 48, 37, 1])
def test_topk_remap_through_a_page_table_is_bit_exact(page):
    """Page sizes that are not powers of two divide by their precomputed reciprocal; with 48 and
    37 the table's pages end before N, so the last positions fall past max_pages (-1)."""
    B, Q, N, K = 3, 2, 2048, 128
    say("topk remap", page)
    rng = np.random.default_rng(5 + page)
    pages = N // page
    table = rng.permutation(B * pages).astype(np.int32).reshape(B, pages)
    table[2, -3:] = 2 ** 31 - 1
    num_rows = B * pages * page
    bits = _logits(B * Q, N, seed=77, tie_levels=8)
    ends = rng.integers(0, N + 1, size=B * Q).astype(np.int32)
    rows, valid = _run(bits, ends, K, block_table=torch.from_numpy(table).to(DEV), page_size=page,
                       q_per_request=Q, num_rows=num_rows)
    cols, cnt = otopk.select(bits, ends, K)
    assert np.array_equal(valid, cnt)
    assert np.array_equal(rows, otopk.remap(cols, table, page, Q, num_rows))


def test_topk_then_sparse_decode_matches_the_oracle():
    """Indexer logits -> top-k cache rows -> sparse decode, against the oracle's decode over the
    oracle's lists (the lists themselves are bit-exact)."""
    B, Q, H, ctx, K, page = 2, 3, 32, 3000, 512, 64
    x = wl.dense_case(B, Q, H, [ctx, 2100], page, seed=123)
    rng = np.random.default_rng(8)
    N = ((ctx + 7) // 8) * 8
    bits = _logits(B * Q, N, seed=99)
    seq = x.seq_lens.astype(np.int64)
    ends = np.array([seq[r // Q] - Q + (r % Q) + 1 for r in range(B * Q)], np.int32)   # causal
    dev = upload(x)
    rows, valid = mla.topk_rows(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV),
                                torch.from_numpy(ends).to(DEV), K, block_table=dev["table"],
                                page_size=page, q_per_request=Q, num_rows=x.kv.shape[0])
    o, lse = mla.sparse(dev["q"], dev["kv"], rows.view(B, Q, K), valid.view(B, Q), x.scale,
                        x.k_scale, plan=(1, 2))
    torch.cuda.synchronize()
    cols, cnt = otopk.select(bits, ends, K)
    ref_rows = otopk.remap(cols, x.block_table, page, Q, x.kv.shape[0])
    assert np.array_equal(rows.cpu().numpy(), ref_rows) and np.array_equal(valid.cpu().numpy(), cnt)
    o_ref, lse_ref, amb = oracle.sparse(x.q_bits, x.kv, x.k_scale, ref_rows.reshape(B, Q, K),
                                        cnt.reshape(B, Q), x.scale, mode=oracle.METHOD, chunk=128,
                                        allowance=True)
    assert_parity(o, lse, o_ref, lse_ref, amb, what="top-k -> sparse decode")


def test_topk_rows_whose_first_span_holds_fewer_than_k_candidates():
    """Spans of 32768 columns: the first span of row 0 holds only 1000 candidates (the rest NaN),
    so the threshold and most of the list come from the second; row 1 has fewer than K candidates
    in all (every one is taken, in column order, across spans); row 2 has exactly K."""
    N, K = 40000, 3000
    bits = _logits(3, N, seed=91, tie_levels=4)
    rng = np.random.default_rng(92)
    nan_cols = rng.permutation(32768)[:32768 - 1000]
    bits[0, nan_cols] = 0x7FC0
    bits[1, :] = 0x7FC0
    keep = np.sort(rng.permutation(N)[:2500])
    bits[1, keep] = _logits(1, N, seed=93)[0, keep]
    bits[2, :] = 0x7FC0
    keep2 = np.sort(rng.permutation(N)[:K])
    bits[2, keep2] = _logits(1, N, seed=94, tie_levels=2)[0, keep2]
    ends = [N, N, N]
    rows, valid = _run(bits, ends, K)
    ref, cnt = otopk.select(bits, np.asarray(ends), K)
    assert list(cnt) == [K, 2500, K]
    assert np.array_equal(valid, cnt)
    assert np.array_equal(rows, ref)


@pytest.mark.parametrize("K", [2048, 1024, 1500, 2049])
def test_topk_rows_built_around_the_per_thread_bound(K):
    """Rows of one 32768-column span whose structure sits on the lower bound the kernel derives
    from each thread's 32 consecutive columns (the least of their m-th largest keys, m = ceil(K /
    1024)): row 0 puts two high values (with ties) in every 32-column group and low ones elsewhere,
    so the bound meets the threshold; row 1 ascends, so the first group's bound is far below it;
    row 2 gives half the groups one candidate only (the rest NaN), so too few groups qualify for
    a bound; row 3 is a plain N(0, 1) row ending mid-group."""
    N = 32768
    rng = np.random.default_rng(700 + K)
    x = rng.standard_normal((4, N)).astype(np.float32) - 3.0
    g = N // 32
    hi_cols = (np.arange(g)[:, None] * 32 + np.stack([rng.choice(32, 2, replace=False)
                                                     for _ in range(g)])).ravel()
    x[0, hi_cols] = np.round((rng.standard_normal(hi_cols.size) + 3.0) * 2) / 2
    x[1] = np.sort(rng.standard_normal(N)).astype(np.float32)
    x[3] = rng.standard_normal(N).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    lone = np.arange(0, g, 2) * 32 + rng.integers(0, 32, g // 2)
    keep = np.zeros(N, bool)
    keep[lone] = True
    keep[(np.arange(g) % 2 == 1).repeat(32)] = True
    bits[2, ~keep] = 0x7FC0
    ends = [N, N, N, N - 17]
    rows, valid = _run(bits, ends, K)
    ref, cnt = otopk.select(bits, np.asarray(ends), K)
    assert np.array_equal(valid, cnt)
    assert np.array_equal(rows, ref)


@pytest.mark.parametrize("K", [2048, 700, 3000])
def test_topk_rows_of_wide_and_narrow_value_ranges(K):
    """The first histogram spans the row's ranks from a lower bound to the largest, in bins of 1, 2,
    4, 8 or 16 ranks as the span needs: rows of log-normal values over many binades (wide), of
    values near 1e-30 (narrow, negative and positive), a row of +inf and NaN only, and a row where
    a few huge values sit above a mass of ordinary ones; every row bit-exact against the oracle."""
    N = 32768
    rng = np.random.default_rng(900 + K)
    x = np.empty((5, N), np.float32)
    with np.errstate(over="ignore"):
        x[0] = np.exp(rng.standard_normal(N) * 20.0).astype(np.float32)
    x[1] = (rng.standard_normal(N) * 1e-30).astype(np.float32)
    x[2] = np.inf
    x[3] = rng.standard_normal(N).astype(np.float32)
    x[3, rng.choice(N, 40, replace=False)] = 3e38
    x[4] = -np.abs(rng.standard_normal(N)).astype(np.float32) * 1e20
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    bits[2, rng.random(N) < 0.5] = 0x7FC0
    bits[2, rng.random(N) < 0.2] = 0xFFC1
    ends = [N, N - 3, N, N, 31000]
    rows, valid = _run(bits, ends, K)
    ref, cnt = otopk.select(bits, np.asarray(ends), K)
    assert np.array_equal(valid, cnt)
    assert np.array_equal(rows, ref)


@pytest.mark.parametrize("K", [1, 100, 2048, 30000])
def test_topk_over_every_bf16_pattern(K):
    """Rows that hold every 16-bit pattern once, shuffled (all NaNs of both signs, both zeros, both
    infinities, the subnormals): row 0 all 65536 (two spans, reloaded per pass), rows 1 and 2 the
    even and the odd patterns in one 32768-column span each (held in registers, with the lower
    bound), row 3 the first 20000 of row 1 (a short row). Bit-exact against the oracle's select,
    which ranks by its own order key: the kernel's ranks must order every pair of patterns the
    same way and put every NaN out of the race."""
    rng = np.random.default_rng(1234 + K)
    allp = rng.permutation(65536).astype(np.uint16)
    ev = rng.permutation(np.arange(0, 65536, 2)).astype(np.uint16)
    od = rng.permutation(np.arange(1, 65536, 2)).astype(np.uint16)
    bits = np.full((4, 65536), 0x7FC0, np.uint16)
    bits[0] = allp
    bits[1, :32768] = ev
    bits[2, :32768] = od
    bits[3, :32768] = ev
    ends = [65536, 32768, 32768, 20000]
    rows, valid = _run(bits, ends, K)
    ref, cnt = otopk.select(bits, np.asarray(ends), K)
    assert np.array_equal(valid, cnt)
    assert np.array_equal(rows, ref)
    # the same halves as rows of one 32768-column span (the one-span kernel)
    rows2, valid2 = _run(bits[1:, :32768].copy(), [32768, 32768, 20000], K)
    ref2, cnt2 = otopk.select(bits[1:, :32768].copy(), np.asarray([32768, 32768, 20000]), K)
    assert np.array_equal(valid2, cnt2)
    assert np.array_equal(rows2, ref2)
