"""GPU parity of the candidate-block path of the top-k producer against the oracle (index work:
bit-exact): the candidate expansion (C ABI mla_expand_candidates), the top-k over sparse logit
columns remapped to positions and cache rows (mla_topk_sparse_rows), and end to end: candidate
blocks -> sparse blocks -> top-k over sparse logits -> cache rows -> mla_decode_sparse, against the
oracle's decode over the oracle's lists."""
import numpy as np
import pytest
import torch

import oracle
import paged_mla_decode_fp8_amd as mla
import workloads as wl
from gpu_util import assert_parity, say, upload
from oracle import topk as otopk

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def _cands(rows, K, n_blocks, rng, unique=True, fill=None):
    cand = np.full((rows, K), -1, np.int32)
    for r in range(rows):
        n = int(rng.integers(0, K + 1)) if fill is None else fill
        if unique:
            cand[r, :n] = rng.permutation(n_blocks)[:n]
        else:
            cand[r, :n] = rng.integers(0, n_blocks, n)
        cand[r] = cand[r, rng.permutation(K)]          # -1 padding anywhere in the row
    return cand


EXPAND_CASES = [
    # rows, K, candidate_block_size, sparse_block_kv, candidate id range, ks range, unique
    (6, 8, 16, 16, 20, 0, True),
    (9, 64, 32, 16, 90, 0, True),
    (5, 100, 16, 8, 300, 2000, True),       # K not a power of two, unaligned K range starts
    (4, 2048, 64, 64, 5000, 0, True),
    (3, 8192, 32, 16, 20000, 100000, True),  # 16384 sparse blocks: the largest sort
    (7, 40, 16, 16, 30, 50, False),          # repeats kept
]


@pytest.mark.parametrize("case", range(len(EXPAND_CASES)))
def test_expand_candidates_is_bit_exact(case):
    rows, K, cbs, sbk, nb, ks_hi, unique = EXPAND_CASES[case]
    say("expand", rows, K, cbs, sbk)
    rng = np.random.default_rng(2000 + case)
    cand = _cands(rows, K, nb, rng, unique)
    ks = rng.integers(0, ks_hi + 1, rows).astype(np.int32)
    ke = (ks + rng.integers(0, nb * cbs, rows)).astype(np.int32)
    ke[0] = ks[0] - 3                                  # an empty K range
    si, end = mla.expand_candidates(_t(cand), _t(ks), _t(ke), cbs, sbk)
    torch.cuda.synchronize()
    ref_si, ref_end = otopk.expand_candidates(cand, ks, ke, cbs, sbk)
    assert np.array_equal(end.cpu().numpy(), ref_end)
    assert np.array_equal(si.cpu().numpy(), ref_si)


def _bits(R, N, seed, ties=None, nan=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, N)).astype(np.float32)
    if ties:
        x = np.round(x * ties) / ties
    b = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if nan:
        b[rng.random((R, N)) < nan] = 0x7FC0
    return b


@pytest.mark.parametrize("sbk,K,ties,page", [(16, 64, None, 64), (8, 300, 4, 64), (16, 2048, 2, 64),
                                             (12, 500, 3, 48), (7, 1024, None, 37)])
def test_topk_over_sparse_columns_is_bit_exact(sbk, K, ties, page):
    """Expanded candidates -> synthetic sparse logits (columns past each row's valid count poisoned
    with +inf) -> the top-k remapped to positions, then through a page table to cache rows."""
    say("sparse topk", sbk, K, page)
    rng = np.random.default_rng(sbk * 1000 + K)
    R, Kc, cbs = 6, 512, 2 * sbk
    cand = _cands(R, Kc, 4000, rng, fill=int(Kc * 0.8))
    ks = np.zeros(R, np.int32)
    ke = rng.integers(20000, 4000 * cbs, R).astype(np.int32)
    si, end = otopk.expand_candidates(cand, ks, ke, cbs, sbk)
    width = si.shape[1] * sbk
    bits = _bits(R, width, seed=K, ties=ties, nan=0.01)
    for r in range(R):
        bits[r, end[r]:] = 0x7F80
    lg = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    pos, cnt = mla.topk_sparse_rows(lg, _t(end), K, _t(si), _t(ks), sbk)
    torch.cuda.synchronize()
    ref, ref_cnt = otopk.sparse_topk(bits, end, K, si, ks, sbk)
    assert np.array_equal(cnt.cpu().numpy(), ref_cnt)
    assert np.array_equal(pos.cpu().numpy(), ref)
    # through a page table (two query rows per request); block and page sizes that are not powers
    # of two divide by their precomputed reciprocals
    Q = 2
    pages = int(ke.max()) // page + 1
    table = rng.permutation((R // Q) * pages).astype(np.int32).reshape(R // Q, pages)
    table[0, 5] = -1
    num_rows = (R // Q) * pages * page
    rows, cnt2 = mla.topk_sparse_rows(lg, _t(end), K, _t(si), _t(ks), sbk, block_table=_t(table),
                                      page_size=page, q_per_request=Q, num_rows=num_rows)
    torch.cuda.synchronize()
    assert np.array_equal(cnt2.cpu().numpy(), ref_cnt)
    assert np.array_equal(rows.cpu().numpy(), otopk.remap(ref, table, page, Q, num_rows))


def test_candidate_blocks_to_sparse_decode_matches_the_oracle():
    """The indexer's candidate blocks of each verify row -> sparse blocks -> top-k over (synthetic)
    sparse logits -> cache rows -> sparse decode, against the oracle's decode over the oracle's
    lists (the lists themselves bit-exact)."""
    B, Q, H, page, cbs, sbk, Kc, K = 2, 3, 32, 64, 32, 16, 48, 512
    x = wl.dense_case(B, Q, H, [5000, 2600], page, seed=2100)
    rng = np.random.default_rng(2101)
    R = B * Q
    seq = x.seq_lens.astype(np.int64)
    ke = np.array([seq[r // Q] - Q + (r % Q) + 1 for r in range(R)], np.int32)   # causal bound
    ks = np.zeros(R, np.int32)
    cand = np.full((R, Kc), -1, np.int32)
    for r in range(R):
        nblk = -(-int(ke[r]) // cbs)
        n = min(Kc - 2, nblk)
        cand[r, :n] = rng.permutation(nblk)[:n]
    si, end = mla.expand_candidates(_t(cand), _t(ks), _t(ke), cbs, sbk)
    width = si.shape[1] * sbk
    bits = _bits(R, width, seed=2102)
    lg = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    dev = upload(x)
    rows, valid = mla.topk_sparse_rows(lg, end, K, si, _t(ks), sbk, block_table=dev["table"],
                                       page_size=page, q_per_request=Q, num_rows=x.kv.shape[0])
    o, lse = mla.sparse(dev["q"], dev["kv"], rows.view(B, Q, K), valid.view(B, Q), x.scale,
                        x.k_scale, plan=(2, 2))
    torch.cuda.synchronize()
    ref_si, ref_end = otopk.expand_candidates(cand, ks, ke, cbs, sbk)
    assert np.array_equal(si.cpu().numpy(), ref_si) and np.array_equal(end.cpu().numpy(), ref_end)
    pos, cnt = otopk.sparse_topk(bits, ref_end, K, ref_si, ks, sbk)
    ref_rows = otopk.remap(pos, x.block_table, page, Q, x.kv.shape[0])
    assert np.array_equal(rows.cpu().numpy(), ref_rows) and np.array_equal(valid.cpu().numpy(), cnt)
    # every chosen position lies under its row's causal bound
    assert all(np.all(pos[r, :cnt[r]] < ke[r]) for r in range(R))
    o_ref, lse_ref, amb = oracle.sparse(x.q_bits, x.kv, x.k_scale, ref_rows.reshape(B, Q, K),
                                        cnt.reshape(B, Q), x.scale, mode=oracle.METHOD, splits=2,
                                        chunk=128, allowance=True)
    assert_parity(o, lse, o_ref, lse_ref, amb, what="candidates -> sparse decode")
