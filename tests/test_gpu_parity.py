"""GPU parity of the HIP library (called through its C ABI) against the FP64 oracle in METHOD
mode with the same split plan, plus the bit-level properties of the kernels (determinism, tiles
invariance, sparse == dense, page permutation, poisoning, empty rows, single key)."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import (BALANCED, assert_parity, bits, run_gpu, run_oracle, sample_rows, say,
                      upload)

pytestmark = pytest.mark.gpu


def _parity(x, plan, what, sel=None):
    say(what, x.kind, "B,Q,H =", x.B, x.Q, x.H, "plan", plan)
    dev = upload(x)
    o, lse = run_gpu(x, dev, plan)
    o_ref, lse_ref, amb = run_oracle(x, plan, sel=sel)
    return assert_parity(o, lse, o_ref, lse_ref, amb, sel=sel, what=what), o, lse


# ---- the small named workloads, whole ----------------------------------------------------------

@pytest.mark.parametrize("splits", [1, 2, 3])
def test_tiny_sparse(splits):
    _parity(wl.tiny_sparse(), (splits, 1), f"tiny_sparse S={splits}")


@pytest.mark.parametrize("splits", [1, 2, 4])
def test_latency_sparse(splits):
    _parity(wl.latency_sparse(), (splits, 1), f"latency_sparse S={splits}")


# ---- shape fuzz: ragged counts around the 16-key subtile and 128-key block ---------------------

SPARSE_CASES = [
    # B, Q, H, K, valid pattern, cache rows, plan
    (1, 1, 16, 1, [[1]], 64, (1, 1)),
    (2, 3, 16, 33, [[0, 1, 15], [16, 17, 33]], 200, (1, 1)),
    (2, 2, 32, 129, [[127, 128], [129, 31]], 500, (2, 2)),
    (3, 2, 64, 300, [[300, 257, 0], [1, 2, 255]], 4096, (3, 4)),
    (1, 5, 16, 256, [[200, 256, 231, 255, 129]], 65536, (5, 1)),
    (2, 1, 128, 1000, [[1000], [999]], 8000, (4, 4)),
    (1, 1, 48, 77, [[77]], 100, (2, 1)),
    (2, 2, 16, 130, [[63, 64], [65, 130]], 400, (1, 1)),
    (1, 3, 32, 200, [[191, 193, 200]], 1000, (3, 2)),
]


@pytest.mark.parametrize("case", range(len(SPARSE_CASES)))
def test_sparse_fuzz(case):
    B, Q, H, K, valid, N, plan = SPARSE_CASES[case]
    valid = np.array(valid, np.int32).reshape(-1)[: B * Q].reshape(B, Q)
    x = wl.sparse_case(B, Q, H, K, valid, N, seed=500 + case)
    _parity(x, plan, f"sparse fuzz {case}")


DENSE_CASES = [
    # B, Q, H, seq_lens, page_size, plan
    (1, 1, 16, [1], 64, (1, 1)),
    (2, 1, 16, [127, 129], 64, (1, 1)),
    (2, 4, 16, [130, 3], 16, (2, 2)),
    (3, 2, 32, [500, 64, 1], 64, (3, 4)),
    (1, 5, 16, [1031], 1, (4, 1)),
    (2, 3, 64, [0, 700], 32, (2, 4)),
    (1, 2, 128, [2100], 64, (5, 4)),
    (2, 1, 16, [63, 65], 16, (2, 1)),
    (1, 2, 16, [200], 48, (3, 1)),
    (2, 1, 16, [300, 517], 7, (2, 1)),
    (1, 1, 32, [1000], 256, (1, 2)),
]


@pytest.mark.parametrize("case", range(len(DENSE_CASES)))
def test_dense_fuzz(case):
    B, Q, H, seq, ps, plan = DENSE_CASES[case]
    x = wl.dense_case(B, Q, H, seq, page_size=ps, seed=600 + case, extra_pages=3)
    _parity(x, plan, f"dense fuzz {case}")


# ---- exact properties ----------------------------------------------------------------------

def test_single_key_gives_v_row_bits_exactly():
    """n = 1: P = 448 exactly, O / l = v exactly, so o = BF16_RNE(fp32(k_scale * v))."""
    x = wl.sparse_case(3, 2, 32, 4, [[1, 1], [1, 1], [1, 1]], 300, seed=700)
    dev = upload(x)
    o, lse = run_gpu(x, dev, (1, 2))
    v = torch.from_numpy(x.kv[x.rows[:, :, 0]][..., :512]).view(torch.float8_e4m3fn).float()
    ref = (v * torch.tensor(x.k_scale, dtype=torch.float32)).to(torch.bfloat16)
    ref = ref[:, :, None, :].expand(3, 2, 32, 512).contiguous()
    assert np.array_equal(bits(o), ref.view(torch.int16).numpy().view(np.uint16))


def _case_for_bits():
    return wl.sparse_case(2, 2, 64, 700, [[700, 513], [0, 257]], 3000, seed=800)


def test_determinism_three_runs_bit_equal():
    x = _case_for_bits()
    dev = upload(x)
    runs = [run_gpu(x, dev, (5, 2)) for _ in range(3)]
    for o, lse in runs[1:]:
        assert np.array_equal(bits(o), bits(runs[0][0]))
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), runs[0][1].cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("splits", [1, 3])
def test_tiles_per_workgroup_do_not_change_bits(splits):
    x = _case_for_bits()
    dev = upload(x)
    ref = run_gpu(x, dev, (splits, 1))
    for tiles in (2, 4):
        o, lse = run_gpu(x, dev, (splits, tiles))
        assert np.array_equal(bits(o), bits(ref[0])), tiles
        assert np.array_equal(lse.cpu().numpy(), ref[1].cpu().numpy()), tiles


@pytest.mark.parametrize("splits", [1, 4])
def test_sparse_over_all_keys_bit_equals_dense(splits):
    d = wl.dense_case(3, 1, 32, [700, 129, 1], page_size=64, seed=900, extra_pages=2)
    K = 700
    rows = np.zeros((3, 1, K), np.int32)
    for b in range(3):
        for j in range(d.seq_lens[b]):
            rows[b, 0, j] = d.block_table[b, j // 64] * 64 + j % 64
    s = wl.Inputs("sparse", d.q_bits, d.kv, d.k_scale, d.scale, rows=rows,
                  valid=d.seq_lens.reshape(3, 1).copy())
    od, ld = run_gpu(d, upload(d), (splits, 2))
    os_, ls = run_gpu(s, upload(s), (splits, 2))
    assert np.array_equal(bits(od), bits(os_))
    assert np.array_equal(ld.cpu().numpy(), ls.cpu().numpy())


def test_page_permutation_bit_invariance():
    d = wl.dense_case(2, 3, 16, [900, 333], page_size=16, seed=1000, extra_pages=7)
    ref = run_gpu(d, upload(d), (3, 1))
    pool = d.kv.shape[0] // 16
    perm = np.random.default_rng(1).permutation(pool)
    kv2 = np.empty_like(d.kv).reshape(pool, 16, 576)
    kv2[perm] = d.kv.reshape(pool, 16, 576)
    t2 = d.block_table.copy()
    used = t2 != wl.INT32_MAX
    t2[used] = perm[t2[used]]
    d2 = wl.Inputs("dense", d.q_bits, kv2.reshape(-1, 576), d.k_scale, d.scale, page_size=16,
                   block_table=t2, seq_lens=d.seq_lens)
    got = run_gpu(d2, upload(d2), (3, 1))
    assert np.array_equal(bits(got[0]), bits(ref[0]))
    assert np.array_equal(got[1].cpu().numpy(), ref[1].cpu().numpy())


def test_poisoned_unread_memory_leaves_bits_unchanged():
    """NaN (0x7F) in every cache row no key reads, INT32_MAX table entries past seq_len, and
    index entries past valid pointing outside the cache: outputs stay bit-equal."""
    # sparse
    x = wl.sparse_case(2, 2, 32, 300, [[300, 17], [0, 129]], 4000, seed=1100)
    ref = run_gpu(x, upload(x), (2, 2))
    read = set()
    for b in range(2):
        for i in range(2):
            read.update(x.rows[b, i, : x.valid[b, i]].tolist())
    kv = x.kv.copy()
    unread = np.setdiff1d(np.arange(kv.shape[0]), np.array(sorted(read)))
    kv[unread] = 0x7F
    rows = x.rows.copy()
    for b in range(2):
        for i in range(2):
            rows[b, i, x.valid[b, i]:] = 2**31 - 1
    xp = wl.Inputs("sparse", x.q_bits, kv, x.k_scale, x.scale, rows=rows, valid=x.valid)
    got = run_gpu(xp, upload(xp), (2, 2))
    assert np.array_equal(bits(got[0]), bits(ref[0]))
    assert np.array_equal(got[1].cpu().numpy(), ref[1].cpu().numpy())
    # dense
    d = wl.dense_case(2, 2, 16, [300, 70], page_size=32, seed=1101, extra_pages=6)
    ref = run_gpu(d, upload(d), (3, 1))
    kv = d.kv.copy().reshape(-1, 32, 576)
    used_rows = np.zeros(kv.shape[0] * 32, bool)
    for b in range(2):
        for j in range(d.seq_lens[b]):
            used_rows[d.block_table[b, j // 32] * 32 + j % 32] = True
    kv = kv.reshape(-1, 576)
    kv[~used_rows] = 0x7F
    dp = wl.Inputs("dense", d.q_bits, kv, d.k_scale, d.scale, page_size=32,
                   block_table=d.block_table, seq_lens=d.seq_lens)
    got = run_gpu(dp, upload(dp), (3, 1))
    assert np.array_equal(bits(got[0]), bits(ref[0]))
    assert np.array_equal(got[1].cpu().numpy(), ref[1].cpu().numpy())


def test_absent_keys_and_clamped_counts_match_oracle():
    x = wl.sparse_case(2, 2, 16, 200, [[10**6, -3], [150, 200]], 1000, seed=1200)
    x.rows[1, 0, [0, 5, 149]] = [-1, 1000, 2**31 - 1]
    x.rows[1, 1, 100:120] = -7
    _parity(x, (2, 1), "absent keys")
    _parity(x, (3, 1, BALANCED), "absent keys, balanced")


# ---- balanced plans: pieces over the call's concatenated blocks ---------------------------------

BALANCED_SPARSE = [
    # B, Q, H, K, valid pattern, cache rows, plan (pieces, tiles)
    # more pieces than blocks: empty pieces, every group cut into several items
    (1, 3, 16, 300, [[300, 129, 1]], 2000, (16, 1)),
    # many short groups per piece, empty groups at the start, middle and end
    (4, 5, 32, 200, [[0, 5, 17, 128, 129], [0, 0, 200, 1, 64], [3, 0, 0, 77, 150],
                     [200, 199, 2, 0, 0]], 3000, (3, 2)),
    # a few long groups over many pieces, tile sets of 4
    (2, 2, 64, 1500, [[1500, 700], [1, 1200]], 9000, (9, 4)),
    # every group empty
    (2, 2, 16, 50, [[0, 0], [0, 0]], 100, (4, 1)),
    # one piece: the whole call in one workgroup per tile set, no partials
    (3, 1, 16, 400, [[400], [129], [0]], 2000, (1, 1)),
]


@pytest.mark.parametrize("case", range(len(BALANCED_SPARSE)))
def test_balanced_sparse(case):
    B, Q, H, K, valid, N, plan = BALANCED_SPARSE[case]
    valid = np.array(valid, np.int32).reshape(B, Q)
    x = wl.sparse_case(B, Q, H, K, valid, N, seed=1300 + case)
    _parity(x, (plan[0], plan[1], BALANCED), f"balanced sparse {case}")


BALANCED_DENSE = [
    # B, Q, H, seq_lens, page_size, plan (pieces, tiles)
    (5, 1, 16, [700, 3, 129, 0, 1300], 64, (7, 1)),
    (3, 4, 32, [2000, 5, 900], 16, (11, 4)),
    (6, 2, 16, [128, 256, 1, 0, 513, 384], 32, (4, 2)),
    (1, 2, 128, [3000], 64, (6, 4)),
]


@pytest.mark.parametrize("case", range(len(BALANCED_DENSE)))
def test_balanced_dense(case):
    B, Q, H, seq, ps, plan = BALANCED_DENSE[case]
    x = wl.dense_case(B, Q, H, seq, page_size=ps, seed=1400 + case, extra_pages=2)
    _parity(x, (plan[0], plan[1], BALANCED), f"balanced dense {case}")


def test_balanced_determinism_and_tiles_invariance():
    x = wl.sparse_case(3, 2, 64, 900, [[900, 13], [0, 640], [257, 899]], 5000, seed=1500)
    dev = upload(x)
    ref = run_gpu(x, dev, (5, 1, BALANCED))
    for plan in ((5, 1, BALANCED), (5, 2, BALANCED), (5, 4, BALANCED)):
        o, lse = run_gpu(x, dev, plan)
        assert np.array_equal(bits(o), bits(ref[0])), plan
        assert np.array_equal(lse.cpu().numpy().view(np.uint32),
                              ref[1].cpu().numpy().view(np.uint32)), plan


def test_balanced_one_piece_per_group_equals_uniform_single_split():
    """Groups of equal block counts and as many pieces as groups: every piece is one whole group,
    the same work as the uniform plan with one split (bit-equal)."""
    x = wl.sparse_case(2, 3, 32, 256, [[256, 200, 129], [250, 160, 255]], 4000, seed=1600)
    dev = upload(x)
    u = run_gpu(x, dev, (1, 2))
    b = run_gpu(x, dev, (6, 2, BALANCED))
    assert np.array_equal(bits(u[0]), bits(b[0]))
    assert np.array_equal(u[1].cpu().numpy(), b[1].cpu().numpy())


# ---- full-size named workloads, sampled rows ---------------------------------------------------

@pytest.mark.timeout(900)   # the FP64 oracle over 256+ rows of 131072 keys takes about a minute
@pytest.mark.parametrize("name", ["dense_paged", "topk_sparse", "long_dense"])
def test_full_size_workloads_sampled(name):
    w = wl.WORKLOADS[name]
    x = w.make()
    sel = sample_rows(x, 256, seed=3)
    assert len(sel) >= 256
    _parity(x, w.plan, f"{name} sampled ({len(sel)} rows)", sel=sel)


def test_workspace_reused_across_shapes_with_zero_prefix_contract():
    """One caller-owned workspace serves a large split call and then a call of another shape whose
    counters overlap the first call's partials, once its counter prefix is zeroed."""
    import paged_mla_decode_fp8_amd as mla
    a = wl.latency_sparse()
    b = wl.sparse_case(2, 2, 32, 129, [[127, 128], [129, 31]], 500, seed=502)
    plans = ((a, (4, 1)), (b, (3, 2)), (a, (4, 1)), (b, (5, 1, BALANCED)), (a, (7, 1, BALANCED)))
    need = max(mla.workspace_bytes(False, x.B, x.Q, x.H, plan) for x, plan in plans)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    for x, plan in plans:
        say("workspace reuse", x.B, x.Q, x.H, plan)
        zero = mla.workspace_zero_bytes(False, x.B, x.Q, x.H, plan)
        ws[:zero].zero_()
        dev = upload(x)
        o, lse = mla.sparse(dev["q"], dev["kv"], dev["rows"], dev["valid"], x.scale, x.k_scale,
                            plan=plan, workspace=ws)
        torch.cuda.synchronize()
        o_ref, lse_ref, amb = run_oracle(x, plan)
        assert_parity(o, lse, o_ref, lse_ref, amb, what="workspace reuse")
        # the call left its counter prefix zero
        assert int(ws[:zero].count_nonzero()) == 0


# ---- a cache of more than 4 GiB: row offsets beyond 2^32 bytes -----------------------------------

BIG_ROWS = 8_000_000                      # 4.608e9 bytes of cache
FIRST_HIGH_ROW = -(-(1 << 32) // 576)     # 7456541: the first row whose offset needs 33 bits


def _big_pool(n_compact_rows, rng, n_low=None):
    """An increasing injection of the compact cache's rows into the big pool: most land at rows
    whose byte offset is >= 2^32, a few low, the last at the pool's final row."""
    n_low = n_compact_rows // 8 if n_low is None else n_low
    low = np.sort(rng.choice(FIRST_HIGH_ROW, n_low, replace=False))
    high = np.sort(rng.choice(np.arange(FIRST_HIGH_ROW, BIG_ROWS - 1), n_compact_rows - n_low - 1,
                              replace=False))
    return np.concatenate([low, high, [BIG_ROWS - 1]]).astype(np.int64)


def _poisoned_pool():
    big = torch.empty((BIG_ROWS, 576), dtype=torch.uint8, device="cuda:0")
    big.fill_(0x7F)                        # E4M3 NaN in every row no key reads
    return big


def test_sparse_decode_over_a_cache_beyond_4gib():
    """The same lists and rows, once in a compact cache and once scattered over an 8M-row
    (4.6 GB) pool with most rows past byte offset 2^32: the decode must read the same bytes, so
    both runs give the same bits, and both match the oracle on the compact cache."""
    rng = np.random.default_rng(1700)
    x = wl.sparse_case(2, 3, 32, 400, [[400, 1, 257], [129, 0, 399]], 3000, seed=1700)
    where = _big_pool(x.kv.shape[0], rng)
    big = _poisoned_pool()
    big[torch.from_numpy(where).to("cuda:0")] = torch.from_numpy(x.kv).to("cuda:0")
    xb = wl.Inputs("sparse", x.q_bits, None, x.k_scale, x.scale,
                   rows=where[x.rows].astype(np.int32), valid=x.valid)
    assert xb.rows.max() >= FIRST_HIGH_ROW
    for plan in ((1, 2), (3, 1), (5, 2, BALANCED)):
        say("cache beyond 4 GiB, sparse", plan)
        small = run_gpu(x, upload(x), plan)
        devb = upload(wl.Inputs("sparse", x.q_bits, x.kv[:1], x.k_scale, x.scale, rows=xb.rows,
                                valid=x.valid))
        devb["kv"] = big
        got = run_gpu(xb, devb, plan)
        assert np.array_equal(bits(got[0]), bits(small[0])), plan
        assert np.array_equal(got[1].cpu().numpy().view(np.uint32),
                              small[1].cpu().numpy().view(np.uint32)), plan
        o_ref, lse_ref, amb = run_oracle(x, plan)
        assert_parity(got[0], got[1], o_ref, lse_ref, amb, what=f"sparse beyond 4 GiB {plan}")
    del big
    torch.cuda.empty_cache()


def test_dense_decode_over_a_cache_beyond_4gib():
    """Dense: the request's pages scattered over a 125000-page pool (page 64), most of them past
    byte offset 2^32, against the same pages in a compact pool."""
    rng = np.random.default_rng(1701)
    page = 64
    x = wl.dense_case(2, 2, 32, [3000, 700], page_size=page, seed=1701, extra_pages=4)
    n_pages = x.kv.shape[0] // page
    big_pages = BIG_ROWS // page
    first_high_page = -(-FIRST_HIGH_ROW // page)
    low = rng.choice(first_high_page, 3, replace=False)
    high = rng.choice(np.arange(first_high_page, big_pages), n_pages - 3, replace=False)
    where = np.concatenate([low, high]).astype(np.int64)       # compact page p -> pool page
    big = _poisoned_pool()
    big.view(big_pages, page, 576)[torch.from_numpy(where).to("cuda:0")] = \
        torch.from_numpy(x.kv.reshape(n_pages, page, 576)).to("cuda:0")
    table = x.block_table.copy()
    used = table != wl.INT32_MAX
    table[used] = where[table[used]]
    assert table[used].max() >= first_high_page
    for plan in ((1, 4), (3, 2), (7, 4, BALANCED)):
        say("cache beyond 4 GiB, dense", plan)
        small = run_gpu(x, upload(x), plan)
        xb = wl.Inputs("dense", x.q_bits, x.kv[:1], x.k_scale, x.scale, page_size=page,
                       block_table=table, seq_lens=x.seq_lens)
        devb = upload(xb)
        devb["kv"] = big
        got = run_gpu(xb, devb, plan)
        assert np.array_equal(bits(got[0]), bits(small[0])), plan
        assert np.array_equal(got[1].cpu().numpy().view(np.uint32),
                              small[1].cpu().numpy().view(np.uint32)), plan
        o_ref, lse_ref, amb = run_oracle(x, plan)
        assert_parity(got[0], got[1], o_ref, lse_ref, amb, what=f"dense beyond 4 GiB {plan}")
    del big
    torch.cuda.empty_cache()
