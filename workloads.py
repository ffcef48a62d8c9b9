"""Seeded synthetic inputs for MLA decode: the five named workloads and random test cases.

This module only draws numbers and lays them out (query bits, E4M3 cache bytes, block tables, index
lists, counts). It holds none of the decode arithmetic, and both the oracle side and the HIP side of
every test and of the benchmark take their inputs from it.

Recipe (all on the CPU with ``torch.Generator``; draw order: KV, then Q, then lengths / counts, then
tables / indices -- except that lengths come first where the cache size depends on them):
  * KV cache: x ~ N(0, 1) in fp32, stored as the E4M3 (OCP, RNE) code of clamp(x / k_scale, +-448)
    with k_scale = 0.05, so the dequantized K and V are close to N(0, 1);
  * Q: N(0, 1) rounded to bf16;
  * softmax scale 192 ** -0.5 (fp32).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

ROW = 576
LATENT = 512
K_SCALE = float(np.float32(0.05))   # the per-tensor scale as the fp32 the C ABI takes
SCALE = float(np.float32(192.0 ** -0.5))
INT32_MAX = 2**31 - 1


@dataclasses.dataclass
class Inputs:
    kind: str                      # "dense" or "sparse"
    q_bits: np.ndarray             # uint16 [B,Q,H,576] bf16 bits
    kv: np.ndarray                 # uint8 [num_rows,576] E4M3 codes
    k_scale: float
    scale: float
    # dense
    page_size: int = 0
    block_table: np.ndarray | None = None   # int32 [B,max_pages]
    seq_lens: np.ndarray | None = None      # int32 [B]
    # sparse
    rows: np.ndarray | None = None          # int32 [B,Q,K]
    valid: np.ndarray | None = None         # int32 [B,Q]

    @property
    def B(self):
        return self.q_bits.shape[0]

    @property
    def Q(self):
        return self.q_bits.shape[1]

    @property
    def H(self):
        return self.q_bits.shape[2]

    def kv_rows_read(self) -> int:
        """Cache rows a decode gathers: each key of a key group once (dense: a request's seq_len
        keys; sparse: a (request, position) row's valid keys)."""
        if self.kind == "dense":
            cap = self.block_table.shape[1] * self.page_size
            return int(np.clip(self.seq_lens, 0, cap).sum())
        return int(np.clip(self.valid, 0, self.rows.shape[2]).sum())


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def e4m3_cache(num_rows: int, g: torch.Generator, k_scale: float = K_SCALE) -> np.ndarray:
    x = torch.randn(num_rows, ROW, generator=g, dtype=torch.float32)
    codes = (x / k_scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy()


def bf16_query(B: int, Q: int, H: int, g: torch.Generator) -> np.ndarray:
    q = torch.randn(B, Q, H, ROW, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q.view(torch.int16).numpy().view(np.uint16)


def deal_pages(pages_per_req, max_pages: int, g: torch.Generator, pool: int | None = None
               ) -> np.ndarray:
    """Distinct page ids drawn as a random permutation of the pool (``pool`` pages, default exactly
    the pages used), dealt to the requests in order; unused table entries are INT32_MAX."""
    used = int(sum(pages_per_req))
    pool = used if pool is None else pool
    perm = torch.randperm(pool, generator=g).numpy().astype(np.int32)[:used]
    table = np.full((len(pages_per_req), max_pages), INT32_MAX, np.int32)
    off = 0
    for b, n in enumerate(pages_per_req):
        table[b, :n] = perm[off:off + n]
        off += n
    return table


def dense_case(B, Q, H, seq_lens, page_size=64, max_pages=None, seed=0, extra_pages=0,
               k_scale=K_SCALE) -> Inputs:
    """Dense paged case with the given per-request lengths; the pool holds the pages the requests
    use plus ``extra_pages`` unused ones, in random order."""
    g = _gen(seed)
    seq = np.asarray(seq_lens, np.int64).reshape(B)
    pages = [int(math.ceil(max(int(s), 0) / page_size)) for s in seq]
    if max_pages is None:
        max_pages = max([1] + pages)
    pool = sum(pages) + extra_pages
    kv = e4m3_cache(max(pool, 1) * page_size, g, k_scale)
    q = bf16_query(B, Q, H, g)
    table = deal_pages(pages, max_pages, g, pool)
    return Inputs("dense", q, kv, k_scale, SCALE, page_size=page_size, block_table=table,
                  seq_lens=seq.astype(np.int32))


def sparse_case(B, Q, H, K, valid, num_rows, seed=0, distinct=True, k_scale=K_SCALE) -> Inputs:
    """Sparse case: per (b, i) row, K indices drawn from [0, num_rows) (distinct unless K >
    num_rows or ``distinct`` is False), with the given counts ``valid`` [B,Q]."""
    g = _gen(seed)
    kv = e4m3_cache(num_rows, g, k_scale)
    q = bf16_query(B, Q, H, g)
    valid = np.asarray(valid, np.int32).reshape(B, Q)
    rows = np.zeros((B, Q, K), np.int32)
    for b in range(B):
        for i in range(Q):
            if distinct and K <= num_rows:
                rows[b, i] = torch.randperm(num_rows, generator=g)[:K].numpy()
            else:
                rows[b, i] = torch.randint(0, num_rows, (K,), generator=g).numpy()
    return Inputs("sparse", q, kv, k_scale, SCALE, rows=rows, valid=valid)


# ---- the five named workloads ------------------------------------------------------------------

def tiny_sparse(seed=1000) -> Inputs:
    """B=2, Q=1, H=16; 128-row cache; each row's list holds 64 distinct picks from [0,128);
    request 1 has valid = 0."""
    g = _gen(seed)
    kv = e4m3_cache(128, g)
    q = bf16_query(2, 1, 16, g)
    valid = np.array([[64], [0]], np.int32)
    rows = np.stack([torch.randperm(128, generator=g)[:64].numpy() for _ in range(2)])
    return Inputs("sparse", q, kv, K_SCALE, SCALE, rows=rows.reshape(2, 1, 64).astype(np.int32),
                  valid=valid)


def dense_paged(seed=1001) -> Inputs:
    """B=64, Q=1, H=128, page 64, seq_len uniform in [1024, 8192], table a permutation of pages."""
    g = _gen(seed)
    B, Q, H, ps, max_pages = 64, 1, 128, 64, 8192 // 64
    # the cache size depends on the lengths, so they are drawn first
    seq = torch.randint(1024, 8193, (B,), generator=g).numpy().astype(np.int32)
    pages = [int(math.ceil(s / ps)) for s in seq]
    kv = e4m3_cache(sum(pages) * ps, g)
    q = bf16_query(B, Q, H, g)
    table = deal_pages(pages, max_pages, g)
    return Inputs("dense", q, kv, K_SCALE, SCALE, page_size=ps, block_table=table, seq_lens=seq)


def latency_sparse(seed=1002) -> Inputs:
    """B=4, Q=5, H=16; 65536-row cache; per row valid uniform in [200, 256] over 256 distinct ids."""
    g = _gen(seed)
    B, Q, H, K, N = 4, 5, 16, 256, 65536
    kv = e4m3_cache(N, g)
    q = bf16_query(B, Q, H, g)
    valid = torch.randint(200, 257, (B, Q), generator=g).numpy().astype(np.int32)
    rows = np.stack([torch.randperm(N, generator=g)[:K].numpy() for _ in range(B * Q)])
    return Inputs("sparse", q, kv, K_SCALE, SCALE, rows=rows.reshape(B, Q, K).astype(np.int32),
                  valid=valid)


def topk_sparse(seed=1003, ascending=True) -> Inputs:
    """B=32, Q=5, H=64, top-k 2048; request b's position p is cache row b*32768+p; row (b,i) picks
    2048 distinct positions under its causal bound [0, 32768-5+i]; 8 of the 160 rows have valid=0."""
    g = _gen(seed)
    B, Q, H, K, L = 32, 5, 64, 2048, 32768
    kv = e4m3_cache(B * L, g)
    q = bf16_query(B, Q, H, g)
    valid = np.full((B, Q), K, np.int32)
    empty = torch.randperm(B * Q, generator=g)[:8].numpy()
    valid.reshape(-1)[empty] = 0
    rows = np.zeros((B, Q, K), np.int32)
    for b in range(B):
        for i in range(Q):
            pos = torch.randperm(L - Q + i + 1, generator=g)[:K]
            if ascending:
                pos = pos.sort().values
            rows[b, i] = (b * L + pos).numpy()
    return Inputs("sparse", q, kv, K_SCALE, SCALE, rows=rows, valid=valid)


def long_dense(seed=1004) -> Inputs:
    """B=8, Q=4 (causal), H=128, seq_len 131072, page 64, a random block table over 16384 pages."""
    g = _gen(seed)
    B, Q, H, ps, L = 8, 4, 128, 64, 131072
    pages = [L // ps] * B
    kv = e4m3_cache(sum(pages) * ps, g)
    q = bf16_query(B, Q, H, g)
    seq = np.full((B,), L, np.int32)
    table = deal_pages(pages, L // ps, g)
    return Inputs("dense", q, kv, K_SCALE, SCALE, page_size=ps, block_table=table, seq_lens=seq)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    make: object
    splits: int      # the plan the benchmark launches: splits (uniform) or pieces (balanced)
    tiles: int       # 16-row tiles per workgroup
    mode: int        # 0: uniform splits per key group, 1: balanced pieces over the call's blocks
    description: str

    @property
    def plan(self):
        return (self.splits, self.tiles, self.mode)


WORKLOADS = {
    "tiny_sparse": Workload("tiny_sparse", tiny_sparse, 1, 1, 0,
                            "sparse B=2 Q=1 H=16, 64 of 128 rows, one row empty"),
    "dense_paged": Workload("dense_paged", dense_paged, 128, 4, 1,
                            "dense B=64 Q=1 H=128 page 64 seq_len U[1024,8192]"),
    "latency_sparse": Workload("latency_sparse", latency_sparse, 1, 1, 0,
                               "sparse B=4 Q=5 H=16 valid U[200,256] of a 65536-row cache"),
    "topk_sparse": Workload("topk_sparse", topk_sparse, 1, 4, 0,
                            "sparse B=32 Q=5 H=64 top-k 2048 over 32768 positions, 5% empty"),
    "long_dense": Workload("long_dense", long_dense, 32, 4, 1,
                           "dense causal B=8 Q=4 H=128 seq_len 131072 page 64"),
}
