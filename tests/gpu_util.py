"""Shared helpers of the GPU tests: upload seeded inputs, run the HIP library through its C ABI,
run the oracle on the same inputs with the same split plan, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_mla_decode_fp8_amd as mla

CHUNK = 128  # keys per block of the kernels: the oracle's chunk for METHOD mode
O_RTOL = 2e-2
LSE_ATOL = 1e-3
UNIFORM, BALANCED = 0, 1   # plan modes of the C ABI


def say(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def upload(x, device="cuda:0"):
    d = {
        "q": torch.from_numpy(x.q_bits.view(np.int16)).view(torch.bfloat16).to(device),
        "kv": torch.from_numpy(x.kv).to(device),
    }
    if x.kind == "dense":
        d["table"] = torch.from_numpy(x.block_table).to(device)
        d["seq"] = torch.from_numpy(x.seq_lens).to(device)
    else:
        d["rows"] = torch.from_numpy(x.rows).to(device)
        d["valid"] = torch.from_numpy(x.valid).to(device)
    return d


def run_gpu(x, dev, plan, q_precision="split", p_precision="e4m3"):
    if x.kind == "dense":
        o, lse = mla.dense(dev["q"], dev["kv"], dev["table"], dev["seq"], x.scale, x.k_scale,
                           x.page_size, plan=plan, q_precision=q_precision, p_precision=p_precision)
    else:
        o, lse = mla.sparse(dev["q"], dev["kv"], dev["rows"], dev["valid"], x.scale, x.k_scale,
                            plan=plan, q_precision=q_precision, p_precision=p_precision)
    torch.cuda.synchronize()
    return o, lse


def bits(o: torch.Tensor) -> np.ndarray:
    return o.view(torch.int16).cpu().numpy().view(np.uint16)


def as_f64(o: torch.Tensor) -> np.ndarray:
    return o.float().cpu().numpy().astype(np.float64)


def group_keys(x) -> np.ndarray:
    """Key count of each key group: request b (dense, clamped to the table's capacity) or list
    (b, i) in order b*Q+i (sparse, clamped to [0, K])."""
    if x.kind == "dense":
        cap = x.block_table.shape[1] * x.page_size
        return np.clip(x.seq_lens.astype(np.int64), 0, cap)
    return np.clip(x.valid.reshape(-1).astype(np.int64), 0, x.rows.shape[2])


def sample_rows(x, n_min=256, seed=0):
    """Flat query rows (b * Q + i) * H + h of a full-size workload for a sampled comparison: at
    least n_min rows, covering every request and position (every key group's rows, with heads drawn
    at random per position), plus the first and last row and, for sparse lists with no key, their
    first and last head."""
    rng = np.random.default_rng(seed)
    groups = x.B * x.Q
    per = max(1, min(x.H, -(-n_min // groups)))
    sel = [(g * x.H + rng.choice(x.H, per, replace=False)) for g in range(groups)]
    sel.append(np.array([0, groups * x.H - 1]))
    if x.kind == "sparse":
        empty = np.flatnonzero(x.valid.reshape(-1) <= 0)
        sel += [empty * x.H, empty * x.H + x.H - 1]
    return np.unique(np.concatenate(sel)).astype(np.int64)


ITEM_BLOCKS = 6   # virtual blocks a key group's run starts with under the balanced plan


def balanced_cuts(x, pieces: int):
    """Split starts per key group under the balanced plan, from its definition in the C header:
    each group is a run of ITEM_BLOCKS + (its 128-key blocks) virtual blocks, the runs in group
    order (V of them) are cut at virtual blocks floor(p V / pieces), p = 1 .. pieces - 1, and
    block j of a group whose run starts at r sits at r + ITEM_BLOCKS + j; a group is split at
    every cut that falls strictly inside its blocks."""
    nb = -(-group_keys(x) // CHUNK)
    V = int((nb + ITEM_BLOCKS).sum())
    cuts_global = sorted({p * V // pieces for p in range(1, pieces)})
    out, pre = [], 0
    for n in nb.tolist():
        b0 = pre + ITEM_BLOCKS
        out.append([0] + [CHUNK * (c - b0) for c in cuts_global if b0 < c < b0 + n])
        pre += ITEM_BLOCKS + n
    return out


def run_oracle(x, plan, sel=None, mode=oracle.METHOD, q_e4m3=False, p_split=False):
    """The oracle on the same inputs under the same split plan ((splits, tiles[, mode])): o, LSE
    and the per-element rounding allowance (o may move by that much where a P lies within FP32
    accuracy of an E4M3 rounding midpoint, so either rounding is correct). q_e4m3: the oracle's
    E4M3 query; p_split: P as E4M3 hi + lo."""
    plan = tuple(plan)
    kw = {"splits": plan[0], "allowance": True, "q_e4m3": q_e4m3}
    if len(plan) > 2 and plan[2] == BALANCED:
        kw = {"cuts": balanced_cuts(x, plan[0]), "allowance": True, "q_e4m3": q_e4m3}
    if p_split:
        kw["p_split"] = True
    if x.kind == "dense":
        return oracle.dense(x.q_bits, x.kv, x.page_size, x.k_scale, x.block_table, x.seq_lens,
                            x.scale, mode=mode, chunk=CHUNK, sel=sel, **kw)
    return oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=mode,
                         chunk=CHUNK, sel=sel, **kw)


def assert_parity(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, o_ref, lse_ref, amb=None, sel=None,
                  what=""):
    """max|do| <= 2e-2 max(1, |o|) per element (plus the oracle's rounding allowance, which may be
    needed by few elements only), |dLSE| <= 1e-3, and rows with no key bit-exact (o = +0.0,
    LSE = -inf)."""
    og = as_f64(o_gpu).reshape(-1, 512)
    lg = lse_gpu.cpu().numpy().astype(np.float64).reshape(-1)
    ob = bits(o_gpu).reshape(-1, 512)
    if sel is not None:
        og, lg, ob = og[sel], lg[sel], ob[sel]
    o_ref = np.asarray(o_ref).reshape(-1, 512)
    lse_ref = np.asarray(lse_ref).reshape(-1)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty), f"{what}: empty-row pattern differs"
    assert np.all(ob[empty] == 0), f"{what}: empty rows must be +0.0"
    err = np.abs(og - o_ref)
    tol = O_RTOL * np.maximum(1.0, np.abs(o_ref))
    allow = 0.0 if amb is None else np.asarray(amb).reshape(-1, 512)
    bad = err > tol + allow
    assert not bad.any(), (f"{what}: {bad.sum()} o elements out of tolerance, max err "
                           f"{err.max():.4g} at {np.unravel_index(err.argmax(), err.shape)}")
    used = int((err > tol).sum())
    if used:
        say(f"{what}: {used} elements within the rounding allowance only")
    assert used <= max(8, err.size // 200), f"{what}: {used} elements need the rounding allowance"
    fin = ~empty
    if fin.any():
        lerr = np.abs(lg[fin] - lse_ref[fin])
        assert lerr.max() <= LSE_ATOL, f"{what}: LSE max err {lerr.max():.3g}"
    return float(err.max()) if err.size else 0.0
