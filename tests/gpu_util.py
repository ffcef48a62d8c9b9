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


def run_gpu(x, dev, plan):
    if x.kind == "dense":
        o, lse = mla.dense(dev["q"], dev["kv"], dev["table"], dev["seq"], x.scale, x.k_scale,
                           x.page_size, plan=plan)
    else:
        o, lse = mla.sparse(dev["q"], dev["kv"], dev["rows"], dev["valid"], x.scale, x.k_scale,
                            plan=plan)
    torch.cuda.synchronize()
    return o, lse


def bits(o: torch.Tensor) -> np.ndarray:
    return o.view(torch.int16).cpu().numpy().view(np.uint16)


def as_f64(o: torch.Tensor) -> np.ndarray:
    return o.float().cpu().numpy().astype(np.float64)


def run_oracle(x, splits, sel=None, mode=oracle.METHOD):
    if x.kind == "dense":
        return oracle.dense(x.q_bits, x.kv, x.page_size, x.k_scale, x.block_table, x.seq_lens,
                            x.scale, mode=mode, splits=splits, chunk=CHUNK, sel=sel)
    return oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale, mode=mode,
                         splits=splits, chunk=CHUNK, sel=sel)


def assert_parity(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, o_ref, lse_ref, sel=None, what=""):
    """max|do| <= 2e-2 max(1, |o|) per element, |dLSE| <= 1e-3, and rows with no key bit-exact
    (o = +0.0, LSE = -inf)."""
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
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} o elements out of tolerance, max err "
                           f"{err.max():.4g} at {np.unravel_index(err.argmax(), err.shape)}")
    fin = ~empty
    if fin.any():
        lerr = np.abs(lg[fin] - lse_ref[fin])
        assert lerr.max() <= LSE_ATOL, f"{what}: LSE max err {lerr.max():.3g}"
    return float(err.max()) if err.size else 0.0
