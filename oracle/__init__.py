"""FP64 CPU oracle of MLA decode over an FP8 E4M3 latent cache (ctypes wrapper of mla_oracle.c).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. It shares no code with the HIP library.

What it computes, and the passages of the vLLM API pages it follows, is stated in the header of
``mla_oracle.c``. Modes:

* ``EXACT``  -- the textbook softmax definition (LSE = ln sum exp, o = softmax-weighted V).
* ``ONLINE`` -- the pages' split / chunked base-2 online softmax and FP32-style merge, P unrounded.
* ``METHOD`` -- as ``ONLINE`` with P rounded to E4M3 at the 448 anchor of the running maximum.

With ``q_e4m3=True`` the logits use the E4M3 query (``q_e4m3_row``) in place of the bf16 one.
With ``p_split=True`` (METHOD mode) each P meets V as E4M3 hi + lo (``p_used``) instead of E4M3.

With ``allowance=True`` the front ends also return, per output element, how far o may move when a
P that an FP8-MFMA / FP32 implementation can only place to within its per-key error bound (the
derivation is at ``logit_error_bound`` in mla_oracle.c; ``logit_bound`` exposes its sum part) of an
E4M3 rounding midpoint is rounded the other way (METHOD mode; zeros otherwise).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

EXACT, ONLINE, METHOD = 0, 1, 2
_QE4M3 = 16   # flag added to a mode: the E4M3 query
_PSPLIT = 32  # flag added to METHOD: P as E4M3 hi + lo

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile mla_oracle.c with gcc (-O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fPIC", "-shared",
             "-o", tmp, _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        lib.mo_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.mo_e4m3_decode.restype = ctypes.c_double
        lib.mo_e4m3_encode.argtypes = [ctypes.c_double]
        lib.mo_e4m3_encode.restype = ctypes.c_uint8
        lib.mo_bf16_decode.argtypes = [ctypes.c_uint16]
        lib.mo_bf16_decode.restype = ctypes.c_double
        lib.mo_q_e4m3_bits.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.mo_q_e4m3_bits.restype = None
        lib.mo_logit_bound.argtypes = [P, P, i32, ctypes.c_double, ctypes.c_double]
        lib.mo_logit_bound.restype = ctypes.c_double
        lib.mo_p_used.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.mo_p_used.restype = ctypes.c_double
        lib.mo_q_shift.argtypes = [ctypes.c_void_p]
        lib.mo_q_shift.restype = ctypes.c_int
        lib.mo_combine_f64.argtypes = [P, P, i32, i64, P, P]
        lib.mo_combine_f64.restype = None
        lib.mo_combine.argtypes = [P, P, i32, i64, P, P]
        lib.mo_combine.restype = None
        lib.mo_dense.argtypes = [P, i32, i32, i32, P, i64, i32, f32, P, i32, P, f32, i32, i32, i32,
                                 P, P, P, i64, i32, P, P, P]
        lib.mo_dense.restype = i32
        lib.mo_sparse.argtypes = [P, i32, i32, i32, P, i64, f32, P, i32, P, f32, i32, i32, i32,
                                  P, P, P, i64, i32, P, P, P]
        lib.mo_sparse.restype = i32
        _lib = lib
    return _lib


def e4m3_decode(code: int) -> float:
    return _load().mo_e4m3_decode(code)


def e4m3_encode(x: float) -> int:
    return _load().mo_e4m3_encode(float(x))


def bf16_decode(bits: int) -> float:
    return _load().mo_bf16_decode(bits)


def p_used(p: float, split: bool) -> float:
    """The P that meets V in METHOD mode for a P of ``p`` (rounded to FP32 first): E4M3(p), or with
    ``split`` hi + lo, hi = E4M3(p), lo = E4M3(p - hi)."""
    return _load().mo_p_used(float(p), int(bool(split)))


def logit_bound(q_bits_row, k_row, scale, k_scale, q_e4m3=False) -> float:
    """The sum's part of the per-key logit error bound, in log2 units: rs (T + gamma(n) sum|p| +
    sum|r K|) for one query row (uint16 bf16 bits [576]) and one cache row (uint8 [576])."""
    q = _as(q_bits_row, np.uint16).reshape(576)
    k = _as(k_row, np.uint8).reshape(576)
    return _load().mo_logit_bound(_ptr(q), _ptr(k), int(bool(q_e4m3)), float(scale), float(k_scale))


def _flags(mode, q_e4m3, p_split):
    if p_split and int(mode) != METHOD:
        raise ValueError("p_split applies to METHOD mode only")
    return int(mode) | (_QE4M3 if q_e4m3 else 0) | (_PSPLIT if p_split else 0)


def q_e4m3_row(q_bits) -> tuple[np.ndarray, int]:
    """The E4M3 query of one row: ``q_bits`` uint16 bf16 bits [576] -> (FP64 values [576], the
    row's power-of-two exponent k), qe = dec(E4M3(q * 2^k)) * 2^-k."""
    q = _as(q_bits, np.uint16).reshape(576)
    qe = np.zeros(576, np.float64)
    _load().mo_q_e4m3_bits(_ptr(q), _ptr(qe))
    qd = np.ascontiguousarray(q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k = _load().mo_q_shift(_ptr(qd))
    return qe, k


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# Worker threads by default: the cores of this process's affinity mask, at most 16 (the host share
# of one GPU on a shared GPU host).
MAX_THREADS = 16


def _threads(threads):
    if threads is not None:
        return int(threads)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(MAX_THREADS, n))


def _as(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _outputs(B, Q, H, sel):
    n = B * Q * H if sel is None else len(sel)
    return np.zeros((n, 512), np.float64), np.zeros((n,), np.float64)


def _shape(B, Q, H, sel, o, lse, amb):
    if sel is None:
        o, lse = o.reshape(B, Q, H, 512), lse.reshape(B, Q, H)
        amb = None if amb is None else amb.reshape(B, Q, H, 512)
    return (o, lse) if amb is None else (o, lse, amb)


def _sel(sel):
    return None if sel is None else _as(sel, np.int64)


def _cuts(cuts, groups):
    """Explicit split starts per key group (a sequence of ``groups`` sequences) -> CSR arrays."""
    if cuts is None:
        return None, None
    assert len(cuts) == groups
    ptr = np.zeros(groups + 1, np.int64)
    ptr[1:] = np.cumsum([len(c) for c in cuts])
    start = np.concatenate([np.asarray(c, np.int64) for c in cuts]) if groups else np.zeros(0, np.int64)
    return ptr, np.ascontiguousarray(start, np.int64)


def dense(q_bits, kv, page_size, k_scale, block_table, seq_lens, scale, *, mode=METHOD, splits=1,
          chunk=128, cuts=None, sel=None, threads=None, allowance=False, q_e4m3=False,
          p_split=False):
    """Paged dense decode. ``q_bits`` uint16 bf16 bits [B,Q,H,576]; ``kv`` uint8 [num_rows,576];
    ``block_table`` int32 [B,max_pages]; ``seq_lens`` int32 [B].

    The split plan: ``splits`` uniform splits per request (per = ceil(n / splits)), or ``cuts``, one
    sequence of split start keys per request (first 0, non-decreasing, each <= the request's keys).

    Returns ``(o, lse)`` in float64: ``o`` [B,Q,H,512] and ``lse`` [B,Q,H], or [n,512] / [n] for a
    ``sel`` list of flat rows ``(b*Q+i)*H+h``."""
    q_bits = _as(q_bits, np.uint16)
    B, Q, H, D = q_bits.shape
    assert D == 576
    kv = _as(kv, np.uint8).reshape(-1, 576)
    table = _as(block_table, np.int32)
    seq = _as(seq_lens, np.int32)
    assert table.shape[0] == B and seq.shape == (B,)
    sel = _sel(sel)
    o, lse = _outputs(B, Q, H, sel)
    cp, cs = _cuts(cuts, B)
    amb = np.zeros_like(o) if allowance else None
    rc = _load().mo_dense(_ptr(q_bits), B, Q, H, _ptr(kv), kv.shape[0], int(page_size),
                          float(k_scale), _ptr(table), table.shape[1], _ptr(seq), float(scale),
                          _flags(mode, q_e4m3, p_split), int(splits), int(chunk), _ptr(cp),
                          _ptr(cs), _ptr(sel),
                          0 if sel is None else len(sel), _threads(threads), _ptr(o), _ptr(lse),
                          _ptr(amb))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return _shape(B, Q, H, sel, o, lse, amb)


def sparse(q_bits, kv, k_scale, rows, valid, scale, *, mode=METHOD, splits=1, chunk=128, cuts=None,
           sel=None, threads=None, allowance=False, q_e4m3=False, p_split=False):
    """Top-k sparse decode. ``rows`` int32 [B,Q,K] flat cache rows; ``valid`` int32 [B,Q]. The
    split plan as for ``dense``, with ``cuts`` given per (b, i) row list, in order b*Q+i."""
    q_bits = _as(q_bits, np.uint16)
    B, Q, H, D = q_bits.shape
    assert D == 576
    kv = _as(kv, np.uint8).reshape(-1, 576)
    rows = _as(rows, np.int32)
    valid = _as(valid, np.int32)
    assert rows.shape[:2] == (B, Q) and valid.shape == (B, Q)
    sel = _sel(sel)
    o, lse = _outputs(B, Q, H, sel)
    cp, cs = _cuts(cuts, B * Q)
    amb = np.zeros_like(o) if allowance else None
    rc = _load().mo_sparse(_ptr(q_bits), B, Q, H, _ptr(kv), kv.shape[0], float(k_scale),
                           _ptr(rows), rows.shape[2], _ptr(valid), float(scale),
                           _flags(mode, q_e4m3, p_split),
                           int(splits), int(chunk), _ptr(cp), _ptr(cs), _ptr(sel),
                           0 if sel is None else len(sel),
                           _threads(threads), _ptr(o), _ptr(lse), _ptr(amb))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return _shape(B, Q, H, sel, o, lse, amb)


def combine(o_parts, lse_parts):
    """Merge of R partial decodes of the same rows over disjoint key parts (decode-context
    parallelism): ``o_parts`` [R, ..., 512] as float64 values, or uint16 bf16 bits (the decode's
    output format); ``lse_parts`` [R, ...] natural-log LSEs. Returns (o [..., 512], lse [...]) in
    float64."""
    o_parts = np.asarray(o_parts)
    lse_parts = np.asarray(lse_parts)
    R = o_parts.shape[0]
    lead = o_parts.shape[1:-1]
    assert o_parts.shape[-1] == 512 and lse_parts.shape == (R, *lead)
    rows = int(np.prod(lead)) if lead else 1
    o = np.zeros((rows, 512), np.float64)
    lse = np.zeros((rows,), np.float64)
    if o_parts.dtype == np.uint16:
        _load().mo_combine(_ptr(_as(o_parts, np.uint16)), _ptr(_as(lse_parts, np.float32)), R, rows,
                           _ptr(o), _ptr(lse))
    else:
        _load().mo_combine_f64(_ptr(_as(o_parts, np.float64)), _ptr(_as(lse_parts, np.float64)), R,
                               rows, _ptr(o), _ptr(lse))
    return o.reshape(*lead, 512), lse.reshape(lead)
