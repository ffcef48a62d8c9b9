"""Python binding of libmla_decode.so: MLA decode attention over an FP8 E4M3 latent cache on
MI355X (gfx950).

Argument marshalling only: every step of the decode runs in the HIP kernels behind the C ABI
declared in include/mla_decode.h. PyTorch provides device memory and the current stream. There is
no fallback: without the built library (``python -m paged_mla_decode_fp8_amd._build``) every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple

import torch

from ._build import LIB

__all__ = ["MlaError", "Plan", "dense", "dense_noalloc", "sparse", "combine", "topk_rows",
           "expand_candidates", "topk_sparse_rows", "plan_dense", "plan_sparse", "workspace_bytes",
           "workspace_zero_bytes", "library_path", "UNIFORM", "BALANCED"]

MLA_OK = 0
UNIFORM, BALANCED = 0, 1   # mla_plan_t.mode


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"mla_decode status {status}: {msg}")
        self.status = status


class Plan(NamedTuple):
    splits: int
    tiles: int
    mode: int = UNIFORM


class _KV(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("num_rows", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("k_scale", ctypes.c_float)]


class _Plan(ctypes.Structure):
    _fields_ = [("splits", ctypes.c_int32), ("tiles", ctypes.c_int32), ("mode", ctypes.c_int32)]


class _SparseCols(ctypes.Structure):
    _fields_ = [("sparse_indices", ctypes.c_void_p), ("S", ctypes.c_int32),
                ("sparse_block_kv", ctypes.c_int32), ("row_ks", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run python -m paged_mla_decode_fp8_amd._build")
        lib = ctypes.CDLL(LIB)
        P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.mla_status_string.argtypes = [i32]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_workspace_bytes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(_Plan)]
        lib.mla_workspace_bytes.restype = sz
        lib.mla_workspace_zero_bytes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(_Plan)]
        lib.mla_workspace_zero_bytes.restype = sz
        lib.mla_plan_dense.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(_Plan)]
        lib.mla_plan_dense.restype = i32
        lib.mla_plan_sparse.argtypes = [i32, i32, i32, i32, ctypes.POINTER(_Plan)]
        lib.mla_plan_sparse.restype = i32
        lib.mla_decode_dense.argtypes = [P, ctypes.POINTER(_KV), P, i32, P, f32, i32, i32, i32,
                                         ctypes.POINTER(_Plan), P, P, P, sz, P]
        lib.mla_decode_dense.restype = i32
        lib.mla_decode_sparse.argtypes = [P, ctypes.POINTER(_KV), P, i32, P, f32, i32, i32, i32,
                                          ctypes.POINTER(_Plan), P, P, P, sz, P]
        lib.mla_decode_sparse.restype = i32
        lib.mla_decode_dense_q.argtypes = [P, ctypes.POINTER(_KV), P, i32, P, f32, i32, i32, i32,
                                           ctypes.POINTER(_Plan), i32, P, P, P, sz, P]
        lib.mla_decode_dense_q.restype = i32
        lib.mla_decode_sparse_q.argtypes = [P, ctypes.POINTER(_KV), P, i32, P, f32, i32, i32, i32,
                                            ctypes.POINTER(_Plan), i32, P, P, P, sz, P]
        lib.mla_decode_sparse_q.restype = i32
        lib.mla_decode_dense_q_noalloc.argtypes = [P, ctypes.POINTER(_KV), P, i32, P, f32, i32, i32,
                                                   i32, ctypes.POINTER(_Plan), i32, P, P, P]
        lib.mla_decode_dense_q_noalloc.restype = i32
        lib.mla_combine.argtypes = [P, P, i32, ctypes.c_int64, P, P, P]
        lib.mla_combine.restype = i32
        lib.mla_topk_rows.argtypes = [P, P, i32, i32, i32, P, i32, i32, i32, ctypes.c_int64, P, P,
                                      P]
        lib.mla_topk_rows.restype = i32
        lib.mla_topk_sparse_rows.argtypes = [P, P, i32, i32, i32, ctypes.POINTER(_SparseCols), P,
                                             i32, i32, i32, ctypes.c_int64, P, P, P]
        lib.mla_topk_sparse_rows.restype = i32
        lib.mla_expand_candidates.argtypes = [P, i32, i32, P, P, i32, i32, P, P, P]
        lib.mla_expand_candidates.restype = i32
        _lib = lib
    return _lib


def _check(status: int):
    if status != MLA_OK:
        raise MlaError(status, _load().mla_status_string(status).decode())


def plan_dense(B: int, Q: int, H: int, max_pages: int, page_size: int) -> Plan:
    p = _Plan()
    _check(_load().mla_plan_dense(B, Q, H, max_pages, page_size, ctypes.byref(p)))
    return Plan(p.splits, p.tiles, p.mode)


def plan_sparse(B: int, Q: int, H: int, K: int) -> Plan:
    p = _Plan()
    _check(_load().mla_plan_sparse(B, Q, H, K, ctypes.byref(p)))
    return Plan(p.splits, p.tiles, p.mode)


def _as_plan(plan) -> Plan:
    return Plan(*plan)


def _plan_struct(plan) -> _Plan:
    pl = _as_plan(plan)
    return _Plan(int(pl.splits), int(pl.tiles), int(pl.mode))


def workspace_bytes(dense: bool, B: int, Q: int, H: int, plan) -> int:
    """Bytes of workspace a call needs (``plan``: a Plan or a (splits, tiles[, mode]) tuple)."""
    return int(_load().mla_workspace_bytes(int(dense), B, Q, H, ctypes.byref(_plan_struct(plan))))


def workspace_zero_bytes(dense: bool, B: int, Q: int, H: int, plan) -> int:
    return int(_load().mla_workspace_zero_bytes(int(dense), B, Q, H,
                                                ctypes.byref(_plan_struct(plan))))


# One workspace per (device, stream) and the length of its prefix known to be zero: a call needs
# its counter prefix zero and leaves exactly that prefix zero (the rest holds partials).
_workspaces: dict = {}


def _workspace(device: torch.device, stream: int, dense, B, Q, H, plan) -> torch.Tensor | None:
    nbytes = workspace_bytes(dense, B, Q, H, plan)
    if nbytes == 0:
        return None
    need_zero = workspace_zero_bytes(dense, B, Q, H, plan)
    key = (device.index, stream)
    ws, zero = _workspaces.get(key, (None, 0))
    if ws is None or ws.numel() < nbytes:
        ws, zero = torch.zeros(nbytes, dtype=torch.uint8, device=device), nbytes
    elif zero < need_zero:
        ws[:need_zero].zero_()   # a fill kernel on the current stream
    _workspaces[key] = (ws, need_zero)
    return ws


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _out_tensor(name, t, shape, dtype, device):
    """A caller's output tensor must have exactly the shape the kernel writes."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _check_tensor(name, t, dtype, device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _outputs(q, o, lse):
    B, Q, H, _ = q.shape
    o = _out_tensor("o", o, (B, Q, H, 512), torch.bfloat16, q.device)
    lse = _out_tensor("lse", lse, (B, Q, H), torch.float32, q.device)
    return o, lse


def _check_tensor(name, t, dtype, device):
    if t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor on {device}")


def _query_shape(q):
    if q.dim() != 4 or q.shape[3] != 576:
        raise ValueError(f"q: expected [B, Q, H, 576], got {tuple(q.shape)}")
    return tuple(q.shape[:3])


def _kv_rows(kv):
    if kv.numel() % 576 != 0 or kv.shape[-1] != 576:
        raise ValueError(f"kv: expected rows of 576 bytes, got {tuple(kv.shape)}")


def _dense_index_shapes(B, kv, block_table, seq_lens):
    """The kernel reads seq_lens[b] and block_table[b, :] for every request b < B."""
    _kv_rows(kv)
    if block_table.dim() != 2 or block_table.shape[0] < B or block_table.shape[1] < 1:
        raise ValueError(f"block_table: expected [>= {B}, max_pages >= 1], got "
                         f"{tuple(block_table.shape)}")
    if tuple(seq_lens.shape) != (B,):
        raise ValueError(f"seq_lens: expected [{B}], got {tuple(seq_lens.shape)}")


def _sparse_index_shapes(B, Q, kv, rows, valid):
    """The kernel reads valid[b, i] and rows[b, i, :] for every list (b, i)."""
    _kv_rows(kv)
    if rows.dim() != 3 or tuple(rows.shape[:2]) != (B, Q) or rows.shape[2] < 1:
        raise ValueError(f"rows: expected [{B}, {Q}, K >= 1], got {tuple(rows.shape)}")
    if tuple(valid.shape) != (B, Q):
        raise ValueError(f"valid: expected [{B}, {Q}], got {tuple(valid.shape)}")


# query precisions of the QK product (C ABI MLA_Q_SPLIT, MLA_Q_E4M3) and P precisions of the PV
# product (MLA_P_E4M3, MLA_P_SPLIT); the entry points take their sum
Q_PRECISIONS = {"split": 0, "e4m3": 1}
P_PRECISIONS = {"e4m3": 0, "split": 2}


def _precision(q_precision: str, p_precision: str) -> int:
    if q_precision not in Q_PRECISIONS:
        raise ValueError(f"q_precision must be one of {sorted(Q_PRECISIONS)}, not {q_precision!r}")
    if p_precision not in P_PRECISIONS:
        raise ValueError(f"p_precision must be one of {sorted(P_PRECISIONS)}, not {p_precision!r}")
    return Q_PRECISIONS[q_precision] | P_PRECISIONS[p_precision]


def _q_precision(name: str) -> int:
    return _precision(name, "e4m3")


def cap_plan(plan, p_precision: str = "e4m3") -> Plan:
    """The plan a call runs: with P as E4M3 hi + lo, at most two tiles per workgroup (the P lo
    tile does not fit in LDS beside four)."""
    pl = _as_plan(plan)
    if P_PRECISIONS.get(p_precision) == P_PRECISIONS["split"] and pl.tiles == 4:
        pl = pl._replace(tiles=2)
    return pl


def _plan_arg(plan):
    if plan is None:
        return None
    return ctypes.byref(_plan_struct(plan))


def dense(q: torch.Tensor, kv: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
          scale: float, k_scale: float, page_size: int, *, plan=None, o=None, lse=None,
          workspace: torch.Tensor | None = None, q_precision: str = "split",
          p_precision: str = "e4m3"):
    """Paged dense decode (C ABI mla_decode_dense_q; mla_decode_dense is its default precision).
    q bf16 [B,Q,H,576]; kv uint8 [rows,576] (or [pages,page_size,576]); block_table int32
    [B,max_pages]; seq_lens int32 [B]. Returns (o bf16 [B,Q,H,512], lse f32 [B,Q,H]) on the
    current stream. With p_precision "split" a plan of four tiles runs as two (cap_plan)."""
    qp = _precision(q_precision, p_precision)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, dev)
    _check_tensor("kv", kv, torch.uint8, dev)
    _check_tensor("block_table", block_table, torch.int32, dev)
    _check_tensor("seq_lens", seq_lens, torch.int32, dev)
    B, Q, H = _query_shape(q)
    _dense_index_shapes(B, kv, block_table, seq_lens)
    o, lse = _outputs(q, o, lse)
    stream = torch.cuda.current_stream(dev).cuda_stream
    pl = cap_plan(plan if plan is not None else plan_dense(B, Q, H, block_table.shape[1], page_size),
                  p_precision)
    if workspace is None:
        workspace = _workspace(dev, stream, True, B, Q, H, pl)
    kvs = _KV(kv.data_ptr(), kv.numel() // 576, int(page_size), float(k_scale))
    _check(_load().mla_decode_dense_q(
        _ptr(q), ctypes.byref(kvs), _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        float(scale), B, Q, H, _plan_arg(pl), qp, _ptr(o), _ptr(lse), _ptr(workspace),
        0 if workspace is None else workspace.numel(), ctypes.c_void_p(stream)))
    return o, lse


def dense_noalloc(q: torch.Tensor, kv: torch.Tensor, block_table: torch.Tensor,
                  seq_lens: torch.Tensor, scale: float, k_scale: float, page_size: int, *,
                  plan=None, o=None, lse=None, q_precision: str = "split",
                  p_precision: str = "e4m3"):
    """``dense`` through the C ABI's mla_decode_dense_q_noalloc: no workspace; the split partials
    live in the library's per-device scratch array (for callers that cannot allocate; calls that
    overlap on one GPU race). Same results as ``dense`` with the same plan."""
    qp = _precision(q_precision, p_precision)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, dev)
    _check_tensor("kv", kv, torch.uint8, dev)
    _check_tensor("block_table", block_table, torch.int32, dev)
    _check_tensor("seq_lens", seq_lens, torch.int32, dev)
    B, Q, H = _query_shape(q)
    _dense_index_shapes(B, kv, block_table, seq_lens)
    o, lse = _outputs(q, o, lse)
    stream = torch.cuda.current_stream(dev).cuda_stream
    pl = None if plan is None else cap_plan(plan, p_precision)
    kvs = _KV(kv.data_ptr(), kv.numel() // 576, int(page_size), float(k_scale))
    _check(_load().mla_decode_dense_q_noalloc(
        _ptr(q), ctypes.byref(kvs), _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        float(scale), B, Q, H, _plan_arg(pl), qp, _ptr(o), _ptr(lse), ctypes.c_void_p(stream)))
    return o, lse


def sparse(q: torch.Tensor, kv: torch.Tensor, rows: torch.Tensor, valid: torch.Tensor,
           scale: float, k_scale: float, *, plan=None, o=None, lse=None,
           workspace: torch.Tensor | None = None, q_precision: str = "split",
           p_precision: str = "e4m3"):
    """Top-k sparse decode (C ABI mla_decode_sparse_q; mla_decode_sparse is its default
    precision). rows int32 [B,Q,K] flat cache rows; valid int32 [B,Q]. Precisions as for dense."""
    qp = _precision(q_precision, p_precision)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, dev)
    _check_tensor("kv", kv, torch.uint8, dev)
    _check_tensor("rows", rows, torch.int32, dev)
    _check_tensor("valid", valid, torch.int32, dev)
    B, Q, H = _query_shape(q)
    _sparse_index_shapes(B, Q, kv, rows, valid)
    K = rows.shape[2]
    o, lse = _outputs(q, o, lse)
    stream = torch.cuda.current_stream(dev).cuda_stream
    pl = cap_plan(plan if plan is not None else plan_sparse(B, Q, H, K), p_precision)
    if workspace is None:
        workspace = _workspace(dev, stream, False, B, Q, H, pl)
    kvs = _KV(kv.data_ptr(), kv.numel() // 576, 1, float(k_scale))
    _check(_load().mla_decode_sparse_q(
        _ptr(q), ctypes.byref(kvs), _ptr(rows), K, _ptr(valid), float(scale), B, Q, H,
        _plan_arg(pl), qp, _ptr(o), _ptr(lse), _ptr(workspace),
        0 if workspace is None else workspace.numel(), ctypes.c_void_p(stream)))
    return o, lse


def combine(o_parts: torch.Tensor, lse_parts: torch.Tensor, *, o=None, lse=None):
    """Merge of R partial decodes of the same rows (C ABI mla_combine): o_parts bf16 [R, ..., 512],
    lse_parts f32 [R, ...] (natural log). Returns (o bf16 [..., 512], lse f32 [...]) on the
    current stream."""
    dev = o_parts.device
    _check_tensor("o_parts", o_parts, torch.bfloat16, dev)
    _check_tensor("lse_parts", lse_parts, torch.float32, dev)
    R = o_parts.shape[0]
    lead = tuple(o_parts.shape[1:-1])
    if o_parts.shape[-1] != 512 or tuple(lse_parts.shape) != (R, *lead):
        raise ValueError("o_parts must be [R, ..., 512] and lse_parts [R, ...]")
    rows = 1
    for d in lead:
        rows *= d
    o = _out_tensor("o", o, (*lead, 512), torch.bfloat16, dev)
    lse = _out_tensor("lse", lse, lead, torch.float32, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(_load().mla_combine(_ptr(o_parts), _ptr(lse_parts), R, rows, _ptr(o), _ptr(lse),
                               ctypes.c_void_p(stream)))
    return o, lse


def topk_rows(logits: torch.Tensor, row_ends: torch.Tensor, k: int, *, block_table=None,
              page_size: int = 1, q_per_request: int = 1, num_rows: int = 0, rows=None,
              valid=None):
    """Top-k key positions of bf16 logits [R, N] (C ABI mla_topk_rows), remapped to cache rows
    through ``block_table`` [R / q_per_request, max_pages] when given. Returns (rows int32 [R, k]
    with -1 padding, valid int32 [R]) on the current stream."""
    dev = logits.device
    _check_tensor("logits", logits, torch.bfloat16, dev)
    _check_tensor("row_ends", row_ends, torch.int32, dev)
    R, N = logits.shape
    if tuple(row_ends.shape) != (R,):
        raise ValueError("row_ends must be [R]")
    max_pages = 0
    if block_table is not None:
        _check_tensor("block_table", block_table, torch.int32, dev)
        max_pages = block_table.shape[1]
        if block_table.shape[0] * q_per_request < R:
            raise ValueError("block_table needs a row per request")
    rows = _out_tensor("rows", rows, (R, k), torch.int32, dev)
    valid = _out_tensor("valid", valid, (R,), torch.int32, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(_load().mla_topk_rows(_ptr(logits), _ptr(row_ends), R, N, int(k), _ptr(block_table),
                                 max_pages, int(page_size), int(q_per_request), int(num_rows),
                                 _ptr(rows), _ptr(valid), ctypes.c_void_p(stream)))
    return rows, valid


def expand_candidates(candidate_blocks: torch.Tensor, row_ks: torch.Tensor, row_ke: torch.Tensor,
                      candidate_block_size: int, sparse_block_kv: int, *, sparse_indices=None,
                      end=None):
    """Candidate blocks [rows, K] (request-local ids, -1 padded) -> (sparse block ids [rows, K *
    ratio], valid sparse-token column counts [rows]) (C ABI mla_expand_candidates), on the current
    stream."""
    dev = candidate_blocks.device
    _check_tensor("candidate_blocks", candidate_blocks, torch.int32, dev)
    _check_tensor("row_ks", row_ks, torch.int32, dev)
    _check_tensor("row_ke", row_ke, torch.int32, dev)
    if candidate_blocks.dim() != 2:
        raise ValueError("candidate_blocks must be [rows, K]")
    rows, K = candidate_blocks.shape
    if tuple(row_ks.shape) != (rows,) or tuple(row_ke.shape) != (rows,):
        raise ValueError("row_ks and row_ke must be [rows]")
    ratio = candidate_block_size // sparse_block_kv if sparse_block_kv > 0 else 0
    sparse_indices = _out_tensor("sparse_indices", sparse_indices, (rows, K * max(ratio, 1)),
                                 torch.int32, dev)
    end = _out_tensor("end", end, (rows,), torch.int32, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(_load().mla_expand_candidates(_ptr(candidate_blocks), rows, K, _ptr(row_ks),
                                         _ptr(row_ke), int(candidate_block_size),
                                         int(sparse_block_kv), _ptr(sparse_indices), _ptr(end),
                                         ctypes.c_void_p(stream)))
    return sparse_indices, end


def topk_sparse_rows(logits: torch.Tensor, end: torch.Tensor, k: int, sparse_indices: torch.Tensor,
                     row_ks: torch.Tensor, sparse_block_kv: int, *, block_table=None,
                     page_size: int = 1, q_per_request: int = 1, num_rows: int = 0, rows=None,
                     valid=None):
    """Top-k over sparse logits [R, N] bounded by ``end`` [R], the chosen columns remapped to
    request-local positions through ``sparse_indices`` [R, S] and ``row_ks`` [R] (C ABI
    mla_topk_sparse_rows), then to cache rows through ``block_table`` when given. Returns
    (rows int32 [R, k], -1 padded; valid int32 [R]) on the current stream."""
    dev = logits.device
    _check_tensor("logits", logits, torch.bfloat16, dev)
    _check_tensor("end", end, torch.int32, dev)
    _check_tensor("sparse_indices", sparse_indices, torch.int32, dev)
    _check_tensor("row_ks", row_ks, torch.int32, dev)
    R, N = logits.shape
    if tuple(end.shape) != (R,) or tuple(row_ks.shape) != (R,):
        raise ValueError("end and row_ks must be [R]")
    if sparse_indices.dim() != 2 or sparse_indices.shape[0] != R:
        raise ValueError("sparse_indices must be [R, S]")
    max_pages = 0
    if block_table is not None:
        _check_tensor("block_table", block_table, torch.int32, dev)
        max_pages = block_table.shape[1]
        if block_table.shape[0] * q_per_request < R:
            raise ValueError("block_table needs a row per request")
    rows = _out_tensor("rows", rows, (R, k), torch.int32, dev)
    valid = _out_tensor("valid", valid, (R,), torch.int32, dev)
    cols = _SparseCols(sparse_indices.data_ptr(), sparse_indices.shape[1], int(sparse_block_kv),
                       row_ks.data_ptr())
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(_load().mla_topk_sparse_rows(_ptr(logits), _ptr(end), R, N, int(k), ctypes.byref(cols),
                                        _ptr(block_table), max_pages, int(page_size),
                                        int(q_per_request), int(num_rows), _ptr(rows), _ptr(valid),
                                        ctypes.c_void_p(stream)))
    return rows, valid
