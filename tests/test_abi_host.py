"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/mla_decode.h declares, and rejects bad arguments with the documented status before
touching the device."""
import ctypes
import os
import re

import pytest

import paged_mla_decode_fp8_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")

OK, NULL, SHAPE, ALIGN, WORKSPACE, UNSUPPORTED = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = mla._load()
    names = declared_functions()
    assert {"mla_decode_dense", "mla_decode_sparse", "mla_plan_dense", "mla_plan_sparse",
            "mla_workspace_bytes", "mla_workspace_zero_bytes", "mla_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = mla._load()
    for s in range(7):
        assert lib.mla_status_string(s)
    assert lib.mla_status_string(99) == b"unknown status"


def _kv(ptr=0x1000, rows=100, page=64):
    return mla._KV(ptr, rows, page, 0.05)


def _dense(q=0x1000, kv=None, table=0x2000, max_pages=4, seq=0x3000, B=2, Q=1, H=16, plan=None,
           o=0x4000, lse=0x5000, ws=None, ws_bytes=0):
    lib = mla._load()
    kvs = kv if kv is not None else _kv()
    return lib.mla_decode_dense(q, ctypes.byref(kvs), table, max_pages, seq, 0.07, B, Q, H, plan,
                                o, lse, ws, ws_bytes, None)


def _sparse(q=0x1000, kv=None, rows=0x2000, K=8, valid=0x3000, B=2, Q=1, H=16, plan=None,
            o=0x4000, lse=0x5000, ws=None, ws_bytes=0):
    lib = mla._load()
    kvs = kv if kv is not None else _kv()
    return lib.mla_decode_sparse(q, ctypes.byref(kvs), rows, K, valid, 0.07, B, Q, H, plan,
                                 o, lse, ws, ws_bytes, None)


def test_bad_arguments_return_status_without_launching():
    P = lambda s, t, m=0: ctypes.byref(mla._Plan(s, t, m))  # noqa: E731
    assert _dense(q=None) == NULL
    assert _dense(table=None) == NULL
    assert _dense(kv=_kv(ptr=0)) == NULL
    assert _dense(H=24) == SHAPE
    assert _dense(H=8) == SHAPE
    assert _dense(Q=0) == SHAPE
    assert _dense(max_pages=0) == SHAPE
    assert _dense(kv=_kv(page=0)) == SHAPE
    assert _dense(q=0x1008) == ALIGN
    assert _dense(kv=_kv(ptr=0x1004)) == ALIGN
    assert _dense(o=0x4002) == ALIGN
    assert _dense(o=0x4008) == ALIGN   # 16-byte output stores
    assert _dense(plan=P(0, 1)) == UNSUPPORTED
    assert _dense(plan=P(1, 3)) == UNSUPPORTED
    assert _dense(plan=P(1, 2)) == UNSUPPORTED       # 1 row tile per group: tiles must divide it
    assert _dense(plan=P(2, 1)) == WORKSPACE         # splits > 1 need a workspace
    need = mla.workspace_bytes(True, 2, 1, 16, (2, 1))
    assert _dense(plan=P(2, 1), ws=0x10000, ws_bytes=need - 1) == WORKSPACE
    assert _dense(plan=P(2, 1), ws=0x10010, ws_bytes=need) == ALIGN
    assert _dense(plan=P(1, 1, 2)) == UNSUPPORTED    # unknown mode
    assert _dense(plan=P(3, 1, 1)) == WORKSPACE      # balanced with pieces > 1 needs one too
    need = mla.workspace_bytes(True, 2, 1, 16, (3, 1, 1))
    assert _dense(plan=P(3, 1, 1), ws=0x10000, ws_bytes=need - 1) == WORKSPACE
    assert _sparse(B=36864, plan=P(2, 1, 1), ws=0x10000, ws_bytes=1 << 40) == UNSUPPORTED
    assert _sparse(B=20000, K=1 << 24, plan=P(2, 1, 1), ws=0x10000, ws_bytes=1 << 40) == UNSUPPORTED
    assert _dense(plan=P(4097, 1, 1)) == UNSUPPORTED
    assert _sparse(K=0) == SHAPE
    assert _sparse(valid=None) == NULL
    assert _sparse(rows=0x2002) == ALIGN
    assert _sparse(B=0) == OK                        # nothing to do, nothing launched


def test_query_precision_entry_points_check_the_precision_first():
    lib = mla._load()
    kvs = _kv()
    for bad in (-1, 4, 7, 8):
        assert lib.mla_decode_dense_q(None, ctypes.byref(kvs), None, 0, None, 0.07, 2, 1, 16, None,
                                      bad, None, None, None, 0, None) == UNSUPPORTED
        assert lib.mla_decode_sparse_q(None, ctypes.byref(kvs), None, 0, None, 0.07, 2, 1, 16, None,
                                       bad, None, None, None, 0, None) == UNSUPPORTED
    # P as hi + lo with a plan of four tiles: refused before anything else is checked
    four = ctypes.byref(mla._plan_struct((1, 4)))
    for prec in (2, 3):
        assert lib.mla_decode_dense_q(None, ctypes.byref(kvs), None, 0, None, 0.07, 2, 1, 64, four,
                                      prec, None, None, None, 0, None) == UNSUPPORTED
        assert lib.mla_decode_sparse_q(None, ctypes.byref(kvs), None, 0, None, 0.07, 2, 1, 64, four,
                                       prec, None, None, None, 0, None) == UNSUPPORTED
    for good in (0, 1, 2, 3):
        # then the same checks as the plain entry points
        assert lib.mla_decode_dense_q(None, ctypes.byref(kvs), 0x2000, 4, 0x3000, 0.07, 2, 1, 16,
                                      None, good, 0x4000, 0x5000, None, 0, None) == NULL
        assert lib.mla_decode_sparse_q(0x1000, ctypes.byref(kvs), 0x2000, 0, 0x3000, 0.07, 2, 1, 16,
                                       None, good, 0x4000, 0x5000, None, 0, None) == SHAPE
        assert lib.mla_decode_sparse_q(0x1000, ctypes.byref(kvs), 0x2000, 8, 0x3000, 0.07, 0, 1, 16,
                                       None, good, 0x4000, 0x5000, None, 0, None) == OK
    with pytest.raises(ValueError):
        mla._q_precision("fp8")
    with pytest.raises(ValueError):
        mla._precision("split", "bf16")
    assert [mla._precision(a, b) for a in ("split", "e4m3") for b in ("e4m3", "split")] == [0, 2, 1, 3]
    # the binding runs P hi + lo with at most two tiles
    assert mla.cap_plan((3, 4), "split") == mla.Plan(3, 2) and mla.cap_plan((3, 4)) == mla.Plan(3, 4)
    assert mla.cap_plan((3, 1, 1), "split") == mla.Plan(3, 1, 1)


def test_workspace_sizes_and_plans():
    for dense in (True, False):
        assert mla.workspace_bytes(dense, 4, 5, 16, (1, 1)) == 0
        assert mla.workspace_zero_bytes(dense, 4, 5, 16, (1, 1)) == 0
        assert mla.workspace_bytes(dense, 4, 5, 16, (1, 1, 1)) == 0
        n = mla.workspace_bytes(dense, 4, 5, 16, (3, 1))
        z = mla.workspace_zero_bytes(dense, 4, 5, 16, (3, 1))
        rows = 4 * 5 * 16
        assert 0 < z < n and z % 256 == 0 and n % 256 == 0
        assert n >= rows * 3 * (512 + 2) * 4 + rows // 16 * 4
        # balanced: at most two partials per piece, each of a key group's rows
        nb = mla.workspace_bytes(dense, 4, 5, 16, (7, 1, 1))
        rows_per_group = 5 * 16 if dense else 16
        assert nb >= 2 * 7 * rows_per_group * (512 + 2) * 4 + rows // 16 * 4
        assert mla.workspace_zero_bytes(dense, 4, 5, 16, (7, 1, 1)) == z
    for B, Q, H, K in ((2, 1, 16, 64), (4, 5, 16, 256), (32, 5, 64, 2048)):
        p = mla.plan_sparse(B, Q, H, K)
        assert p.splits >= 1 and p.tiles in (1, 2, 4) and (H // 16) % p.tiles == 0
    for B, Q, H, mp in ((64, 1, 128, 128), (8, 4, 128, 2048)):
        p = mla.plan_dense(B, Q, H, mp, 64)
        assert p.splits >= 1 and (Q * H // 16) % p.tiles == 0
    with pytest.raises(mla.MlaError):
        mla.plan_dense(1, 1, 20, 4, 64)


def test_chooser_picks_the_benchmark_plans():
    """The shapes-only plan chooser agrees with the plans the benchmark launches."""
    import workloads as wl
    shapes = {
        "tiny_sparse": ("sparse", 2, 1, 16, 64),
        "dense_paged": ("dense", 64, 1, 128, 128),
        "latency_sparse": ("sparse", 4, 5, 16, 256),
        "topk_sparse": ("sparse", 32, 5, 64, 2048),
        "long_dense": ("dense", 8, 4, 128, 2048),
    }
    for name, (kind, B, Q, H, n) in shapes.items():
        p = mla.plan_dense(B, Q, H, n, 64) if kind == "dense" else mla.plan_sparse(B, Q, H, n)
        w = wl.WORKLOADS[name]
        assert (p.splits, p.tiles, p.mode) == w.plan, name


def test_combine_checks_arguments_without_launching():
    lib = mla._load()
    c = lib.mla_combine
    assert c(0x1000, 0x2000, 0, 4, 0x3000, 0x4000, None) == SHAPE      # R < 1
    assert c(0x1000, 0x2000, 2, -1, 0x3000, 0x4000, None) == SHAPE     # rows < 0
    assert c(0x1000, 0x2000, 2, 1 << 40, 0x3000, 0x4000, None) == SHAPE
    assert c(None, None, 2, 0, None, None, None) == OK                  # nothing to do
    assert c(None, 0x2000, 2, 4, 0x3000, 0x4000, None) == NULL
    assert c(0x1000, 0x2000, 2, 4, 0x3000, None, None) == NULL
    assert c(0x1008, 0x2000, 2, 4, 0x3000, 0x4000, None) == ALIGN
    assert c(0x1000, 0x2002, 2, 4, 0x3000, 0x4000, None) == ALIGN
    assert c(0x1000, 0x2000, 2, 4, 0x3004, 0x4000, None) == ALIGN


def test_binding_rejects_output_tensors_of_the_wrong_shape():
    import torch
    q = torch.zeros(2, 1, 16, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mla._outputs(q, torch.zeros(2, 1, 16, 511, dtype=torch.bfloat16), None)
    with pytest.raises(ValueError):
        mla._outputs(q, None, torch.zeros(2, 16, dtype=torch.float32))
    with pytest.raises(ValueError):
        mla._outputs(q, torch.zeros(2, 1, 16, 512, dtype=torch.float32), None)
    o, lse = mla._outputs(q, None, None)
    assert tuple(o.shape) == (2, 1, 16, 512) and tuple(lse.shape) == (2, 1, 16)


def test_topk_checks_arguments_without_launching():
    lib = mla._load()
    f = lib.mla_topk_rows
    args = lambda **kw: dict(dict(lg=0x1000, re=0x2000, R=4, N=64, K=8, tb=None, mp=0, ps=1, Q=1,  # noqa: E731
                                  nr=0, ro=0x3000, vo=0x4000), **kw)
    call = lambda a: f(a["lg"], a["re"], a["R"], a["N"], a["K"], a["tb"], a["mp"], a["ps"], a["Q"],  # noqa: E731
                       a["nr"], a["ro"], a["vo"], None)
    assert call(args(R=-1)) == SHAPE
    assert call(args(N=60)) == SHAPE           # not a multiple of 8
    assert call(args(N=0)) == SHAPE
    assert call(args(N=0x7FFFFFF8)) == SHAPE   # the last span's columns would overflow int
    assert call(args(N=0x7FFF8000)) == SHAPE
    assert call(args(N=0x7FFF7FF8, R=0)) == OK   # the largest accepted N
    assert call(args(K=0)) == SHAPE
    assert call(args(Q=0)) == SHAPE
    assert call(args(tb=0x5000, mp=0)) == SHAPE
    assert call(args(tb=0x5000, mp=4, ps=0)) == SHAPE
    assert call(args(tb=0x5000, mp=1 << 20, ps=1 << 12)) == SHAPE
    assert call(args(R=0, lg=None)) == OK
    assert call(args(lg=None)) == NULL
    assert call(args(vo=None)) == NULL
    assert call(args(lg=0x1008)) == ALIGN
    assert call(args(ro=0x3002)) == ALIGN


def test_binding_rejects_index_tensors_of_the_wrong_shape():
    """The kernels read seq_lens / block_table (dense) and valid / rows (sparse) for every key
    group that q implies: short or misshapen index tensors are refused before any launch."""
    import torch
    B, Q, H = 2, 3, 16
    q = torch.zeros(B, Q, H, 576, dtype=torch.bfloat16)
    kv = torch.zeros(64, 576, dtype=torch.uint8)
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)  # noqa: E731
    dense = lambda table, seq, kv=kv, q=q: mla.dense(q, kv, table, seq, 0.07, 0.05, 16)  # noqa: E731
    sparse = lambda rows, valid, kv=kv, q=q: mla.sparse(q, kv, rows, valid, 0.07, 0.05)  # noqa: E731
    with pytest.raises(ValueError, match="block_table"):
        dense(i32(B - 1, 4), i32(B))               # a request without a table row
    with pytest.raises(ValueError, match="block_table"):
        dense(i32(B * 4), i32(B))                  # not 2-D
    with pytest.raises(ValueError, match="seq_lens"):
        dense(i32(B, 4), i32(B - 1))
    with pytest.raises(ValueError, match="seq_lens"):
        dense(i32(B, 4), i32(B, 1))
    with pytest.raises(ValueError, match="rows"):
        sparse(i32(B, Q - 1, 8), i32(B, Q))
    with pytest.raises(ValueError, match="rows"):
        sparse(i32(B * Q, 8), i32(B, Q))
    with pytest.raises(ValueError, match="valid"):
        sparse(i32(B, Q, 8), i32(B * Q))
    with pytest.raises(ValueError, match="valid"):
        sparse(i32(B, Q, 8), i32(B, Q - 1))
    with pytest.raises(ValueError, match="q"):
        sparse(i32(B, Q, 8), i32(B, Q), q=torch.zeros(B, Q, H, 512, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="kv"):
        sparse(i32(B, Q, 8), i32(B, Q), kv=torch.zeros(64, 512, dtype=torch.uint8))


def test_candidate_expansion_and_sparse_topk_check_arguments_without_launching():
    lib = mla._load()
    ex = lambda cb=0x1000, rows=4, K=8, ks=0x2000, ke=0x3000, cbs=16, sbk=16, si=0x4000, end=0x5000: \
        lib.mla_expand_candidates(cb, rows, K, ks, ke, cbs, sbk, si, end, None)  # noqa: E731
    assert ex(rows=-1) == SHAPE
    assert ex(K=0) == SHAPE
    assert ex(sbk=0) == SHAPE
    assert ex(cbs=48) == SHAPE                 # ratio 3
    assert ex(cbs=24) == SHAPE                 # not a multiple
    assert ex(cbs=8) == SHAPE                  # ratio 0
    assert ex(K=16385) == SHAPE                # beyond the in-LDS sort
    assert ex(K=8193, cbs=32) == SHAPE         # K * ratio beyond it
    assert ex(rows=0, cb=None) == OK
    assert ex(cb=None) == NULL
    assert ex(end=None) == NULL
    assert ex(si=0x4002) == ALIGN
    cols = lambda S=4, sbk=8, si=0x6000, ks=0x7000: ctypes.byref(mla._SparseCols(si, S, sbk, ks))  # noqa: E731
    tk = lambda c, N=32, R=2: lib.mla_topk_sparse_rows(0x1000, 0x2000, R, N, 8, c, None, 0, 1, 1, 0,  # noqa: E731
                                                       0x3000, 0x4000, None)
    assert tk(cols(S=3)) == SHAPE               # 3 blocks of 8 do not cover 32 columns
    assert tk(cols(sbk=0)) == SHAPE
    assert tk(cols(S=0)) == SHAPE
    assert tk(cols(si=None)) == NULL
    assert tk(cols(ks=None)) == NULL
    assert tk(cols(ks=0x7002)) == ALIGN
    assert tk(cols(), R=0) == OK
