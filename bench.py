"""Benchmark of MLA decode over an FP8 E4M3 latent cache on one MI355X.

One step = one decode call (mla_decode_dense / mla_decode_sparse through the C ABI) over one batch
of the workload: Q-stage, KV gather, QK, softmax, PV, split emit and FP32 merge all run inside it.
The headline line is the long-context dense causal verify workload (B=8, Q=4 causal rows, H=128,
seq_len 131072, page 64; the largest of the five, MFMA-bound with the split query); the other four
workloads are timed the same way and reported under "workloads".

Timing is cold with respect to the 256 MB Infinity Cache: the timed calls rotate over several
copies of the KV cache (together well above 256 MB), all resident in HBM before timing starts.
HIP events on the stream the kernel runs on bracket the timed calls. The reported time per call is
measured on a HIP graph that holds one call per KV copy, replayed back to back (the GPU time per
call, with no host launch work in between); the time of K eager launches from Python is reported
beside it (us_per_call_eager), and for the large workloads the two agree. Also reported per
workload: the spread of the time per call over the timed graph replays (p10 / p50 / p90, each
replay being one call per KV copy; an event is recorded between every two replays) and the hot
time per call (every call on one KV copy, so whatever of it fits stays in the caches).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12        # B/s, MI355X
FP8_PEAK = 5.0e15        # dense FP8 MFMA flop/s, MI355X
FLOP_PER_HEAD_KEY = 2 * 2 * 576 + 2 * 512   # QK with the hi + lo query (two E4M3 passes) + PV
FLOP_PER_HEAD_KEY_E4M3Q = 2 * 576 + 2 * 512  # QK with the E4M3 query (one pass) + PV
FLOP_PER_HEAD_KEY_PLO = 2 * 512                # PV's second pass with P as E4M3 hi + lo
HEADLINE = "long_dense"
METRIC = ("µs/call and KV HBM GB/s (fraction of 8 TB/s peak), dense + top-k sparse MLA "
          "decode")
KERNEL_SRC = os.path.join(ROOT, "paged_mla_decode_fp8_amd", "csrc", "mla_decode.hip")


def kernel_source_hash(text: str | None = None) -> str:
    """Hash of the decode kernel's device code (the source up to its host-side section) with //
    comments, blank lines and #include lines removed, so that counter summaries stay valid across
    comment edits and host-side changes and go stale on any change of the kernel's code."""
    if text is None:
        with open(KERNEL_SRC) as f:
            text = f.read()
    lines = []
    for ln in text.splitlines():
        if "---- host side" in ln:
            break
        if not ln.startswith("#include"):
            lines.append(re.sub(r"//.*", "", ln).rstrip())
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def algorithmic(x, q_precision="split", p_precision="e4m3"):
    """Algorithmic HBM bytes and MFMA flops of one call: every gathered KV row once per key group,
    Q read once, o and lse written once, indices / block-table entries read once. The flops count
    the QK product once per query pass (two for the split query, one for the E4M3 query) and the
    PV product once per P pass (two for P as hi + lo)."""
    rows = x.B * x.Q * x.H
    q_bytes = rows * 576 * 2
    o_bytes = rows * 512 * 2 + rows * 4
    if x.kind == "dense":
        cap = x.block_table.shape[1] * x.page_size
        seq = np.clip(x.seq_lens.astype(np.int64), 0, cap)
        kv_rows = int(seq.sum())
        idx_bytes = int(np.ceil(seq / x.page_size).sum()) * 4 + x.B * 4
        head_keys = 0
        for i in range(x.Q):
            head_keys += int(np.clip(seq - x.Q + i + 1, 0, seq).sum()) * x.H
    else:
        cnt = np.clip(x.valid.astype(np.int64), 0, x.rows.shape[2])
        kv_rows = int(cnt.sum())
        idx_bytes = kv_rows * 4 + x.B * x.Q * 4
        head_keys = kv_rows * x.H
    kv_bytes = kv_rows * 576
    return {
        "kv_bytes": kv_bytes,
        "bytes": kv_bytes + q_bytes + o_bytes + idx_bytes,
        "flops": head_keys * ((FLOP_PER_HEAD_KEY_E4M3Q if q_precision == "e4m3" else FLOP_PER_HEAD_KEY)
                              + (FLOP_PER_HEAD_KEY_PLO if p_precision == "split" else 0)),
        "head_keys": head_keys,
    }


def bench_workload(name, steps, warmup, min_rotation_bytes=768 << 20, q_precision="split", x=None,
                   p_precision="e4m3", plan=None, min_timed_ms=0.0):
    import torch

    import paged_mla_decode_fp8_amd as mla
    import workloads as wl

    w = wl.WORKLOADS[name]
    if x is None:
        x = w.make()
    alg = algorithmic(x, q_precision, p_precision)
    dev = torch.device("cuda:0")
    plan = mla.cap_plan(w.plan if plan is None else plan, p_precision)
    kv_host = torch.from_numpy(x.kv)
    copies = max(1, min(8, math.ceil(min_rotation_bytes / max(1, x.kv.nbytes))))
    kvs = [kv_host.to(dev) for _ in range(copies)]
    q = torch.from_numpy(x.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    o = torch.empty((x.B, x.Q, x.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((x.B, x.Q, x.H), dtype=torch.float32, device=dev)
    nbytes = mla.workspace_bytes(x.kind == "dense", x.B, x.Q, x.H, plan)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
    if x.kind == "dense":
        table = torch.from_numpy(x.block_table).to(dev)
        seq = torch.from_numpy(x.seq_lens).to(dev)

        def call(k):
            mla.dense(q, kvs[k % copies], table, seq, x.scale, x.k_scale, x.page_size, plan=plan,
                      o=o, lse=lse, workspace=ws, q_precision=q_precision, p_precision=p_precision)
    else:
        rows = torch.from_numpy(x.rows).to(dev)
        valid = torch.from_numpy(x.valid).to(dev)

        def call(k):
            mla.sparse(q, kvs[k % copies], rows, valid, x.scale, x.k_scale, plan=plan, o=o,
                       lse=lse, workspace=ws, q_precision=q_precision, p_precision=p_precision)

    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # eager: one stream launch per call from Python
    start.record(stream)
    for k in range(steps):
        call(warmup + k)
    end.record(stream)
    torch.cuda.synchronize()
    ms_eager = start.elapsed_time(end) / steps
    o_eager = o.clone()
    # graph replay: the calls over all KV copies captured once (no host work between launches)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(copies):
            call(k)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(o.view(torch.int16), o_eager.view(torch.int16)):
        raise RuntimeError(f"{name}: graph replay output differs from the eager call")
    # the timed calls: reps replays back to back, an event between every two (the spread of the
    # time per call comes from the same replays as its mean); with min_timed_ms, at least that long
    # a timed region by the eager estimate (short workloads: enough replays for a steady figure)
    reps = max(1, steps // copies)
    if min_timed_ms > 0.0:
        reps = max(reps, math.ceil(min_timed_ms / max(ms_eager * copies, 1e-3)))
    stream = torch.cuda.current_stream(dev)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for r in range(reps):
        graph.replay()
        marks[r + 1].record(stream)
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[reps]) / (reps * copies)
    per_call = np.array([marks[r].elapsed_time(marks[r + 1]) / copies for r in range(reps)])
    del graph
    # hot: the same number of calls, all on KV copy 0
    hot = torch.cuda.CUDAGraph()
    with torch.cuda.graph(hot):
        for k in range(copies):
            call(0)
    torch.cuda.synchronize()
    hot.replay()
    start.record(stream)
    for _ in range(reps):
        hot.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms_hot = start.elapsed_time(end) / (reps * copies)
    del hot
    sec = ms * 1e-3
    res = {
        "workload": name,
        "description": w.description,
        "plan": {"splits": plan[0], "tiles": plan[1],
                 "mode": "balanced" if plan[2] == mla.BALANCED else "uniform"},
        "us_per_call": round(ms * 1e3, 3),
        "us_per_call_eager": round(ms_eager * 1e3, 3),
        "us_per_call_hot": round(ms_hot * 1e3, 3),
        "us_p10_p50_p90": [round(float(np.percentile(per_call, q)) * 1e3, 3) for q in (10, 50, 90)],
        "spread_samples": f"{reps} graph replays of {copies} call(s) each (one per KV copy)",
        "timed_calls": reps * copies,
        "kv_bytes": alg["kv_bytes"],
        "alg_bytes": alg["bytes"],
        "alg_flops": alg["flops"],
        "kv_GBps": round(alg["kv_bytes"] / sec / 1e9, 2),
        "hbm_frac": round(alg["bytes"] / sec / HBM_PEAK, 4),
        "mfma_frac": round(alg["flops"] / sec / FP8_PEAK, 4),
        "hbm_floor_us": round(alg["bytes"] / HBM_PEAK * 1e6, 3),
        "mfma_floor_us": round(alg["flops"] / FP8_PEAK * 1e6, 3),
        "kv_copies_rotated": copies,
    }
    res["bound"] = "hbm" if res["hbm_floor_us"] >= res["mfma_floor_us"] else "mfma"
    del kvs
    torch.cuda.empty_cache()
    return res, x


# The decode-context-parallel combine: R ranks' (o, LSE) partials of the latency checkpoint's
# rows (B=4, Q=5, H=16: one rank's share at DCP8) and of the top-k workload's rows (B=32, Q=5, H=64).
COMBINE_CASES = {"dcp8_latency_rows": (8, 4 * 5 * 16), "dcp8_topk_rows": (8, 32 * 5 * 64)}


def bench_combine(R, rows, steps, warmup, min_rotation_bytes=768 << 20, seed=0):
    """mla.combine on synthetic partials (bf16 o ~ N(0,1) * 3, LSE ~ N(0,16), 10 % of the rank
    rows empty), timed like the decode: graph replay over rotated input copies."""
    import torch

    import paged_mla_decode_fp8_amd as mla

    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(seed)
    o_host = (torch.randn((R, rows, 512), generator=g) * 3).to(torch.bfloat16)
    lse_host = torch.randn((R, rows), generator=g) * 4
    lse_host[torch.rand((R, rows), generator=g) < 0.1] = -math.inf
    in_bytes = R * rows * (512 * 2 + 4)
    copies = max(1, min(8, math.ceil(min_rotation_bytes / in_bytes)))
    parts = [(o_host.to(dev), lse_host.to(dev)) for _ in range(copies)]
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev)

    def call(k):
        mla.combine(parts[k % copies][0], parts[k % copies][1], o=o, lse=lse)

    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(copies):
            call(k)
    torch.cuda.synchronize()
    reps = max(1, steps // copies)
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / (reps * copies) * 1e3
    alg = in_bytes + rows * (512 * 2 + 4)
    del graph, parts
    torch.cuda.empty_cache()
    return {"R": R, "rows": rows, "us_per_call": round(us, 3), "alg_bytes": alg,
            "GBps": round(alg / (us * 1e-6) / 1e9, 2), "hbm_frac": round(alg / (us * 1e-6) / HBM_PEAK, 4),
            "hbm_floor_us": round(alg / HBM_PEAK * 1e6, 3), "input_copies_rotated": copies}


# The top-k producer at the top-k workload's shape: B=32 requests x Q=5 rows of indexer logits over
# a 32768-position context, K=2048, positions remapped through 64-row pages (request b's position p
# is cache row b * 32768 + p, as in that workload's cache).
TOPK_CASE = {"B": 32, "Q": 5, "N": 32768, "K": 2048, "page": 64}


# Plans timed beside the chooser's: the latency checkpoint's configuration names the many-split
# path and its FP32 LSE combine, which the chooser does not pick there (one split measures faster).
SPLIT_PLANS = {"latency_sparse": [(2, 1, 0), (4, 1, 0)]}

# The headline times exactly --steps calls; the other workloads time at least this long (by the
# eager estimate), so that the short ones average over enough replays for a steady figure.
MIN_TIMED_MS = 10.0

TOPK_CALLS_PER_GRAPH = 16


def bench_topk(steps, warmup, seed=0):
    """mla.topk_rows on synthetic bf16 logits ~ N(0,1), causal row ends (row (b, i) sees
    N - Q + i + 1 positions), timed by graph replay (the 10 MB of logits stay L2/MALL-resident).
    A graph holds TOPK_CALLS_PER_GRAPH calls, so that the replay's launch cost (about 18 us for a
    graph of one small kernel) does not stand in for the kernel's own time."""
    import torch

    import paged_mla_decode_fp8_amd as mla

    c = TOPK_CASE
    B, Q, N, K, page = c["B"], c["Q"], c["N"], c["K"], c["page"]
    R = B * Q
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(seed)
    logits = torch.randn((R, N), generator=g).to(torch.bfloat16).to(dev)
    ends = torch.tensor([N - Q + (r % Q) + 1 for r in range(R)], dtype=torch.int32, device=dev)
    pages = N // page
    table = (torch.arange(B * pages, dtype=torch.int32).view(B, pages)).to(dev)
    rows = torch.empty((R, K), dtype=torch.int32, device=dev)
    valid = torch.empty((R,), dtype=torch.int32, device=dev)

    def call():
        mla.topk_rows(logits, ends, K, block_table=table, page_size=page, q_per_request=Q,
                      num_rows=B * N, rows=rows, valid=valid)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(TOPK_CALLS_PER_GRAPH):
            call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    reps = max(1, steps // 4)
    start.record(stream)
    for _ in range(reps):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / (reps * TOPK_CALLS_PER_GRAPH) * 1e3
    alg = R * N * 2 + R * K * 4 + R * 8 + B * pages * 4
    del graph
    return {**c, "rows": R, "us_per_call": round(us, 3), "alg_bytes": alg,
            "GBps": round(alg / (us * 1e-6) / 1e9, 2), "hbm_floor_us": round(alg / HBM_PEAK * 1e6, 3),
            "calls_per_graph": TOPK_CALLS_PER_GRAPH}


def read_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this workload, or
    None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"mla_decode_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Host threads the CPU oracle may use: the cores of this process's affinity mask, at most 16 (the
# host share of one GPU on a shared GPU host).
MAX_CPU_THREADS = 16


def cpu_baseline(x, seconds=15.0, single_seconds=4.0, seed=0):
    """The FP64 oracle (as it stands, METHOD mode, one split per row) on a bounded random sample of
    the workload's query rows: batches of one row per thread until about ``seconds`` of wall time
    have passed, on every core of this process's affinity mask (at most 16); then single rows on
    one thread for about ``single_seconds``. The time per full call is scaled from each sample by
    the rows' key counts."""
    import oracle

    threads = max(1, min(MAX_CPU_THREADS, len(os.sched_getaffinity(0))))
    n_rows = x.B * x.Q * x.H
    order = np.random.default_rng(seed).permutation(n_rows)
    if x.kind == "dense":
        seq = np.clip(x.seq_lens.astype(np.int64), 0, x.block_table.shape[1] * x.page_size)
        keys = np.repeat(seq, x.Q * x.H)
    else:
        keys = np.repeat(np.clip(x.valid.astype(np.int64), 0, x.rows.shape[2]).reshape(-1), x.H)
    all_keys = int(keys.sum())

    def run(sel, nthreads):
        sel = np.sort(sel)
        if x.kind == "dense":
            oracle.dense(x.q_bits, x.kv, x.page_size, x.k_scale, x.block_table, x.seq_lens,
                         x.scale, mode=oracle.METHOD, splits=1, sel=sel, threads=nthreads)
        else:
            oracle.sparse(x.q_bits, x.kv, x.k_scale, x.rows, x.valid, x.scale,
                          mode=oracle.METHOD, splits=1, sel=sel, threads=nthreads)

    def timed(nthreads, batch, budget, pos):
        t0 = time.perf_counter()
        used = 0
        while used < n_rows and (used == 0 or time.perf_counter() - t0 < budget):
            sel = order[pos + used: pos + used + batch]
            if sel.size == 0:
                break
            run(sel, nthreads)
            used += sel.size
        dt = time.perf_counter() - t0
        sample_keys = int(keys[order[pos: pos + used]].sum())
        return used, dt, dt * all_keys / max(1, sample_keys)

    used, dt, per_call = timed(threads, threads, seconds, 0)
    used1, dt1, per_call1 = timed(1, 1, single_seconds, used if used < n_rows else 0)
    kv_bytes = algorithmic(x)["kv_bytes"]
    return {
        "value": float(f"{kv_bytes / per_call / 1e9:.4g}"),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{used} of {n_rows} query rows (uniform random, seed {seed}), METHOD mode, one "
                   f"split per row, {threads} threads: {dt:.2f} s measured, scaled by key counts "
                   f"to {per_call:.1f} s per call; single thread: {used1} rows in "
                   f"{dt1:.2f} s, {per_call1:.1f} s per call"),
        "us_per_call": round(per_call * 1e6, 1),
        "single_thread": {"value": float(f"{kv_bytes / per_call1 / 1e9:.4g}"), "unit": "GB/s",
                          "us_per_call": round(per_call1 * 1e6, 1), "rows": used1},
        "cpu_model": cpu_model(),
        "affinity_cores": len(os.sched_getaffinity(0)),
    }


def headline_config(x, res):
    """The headline workload's shape, from its inputs."""
    cfg = {"workload": res["workload"], "description": res["description"], "kind": x.kind,
           "B": x.B, "Q": x.Q, "H": x.H}
    if x.kind == "dense":
        seq = np.unique(x.seq_lens)
        cfg.update(page_size=x.page_size, max_pages=int(x.block_table.shape[1]),
                   seq_len=int(seq[0]) if seq.size == 1 else f"{int(seq.min())}..{int(seq.max())}",
                   causal_rows=x.Q)
    else:
        cfg.update(K=int(x.rows.shape[2]), cache_rows=int(x.kv.shape[0]))
    cfg.update(kv_bytes=res["kv_bytes"], plan=res["plan"], parallelism="single GPU")
    return cfg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default="all",
                    help="comma-separated workload names, or 'all' (headline first)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall time of the CPU oracle sample on all threads (a single-thread sample "
                         "of about 4 s follows)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the E4M3-query and P hi + lo precision runs of every workload")
    ap.add_argument("--no-combine", action="store_true",
                    help="skip the decode-context-parallel combine and top-k producer runs")
    ap.add_argument("--plan", default=None,
                    help="splits,tiles,mode: run the named workloads with this launch plan instead of "
                         "the chooser's (for counter runs; mode 0 uniform, 1 balanced)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device copy (a known-size reference for "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the decode of one GPU's share of the keys; the "
              "library has no multi-GPU path). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as wl
    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = list(wl.WORKLOADS) if args.workloads == "all" else args.workloads.split(",")
    if HEADLINE in names:
        names.remove(HEADLINE)
    names = [HEADLINE] + names

    results = {}
    variants = {}
    p_variants = {}
    split_plans = {}
    head_x = None
    plan_override = tuple(int(v) for v in args.plan.split(",")) if args.plan else None
    for name in names:
        mt = 0.0 if name == HEADLINE else MIN_TIMED_MS
        res, x = bench_workload(name, args.steps, args.warmup, min_timed_ms=mt,
                                plan=plan_override if name in args.workloads.split(",") else None)
        results[name] = res
        print(f"[bench] {name}: {res['us_per_call']} us/call, {res['kv_GBps']} KV GB/s, "
              f"hbm {res['hbm_frac']:.3f}, mfma {res['mfma_frac']:.3f}", file=sys.stderr,
              flush=True)
        if not args.no_variants:
            v, _ = bench_workload(name, args.steps, args.warmup, q_precision="e4m3", x=x, min_timed_ms=mt)
            variants[name] = {k: v[k] for k in ("us_per_call", "kv_GBps", "hbm_frac", "mfma_frac",
                                                "alg_flops", "mfma_floor_us", "timed_calls")}
            print(f"[bench] {name} (E4M3 query): {v['us_per_call']} us/call, {v['kv_GBps']} KV "
                  f"GB/s, hbm {v['hbm_frac']:.3f}, mfma {v['mfma_frac']:.3f}", file=sys.stderr,
                  flush=True)
            v, _ = bench_workload(name, args.steps, args.warmup, p_precision="split", x=x, min_timed_ms=mt)
            p_variants[name] = {k: v[k] for k in ("us_per_call", "kv_GBps", "hbm_frac", "mfma_frac",
                                                  "alg_flops", "mfma_floor_us", "plan", "timed_calls")}
            print(f"[bench] {name} (P hi + lo): {v['us_per_call']} us/call, {v['kv_GBps']} KV "
                  f"GB/s, hbm {v['hbm_frac']:.3f}, mfma {v['mfma_frac']:.3f}", file=sys.stderr,
                  flush=True)
        for sp in SPLIT_PLANS.get(name, ()) if not args.no_variants else ():
            v, _ = bench_workload(name, args.steps, args.warmup, x=x, plan=sp, min_timed_ms=mt)
            key = f"{sp[0]},{sp[1]},{'balanced' if sp[2] else 'uniform'}"
            split_plans.setdefault(name, {})[key] = {k: v[k] for k in ("us_per_call", "kv_GBps", "hbm_frac",
                                                                        "us_p10_p50_p90", "timed_calls")}
            print(f"[bench] {name} (plan {key}): {v['us_per_call']} us/call, {v['kv_GBps']} KV GB/s",
                  file=sys.stderr, flush=True)
        if name == HEADLINE:
            head_x = x
        else:
            del x

    combine = {}
    if not args.no_combine:
        for cname, (R, rows) in COMBINE_CASES.items():
            combine[cname] = bench_combine(R, rows, args.steps, args.warmup)
            c = combine[cname]
            print(f"[bench] combine {cname} (R={R}, rows={rows}): {c['us_per_call']} us/call, "
                  f"{c['GBps']} GB/s, hbm {c['hbm_frac']:.3f}", file=sys.stderr, flush=True)
        topk_res = bench_topk(args.steps, args.warmup)
        print(f"[bench] top-k producer ({topk_res['rows']} rows x {topk_res['N']} -> "
              f"{topk_res['K']}): {topk_res['us_per_call']} us/call", file=sys.stderr, flush=True)
    else:
        topk_res = None

    h = results[HEADLINE]
    sec = h["us_per_call"] * 1e-6
    if h["bound"] == "hbm":
        achieved, peak, unit = h["alg_bytes"] / sec / 1e9, HBM_PEAK / 1e9, "GB/s"
    else:
        achieved, peak, unit = h["alg_flops"] / sec / 1e12, FP8_PEAK / 1e12, "TFLOP/s"
    roofline = {
        "bound": h["bound"],
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "traffic": read_traffic(HEADLINE),
        "kernel": (f"mla_decode_kernel<{h['plan']['tiles']}, {str(head_x.kind == 'dense').lower()}, "
                   f"false, false> ({head_x.kind}, split query, E4M3 P)"),
        "hbm_frac": h["hbm_frac"],
        "mfma_frac": h["mfma_frac"],
    }
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(head_x, seconds=args.cpu_seconds)
        print(f"[bench] cpu oracle: {cpu['sample']}", file=sys.stderr, flush=True)
    line = {
        "metric": METRIC,
        "value": h["kv_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["us_per_call"] / 1e3, 6),
        "us_per_call": h["us_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded; E4M3 cache of N(0,1)/0.05, bf16 N(0,1) queries)",
        "config": headline_config(head_x, h),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "workloads": results,
        "q_e4m3": variants or None,
        "p_split": p_variants or None,
        "split_plans": split_plans or None,
        "dcp_combine": combine or None,
        "topk_producer": topk_res,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
