"""GPU test of mla_decode_dense_q_noalloc (C ABI): the decode without a caller workspace, its split
partials and arrival counters in the library's per-device scratch array, against
mla_decode_dense_q with a workspace under the same plan. Same kernels, same plan: bit-identical
results are required, on calls in a row with inputs that shrink and grow (the scratch keeps the
last call's contents), and a plan too large for the scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import paged_mla_decode_fp8_amd as mla
import workloads as wl
from gpu_util import BALANCED, assert_parity, bits, run_oracle, say, upload

pytestmark = pytest.mark.gpu


def _both(x, plan, q_precision="split"):
    dev = upload(x)
    ref = mla.dense(dev["q"], dev["kv"], dev["table"], dev["seq"], x.scale, x.k_scale, x.page_size,
                    plan=plan, q_precision=q_precision)
    got = mla.dense_noalloc(dev["q"], dev["kv"], dev["table"], dev["seq"], x.scale, x.k_scale,
                            x.page_size, plan=plan, q_precision=q_precision)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, what):
    assert np.array_equal(bits(got[0]), bits(ref[0])), what
    assert np.array_equal(got[1].cpu().numpy().view(np.uint32), ref[1].cpu().numpy().view(np.uint32)), what


def test_noalloc_matches_the_workspace_entry_point_on_calls_in_a_row():
    # 1: the dense paged workload with its balanced plan (128 pieces, four tiles: 64 MiB of partials)
    x1 = wl.dense_paged()
    say("noalloc", "dense_paged", wl.WORKLOADS["dense_paged"].plan)
    ref, got = _both(x1, wl.WORKLOADS["dense_paged"].plan)
    _same(ref, got, "dense_paged")
    # 2: a smaller call right after, uniform splits (its partials overwrite the first call's)
    x2 = wl.dense_case(3, 2, 32, [500, 64, 1], page_size=64, seed=1900, extra_pages=2)
    say("noalloc", "small uniform", (3, 2))
    ref2, got2 = _both(x2, (3, 2))
    _same(ref2, got2, "small uniform")
    o_ref, lse_ref, amb = run_oracle(x2, (3, 2))
    assert_parity(got2[0], got2[1], o_ref, lse_ref, amb, what="noalloc small uniform vs oracle")
    # 3: more key groups than the first call, a balanced plan with the E4M3 query, then the plan
    # chosen by the library (planner's choice: plan=None on both sides)
    x3 = wl.dense_case(24, 4, 64, np.random.default_rng(3).integers(0, 3000, 24), page_size=16,
                       seed=1901, extra_pages=5)
    say("noalloc", "balanced E4M3 query", (40, 2, BALANCED))
    ref3, got3 = _both(x3, (40, 2, BALANCED), q_precision="e4m3")
    _same(ref3, got3, "balanced e4m3")
    ref4, got4 = _both(x3, None)
    _same(ref4, got4, "planner's plan")
    # 4: the first shape again: the counters were left zero by every call
    ref5, got5 = _both(x1, wl.WORKLOADS["dense_paged"].plan)
    _same(ref5, got5, "dense_paged again")
    _same(ref, got5, "dense_paged repeat is deterministic")


def test_noalloc_refuses_plans_beyond_its_scratch():
    x = wl.dense_case(64, 4, 128, [400] * 64, page_size=64, seed=1902)
    dev = upload(x)
    # 32768 query rows x 4 splits of 2 KB partials: 268 MB, beyond the 80 MiB scratch
    with pytest.raises(mla.MlaError) as e:
        mla.dense_noalloc(dev["q"], dev["kv"], dev["table"], dev["seq"], x.scale, x.k_scale, 64,
                          plan=(4, 4))
    assert e.value.status == 4   # MLA_ERR_WORKSPACE
    # one split needs no scratch at all
    ref, got = _both(x, (1, 4))
    _same(ref, got, "one split")
