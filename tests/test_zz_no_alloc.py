"""The allocation-free grouped prefill (mm_id_prefill_noalloc) against the
same prefill with caller-owned scratch (mm_id, route 1): identical output
bits on two calls in a row, the second with a smaller problem, so the
library's shared scratch keeps the first call's contents when the second
starts. Both are also held to the oracle's tolerance."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gemv_expert_id_amd as mm
import workloads as wl
from gpu_util import IdRun, assert_close, empty_like_bits, from_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc_out(run: IdRun) -> np.ndarray:
    c = run.case
    out = empty_like_bits(c.m * c.top_k * c.n, wl.F32)
    rec = mm.mm_id_prefill_noalloc(run.params, c.wdtype, mm.buf(run.w), mm.buf(run.x),
                                   mm.buf(run.ids), mm.buf(out),
                                   stream=torch.cuda.current_stream())
    assert rec.route == mm.MM_ROUTE_ID_PREFILL and rec.dispatch_count == 2
    torch.cuda.synchronize()
    return from_dev(out, np.float32).reshape(c.m * c.top_k, c.n)


@pytest.mark.parametrize("wdt", [wl.BF16, wl.F16, wl.F32])
def test_noalloc_matches_caller_scratch_twice(wdt):
    shapes = [(256, 1000, 256, 8, 64), (9, 96, 128, 3, 8)]  # second call smaller
    for i, (m, n, k, top_k, E) in enumerate(shapes):
        _say(f"no-alloc prefill call {i} wdt={wl.DTYPE_NAMES[wdt]} m={m} n={n} k={k} "
             f"top_k={top_k} E={E}")
        case = wl.random_id_case(200 + i, wdt, m, n, k, top_k, E)
        case.ids.reshape(-1)[1] = E + 3  # an out-of-range id: a +0.0 row
        run = IdRun(case, route=1)
        got = _noalloc_out(run)
        run.run()
        ref_bits = from_dev(run.out, np.float32).reshape(m * top_k, n)
        np.testing.assert_array_equal(got.view(np.uint32), ref_bits.view(np.uint32))
        wmax, xmax = run.absmax()
        assert_close(got.astype(np.float64), run.oracle(), wdt, k, wmax, xmax, "no-alloc")


@pytest.mark.parametrize("n,variant", [(704, 4), (1408, 3 | (8 << 8))])
def test_noalloc_under_graph_capture_replays(n, variant):
    """Captured in a HIP graph after one eager call on the GPU (which looks up
    the array's address), the allocation-free prefill replays correctly: three
    replays, with eager calls between them that overwrite the library's array
    with another problem's counts and lists, each replay's output bit-equal
    to the eager result with caller-owned scratch. 704 outputs land on the
    4-wave grouped instance, 1408 on the 8-wave one."""
    wdt = wl.BF16
    m, k, top_k, E = 128, 256, 8, 64
    _say(f"no-alloc prefill under graph capture m={m} n={n} k={k} top_k={top_k} E={E}")
    case = wl.random_id_case(210, wdt, m, n, k, top_k, E)
    case.ids.reshape(-1)[5] = E + 1  # an out-of-range id: a +0.0 row
    run = IdRun(case, route=1)
    rec0 = run.run()
    assert rec0.kernel == mm.MM_KERNEL_ID_GROUPED_MFMA and rec0.variant == variant, rec0.variant
    ref = from_dev(run.out, np.float32).reshape(m * top_k, n).view(np.uint32).copy()

    other = IdRun(wl.random_id_case(211, wdt, 40, 96, 128, 4, 32), route=1)
    _noalloc_out(other)  # eager: the first call on this GPU looks up the address

    out = empty_like_bits(m * top_k * n, wl.F32)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        rec = mm.mm_id_prefill_noalloc(run.params, wdt, mm.buf(run.w), mm.buf(run.x),
                                       mm.buf(run.ids), mm.buf(out), stream=side)
    assert rec.route == mm.MM_ROUTE_ID_PREFILL and rec.dispatch_count == 2
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(-1)  # a fill kernel, not a memset node: every replay rewrites all of it
        _noalloc_out(other)  # overwrites the shared array with another problem
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = from_dev(out, np.float32).reshape(m * top_k, n).view(np.uint32)
        _say(f"  replay {rep}")
        np.testing.assert_array_equal(got, ref)
