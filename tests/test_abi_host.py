"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/mm.h declares, compute
capability extents on the host, and reject every invalid call before it
enqueues anything (the launch counter does not move). Buffers here are fake
device addresses: validation never dereferences them.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import gemv_expert_id_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mm.LIB_PATH):
        from gemv_expert_id_amd import build
        build.build()
    return mm.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mm_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(mm.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"
    out = os.popen(f"nm -D --defined-only {mm.LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}\b", out), f"{name} missing from the dynamic symbol table"


def test_status_strings(lib):
    for code in range(8):
        assert mm.mm_status_string(code) != "unknown status"


A = 0x10000000
B = 0x20000000
C = 0x30000000


def _fails(status, fn, *args, **kw):
    before = mm.load().mm_test_launch_count()
    with pytest.raises(mm.MmError) as ei:
        fn(*args, **kw)
    assert ei.value.status == status, str(ei.value)
    assert mm.load().mm_test_launch_count() == before, "enqueued despite the error"
    assert mm.mm_last_error()
    return str(ei.value)


def _gemm_bufs(dt, m, n, k, batch=1):
    e = 4 if dt == mm.MM_F32 else 2
    return (mm.Buf(A, batch * m * k * e), mm.Buf(B, batch * n * k * e),
            mm.Buf(C, batch * m * n * e))


def test_gemm_rejects(lib):
    d = mm.gemm_desc(mm.MM_F16, 8, 8, 8)
    a, b, c = _gemm_bufs(mm.MM_F16, 8, 8, 8)
    _fails(2, mm.mm_gemm, mm.gemm_desc(7, 8, 8, 8), a, b, c)                 # dtype
    for bad in ({"m": 0}, {"n": 0}, {"k": 0}):
        kw = dict(m=8, n=8, k=8)
        kw.update(bad)
        _fails(1, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, kw["m"], kw["n"], kw["k"]), a, b, c)
    _fails(1, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, batch=0), a, b, c)
    _fails(1, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, lda=7), a, b, c)   # ld below tight
    _fails(1, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, ldb=7), a, b, c)
    _fails(1, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, ldc=7), a, b, c)
    _fails(1, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, trans_a=2), a, b, c)
    _fails(1, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, batch=2, stride_c=10),
           *_gemm_bufs(mm.MM_F16, 8, 8, 8, 2))                                 # C batches overlap
    _fails(1, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, stride_a=-1), a, b, c)
    _fails(4, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, offset_a=1), a, b, c)  # odd offset
    _fails(4, mm.mm_gemm, d, mm.Buf(A + 1, 1000), b, c)                     # misaligned ptr
    _fails(3, mm.mm_gemm, d, mm.Buf(A, 127), b, c)                          # too small
    _fails(3, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, offset_c=2), a, b, c)
    _fails(1, mm.mm_gemm, d, mm.Buf(None, 128), b, c)                       # null
    _fails(5, mm.mm_gemm, d, a, b, mm.Buf(A + 64, 128))                     # C overlaps A
    _fails(5, mm.mm_gemm, d, a, b, mm.Buf(B, 128))                          # C overlaps B
    # batch extents: broadcast A needs one matrix only, a strided one needs all
    _fails(3, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 8, 8, 8, batch=3, stride_a=64),
           mm.Buf(A, 128), mm.Buf(B, 3 * 128), mm.Buf(C, 3 * 128))
    # GEMV entry needs m == 1 or n == 1
    _fails(1, mm.mm_gemv, d, a, b, c)


def test_gemm_valid_call_reaches_launch(lib):
    """Without a GPU a fully valid call gets as far as the launch (and fails
    there); with the resolution failure injected it stops before."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("the CPU-only variant of this check")
    d = mm.gemm_desc(mm.MM_F16, 8, 8, 8, batch=3, stride_a=0)
    a, b, c = mm.Buf(A, 128), mm.Buf(B, 3 * 128), mm.Buf(C, 3 * 128)
    before = lib.mm_test_launch_count()
    with pytest.raises(mm.MmError) as ei:
        mm.mm_gemm(d, a, b, c)
    assert ei.value.status == 7
    assert lib.mm_test_launch_count() == before + 1
    lib.mm_test_inject_resolve_failure(b"gemm")
    _fails(2, mm.mm_gemm, d, a, b, c)
    lib.mm_test_inject_resolve_failure(b"gemv")
    _fails(2, mm.mm_gemm, mm.gemm_desc(mm.MM_F16, 1, 8, 8), mm.Buf(A, 16), mm.Buf(B, 128),
           mm.Buf(C, 16))


MOE = dict(m=512, n=1408, k=2048, top_k=8, n_experts=64, expert_stride_bytes=1408 * 2048 * 2)


def test_id_query_extents_moe():
    p = mm.id_params(**MOE, input_layout=0, multiplicity=0, route=1)
    cap = mm.mm_id_query(mm.MM_BF16, p)
    assert cap.schema_version == mm.MM_ID_SCHEMA_VERSION == 5
    assert cap.weight_bytes == 64 * 1408 * 2048 * 2 == 369_098_752
    assert cap.input_bytes == 512 * 2048 * 4 == 4_194_304
    assert cap.ids_bytes == 512 * 8 * 4 == 16_384
    assert cap.output_bytes == 512 * 8 * 1408 * 4 == 23_068_672
    assert cap.counts_bytes == 256 and cap.routed_rows_bytes == 64 * 512 * 4 == 131_072
    d = mm.mm_id_query(mm.MM_BF16, mm.id_params(**dict(MOE, m=1), multiplicity=1, route=0))
    assert d.ids_bytes == 32 and d.output_bytes == 8 * 1408 * 4 and d.input_bytes == 8192
    assert d.counts_bytes == 0 and d.routed_rows_bytes == 0
    s = mm.mm_id_query(mm.MM_F32, mm.id_params(**dict(MOE, expert_stride_bytes=1408 * 2048 * 4 + 64),
                                               input_layout=1, route=0))
    assert s.input_bytes == 512 * 8 * 2048 * 4
    assert s.weight_bytes == 63 * (1408 * 2048 * 4 + 64) + 1408 * 2048 * 4


def test_id_query_rejects():
    def q(wdt=mm.MM_BF16, **kw):
        base = dict(MOE, input_layout=0, multiplicity=0, route=1)
        base.update(kw)
        return mm.mm_id_query(wdt, mm.id_params(**base))
    for dim in ("m", "n", "k", "top_k", "n_experts"):
        _fails(1, q, **{dim: 0})
    _fails(1, q, top_k=65)                                            # distinct top_k > E
    q(top_k=65, multiplicity=1, route=0)                              # fine when repeats allowed
    _fails(1, q, expert_stride_bytes=1408 * 2048 * 2 - 2)             # stride below one matrix
    _fails(1, q, expert_stride_bytes=1408 * 2048 * 2 + 1)             # stride not elt aligned
    _fails(1, q, multiplicity=1)                                      # grouped needs distinct
    _fails(1, q, n_experts=1025, top_k=8)                             # grouped expert limit
    q(n_experts=1025, route=0)                                        # direct has no limit
    _fails(1, q, m=2 ** 30, top_k=8)                                  # rows beyond u32
    _fails(1, q, input_layout=2)
    _fails(1, q, route=2)
    _fails(2, q, wdt=5)
    _fails(1, q, expert_stride_bytes=2 ** 63, n_experts=4)            # weight extent overflow


def _id_bufs(cap, base=0x40000000):
    w = mm.Buf(base, cap.weight_bytes)
    x = mm.Buf(base + 2 ** 32, cap.input_bytes)
    ids = mm.Buf(base + 2 ** 33, cap.ids_bytes)
    out = mm.Buf(base + 2 ** 34, cap.output_bytes)
    cnt = mm.Buf(base + 2 ** 35, max(cap.counts_bytes, 4))
    rr = mm.Buf(base + 2 ** 36, max(cap.routed_rows_bytes, 4))
    return w, x, ids, out, cnt, rr


def test_id_route_hint():
    """Host-only route suggestion: grouped from 2 routed rows per expert
    (16 when f16/f32 weights would take FMA tiles, k % 128 != 0), never with
    may-repeat ids or above the grouped expert limit; params.route is
    ignored; invalid params are rejected."""
    def hint(wdt, m, top_k, E, mult=0, route=0, n=1408, k=2048):
        es = 4 if wdt == mm.MM_F32 else 2
        return mm.mm_id_route_hint(wdt, mm.id_params(m, n, k, top_k, E, n * k * es, 0, mult, route))
    assert hint(mm.MM_BF16, 1, 8, 64) == 0
    assert hint(mm.MM_BF16, 15, 8, 64) == 0
    assert hint(mm.MM_BF16, 16, 8, 64) == 1
    assert hint(mm.MM_F16, 16, 8, 64, route=1) == 1
    assert hint(mm.MM_BF16, 512, 8, 64) == 1
    assert hint(mm.MM_BF16, 512, 8, 64, mult=1) == 0
    assert hint(mm.MM_BF16, 4096, 2, 2000) == 0      # above the grouped expert limit
    assert hint(mm.MM_F32, 15, 8, 64) == 0 and hint(mm.MM_F32, 16, 8, 64) == 1
    assert hint(mm.MM_F32, 64, 8, 64, k=2000) == 0 and hint(mm.MM_F32, 128, 8, 64, k=2000) == 1
    assert hint(mm.MM_F16, 64, 8, 64, k=2000) == 0 and hint(mm.MM_BF16, 16, 8, 64, k=2000) == 1
    assert hint(mm.MM_BF16, 8, 4, 16) == 1 and hint(mm.MM_BF16, 7, 4, 16) == 0
    with pytest.raises(mm.MmError) as e:
        hint(mm.MM_BF16, 0, 8, 64)
    assert e.value.status == 1
    with pytest.raises(mm.MmError):
        hint(mm.MM_BF16, 4, 9, 8)                     # distinct top_k > n_experts


def test_id_call_rejects():
    pd = mm.id_params(9, 7, 35, 2, 4, 7 * 35 * 4, 0, 1, 0)
    pg = mm.id_params(9, 7, 35, 2, 4, 7 * 35 * 4, 0, 0, 1)
    capd = mm.mm_id_query(mm.MM_F32, pd)
    capg = mm.mm_id_query(mm.MM_F32, pg)
    w, x, ids, out, cnt, rr = _id_bufs(capg)
    # route must match the entry point
    _fails(1, mm.mm_id_direct, pg, mm.MM_F32, w, x, ids, out)
    _fails(1, mm.mm_id_map, pd, ids, cnt, rr, out)
    _fails(1, mm.mm_id_grouped, pd, mm.MM_F32, w, x, cnt, rr, out)
    # short buffers, misalignment, overlap
    _fails(3, mm.mm_id_direct, pd, mm.MM_F32, mm.Buf(w.ptr, capd.weight_bytes - 1), x, ids, out)
    _fails(3, mm.mm_id_direct, pd, mm.MM_F32, w, x, ids, mm.Buf(out.ptr, capd.output_bytes - 4))
    _fails(4, mm.mm_id_direct, pd, mm.MM_F32, mm.Buf(w.ptr + 2, 10 ** 6), x, ids, out)
    _fails(4, mm.mm_id_direct, pd, mm.MM_F32, w, x, mm.Buf(ids.ptr + 1, 100), out)
    _fails(5, mm.mm_id_direct, pd, mm.MM_F32, w, x, ids, mm.Buf(w.ptr + 16, capd.output_bytes))
    _fails(5, mm.mm_id_direct, pd, mm.MM_F32, w, x, ids, mm.Buf(x.ptr, capd.output_bytes))
    _fails(5, mm.mm_id_direct, pd, mm.MM_F32, w, x, ids, mm.Buf(ids.ptr, capd.output_bytes))
    _fails(1, mm.mm_id_direct, pd, mm.MM_F32, mm.Buf(None, 0), x, ids, out)
    # scratch: missing, too small, overlapping
    _fails(6, mm.mm_id, pg, mm.MM_F32, w, x, ids, out)
    _fails(6, mm.mm_id, pg, mm.MM_F32, w, x, ids, out, mm.Buf(cnt.ptr, 15), rr)
    _fails(6, mm.mm_id, pg, mm.MM_F32, w, x, ids, out, cnt, mm.Buf(rr.ptr, 4 * 9 * 4 - 4))
    _fails(5, mm.mm_id, pg, mm.MM_F32, w, x, ids, out, cnt, mm.Buf(cnt.ptr + 4, 4 * 9 * 4))
    _fails(5, mm.mm_id, pg, mm.MM_F32, w, x, ids, out, mm.Buf(out.ptr, 16), rr)
    _fails(5, mm.mm_id_map, pg, ids, cnt, mm.Buf(ids.ptr, 4 * 9 * 4), out)
    _fails(4, mm.mm_id_map, pg, ids, mm.Buf(cnt.ptr + 2, 64), rr, out)


def test_prefill_fails_closed_on_grouped_resolution():
    """mlx-native `grouped_pipeline_resolution_failure_does_not_mutate_encoder`:
    when the grouped kernel cannot be resolved, the map launch must not be
    enqueued either. Same ragged shape: m=9, n=7, k=35, top_k=2, E=4, f32."""
    lib = mm.load()
    pg = mm.id_params(9, 7, 35, 2, 4, 7 * 35 * 4, 0, 0, 1)
    cap = mm.mm_id_query(mm.MM_F32, pg)
    w, x, ids, out, cnt, rr = _id_bufs(cap)
    lib.mm_test_inject_resolve_failure(b"id_grouped")
    msg = _fails(2, mm.mm_id, pg, mm.MM_F32, w, x, ids, out, cnt, rr)
    assert "id_grouped" in msg
    lib.mm_test_inject_resolve_failure(b"id_map")
    _fails(2, mm.mm_id, pg, mm.MM_F32, w, x, ids, out, cnt, rr)
    lib.mm_test_inject_resolve_failure(None)


def test_noalloc_prefill_rejects_before_enqueue():
    """The allocation-free prefill: a problem whose scratch exceeds the
    library's array, a direct-route params block and an unresolvable grouped
    kernel all fail before anything is enqueued."""
    lib = mm.load()
    E, m, top_k = 1024, 1024, 1
    pg = mm.id_params(m, 1, 1, top_k, E, 4, 0, 0, 1)
    cap = mm.mm_id_query(mm.MM_F32, pg)
    need = -(-cap.counts_bytes // 256) * 256 + cap.routed_rows_bytes
    assert need > mm.MM_ID_NOALLOC_SCRATCH_BYTES
    w, x, ids, out, _, _ = _id_bufs(cap)
    msg = _fails(6, mm.mm_id_prefill_noalloc, pg, mm.MM_F32, w, x, ids, out)
    assert "holds" in msg
    pd = mm.id_params(9, 7, 35, 2, 4, 7 * 35 * 4, 0, 1, 0)
    capd = mm.mm_id_query(mm.MM_F32, pd)
    w, x, ids, out, _, _ = _id_bufs(capd)
    _fails(1, mm.mm_id_prefill_noalloc, pd, mm.MM_F32, w, x, ids, out)
    pg = mm.id_params(9, 7, 35, 2, 4, 7 * 35 * 4, 0, 0, 1)
    lib.mm_test_inject_resolve_failure(b"id_grouped")
    _fails(2, mm.mm_id_prefill_noalloc, pg, mm.MM_F32, w, x, ids, out)
    lib.mm_test_inject_resolve_failure(None)


def test_gemm_route_refusals():
    """mm_gemm_route refuses a route that cannot take the problem, before
    anything is enqueued: GEMV with m, n > 1; skinny with 65 rows or more on
    both sides or a transposed A; an unknown route value."""
    d = mm.gemm_desc(mm.MM_F16, 8, 300, 256, trans_b=True)
    bufs = _gemm_bufs(mm.MM_F16, 8, 300, 256)
    _fails(2, mm.mm_gemm_route, d, mm.MM_ROUTE_GEMV, *bufs)
    d65 = mm.gemm_desc(mm.MM_F16, 65, 300, 256, trans_b=True)
    _fails(2, mm.mm_gemm_route, d65, mm.MM_ROUTE_GEMV_WIDE, *_gemm_bufs(mm.MM_F16, 65, 300, 256))
    dta = mm.gemm_desc(mm.MM_F16, 8, 300, 256, trans_a=True, trans_b=True)
    _fails(2, mm.mm_gemm_route, dta, mm.MM_ROUTE_GEMV_WIDE, *bufs)
    _fails(1, mm.mm_gemm_route, d, mm.MM_ROUTE_ID_DIRECT, *bufs)
    _fails(1, mm.mm_gemm_route, d, 99, *bufs)


@pytest.mark.parametrize("dt", [mm.MM_F32, mm.MM_F16, mm.MM_BF16])
def test_dispatch_crossover_skinny_vs_tiled(dt):
    """The measured route crossover of mm_gemm for x[m,k] . W[n,k]^T: the
    skinny route up to 64 rows on either side (faster than the tiled GEMM at
    every calibrated m <= 64 and (n, k)), the tiled GEMM from 65 rows, the
    GEMV route at one row. The resolve-failure hook names the family the
    dispatch chose, before anything is enqueued."""
    lib = mm.load()
    n, k = 4096, 4096

    def family(m, nn):
        d = mm.gemm_desc(dt, m, nn, k, trans_b=True)
        for fam in (b"gemv_wide", b"gemm", b"gemv"):
            lib.mm_test_inject_resolve_failure(fam)
            before = lib.mm_test_launch_count()
            try:
                mm.mm_gemm(d, *_gemm_bufs(dt, m, nn, k))
            except mm.MmError as e:
                if e.status == 2 and "injected" in str(e):
                    lib.mm_test_inject_resolve_failure(None)
                    assert lib.mm_test_launch_count() == before
                    return fam.decode()
            lib.mm_test_inject_resolve_failure(None)
        raise AssertionError("no family resolved")

    for m in (2, 16, 17, 32, 33, 48, 64):
        assert family(m, n) == "gemv_wide", m
        assert family(n, m) == "gemv_wide", ("mirrored", m)
    for m in (65, 128):
        assert family(m, n) == "gemm", m
    assert family(1, n) == "gemv"


def _dispatch_family(lib, dt, batch, m, n, k):
    """The launch family mm_gemm resolves for C[b] = A[b] . B[b]^T, found with
    the resolve-failure hook before anything is enqueued."""
    d = mm.gemm_desc(dt, m, n, k, batch=batch, trans_b=True, stride_a=m * k, stride_b=n * k,
                     stride_c=m * n)
    for fam in (b"gemv_wide", b"gemm", b"gemv"):
        lib.mm_test_inject_resolve_failure(fam)
        before = lib.mm_test_launch_count()
        try:
            mm.mm_gemm(d, *_gemm_bufs(dt, m, n, k, batch))
        except mm.MmError as e:
            if e.status == 2 and "injected" in str(e):
                lib.mm_test_inject_resolve_failure(None)
                assert lib.mm_test_launch_count() == before
                return fam.decode()
        lib.mm_test_inject_resolve_failure(None)
    raise AssertionError("no family resolved")


@pytest.mark.parametrize("dt,batch,m,n,k,fam", [
    (mm.MM_F16, 32, 64, 512, 64, "gemm"),         # 4 rounds of 1-per-CU blocks
    (mm.MM_F16, 32, 4, 512, 128, "gemm"),         # 2 rounds, 256-byte rows
    (mm.MM_F16, 32, 4, 512, 256, "gemv_wide"),    # 2 rounds, 512-byte rows
    (mm.MM_F16, 32, 4, 4096, 256, "gemm"),        # 11 rounds, 512-byte rows
    (mm.MM_F16, 32, 4, 4096, 512, "gemv_wide"),   # 11 rounds, 1 KiB rows
    (mm.MM_BF16, 3, 40, 4096, 64, "gemv_wide"),   # 3 rounds, three fragments
    (mm.MM_BF16, 4, 40, 4096, 64, "gemm"),        # 4 rounds, three fragments
    (mm.MM_F32, 16, 20, 2048, 256, "gemv_wide"),  # 4 rounds of 2-per-CU blocks, 1 KiB rows
    (mm.MM_F32, 16, 20, 2048, 128, "gemm"),       # same, 512-byte rows
    (mm.MM_F16, 32, 512, 4, 128, "gemm"),         # mirrored: few rows in B
    (mm.MM_F16, 32, 512, 4, 256, "gemv_wide"),
    (mm.MM_F16, 1, 64, 11008, 4096, "gemv_wide"),  # 3 rounds, four fragments
])
def test_dispatch_skinny_rounds_rule(dt, batch, m, n, k, fam):
    """The skinny route's rounds rule (mm.h, mm_gemm): when its blocks do not
    all fit on the GPU at once, the dispatch keeps it only for long rows (one
    or two activation fragments) or few rounds (three or four), else the
    tiled GEMM, as the short-k calibration measured."""
    assert _dispatch_family(mm.load(), dt, batch, m, n, k) == fam


def test_capabilities_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("CPU-only check")
    with pytest.raises(mm.MmError) as ei:
        mm.mm_capabilities(0)
    assert ei.value.status == 7


def test_struct_layouts_match_header():
    """ctypes mirrors must have the C sizes (offsets follow natural alignment)."""
    assert ctypes.sizeof(mm.GemmDesc) == 4 * 3 + 4 + 8 * 13
    assert ctypes.sizeof(mm.IdParams) == 48
    assert ctypes.sizeof(mm.IdCapability) == 16 + 48
    assert ctypes.sizeof(mm.Receipt) == 24
    assert ctypes.sizeof(mm.DeviceCaps) == 64 + 16 + 8 + 16
