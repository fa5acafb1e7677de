"""Host-side checks of the C ABI (no GPU needed).

The library is loaded (built first if missing), every function declared in
include/sa_indexer.h must be exported, and argument validation must reject bad
shapes and budgets with the documented codes before anything is launched.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa_indexer.h")


@pytest.fixture(scope="module")
def api():
    from sparse_attention_token_dsa_amd import api as a
    if not os.path.exists(a.LIB_PATH):
        from sparse_attention_token_dsa_amd import build
        build.build()
    a.load()
    return a


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("indexer_score_topk", "misa_route", "hisa_coarse_fine", "sa_pool_blocks",
              "sa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(api):
    lib = api.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(api.EXPORTS) == set(declared_functions())
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True).stdout
    for n in declared_functions():
        assert re.search(r"\bT %s$" % n, out, flags=re.M), n


def shape(api, **kw):
    d = dict(batch=2, T=1, H=64, d=128, L=4096, causal_offset=4095, topk=64)
    d.update(kw)
    return api.Shape(**d)


def ws_rc(api, s):
    n = ctypes.c_size_t()
    return api.load().indexer_score_topk_ws(ctypes.byref(s), ctypes.byref(n)), n.value


def test_workspace_sizes_and_shape_validation(api):
    rc, n = ws_rc(api, shape(api))
    assert rc == api.SA_OK and n > 0
    # decode path: score row + histogram + candidates per row
    assert n >= 2 * 4096 * 4
    assert ws_rc(api, shape(api, d=64))[0] == api.SA_EUNSUPPORTED
    assert ws_rc(api, shape(api, H=65))[0] == api.SA_EUNSUPPORTED
    assert ws_rc(api, shape(api, causal_offset=4090, T=7))[0] == api.SA_EINVAL
    assert ws_rc(api, shape(api, causal_offset=-1))[0] == api.SA_EINVAL
    assert ws_rc(api, shape(api, topk=0))[0] == api.SA_EINVAL
    assert ws_rc(api, shape(api, L=0, causal_offset=0))[0] == api.SA_EINVAL
    assert "causal_offset" in api.last_error() or api.last_error()


def test_budget_validation(api):
    lib = api.load()
    n = ctypes.c_size_t()
    s = shape(api, topk=2048, L=131072, causal_offset=131071)
    # MISA: h in [1, H], k' = 0 or >= k
    assert lib.misa_route_ws(ctypes.byref(s), 1024, 8, 0, 0, ctypes.byref(n)) == api.SA_OK
    assert lib.misa_route_ws(ctypes.byref(s), 1024, 8, 8192, 1, ctypes.byref(n)) == api.SA_OK
    assert lib.misa_route_ws(ctypes.byref(s), 1024, 0, 0, 0, ctypes.byref(n)) == api.SA_EINVAL
    assert lib.misa_route_ws(ctypes.byref(s), 1024, 65, 0, 0, ctypes.byref(n)) == api.SA_EINVAL
    assert lib.misa_route_ws(ctypes.byref(s), 1024, 8, 1000, 0, ctypes.byref(n)) == api.SA_EINVAL
    assert lib.misa_route_ws(ctypes.byref(s), 0, 8, 0, 0, ctypes.byref(n)) == api.SA_EINVAL
    # HISA: r * b >= k (PaperTrace section 2.3)
    assert lib.hisa_coarse_fine_ws(ctypes.byref(s), 128, 64, 0, ctypes.byref(n)) == api.SA_OK
    assert lib.hisa_coarse_fine_ws(ctypes.byref(s), 128, 15, 0, ctypes.byref(n)) == api.SA_EINVAL
    assert "r * block_b" in api.last_error()
    assert lib.hisa_coarse_fine_ws(ctypes.byref(s), 0, 64, 0, ctypes.byref(n)) == api.SA_EINVAL


def test_entry_points_reject_before_launch(api):
    """Bad arguments return an error without touching the GPU."""
    lib = api.load()
    s = shape(api)
    buf = ctypes.create_string_buffer(16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    # NULL q
    assert lib.indexer_score_topk(None, p, p, ctypes.byref(s), p, None, p, 16, None) == \
        api.SA_EINVAL
    # workspace too small
    assert lib.indexer_score_topk(p, p, p, ctypes.byref(s), p, None, p, 16, None) == \
        api.SA_EWORKSPACE
    assert "workspace" in api.last_error()
    # bad shape
    s2 = shape(api, d=96)
    assert lib.indexer_score_topk(p, p, p, ctypes.byref(s2), p, None, p, 16, None) == \
        api.SA_EUNSUPPORTED
    assert lib.misa_route(p, p, p, ctypes.byref(s), 1024, 9999, 0, None, None, None, p, None,
                          p, 16, None) == api.SA_EINVAL
    assert lib.hisa_coarse_fine(p, p, p, ctypes.byref(s), 8, 2, None, None, p, None, p, 16,
                                None) == api.SA_EINVAL
    assert lib.sa_pool_blocks(p, 1, 100, 128, 0, p, None) == api.SA_EINVAL
    assert lib.sa_pool_blocks2(p, 1, 100, 128, 128, 1000, p, p, None) == api.SA_EINVAL


def test_kernel_names(api):
    names = api.kernel_names()
    assert "scan_dsa" in names and "prefill_fused" in names and "topk_select" in names
    assert len(set(names)) == len(names)


def test_grid_row_limits(api):
    """Paths that put query rows on the grid's y axis take at most 65535 rows per call; the
    fused prefill puts sequences there instead."""
    lib = api.load()
    n = ctypes.c_size_t()
    big_decode = shape(api, batch=65536, T=1, L=64, causal_offset=63)
    assert ws_rc(api, big_decode)[0] == api.SA_EUNSUPPORTED
    assert "65535" in api.last_error()
    assert ws_rc(api, shape(api, batch=65535, T=1, L=64, causal_offset=63))[0] == api.SA_OK
    prefill_rows = shape(api, batch=5, T=16384, L=16384, causal_offset=0)   # 81920 rows
    assert ws_rc(api, prefill_rows)[0] == api.SA_OK
    assert lib.hisa_coarse_fine_ws(ctypes.byref(prefill_rows), 128, 64, 0,
                                   ctypes.byref(n)) == api.SA_EUNSUPPORTED
    assert lib.misa_route_ws(ctypes.byref(prefill_rows), 1024, 8, 0, 0,
                             ctypes.byref(n)) == api.SA_EUNSUPPORTED
    assert lib.lisa_score_topk_ws(ctypes.byref(prefill_rows), ctypes.byref(n)) == api.SA_OK
    assert lib.resmisa_route_ws(ctypes.byref(prefill_rows), 128, 7, 0,
                                ctypes.byref(n)) == api.SA_EUNSUPPORTED


def test_new_entry_points_validate(api):
    lib = api.load()
    n = ctypes.c_size_t()
    buf = ctypes.create_string_buffer(16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    s = shape(api)
    # FP8 keys: decode-style rows only
    assert lib.indexer_score_topk_fp8_ws(ctypes.byref(s), ctypes.byref(n)) == api.SA_OK
    s16 = shape(api, T=16, causal_offset=4080)
    assert lib.indexer_score_topk_fp8_ws(ctypes.byref(s16), ctypes.byref(n)) == api.SA_EUNSUPPORTED
    # with the query in E4M3, prefill rows take the fused prefill
    assert lib.indexer_score_topk_fp8q_ws(ctypes.byref(s16), ctypes.byref(n)) == api.SA_OK
    n16 = n.value
    assert lib.indexer_score_topk_ws(ctypes.byref(s16), ctypes.byref(n)) == api.SA_OK
    assert n16 == n.value
    assert lib.sa_quantize_keys_fp8(p, 1, 10, 64, p, p, None) == api.SA_EUNSUPPORTED
    assert lib.sa_quantize_keys_fp8(None, 1, 10, 128, p, p, None) == api.SA_EINVAL
    # ResMiSA: 0 <= r <= H and 4 + r <= 64 unless r == H
    assert lib.resmisa_route_ws(ctypes.byref(s), 128, 60, 0, ctypes.byref(n)) == api.SA_OK
    assert lib.resmisa_route_ws(ctypes.byref(s), 128, 64, 0, ctypes.byref(n)) == api.SA_OK
    assert lib.resmisa_route_ws(ctypes.byref(s), 128, 61, 0, ctypes.byref(n)) == \
        api.SA_EUNSUPPORTED
    assert lib.resmisa_route_ws(ctypes.byref(s), 128, 65, 0, ctypes.byref(n)) == api.SA_EINVAL
    assert lib.resmisa_route_ws(ctypes.byref(s), 0, 7, 0, ctypes.byref(n)) == api.SA_EINVAL
    assert lib.sa_block_extrema(p, 1, 100, 128, 0, p, None) == api.SA_EINVAL
    # MISA x HISA: both budgets
    s2 = shape(api, topk=2048, L=131072, causal_offset=131071)
    assert lib.misa_hisa_ws(ctypes.byref(s2), 1024, 8, 128, 64, 0, 0, ctypes.byref(n)) == api.SA_OK
    assert lib.misa_hisa_ws(ctypes.byref(s2), 1024, 8, 128, 15, 0, 0, ctypes.byref(n)) == \
        api.SA_EINVAL
    assert lib.misa_hisa_ws(ctypes.byref(s2), 1024, 0, 128, 64, 0, 0, ctypes.byref(n)) == \
        api.SA_EINVAL
    # ragged: causal_offset = L - T, seq_lens required, total_len >= 0; decode
    # rows and prefill rows (T >= 16) both taken
    assert lib.indexer_score_topk_ragged_ws(ctypes.byref(s), ctypes.byref(n)) == api.SA_OK
    s16r = shape(api, T=16, causal_offset=4096 - 16)
    assert lib.indexer_score_topk_ragged_ws(ctypes.byref(s16r), ctypes.byref(n)) == api.SA_OK
    s3 = shape(api, causal_offset=100)
    assert lib.indexer_score_topk_ragged_ws(ctypes.byref(s3), ctypes.byref(n)) == api.SA_EINVAL
    assert lib.indexer_score_topk_ragged(p, p, p, None, 0, ctypes.byref(s), p, None, p, 16,
                                         None) == api.SA_EINVAL
    assert lib.indexer_score_topk_ragged(p, p, p, p, -1, ctypes.byref(s), p, None, p, 16,
                                         None) == api.SA_EINVAL
    # FP8 MISA / HISA / ragged: same shape rules as their bf16 forms; the FP8
    # cache pointers are required; ragged FP8 takes decode-style rows with
    # causal_offset = L - T
    s4 = shape(api, topk=64, L=4096, causal_offset=4095)
    assert lib.misa_route_fp8_ws(ctypes.byref(s4), 256, 8, 0, 0, ctypes.byref(n)) == api.SA_OK
    assert lib.misa_route_fp8_ws(ctypes.byref(s4), 256, 65, 0, 0, ctypes.byref(n)) == \
        api.SA_EINVAL
    assert lib.misa_route_fp8(p, p, None, p, ctypes.byref(s4), 256, 8, 0, None, None, None, p,
                              None, p, 16, None) == api.SA_EINVAL
    assert lib.hisa_coarse_fine_fp8_ws(ctypes.byref(s4), 64, 8, 0, ctypes.byref(n)) == api.SA_OK
    assert lib.hisa_coarse_fine_fp8(p, p, p, None, ctypes.byref(s4), 64, 8, None, None, p, None,
                                    p, 16, None) == api.SA_EINVAL
    assert lib.indexer_score_topk_fp8_ragged_ws(ctypes.byref(s), ctypes.byref(n)) == api.SA_OK
    assert lib.indexer_score_topk_fp8_ragged_ws(ctypes.byref(s3), ctypes.byref(n)) == \
        api.SA_EINVAL
    # prefill rows: sized for the fused prefill (a bf16 query is refused by the call)
    assert lib.indexer_score_topk_fp8_ragged_ws(ctypes.byref(s16r), ctypes.byref(n)) == \
        api.SA_OK
    assert lib.indexer_score_topk_fp8_ragged(p, p, p, p, None, 0, 0, ctypes.byref(s), p, None, p,
                                             16, None) == api.SA_EINVAL
    # tidy-up: k <= 4096 unless a slot bound <= 2^18 is given
    assert lib.sa_tidy_indices(p, 4, 1, 5000, None, 0, 64, 0, p, None, None) == \
        api.SA_EUNSUPPORTED
    assert lib.sa_tidy_indices(p, 4, 3, 64, None, 0, 64, 0, p, None, None) == api.SA_EINVAL
    assert lib.sa_tidy_indices(p, 4, 1, 64, None, 0, 0, 0, p, None, None) == api.SA_EINVAL
    assert lib.sa_tidy_indices(p, 4, 1, 64, p, 0, 64, 0, p, None, None) == api.SA_EINVAL


def test_phase_entry_points_validate(api):
    """The decode selectors in phases: bad phase masks, and shapes that cannot
    be split, are rejected before anything is launched."""
    lib = api.load()
    buf = ctypes.create_string_buffer(16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    s = shape(api, L=4096, causal_offset=4095)
    for bad in (0, 4, -1):
        assert lib.indexer_score_topk_pooled_phase(p, p, p, ctypes.byref(s), 128, 1024, p, p, p,
                                                   None, p, 1 << 40, bad, None) == api.SA_EINVAL
        assert lib.misa_route_phase(p, p, p, ctypes.byref(s), 1024, 8, 0, None, None, None, p,
                                    None, p, 1 << 40, bad, None) == api.SA_EINVAL
    n = ctypes.c_size_t()
    # prefill rows (T >= 16) and decode rows with a pooling block cut by the
    # causal bound (the rows before the last of T = 3) take other paths,
    # which are not split
    for s2 in (shape(api, T=32, L=4096, causal_offset=4064),
               shape(api, T=3, L=4096, causal_offset=4093)):
        assert lib.misa_route_ws(ctypes.byref(s2), 1024, 8, 0, 1, ctypes.byref(n)) == api.SA_OK
        for ph in (api.PHASE_SCAN, api.PHASE_SELECT):
            assert lib.misa_route_phase(p, p, p, ctypes.byref(s2), 1024, 8, 0, p, None, None, p,
                                        None, p, n.value, ph, None) == api.SA_EUNSUPPORTED
            assert "phases" in api.last_error()
    # the binding checks the mask and the workspace before touching tensors
    with pytest.raises(ValueError):
        api.indexer_score_topk_pooled(None, None, None, 0, 64, 128, 1024, phases=4)
    with pytest.raises(ValueError):
        api.indexer_score_topk_pooled(None, None, None, 0, 64, 128, 1024, phases=api.PHASE_SCAN)
    with pytest.raises(ValueError):
        api.misa_route(None, None, None, 0, 64, 1024, 8, phases=api.PHASE_SELECT)


def test_bench_refuses_more_than_one_gpu():
    # bench.py measures one GPU; asking for more exits with a message before
    # any device work.
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
