"""GPU: the decode selectors called in phases (scan, then select) give the
same outputs as the whole calls: the same top-k sets with bit-identical
scores, the same block means, routed heads and k' pools (the same kernels run
on the same workspace, only later).  Also with several selectors' scans
issued first and their selections afterwards on other streams, as a caller
that runs the latency-bound selections side by side would."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from sparse_attention_token_dsa_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_token_dsa_amd import api as a
    a.load()
    return a


def _inputs(p):
    q = torch.from_numpy(p["q"].view(np.int16)).to(DEV)
    w = torch.from_numpy(p["w"]).to(DEV)
    K = torch.from_numpy(p["K"].view(np.int16)).to(DEV)
    return q, w, K


def _ws(api, n):
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def _sorted(idx, sc):
    i, perm = torch.sort(idx, dim=-1)
    return i, (None if sc is None else torch.gather(sc, -1, perm))


def _same(a, b):
    """(idx, score, x, y) of two calls: the same top-k set with the same
    scores (the order of a set is not fixed: winners are appended through
    atomics), x and y (block means, or routed heads and the k' pool) equal,
    the pool as a set."""
    ia, sa = _sorted(a[0], a[1])
    ib, sb = _sorted(b[0], b[1])
    assert torch.equal(ia, ib)
    assert (sa is None and sb is None) or torch.equal(sa, sb)
    for n, (x, y) in enumerate(zip(a[2:], b[2:])):
        if x is None:
            assert y is None
        elif n == 1 and x.dtype == torch.int32:
            assert torch.equal(torch.sort(x, -1)[0], torch.sort(y, -1)[0])
        else:
            assert torch.equal(x, y)


@pytest.mark.parametrize("name,L", [("misa_128k_h64", None), ("small", 5000)])
def test_phases_equal_whole_calls(api, name, L):
    say("phases %s" % name)
    if name == "small":
        p = synth.make_problem(21, Bt=2, T=1, L=L, H=64, needles=8, needle_mode="decode")
    else:
        p = synth.make_config(name)
    q, w, K = _inputs(p)
    off, k, B, h, b = p["offset"], min(2048, p["L"]), 1024, 8, 128
    shape = api.Shape(q.shape[0], 1, q.shape[2], 128, p["L"], off, k)
    ws = _ws(api, api.indexer_score_topk_pooled_ws(shape, b, B))
    whole = api.indexer_score_topk_pooled(q, w, K, off, k, b, B, ws=ws)
    a = api.indexer_score_topk_pooled(q, w, K, off, k, b, B, ws=ws, phases=api.PHASE_SCAN)
    a = api.indexer_score_topk_pooled(q, w, K, off, k, b, B, out_small=a[2], out_large=a[3],
                                      out_idx=a[0], out_score=a[1], ws=ws,
                                      phases=api.PHASE_SELECT)
    torch.cuda.synchronize()
    _same(whole, a)
    reps = whole[3]
    for kp in (0, 4 * k):
        wsm = _ws(api, api.misa_route_ws(shape, B, h, kp, True))
        whole = api.misa_route(q, w, K, off, k, B, h, kp, pooled=reps, want_pool=kp > 0, ws=wsm)
        m = api.misa_route(q, w, K, off, k, B, h, kp, pooled=reps, want_pool=kp > 0, ws=wsm,
                           phases=api.PHASE_SCAN)
        m = api.misa_route(q, w, K, off, k, B, h, kp, pooled=reps, ws=wsm, out_idx=m[0],
                           out_score=m[1], out_heads=m[2], out_pool=m[3],
                           phases=api.PHASE_SELECT)
        torch.cuda.synchronize()
        _same(whole, m)
    # MISA pooling the keys itself in its scan phase
    wsm = _ws(api, api.misa_route_ws(shape, B, h, 0, False))
    whole = api.misa_route(q, w, K, off, k, B, h, 0, ws=wsm)
    m = api.misa_route(q, w, K, off, k, B, h, 0, ws=wsm, phases=api.PHASE_SCAN)
    m = api.misa_route(q, w, K, off, k, B, h, 0, ws=wsm, out_idx=m[0], out_score=m[1],
                       out_heads=m[2], phases=api.PHASE_SELECT)
    torch.cuda.synchronize()
    _same(whole, m)


def test_scans_first_selects_on_other_streams(api):
    # The decode step's selectors: every key scan first on one stream, then
    # the selections on three side streams behind one event; each output
    # equals the selector's whole call.
    say("scans first, selections on side streams")
    p = synth.make_config("misa_128k_h64")
    q, w, K = _inputs(p)
    off, k, B, h, kp, b = p["offset"], 2048, 1024, 8, 8192, 128
    shape = api.Shape(q.shape[0], 1, q.shape[2], 128, p["L"], off, k)
    ref_d = api.indexer_score_topk_pooled(q, w, K, off, k, b, B)
    reps = ref_d[3]
    ref_md = api.misa_route(q, w, K, off, k, B, h, kp, pooled=reps, want_pool=True)
    ref_m = api.misa_route(q, w, K, off, k, B, h, 0, pooled=reps)
    torch.cuda.synchronize()
    ws_d = _ws(api, api.indexer_score_topk_pooled_ws(shape, b, B))
    ws_md = _ws(api, api.misa_route_ws(shape, B, h, kp, True))
    ws_m = _ws(api, api.misa_route_ws(shape, B, h, 0, True))
    d = api.indexer_score_topk_pooled(q, w, K, off, k, b, B, ws=ws_d, phases=api.PHASE_SCAN)
    md = api.misa_route(q, w, K, off, k, B, h, kp, pooled=d[3], want_pool=True, ws=ws_md,
                        phases=api.PHASE_SCAN)
    m = api.misa_route(q, w, K, off, k, B, h, 0, pooled=d[3], ws=ws_m, phases=api.PHASE_SCAN)
    scans = torch.cuda.Event()
    scans.record()
    side = [torch.cuda.Stream(device=DEV) for _ in range(3)]
    for s_ in side:
        s_.wait_event(scans)
    with torch.cuda.stream(side[0]):
        d = api.indexer_score_topk_pooled(q, w, K, off, k, b, B, out_small=d[2], out_large=d[3],
                                          out_idx=d[0], out_score=d[1], ws=ws_d,
                                          phases=api.PHASE_SELECT)
    with torch.cuda.stream(side[1]):
        md = api.misa_route(q, w, K, off, k, B, h, kp, pooled=d[3], ws=ws_md, out_idx=md[0],
                            out_score=md[1], out_heads=md[2], out_pool=md[3],
                            phases=api.PHASE_SELECT)
    with torch.cuda.stream(side[2]):
        m = api.misa_route(q, w, K, off, k, B, h, 0, pooled=d[3], ws=ws_m, out_idx=m[0],
                           out_score=m[1], out_heads=m[2], phases=api.PHASE_SELECT)
    torch.cuda.synchronize()
    _same(ref_d, d)
    _same(ref_md, md)
    _same(ref_m, m)
