"""GPU: the selectors captured into HIP graphs give, on every replay, the
outputs of the same calls run eagerly.  The library clears its state with a
fill kernel (no memset node), and every launch goes through the capture
stream, so a replay runs the same kernels on the same buffers.  Each test
replays several times with eager work and synchronizations in between, and
clears the outputs before each replay so that a replay that wrote nothing
would show.  Cases: the decode step of all four selectors on two streams (as
bench.py times it), and prefill rows of DSA, MISA, MISA-dagger and HISA at a
size that takes the many-row kernels (a router row per wave, the 512-thread
select, the rescoring that sweeps each row's list)."""
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


def _sets(outs):
    """Per output: sorted indices and sorted scores (the emit order of a set
    is not specified)."""
    return {m: (torch.sort(i, -1)[0].cpu(), torch.sort(s, -1)[0].cpu()) for m, (i, s) in outs.items()}


def _replays_match(step, outs, replays=4):
    step()
    torch.cuda.synchronize()
    ref = _sets(outs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for n in range(replays):
        for i, s in outs.values():
            i.fill_(-7)
            s.fill_(0.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _sets(outs)
        for m in outs:
            assert torch.equal(got[m][0], ref[m][0]), "replay %d: %s indices" % (n, m)
            assert torch.equal(got[m][1], ref[m][1]), "replay %d: %s scores" % (n, m)
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_graph_decode_step_two_streams(api):
    say("graph: decode step, 4 selectors, 2 streams")
    p = synth.make_problem(81, Bt=4, T=1, L=16384, H=64, needles=8, needle_mode="decode")
    q, w, K = _inputs(p)
    Bt, L, H, d, off, k = p["Bt"], p["L"], p["H"], p["d"], p["offset"], 512
    B, h, kp, b, r = 1024, 8, 2048, 128, 16
    shape = api.Shape(Bt, 1, H, d, L, off, k)
    ws = {"dsa": api.indexer_score_topk_pooled_ws(shape, b, B),
          "misa": api.misa_route_ws(shape, B, h, 0, True),
          "misa_dagger": api.misa_route_ws(shape, B, h, kp, True),
          "hisa": api.hisa_coarse_fine_ws(shape, b, r, True)}
    ws = {m: torch.empty(n, dtype=torch.uint8, device=DEV) for m, n in ws.items()}
    reps_b = torch.empty((Bt, L // b, 2, d), dtype=torch.int16, device=DEV)
    reps_B = torch.empty((Bt, L // B, 2, d), dtype=torch.int16, device=DEV)
    outs = {m: (torch.empty((Bt, 1, k), dtype=torch.int32, device=DEV),
                torch.empty((Bt, 1, k), dtype=torch.float32, device=DEV)) for m in ws}
    side = torch.cuda.Stream(device=DEV)
    ready = torch.cuda.Event()
    ready.record()

    def step():
        main = torch.cuda.current_stream()
        api.indexer_score_topk_pooled(q, w, K, off, k, b, B, out_small=reps_b, out_large=reps_B,
                                      out_idx=outs["dsa"][0], out_score=outs["dsa"][1],
                                      ws=ws["dsa"], pools_ready=ready)
        side.wait_event(ready)
        with torch.cuda.stream(side):
            api.hisa_coarse_fine(q, w, K, off, k, b, r, reps=reps_b, want_blocks=False,
                                 out_idx=outs["hisa"][0], out_score=outs["hisa"][1],
                                 ws=ws["hisa"])
            api.misa_route(q, w, K, off, k, B, h, 0, pooled=reps_B, want_heads=False,
                           out_idx=outs["misa"][0], out_score=outs["misa"][1], ws=ws["misa"])
        api.misa_route(q, w, K, off, k, B, h, kp, pooled=reps_B, want_heads=False,
                       out_idx=outs["misa_dagger"][0], out_score=outs["misa_dagger"][1],
                       ws=ws["misa_dagger"])
        main.wait_stream(side)

    _replays_match(step, outs)


def test_graph_prefill_rows(api):
    say("graph: prefill rows T=1024, DSA, MISA, MISA-dagger, HISA")
    p = synth.make_problem(82, Bt=1, T=1024, L=10240, H=64, offset=10240 - 1024, needles=8,
                           needle_mode="rows")
    q, w, K = _inputs(p)
    T, L, H, d, off, k = p["T"], p["L"], p["H"], p["d"], p["offset"], 256
    B, h, kp, b, r = 1024, 8, 2048, 128, 16
    shape = api.Shape(1, T, H, d, L, off, k)
    pooled = api.pool_blocks(K, B)
    reps = api.pool_blocks(K, b)
    ws = {"dsa": api.indexer_score_topk_ws(shape),
          "misa": api.misa_route_ws(shape, B, h, 0, True),
          "misa_dagger": api.misa_route_ws(shape, B, h, kp, True),
          "hisa": api.hisa_coarse_fine_ws(shape, b, r, True)}
    ws = {m: torch.empty(n, dtype=torch.uint8, device=DEV) for m, n in ws.items()}
    outs = {m: (torch.empty((1, T, k), dtype=torch.int32, device=DEV),
                torch.empty((1, T, k), dtype=torch.float32, device=DEV)) for m in ws}

    def step():
        api.indexer_score_topk(q, w, K, off, k, outs["dsa"][0], outs["dsa"][1], ws=ws["dsa"])
        api.misa_route(q, w, K, off, k, B, h, 0, pooled=pooled, want_heads=False,
                       out_idx=outs["misa"][0], out_score=outs["misa"][1], ws=ws["misa"])
        api.misa_route(q, w, K, off, k, B, h, kp, pooled=pooled, want_heads=False,
                       out_idx=outs["misa_dagger"][0], out_score=outs["misa_dagger"][1],
                       ws=ws["misa_dagger"])
        api.hisa_coarse_fine(q, w, K, off, k, b, r, reps=reps, want_blocks=False,
                             out_idx=outs["hisa"][0], out_score=outs["hisa"][1], ws=ws["hisa"])

    _replays_match(step, outs)
