"""GPU parity of the MISA x HISA composition through the C ABI (staged:
routed heads, then blocks scored over those heads, then every-head token
rescoring), against the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from parity import _np, check_hisa, check_misa_hisa, rows_of, to_device
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


@pytest.mark.parametrize("Bt,T,L,offset,H,B,h,b,r,k", [
    (3, 1, 5000, None, 64, 1024, 8, 128, 8, 512),    # decode, cut last blocks
    (2, 3, 9001, None, 64, 512, 8, 64, 16, 257),     # several decode rows
    (1, 2, 20000, None, 32, 1024, 4, 128, 32, 2048),  # H = 32
    (2, 1, 4100, None, 40, 256, 5, 100, 4, 64),      # H not a multiple of 16
    (1, 40, 700, 660, 64, 128, 8, 64, 4, 64),        # prefill-sized rows, causal cut blocks
    (1, 1, 1, None, 64, 64, 8, 8, 1, 1),             # a single key
])
def test_misa_hisa(api, Bt, T, L, offset, H, B, h, b, r, k):
    say("misa x hisa Bt=%d T=%d L=%d H=%d B=%d h=%d b=%d r=%d k=%d" % (Bt, T, L, H, B, h, b, r, k))
    p = synth.make_problem(900 + T + L % 19, Bt=Bt, T=T, L=L, H=H, offset=offset, needles=8,
                           needle_mode="decode" if T == 1 else "rows")
    q, w, K = to_device(p, DEV)
    idx, sc, heads, blocks = api.misa_hisa(q, w, K, p["offset"], k, B, h, b, r)
    torch.cuda.synchronize()
    check_misa_hisa(p, k, B, h, b, r, _np(idx), _np(sc), _np(heads), _np(blocks), rows_of(p))


def test_misa_hisa_many_prefill_rows(api):
    # 2048 prefill rows: a router row per wave, the routed block scores with
    # a row's whole block range per workgroup, the rescoring sweeping each
    # row's list and the 512-thread selects; one row of each 8-row group.
    say("misa x hisa T=2048 L=8192")
    from parity import prefill_group_rows
    p = synth.make_problem(913, Bt=1, T=2048, L=8192, H=64, offset=8192 - 2048, needles=8,
                           needle_mode="rows")
    q, w, K = to_device(p, DEV)
    idx, sc, heads, blocks = api.misa_hisa(q, w, K, p["offset"], 512, 1024, 8, 128, 16)
    torch.cuda.synchronize()
    check_misa_hisa(p, 512, 1024, 8, 128, 16, _np(idx), _np(sc), _np(heads), _np(blocks),
                    prefill_group_rows(2048, 4))


def test_misa_hisa_all_heads_is_hisa(api):
    say("misa x hisa h = H")
    p = synth.make_problem(911, Bt=2, T=1, L=6000, H=64, needles=8, needle_mode="hisa")
    q, w, K = to_device(p, DEV)
    idx, sc, heads, blocks = api.misa_hisa(q, w, K, p["offset"], 200, 1024, 64, 128, 8)
    torch.cuda.synchronize()
    assert np.array_equal(_np(heads).reshape(-1, 64), np.tile(np.arange(64), (2, 1)))
    check_hisa(p, 200, 128, 8, _np(idx), _np(sc), _np(blocks), rows_of(p))


def test_misa_hisa_pools_given_match_internal(api):
    say("misa x hisa pools given")
    p = synth.make_problem(912, Bt=2, T=1, L=8192, H=64, needles=8, needle_mode="hisa")
    q, w, K = to_device(p, DEV)
    pb, pB = api.pool_blocks2(K, 128, 1024)
    a = [_np(x) for x in api.misa_hisa(q, w, K, p["offset"], 256, 1024, 8, 128, 16, pooled=pB,
                                       reps=pb)]
    c = [_np(x) for x in api.misa_hisa(q, w, K, p["offset"], 256, 1024, 8, 128, 16)]
    torch.cuda.synchronize()
    assert np.array_equal(a[2], c[2]) and np.array_equal(np.sort(a[3], -1), np.sort(c[3], -1))
    oa, oc = np.argsort(a[0], -1), np.argsort(c[0], -1)
    assert np.array_equal(np.take_along_axis(a[0], oa, -1), np.take_along_axis(c[0], oc, -1))
    assert np.array_equal(np.take_along_axis(a[1], oa, -1), np.take_along_axis(c[1], oc, -1))


def test_misa_hisa_128k(api):
    # L = 131072, batch 8, 64 heads: B = 1024, h = 8; b = 128, r = 64; k = 2048.
    say("misa x hisa 128k b8 h64")
    p = synth.make_config("hisa_128k")
    q, w, K = to_device(p, DEV)
    idx, sc, heads, blocks = api.misa_hisa(q, w, K, p["offset"], 2048, 1024, 8, 128, 64)
    torch.cuda.synchronize()
    check_misa_hisa(p, 2048, 1024, 8, 128, 64, _np(idx), _np(sc), _np(heads), _np(blocks),
                    rows_of(p))
