"""GPU parity of LISA and ResMiSA (PaperTrace, "2.2.2 MISA, LISA and
ResMiSA", sections 3.1 and 3.2) through the C ABI against the CPU oracle.

* sa_block_extrema is byte work: every per-block max / min must equal numpy's
  reduction of the same bf16 values bit for bit.
* lisa_score_topk: the linear score g . k, parity rule of tests/parity.py.
* resmisa_route: the routed heads by the near-tie rule on the oracle's S,
  then the tokens against the oracle run with the GPU's heads (staged).
Shapes cover decode and fused-prefill rows, blocks cut by the causal bound,
H not a multiple of 16, the limits r = 0 (LISA) and r = H (DSA), the largest
r that fits, and the L = 131072 batch-8 decode workload.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from parity import _np, check_dsa, check_lisa, check_resmisa, rows_of, to_device
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


@pytest.mark.parametrize("Bt,L,block", [(2, 5000, 128), (1, 1000, 300), (1, 1, 64), (3, 2049, 1)])
def test_block_extrema(api, Bt, L, block):
    say("extrema Bt=%d L=%d block=%d" % (Bt, L, block))
    p = synth.make_problem(500 + L % 97, Bt=Bt, T=1, L=L, H=4)
    K = torch.from_numpy(p["K"].view(np.int16)).to(DEV)
    out = _np(api.block_extrema(K, block)).view(np.uint16)
    Kf = synth.bf16_bits_to_f32(p["K"])
    nb = (L + block - 1) // block
    assert out.shape == (Bt, nb, 2, 128)
    for m in range(nb):
        blk = Kf[:, m * block:min((m + 1) * block, L)]
        assert np.array_equal(synth.bf16_bits_to_f32(out[:, m, 0]), blk.max(1))
        assert np.array_equal(synth.bf16_bits_to_f32(out[:, m, 1]), blk.min(1))


@pytest.mark.parametrize("Bt,T,L,offset,H,k", [
    (3, 1, 5000, None, 64, 100),     # decode, ragged L
    (2, 3, 9001, None, 64, 257),     # several decode rows
    (2, 1, 300, None, 40, 512),      # k > t+1; H not a multiple of 16
    (1, 40, 700, 660, 64, 64),       # fused prefill rows
    (1, 300, 300, 0, 32, 128),       # causal prefill from position 0
])
def test_lisa(api, Bt, T, L, offset, H, k):
    say("lisa Bt=%d T=%d L=%d H=%d k=%d" % (Bt, T, L, H, k))
    p = synth.make_problem(600 + T + L % 13, Bt=Bt, T=T, L=L, H=H, offset=offset, needles=8,
                           needle_mode="decode" if T == 1 else "rows")
    q, w, K = to_device(p, DEV)
    idx, sc = api.lisa_score_topk(q, w, K, p["offset"], k)
    torch.cuda.synchronize()
    check_lisa(p, k, _np(idx), _np(sc), rows_of(p))


@pytest.mark.parametrize("Bt,T,L,offset,H,block,r,k", [
    (3, 1, 5000, None, 64, 128, 7, 100),    # decode, cut last block (5000 % 128)
    (2, 3, 9001, None, 64, 64, 7, 257),     # decode rows with cut blocks
    (1, 2, 20000, None, 32, 128, 3, 2048),  # H = 32
    (2, 1, 4100, None, 40, 100, 5, 64),     # H not a multiple of 16
    (1, 40, 700, 660, 64, 64, 7, 64),       # prefill rows, causal cut blocks
    (1, 16, 3000, 2984, 16, 32, 2, 200),    # prefill at the row-count boundary
    (2, 1, 3000, None, 64, 128, 60, 300),   # the largest r with 64 heads
    (1, 1, 1, None, 64, 8, 7, 8),           # a single key
])
def test_resmisa(api, Bt, T, L, offset, H, block, r, k):
    say("resmisa Bt=%d T=%d L=%d H=%d block=%d r=%d k=%d" % (Bt, T, L, H, block, r, k))
    p = synth.make_problem(700 + T + L % 17, Bt=Bt, T=T, L=L, H=H, offset=offset, needles=8,
                           needle_mode="decode" if T == 1 else "rows")
    q, w, K = to_device(p, DEV)
    idx, sc, heads = api.resmisa_route(q, w, K, p["offset"], k, block, r)
    torch.cuda.synchronize()
    check_resmisa(p, k, block, r, _np(idx), _np(sc), _np(heads), rows_of(p))


def test_resmisa_limits(api):
    # r = 0 gives LISA's selection and r = H the DSA one, through the same entry point.
    say("resmisa limits")
    p = synth.make_problem(801, Bt=2, T=2, L=3000, H=64, needles=8, needle_mode="rows")
    q, w, K = to_device(p, DEV)
    i0, s0, h0 = api.resmisa_route(q, w, K, p["offset"], 150, 128, 0)
    torch.cuda.synchronize()
    assert h0 is None
    check_lisa(p, 150, _np(i0), _np(s0), rows_of(p))
    iH, sH, hH = api.resmisa_route(q, w, K, p["offset"], 150, 128, 64)
    torch.cuda.synchronize()
    assert np.array_equal(_np(hH).reshape(-1, 64), np.tile(np.arange(64), (4, 1)))
    check_dsa(p, 150, _np(iH), _np(sH), rows_of(p))


def test_resmisa_extrema_given_matches_internal(api):
    say("resmisa extrema given")
    p = synth.make_problem(802, Bt=2, T=1, L=6000, H=64, needles=8, needle_mode="decode")
    q, w, K = to_device(p, DEV)
    ext = api.block_extrema(K, 128)
    ia, sa, ha = (_np(x) for x in api.resmisa_route(q, w, K, p["offset"], 200, 128, 7, extrema=ext))
    ib, sb, hb = (_np(x) for x in api.resmisa_route(q, w, K, p["offset"], 200, 128, 7))
    torch.cuda.synchronize()
    assert np.array_equal(ha, hb)
    # same set and the same score per index (the order inside a row is not specified)
    oa, ob = np.argsort(ia, -1), np.argsort(ib, -1)
    assert np.array_equal(np.take_along_axis(ia, oa, -1), np.take_along_axis(ib, ob, -1))
    assert np.array_equal(np.take_along_axis(sa, oa, -1), np.take_along_axis(sb, ob, -1))


def test_resmisa_rejects_r_that_does_not_fit(api):
    say("resmisa r=61 rejected")
    p = synth.make_problem(803, Bt=1, T=1, L=100, H=64)
    q, w, K = to_device(p, DEV)
    with pytest.raises(api.SaError) as e:
        api.resmisa_route(q, w, K, p["offset"], 8, 16, 61)
    assert e.value.code == api.SA_EUNSUPPORTED


def test_lisa_and_resmisa_128k(api):
    # The L = 131072, batch-8, 64-head decode workload: LISA and ResMiSA
    # (block 128, r = 7: one shared expert and 7 residual heads), every row.
    say("lisa / resmisa 128k b8 h64")
    p = synth.make_config("misa_128k_h64")
    q, w, K = to_device(p, DEV)
    idx, sc = api.lisa_score_topk(q, w, K, p["offset"], 2048)
    torch.cuda.synchronize()
    check_lisa(p, 2048, _np(idx), _np(sc), rows_of(p))
    idx, sc, heads = api.resmisa_route(q, w, K, p["offset"], 2048, 128, 7)
    torch.cuda.synchronize()
    check_resmisa(p, 2048, 128, 7, _np(idx), _np(sc), _np(heads), rows_of(p))
