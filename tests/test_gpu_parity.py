"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases span several key tiles and chunks with ragged tails (L not a
multiple of 64 / 128 / 1024 / 8192); the named workloads run at full size with
sampled rows.  Every comparison uses the rule in tests/parity.py
(tolerance 2e-3 * max |score| per row, near-tie exchanges only).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import parity
from parity import _np, check_dsa, check_hisa, check_misa, rows_of, to_device
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


def run_dsa(api, p, k):
    q, w, K = to_device(p, DEV)
    idx, sc = api.indexer_score_topk(q, w, K, p["offset"], k)
    torch.cuda.synchronize()
    return _np(idx), _np(sc)


# ------------------------------------------------------------------ DSA

@pytest.mark.parametrize("Bt,T,L,H,k,needles", [
    (3, 1, 5000, 64, 100, 16),      # decode, ragged L
    (2, 3, 9001, 64, 257, 8),       # several decode rows per sequence
    (2, 1, 300, 64, 512, 4),        # k > t+1: the whole prefix
    (1, 2, 20000, 32, 2048, 32),    # H = 32 (GLM-5 indexer width)
    (2, 1, 4100, 40, 64, 8),        # H not a multiple of 16: zero-padded head tile
    (1, 1, 1, 64, 8, 0),            # a single key
])
def test_dsa_decode_path(api, Bt, T, L, H, k, needles):
    say("dsa decode Bt=%d T=%d L=%d H=%d k=%d" % (Bt, T, L, H, k))
    p = synth.make_problem(100 + L % 97, Bt=Bt, T=T, L=L, H=H, needles=needles,
                           needle_mode="decode")
    idx, sc = run_dsa(api, p, k)
    check_dsa(p, k, idx, sc, rows_of(p))


@pytest.mark.parametrize("Bt,T,L,offset,H,k", [
    (2, 40, 700, 660, 64, 64),      # chunked prefill, ragged tail of 8-row groups
    (1, 300, 300, 0, 64, 128),      # full causal prefill from position 0 (t < k rows)
    (1, 16, 3000, 2984, 32, 200),   # H = 32
    (1, 77, 1500, 1000, 64, 1000),  # k larger than many rows' survivors
    (1, 32, 6000, 5968, 64, 4000),  # k-th score negative: crowded one-octave bins
    (1, 24, 2000, 1976, 16, 1),     # k = 1, H = 16
])
def test_dsa_prefill_path(api, Bt, T, L, offset, H, k):
    say("dsa prefill Bt=%d T=%d L=%d off=%d H=%d k=%d" % (Bt, T, L, offset, H, k))
    p = synth.make_problem(200 + T, Bt=Bt, T=T, L=L, H=H, offset=offset, needles=12,
                           needle_mode="rows")
    idx, sc = run_dsa(api, p, k)
    check_dsa(p, k, idx, sc, rows_of(p))


def test_dsa_decode_winners_packed_in_few_chunks(api):
    # Every winner sits in one 600-key stretch of each row, i.e. in the
    # slices of a few scan and filter workgroups; the top-k must still be the
    # exact one.
    say("dsa packed winners")
    p = synth.make_problem(7, Bt=2, T=1, L=20000, H=64)
    rng = np.random.default_rng(7)
    for b in range(2):
        j = int(np.argmax(p["w"][b, 0]))
        qj = synth.bf16_bits_to_f32(p["q"][b, 0, j])
        noise = rng.standard_normal((600, 128)).astype(np.float32) * np.float32(0.3 / np.sqrt(128))
        p["K"][b, 5000:5600] = synth.to_bf16_bits(qj[None, :] * np.float32(4.0) + noise)
    idx, sc = run_dsa(api, p, 512)
    check_dsa(p, 512, idx, sc, rows_of(p))
    assert np.all((idx[:, 0] >= 5000) & (idx[:, 0] < 5600)), "winners outside the packed stretch"


def test_dsa_all_equal_keys_take_lowest_positions(api):
    say("dsa ties")
    p = synth.make_problem(5, Bt=1, T=1, L=2000, H=64)
    p["K"][:] = p["K"][0, 0]
    idx, sc = run_dsa(api, p, 50)
    assert sorted(idx[0, 0].tolist()) == list(range(50))
    p2 = synth.make_problem(6, Bt=1, T=20, L=600, H=64, offset=580)
    p2["K"][:] = p2["K"][0, 0]
    idx, sc = run_dsa(api, p2, 50)
    for i in range(20):
        assert sorted(idx[0, i].tolist()) == list(range(50))
    # Prefill rows of 5000 equal scores: one histogram bin holds the whole row,
    # so the selection goes down to the position bits of the key.
    p3 = synth.make_problem(7, Bt=1, T=16, L=5000, H=64, offset=4984)
    p3["K"][:] = p3["K"][0, 0]
    idx, sc = run_dsa(api, p3, 50)
    for i in range(16):
        assert sorted(idx[0, i].tolist()) == list(range(50))


def test_prefill_tiny_full(api):
    """Causal prefill, T = L = 1024, k = 128: every row against the oracle."""
    say("prefill_tiny full")
    p = synth.make_config("prefill_tiny")
    idx, sc = run_dsa(api, p, 128)
    check_dsa(p, 128, idx, sc, rows_of(p))


def test_decode_32k_sampled(api):
    say("decode_32k sampled")
    p = synth.make_config("decode_32k")
    idx, sc = run_dsa(api, p, 2048)
    check_dsa(p, 2048, idx, sc, rows_of(p, sample=8, seed=1))


def test_prefill_chunked_sampled(api):
    say("prefill_chunked sampled")
    p = synth.make_config("prefill_chunked")
    idx, sc = run_dsa(api, p, 2048)
    check_dsa(p, 2048, idx, sc, rows_of(p, sample=32, seed=2))


# ----------------------------------------------------------------- MISA

@pytest.mark.parametrize("Bt,T,L,H,B,h,k,kp", [
    (2, 1, 5000, 64, 256, 8, 64, 0),
    (2, 1, 5000, 64, 256, 8, 64, 320),
    (1, 3, 7000, 32, 1024, 8, 100, 0),     # partial last blocks (causal tail)
    (1, 4, 4000, 64, 300, 4, 50, 200),     # B not a power of two, dagger
    (1, 1, 2100, 64, 512, 64, 32, 0),      # h = H: equals DSA
    (1, 20, 900, 64, 128, 8, 40, 100),     # T >= 16 rows per sequence
])
def test_misa(api, Bt, T, L, H, B, h, k, kp):
    say("misa Bt=%d T=%d L=%d H=%d B=%d h=%d k=%d k'=%d" % (Bt, T, L, H, B, h, k, kp))
    p = synth.make_problem(300 + L % 89, Bt=Bt, T=T, L=L, H=H, needles=8,
                           needle_mode="decode" if T == 1 else "rows")
    q, w, K = to_device(p, DEV)
    idx, sc, heads, pool = api.misa_route(q, w, K, p["offset"], k, B, h, k_prime=kp,
                                          want_pool=kp > 0)
    torch.cuda.synchronize()
    check_misa(p, k, B, h, kp, _np(idx), _np(sc), _np(heads), _np(pool), rows_of(p))


def test_misa_all_heads_equals_dsa(api):
    say("misa h=H vs dsa")
    p = synth.make_problem(31, Bt=2, T=1, L=6000, H=64, needles=8, needle_mode="decode")
    q, w, K = to_device(p, DEV)
    idx, sc, heads, _ = api.misa_route(q, w, K, p["offset"], 128, 1024, 64)
    didx, dsc = api.indexer_score_topk(q, w, K, p["offset"], 128)
    torch.cuda.synchronize()
    assert np.all(np.sort(_np(heads), -1) == np.arange(64))
    for r in range(2):
        assert set(_np(idx)[r, 0].tolist()) == set(_np(didx)[r, 0].tolist())


def test_misa_pooled_given_matches_internal(api):
    say("misa pooled given")
    p = synth.make_problem(32, Bt=2, T=1, L=8192, H=64, needles=8, needle_mode="decode")
    q, w, K = to_device(p, DEV)
    pooled = api.pool_blocks(K, 1024)
    a = api.misa_route(q, w, K, p["offset"], 256, 1024, 8, k_prime=1024, pooled=pooled)
    b = api.misa_route(q, w, K, p["offset"], 256, 1024, 8, k_prime=1024)
    torch.cuda.synchronize()
    assert torch.equal(a[2], b[2])
    assert torch.equal(torch.sort(a[0], -1)[0], torch.sort(b[0], -1)[0])


@pytest.mark.parametrize("name", ["misa_128k_h64", "misa_128k_h32"])
@pytest.mark.parametrize("kp", [0, 8192])
def test_misa_configs(api, name, kp):
    say("%s k'=%d" % (name, kp))
    p = synth.make_config(name)
    q, w, K = to_device(p, DEV)
    idx, sc, heads, pool = api.misa_route(q, w, K, p["offset"], 2048, 1024, 8, k_prime=kp,
                                          want_pool=kp > 0)
    torch.cuda.synchronize()
    check_misa(p, 2048, 1024, 8, kp, _np(idx), _np(sc), _np(heads), _np(pool),
               rows_of(p, sample=4, seed=3))


# ----------------------------------------------------------------- HISA

@pytest.mark.parametrize("Bt,T,L,H,b,r,k", [
    (2, 1, 5000, 64, 64, 8, 64),
    (1, 3, 9000, 64, 128, 16, 300),       # ragged last block, several rows
    (1, 20, 1000, 32, 32, 6, 100),        # T >= 16, causal tails
    (1, 1, 700, 64, 128, 64, 200),        # r > #blocks: equals DSA
])
def test_hisa(api, Bt, T, L, H, b, r, k):
    say("hisa Bt=%d T=%d L=%d H=%d b=%d r=%d k=%d" % (Bt, T, L, H, b, r, k))
    p = synth.make_problem(400 + L % 83, Bt=Bt, T=T, L=L, H=H, needles=8,
                           needle_mode="hisa" if T == 1 else "rows", b=b)
    q, w, K = to_device(p, DEV)
    idx, sc, blocks = api.hisa_coarse_fine(q, w, K, p["offset"], k, b, r)
    torch.cuda.synchronize()
    check_hisa(p, k, b, r, _np(idx), _np(sc), _np(blocks), rows_of(p))


def test_hisa_config(api):
    say("hisa_128k")
    p = synth.make_config("hisa_128k")
    q, w, K = to_device(p, DEV)
    reps = api.pool_blocks(K, 128)
    idx, sc, blocks = api.hisa_coarse_fine(q, w, K, p["offset"], 2048, 128, 64, reps=reps)
    torch.cuda.synchronize()
    check_hisa(p, 2048, 128, 64, _np(idx), _np(sc), _np(blocks), rows_of(p, sample=4, seed=4))


# ----------------------------------------------------------------- pool

@pytest.mark.parametrize("L,block", [(5000, 128), (131072, 1024), (1000, 300)])
def test_pool_blocks(api, L, block):
    say("pool L=%d block=%d" % (L, block))
    p = synth.make_problem(50, Bt=2, T=1, L=L, H=4)
    _, _, K = to_device(p, DEV)
    got = _np(api.pool_blocks(K, block)).view(np.uint16)
    val = synth.bf16_bits_to_f32(got[:, :, 0]).astype(np.float64) + \
        synth.bf16_bits_to_f32(got[:, :, 1]).astype(np.float64)
    ref = oracle.pool(p["K"], block)
    np.testing.assert_allclose(val, ref, rtol=1e-4, atol=2e-6)


def test_pool_blocks2_matches_single(api):
    say("pool2")
    p = synth.make_problem(51, Bt=2, T=1, L=10000, H=4)
    _, _, K = to_device(p, DEV)
    s2, l2 = api.pool_blocks2(K, 128, 1024)
    for got, block in ((s2, 128), (l2, 1024)):
        g = _np(got).view(np.uint16)
        val = synth.bf16_bits_to_f32(g[:, :, 0]).astype(np.float64) + \
            synth.bf16_bits_to_f32(g[:, :, 1]).astype(np.float64)
        np.testing.assert_allclose(val, oracle.pool(p["K"], block), rtol=1e-4, atol=2e-6)


def test_profile_counters(api):
    say("profile")
    p = synth.make_problem(52, Bt=1, T=1, L=4096, H=64)
    q, w, K = to_device(p, DEV)
    api.profile_enable(True)
    api.indexer_score_topk(q, w, K, p["offset"], 64)
    torch.cuda.synchronize()
    prof = api.profile_read()
    api.profile_enable(False)
    assert prof["scan_dsa"][1] == 1 and prof["scan_dsa"][0] > 0
    assert "topk_select" in prof and "topk_filter" in prof


def test_smoke_run_every_entry_point(api):
    # The smoke check's sequence: one small call of every entry point, each
    # checked against the oracle.
    say("smoke run")
    parity.smoke_run(torch.device(DEV))
