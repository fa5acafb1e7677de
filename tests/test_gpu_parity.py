"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases span several key tiles and chunks with ragged tails (L not a
multiple of 64 / 128 / 1024 / 8192); the named workloads run at full size,
every row of the decode-style ones and 512 rows of the chunked prefill (one
of each workgroup's two 8-row groups).  Every comparison uses the rule in
tests/parity.py (tolerance 2e-3 * max |score| per row, near-tie exchanges
only).  Outputs and workspaces sit between guard bytes that must come back
untouched.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import parity
from parity import (_np, check_dsa, check_guards, check_hisa, check_misa, guarded_outputs,
                    prefill_group_rows,
                    rows_of, to_device)
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
    shape = api.Shape(p["Bt"], p["T"], p["H"], p["d"], p["L"], p["offset"], k)
    gi, gs, gw = guarded_outputs(q, k, DEV, api.indexer_score_topk_ws(shape))
    idx, sc = api.indexer_score_topk(q, w, K, p["offset"], k, out_idx=gi.view,
                                     out_score=gs.view, ws=gw.view)
    torch.cuda.synchronize()
    check_guards(gi, gs, gw)
    return _np(idx), _np(sc)


def run_misa(api, p, k, B, h, kp):
    q, w, K = to_device(p, DEV)
    shape = api.Shape(p["Bt"], p["T"], p["H"], p["d"], p["L"], p["offset"], k)
    gi, gs, gw = guarded_outputs(q, k, DEV, api.misa_route_ws(shape, B, h, kp, False))
    idx, sc, heads, pool = api.misa_route(q, w, K, p["offset"], k, B, h, k_prime=kp,
                                          want_pool=kp > 0, out_idx=gi.view, out_score=gs.view,
                                          ws=gw.view)
    torch.cuda.synchronize()
    check_guards(gi, gs, gw)
    return _np(idx), _np(sc), _np(heads), _np(pool)


def run_hisa(api, p, k, b, r, reps_given=False):
    q, w, K = to_device(p, DEV)
    reps = api.pool_blocks(K, b) if reps_given else None
    shape = api.Shape(p["Bt"], p["T"], p["H"], p["d"], p["L"], p["offset"], k)
    gi, gs, gw = guarded_outputs(q, k, DEV, api.hisa_coarse_fine_ws(shape, b, r, reps_given))
    idx, sc, blocks = api.hisa_coarse_fine(q, w, K, p["offset"], k, b, r, reps=reps,
                                           out_idx=gi.view, out_score=gs.view, ws=gw.view)
    torch.cuda.synchronize()
    check_guards(gi, gs, gw)
    return _np(idx), _np(sc), _np(blocks)


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
    # at most 8 heads: a wave's two rows share one head tile
    (2, 37, 1200, 1163, 8, 100),    # H = 8, odd T (a wave with one active row)
    (1, 64, 4000, 3936, 5, 300),    # H = 5: tile rows of heads 5..7 empty
    (1, 20, 900, 0, 1, 50),         # H = 1, from position 0
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


def _bounded(api, T, L, offset, H, k):
    # the survivor list of these rows is shorter than their legal keys, so the
    # kernel compacts it while sweeping
    shape = api.Shape(1, T, H, 128, L, offset, k)
    return api.indexer_score_topk_ws(shape) < T * (offset + T) * 8


def test_prefill_bounded_lists_ascending_scores(api):
    # Scores grow with the position (every key survives the running threshold
    # until the list fills), with runs of exactly equal keys from bf16
    # rounding: the lists are compacted by the threshold bin and, where a bin
    # is too crowded, by the exact k-th key.
    say("prefill bounded lists, ascending scores")
    T, L, H, k = 16, 20000, 64, 100
    assert _bounded(api, T, L, L - T, H, k)
    p = synth.make_problem(61, Bt=1, T=T, L=L, H=H, offset=L - T)
    p["w"] = np.abs(p["w"])
    j = int(np.argmax(p["w"][0, 0]))
    u = synth.bf16_bits_to_f32(p["q"][0, 0, j])
    c = (0.5 + np.arange(L, dtype=np.float32) / np.float32(L))[:, None]
    p["K"][0] = synth.to_bf16_bits(c * u[None, :])
    idx, sc = run_dsa(api, p, k)
    check_dsa(p, k, idx, sc, rows_of(p))


def test_prefill_bounded_lists_all_equal(api):
    # 20000 equal scores per row: no threshold bin can be dropped, so the
    # exact compaction keeps positions 0..k-1 and refuses every later key.
    say("prefill bounded lists, all equal")
    T, L, H, k = 16, 20000, 64, 50
    assert _bounded(api, T, L, L - T, H, k)
    p = synth.make_problem(62, Bt=1, T=T, L=L, H=H, offset=L - T)
    p["K"][:] = p["K"][0, 0]
    idx, sc = run_dsa(api, p, k)
    for i in range(T):
        assert sorted(idx[0, i].tolist()) == list(range(k))


def test_prefill_bounded_lists_negative_scores(api):
    # Every weight negative: the scores are negative, their k-th in a crowded
    # one-octave bin.
    say("prefill bounded lists, negative scores")
    T, L, H, k = 32, 24000, 64, 64
    assert _bounded(api, T, L, L - T, H, k)
    p = synth.make_problem(63, Bt=1, T=T, L=L, H=H, offset=L - T, needles=8, needle_mode="rows")
    p["w"] = -np.abs(p["w"])
    idx, sc = run_dsa(api, p, k)
    check_dsa(p, k, idx, sc, rows_of(p))


def test_prefill_tiny_full(api):
    """Causal prefill, T = L = 1024, k = 128: every row against the oracle."""
    say("prefill_tiny full")
    p = synth.make_config("prefill_tiny")
    idx, sc = run_dsa(api, p, 128)
    check_dsa(p, 128, idx, sc, rows_of(p))


def test_decode_32k_all_rows(api):
    say("decode_32k all rows")
    p = synth.make_config("decode_32k")
    idx, sc = run_dsa(api, p, 2048)
    check_dsa(p, 2048, idx, sc, rows_of(p))


def test_prefill_chunked_rows(api):
    say("prefill_chunked 512 rows")
    p = synth.make_config("prefill_chunked")
    idx, sc = run_dsa(api, p, 2048)
    rows = prefill_group_rows(p["T"], 2)
    assert len(rows) == 512
    check_dsa(p, 2048, idx, sc, rows)


# ----------------------------------------------------------------- MISA

@pytest.mark.parametrize("Bt,T,L,H,B,h,k,kp", [
    (2, 1, 5000, 64, 256, 8, 64, 0),
    (2, 1, 5000, 64, 256, 8, 64, 320),
    (1, 3, 7000, 32, 1024, 8, 100, 0),     # partial last blocks (causal tail)
    (1, 4, 4000, 64, 300, 4, 50, 200),     # B not a power of two, dagger
    (1, 1, 2100, 64, 512, 64, 32, 0),      # h = H: equals DSA
    (1, 20, 900, 64, 128, 8, 40, 100),     # T >= 16 rows per sequence: the fused prefill
    (1, 256, 4096, 64, 1024, 8, 256, 1024),  # prefill rows, MISA-dagger
    (2, 64, 3000, 32, 512, 4, 100, 0),     # prefill rows, H = 32, partial blocks
    # decode rows whose blocks are whole (L a multiple of B): routed inside the scan
    (2, 1, 4096, 64, 512, 24, 100, 0),     # h = 24: two routed head tiles
    (1, 1, 8192, 40, 1024, 40, 64, 200),   # h = H = 40 (three tiles), MISA-dagger
    (3, 1, 2048, 16, 256, 3, 50, 100),     # H = 16, h = 3
    (2, 1, 4096, 64, 4096, 8, 64, 0),      # one block
])
def test_misa(api, Bt, T, L, H, B, h, k, kp):
    say("misa Bt=%d T=%d L=%d H=%d B=%d h=%d k=%d k'=%d" % (Bt, T, L, H, B, h, k, kp))
    p = synth.make_problem(300 + L % 89, Bt=Bt, T=T, L=L, H=H, needles=8,
                           needle_mode="decode" if T == 1 else "rows")
    idx, sc, heads, pool = run_misa(api, p, k, B, h, kp)
    check_misa(p, k, B, h, kp, idx, sc, heads, pool, rows_of(p))


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
    idx, sc, heads, pool = run_misa(api, p, 2048, 1024, 8, kp)
    check_misa(p, 2048, 1024, 8, kp, idx, sc, heads, pool, rows_of(p))


@pytest.mark.parametrize("kp", [0, 8192])
def test_misa_prefill_chunked_rows(api, kp):
    """MISA on the 4096-row prefill chunk over 32768 keys (the routed fused
    prefill, k' = 0 and the MISA-dagger pool): one row of each 8-row group."""
    say("misa prefill_chunked k'=%d 512 rows" % kp)
    p = synth.make_config("prefill_chunked")
    idx, sc, heads, pool = run_misa(api, p, 2048, 1024, 8, kp)
    rows = prefill_group_rows(p["T"], 5 + kp)
    check_misa(p, 2048, 1024, 8, kp, idx, sc, heads, pool, rows)


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
    idx, sc, blocks = run_hisa(api, p, k, b, r)
    check_hisa(p, k, b, r, idx, sc, blocks, rows_of(p))


def test_hisa_prefill_chunked_rows(api):
    """HISA (b = 128, r = 64) on the 4096-row prefill chunk over 32768 keys:
    one row of each 8-row group."""
    say("hisa prefill_chunked 512 rows")
    p = synth.make_config("prefill_chunked")
    idx, sc, blocks = run_hisa(api, p, 2048, 128, 64)
    rows = prefill_group_rows(p["T"], 9)
    check_hisa(p, 2048, 128, 64, idx, sc, blocks, rows)


def test_hisa_config(api):
    say("hisa_128k")
    p = synth.make_config("hisa_128k")
    idx, sc, blocks = run_hisa(api, p, 2048, 128, 64, reps_given=True)
    check_hisa(p, 2048, 128, 64, idx, sc, blocks, rows_of(p))


# ------------------------------------------------- score ranges of the select

def _scaled_keys(p, q_scale, key_scale):
    """q times q_scale, key row i times key_scale[i] (powers of two keep the
    bf16 mantissas as they were)."""
    q = synth.bf16_bits_to_f32(p["q"]) * np.float32(q_scale)
    K = synth.bf16_bits_to_f32(p["K"]) * key_scale.astype(np.float32)[None, :, None]
    p["q"], p["K"] = synth.to_bf16_bits(q), synth.to_bf16_bits(K)
    return p


def test_many_rows_select(api):
    """512 rows or more take the 512-thread select (two rows per CU): ties
    (all keys equal) in HISA's block and token selects and in MISA-dagger's
    rerank, then a MISA-dagger pool of 12000 keys (the general path)."""
    say("many-row select: ties")
    p = synth.make_problem(71, Bt=1, T=512, L=2048, H=64, offset=1536)
    p["K"][:] = p["K"][0, 0]
    idx, sc, blocks = run_hisa(api, p, 128, 64, 8)
    for i in range(512):
        assert sorted(idx[0, i].tolist()) == list(range(128))
        assert sorted(blocks[0, i].tolist()) == list(range(8))
    idx, sc, heads, pool = run_misa(api, p, 128, 256, 8, 512)
    for i in range(512):
        assert sorted(idx[0, i].tolist()) == list(range(128))
    say("many-row select: pool over 8192 keys")
    p = synth.make_problem(72, Bt=1, T=512, L=13000, H=64, offset=13000 - 512, needles=8,
                           needle_mode="rows")
    idx, sc, heads, pool = run_misa(api, p, 2048, 1024, 8, 12000)
    check_misa(p, 2048, 1024, 8, 12000, idx, sc, heads, pool, prefill_group_rows(512, 3))


def test_select_sources_over_8192_keys(api):
    # Sources of more than 8192 keys take the select's general path, not the
    # register-resident one: every key of a 20000-key row on the filter's
    # threshold bin (all keys equal), a MISA-dagger pool of k' = 12000, and
    # HISA's 96 x 128 rescored tokens.
    say("select over 8192 keys")
    p = synth.make_problem(13, Bt=1, T=1, L=20000, H=64)
    p["K"][:] = p["K"][0, 0]
    idx, sc = run_dsa(api, p, 100)
    assert sorted(idx[0, 0].tolist()) == list(range(100))
    idx, sc = run_dsa(api, p, 9000)
    assert sorted(idx[0, 0].tolist()) == list(range(9000))
    p = synth.make_problem(14, Bt=2, T=1, L=20000, H=64, needles=8, needle_mode="decode")
    idx, sc, heads, pool = run_misa(api, p, 2048, 1024, 8, 12000)
    check_misa(p, 2048, 1024, 8, 12000, idx, sc, heads, pool, rows_of(p))
    p = synth.make_problem(15, Bt=2, T=1, L=20000, H=64, needles=8, needle_mode="hisa", b=128)
    idx, sc, blocks = run_hisa(api, p, 2048, 128, 96)
    check_hisa(p, 2048, 128, 96, idx, sc, blocks, rows_of(p))


def test_select_tiny_score_range(api):
    # Scores below 1e-32: the span of a row's scores is too small for
    # equal slices of the score interval, so the selects take radix digits
    # of the ordered score bits from their first level.
    say("tiny score range")
    L = 20000
    p = _scaled_keys(synth.make_problem(11, Bt=2, T=1, L=L, H=64, needles=8,
                                        needle_mode="decode"), 2.0 ** -52, np.full(L, 2.0 ** -52))
    idx, sc = run_dsa(api, p, 2048)
    assert np.abs(sc).max() < 1e-30
    check_dsa(p, 2048, idx, sc, rows_of(p))
    idx, sc, heads, pool = run_misa(api, p, 512, 1024, 8, 2048)
    check_misa(p, 512, 1024, 8, 2048, idx, sc, heads, pool, rows_of(p))
    idx, sc, blocks = run_hisa(api, p, 512, 64, 32)
    check_hisa(p, 512, 64, 32, idx, sc, blocks, rows_of(p))


def test_select_scores_over_many_octaves(api):
    # Key i scaled by 2^-(i mod 40): the scores spread over some 40 octaves,
    # most of them near the bottom of the interval, so a slicing level keeps
    # most of its keys and the selects go on with radix digits.
    say("scores over many octaves")
    L = 20000
    p = _scaled_keys(synth.make_problem(12, Bt=2, T=1, L=L, H=64, needles=8,
                                        needle_mode="decode"), 1.0,
                     2.0 ** -(np.arange(L) % 40).astype(np.float64))
    idx, sc = run_dsa(api, p, 2048)
    check_dsa(p, 2048, idx, sc, rows_of(p))
    idx, sc, heads, pool = run_misa(api, p, 512, 1024, 8, 2048)
    check_misa(p, 512, 1024, 8, 2048, idx, sc, heads, pool, rows_of(p))
    idx, sc, blocks = run_hisa(api, p, 512, 64, 32)
    check_hisa(p, 512, 64, 32, idx, sc, blocks, rows_of(p))


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


@pytest.mark.parametrize("Bt,L,small,large,k", [
    (8, 131072, 128, 1024, 2048),   # the 128K decode batch: full 4096-key chunks
    (3, 5000, 128, 1024, 100),      # partial last chunk and blocks
    (2, 300, 128, 1024, 64),        # one chunk shorter than a large block
    (2, 20000, 256, 2048, 500),     # other block sizes
])
def test_pooled_dsa(api, Bt, L, small, large, k):
    # The DSA decode selector that also pools the keys it streams: the same
    # selection as indexer_score_topk (same scores, so the same set), and the
    # block means of the oracle (as sa_pool_blocks2, up to fp32 rounding).
    say("pooled dsa Bt=%d L=%d small=%d large=%d" % (Bt, L, small, large))
    p = synth.make_problem(70 + L % 61, Bt=Bt, T=1, L=L, H=64, needles=8, needle_mode="decode")
    q, w, K = to_device(p, DEV)
    shape = api.Shape(Bt, 1, 64, 128, L, L - 1, k)
    gi, gs, gw = guarded_outputs(q, k, DEV, api.indexer_score_topk_pooled_ws(shape, small, large))
    ev = torch.cuda.Event()
    idx, sc, ps, pl = api.indexer_score_topk_pooled(q, w, K, L - 1, k, small, large,
                                                    out_idx=gi.view, out_score=gs.view,
                                                    ws=gw.view, pools_ready=ev)
    ridx, rsc = api.indexer_score_topk(q, w, K, L - 1, k)
    torch.cuda.synchronize()
    check_guards(gi, gs, gw)
    a, r = _np(idx).reshape(Bt, k), _np(ridx).reshape(Bt, k)
    for row in range(Bt):
        assert set(a[row].tolist()) == set(r[row].tolist())
    check_dsa(p, k, _np(idx), _np(sc), rows_of(p))
    for got, block in ((ps, small), (pl, large)):
        g = _np(got).view(np.uint16)
        val = synth.bf16_bits_to_f32(g[:, :, 0]).astype(np.float64) + \
            synth.bf16_bits_to_f32(g[:, :, 1]).astype(np.float64)
        np.testing.assert_allclose(val, oracle.pool(p["K"], block), rtol=1e-4, atol=2e-6)


def test_pooled_dsa_rejects_prefill_rows(api):
    say("pooled dsa rejects T > 1")
    p = synth.make_problem(79, Bt=1, T=2, L=500, H=16)
    q, w, K = to_device(p, DEV)
    with pytest.raises(api.SaError) as e:
        api.indexer_score_topk_pooled(q, w, K, 498, 8, 128, 1024)
    assert e.value.code == api.SA_EUNSUPPORTED


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
