"""Pins for the oracle's LISA and ResMiSA functions (no GPU).

PaperTrace, "2.2.2 MISA, LISA and ResMiSA", sections 3.1 and 3.2 define:
* LISA: the linear score l = g . k with the fused query g = sum_j w_j q_j;
* ResMiSA: R = l + sum_{h in A} w_h ReLU(-(q_h . k)) over r residual heads A,
  routed by S_h = |w_h| max_b ReLU(U-_{h,b}), U- the coordinate-box bound over
  the legal keys of block b.

What fixes them, other than the functions themselves:
* the two worked examples of the pages (score 6 = 4.5 + 1.5, and the routed
  second head recovering 6; the box bound 9 of a two-dimensional block);
* the limits the pages state: r = 0 is LISA, r = H is the full DSA score;
* exact rational brute force (tests/brute.py) that scores and routes by an
  independent formulation (per-head linear sums, the box maximum taken
  coordinate by coordinate) on tiny inputs, causal rows and cut blocks;
* the omitted-term bound of section 3.2, |R - I| <= sum_{h not in A} S_h;
* legality: keys past the row's position in its block never enter the bound;
* the sign of w is kept: a routed head with negative w lowers the score.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import brute
import oracle
from sparse_attention_token_dsa_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(q, w, K, offset):
    return oracle.Problem(np.ascontiguousarray(q), np.ascontiguousarray(w),
                          np.ascontiguousarray(K), offset)


def _embed_two_head_example():
    ex = json.load(open(os.path.join(GOLDEN, "pt_3_1_two_head_example.json")))
    d = 128
    q = np.zeros((1, 1, 2, d), np.float32)
    q[0, 0, :, 0] = ex["q"]
    w = np.array(ex["w"], np.float32).reshape(1, 1, 2)
    K = np.zeros((1, 1, d), np.float32)
    K[0, 0, 0] = ex["k"]
    return ex, synth.to_bf16_bits(q), w, synth.to_bf16_bits(K)


def test_two_head_example_lisa_and_resmisa():
    ex, q, w, K = _embed_two_head_example()
    prob = _problem(q, w, K, 0)
    _, _, dsa_rs = oracle.dsa(prob, 1, want_rowscore=True)
    _, lisa_sc, lisa_rs = oracle.lisa(prob, 1, want_rowscore=True)
    assert dsa_rs[0, 0] == ex["score"]
    assert lisa_rs[0, 0] == ex["linear_term"] and lisa_sc[0, 0] == ex["linear_term"]
    # r = 1: the routing must pick the second head (the only one whose box
    # bound is positive), which restores the full score.
    out = oracle.resmisa(prob, 1, 1, 1, want_rowscore=True)
    assert out["heads"].tolist() == [[1]]
    assert out["S"][0].tolist() == [0.0, ex["w"][1] * -ex["q"][1] * ex["k"]]
    assert out["rowscore"][0, 0] == ex["score"]
    assert out["rowscore"][0, 0] - lisa_rs[0, 0] == ex["nonlinear_correction"]
    # forcing the first head instead leaves the linear term (its correction is 0)
    forced = oracle.resmisa(prob, 1, 1, 1, override_heads=np.array([[0]]), want_rowscore=True)
    assert forced["rowscore"][0, 0] == ex["linear_term"]


def test_box_bound_example():
    ex = json.load(open(os.path.join(GOLDEN, "pt_3_2_box_bound_example.json")))
    assert oracle.box_bound(ex["q"], ex["k_min"], ex["k_max"]) == ex["box_bound"]
    q = np.array(ex["q"])
    for key, neg in zip(ex["block_keys"], ex["negative_dots"]):
        assert -float(q @ np.array(key)) == neg <= ex["box_bound"]
    # the same block through the routed selector: one head, two keys, block 2
    d = 128
    qq = np.zeros((1, 1, 1, d), np.float32)
    qq[0, 0, 0, :2] = ex["q"]
    K = np.zeros((1, 2, d), np.float32)
    K[0, :, :2] = ex["block_keys"]
    prob = _problem(synth.to_bf16_bits(qq), np.ones((1, 1, 1), np.float32),
                    synth.to_bf16_bits(K), 1)
    out = oracle.resmisa(prob, 2, 2, 1)
    assert out["S"][0, 0] == ex["box_bound"]


@pytest.mark.parametrize("seed", [11, 12])
def test_limits_r0_is_lisa_and_rH_is_dsa(seed):
    p = synth.make_problem(seed, Bt=2, T=3, L=200, H=8, offset=197)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    k = 17
    li, ls, lrs = oracle.lisa(prob, k, want_rowscore=True)
    r0 = oracle.resmisa(prob, k, 16, 0, want_rowscore=True)
    assert np.array_equal(r0["idx"], li) and np.array_equal(r0["score"], ls)
    di, ds, drs = oracle.dsa(prob, k, want_rowscore=True)
    rH = oracle.resmisa(prob, k, 16, 8, want_rowscore=True)
    assert sorted(rH["heads"][0].tolist()) == list(range(8))
    ok = ~np.isnan(drs)
    scale = np.nanmax(np.abs(drs))
    assert np.allclose(rH["rowscore"][ok], drs[ok], rtol=0, atol=1e-12 * scale)
    assert np.array_equal(np.sort(rH["idx"], 1), np.sort(di, 1))


def test_linear_score_is_the_weighted_head_sum():
    # l = g . k (the oracle's form) against sum_j w_j (q_j . k) by a library
    # matrix product: the head fusion of section 3.1 is exact.
    p = synth.make_problem(13, Bt=1, T=2, L=300, H=16, offset=298)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    _, _, lrs = oracle.lisa(prob, 5, want_rowscore=True)
    q = synth.bf16_bits_to_f32(p["q"][0]).astype(np.float64)      # [T, H, d]
    K = synth.bf16_bits_to_f32(p["K"][0]).astype(np.float64)      # [L, d]
    w = p["w"][0].astype(np.float64)                               # [T, H]
    z = np.einsum("thd,sd->ths", q, K)
    ref = np.einsum("th,ths->ts", w, z)
    for i in range(2):
        t = p["offset"] + i
        assert np.allclose(lrs[i, : t + 1], ref[i, : t + 1], rtol=0,
                           atol=1e-12 * np.abs(ref[i]).max())
        assert np.all(np.isnan(lrs[i, t + 1:]))


@pytest.mark.parametrize("seed,T,L,H,block,r,k", [
    (21, 3, 9, 4, 4, 2, 3),     # cut last block on every row
    (22, 2, 8, 3, 3, 1, 2),     # one residual head
    (23, 2, 7, 4, 2, 3, 4),
    (24, 1, 6, 5, 6, 0, 2),     # LISA
    (25, 2, 6, 3, 1, 3, 3),     # blocks of one key, every head routed
])
def test_brute_force(seed, T, L, H, block, r, k):
    d = 4
    p = synth.make_problem(seed, Bt=1, T=T, L=L, H=H, d=d, offset=L - T)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    out = oracle.resmisa(prob, k, block, r, want_rowscore=True)
    li, _, lrs = oracle.lisa(prob, k, want_rowscore=True)
    qe, we, ke = brute.exact_vectors(p["q"][0], p["w"][0], p["K"][0])
    for i in range(T):
        t = p["offset"] + i
        ref = brute.resmisa_row(qe, we, ke, i, t, k, block, r)
        if r:
            assert set(out["heads"][i].tolist()) == set(ref["heads"])
            assert np.allclose(out["S"][i], [float(ref["S"][j]) for j in range(H)],
                               rtol=1e-12, atol=1e-15)
        assert set(out["idx"][i][out["idx"][i] >= 0].tolist()) == set(ref["sel"])
        assert np.allclose(out["rowscore"][i, : t + 1], [float(ref["R"][s]) for s in range(t + 1)],
                           rtol=1e-12, atol=1e-15)
        lsel, lin = brute.lisa_row(qe, we, ke, i, t, k)
        assert set(li[i][li[i] >= 0].tolist()) == set(lsel)
        assert np.allclose(lrs[i, : t + 1], [float(lin[s]) for s in range(t + 1)],
                           rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed,block,r", [(31, 64, 3), (32, 100, 7), (33, 7, 1)])
def test_omitted_term_bound(seed, block, r):
    # Section 3.2: every omitted correction |w_h ReLU(-z_h)| is at most S_h,
    # so |R - I| <= sum of S_h over the heads not routed, for every legal key.
    p = synth.make_problem(seed, Bt=1, T=5, L=700, H=16, offset=695)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    out = oracle.resmisa(prob, 10, block, r, want_rowscore=True)
    _, _, drs = oracle.dsa(prob, 10, want_rowscore=True)
    for i in range(5):
        t = p["offset"] + i
        left = np.setdiff1d(np.arange(16), out["heads"][i])
        bound = out["S"][i][left].sum()
        diff = np.abs(out["rowscore"][i, : t + 1] - drs[i, : t + 1])
        assert np.all(diff <= bound * (1 + 1e-12))
        assert diff.max() > 0, "the routed score should differ from the full one here"
        # the routed heads are the r largest S (ties to the lower head)
        order = np.lexsort((np.arange(16), -out["S"][i]))
        assert sorted(out["heads"][i].tolist()) == sorted(order[:r].tolist())


def test_future_keys_never_enter_the_bound():
    # Row t sits inside a block whose later keys are huge; S must be the same
    # as with those future keys zeroed.
    p = synth.make_problem(41, Bt=1, T=1, L=64, H=4, offset=40)
    K2 = p["K"].copy()
    big = synth.bf16_bits_to_f32(K2).copy()
    big[0, 41:] = 50.0
    K2 = synth.to_bf16_bits(big)
    a = oracle.resmisa(oracle.Problem(p["q"], p["w"], p["K"], 40), 5, 32, 2)
    b = oracle.resmisa(oracle.Problem(p["q"], p["w"], K2, 40), 5, 32, 2)
    assert np.array_equal(a["S"], b["S"]) and np.array_equal(a["idx"], b["idx"])


def test_negative_weight_residual_lowers_the_score():
    # One key k = 1, two heads: q = (-1, 0.5) on dim 0, w = (-1, 1).
    # z = (-1, 0.5); l = (-1)(-1) + 1(0.5) = 1.5; head 0's correction is
    # w_0 ReLU(1) = -1, so routing it gives R = 0.5 = the DSA score
    # (-1 * ReLU(-1) + 1 * ReLU(0.5) = 0.5).
    d = 128
    q = np.zeros((1, 1, 2, d), np.float32)
    q[0, 0, :, 0] = [-1.0, 0.5]
    K = np.zeros((1, 1, d), np.float32)
    K[0, 0, 0] = 1.0
    w = np.array([-1.0, 1.0], np.float32).reshape(1, 1, 2)
    prob = _problem(synth.to_bf16_bits(q), w, synth.to_bf16_bits(K), 0)
    _, _, lrs = oracle.lisa(prob, 1, want_rowscore=True)
    out = oracle.resmisa(prob, 1, 1, 1, want_rowscore=True)
    _, _, drs = oracle.dsa(prob, 1, want_rowscore=True)
    assert lrs[0, 0] == 1.5
    assert out["heads"].tolist() == [[0]] and out["S"][0].tolist() == [1.0, 0.0]
    assert out["rowscore"][0, 0] == 0.5 == drs[0, 0]
