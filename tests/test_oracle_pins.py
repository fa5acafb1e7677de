"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
* the two-head worked example printed on the PaperTrace page (score 6, its
  linear / correction split 4.5 + 1.5);
* exact rational brute force with exhaustive subset selection (tests/brute.py);
* a special case that reduces to a plain matrix product (all dot products
  non-negative, so every ReLU is the identity);
* the identity ReLU(x) = x + ReLU(-x) (the head-fused linear form);
* the structural invariants the method fixes (causality, whole-prefix rows,
  tie order, MISA with h = H and HISA with all blocks equal DSA, ...).
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


def _prob(seed, Bt=1, T=1, L=8, H=3, d=6, offset=None, needles=0):
    p = synth.make_problem(seed, Bt=Bt, T=T, L=L, H=H, d=d, offset=offset, needles=needles,
                           needle_mode="rows")
    return p, oracle.Problem(p["q"], p["w"], p["K"], p["offset"])


def _bits(x):
    return synth.to_bf16_bits(np.asarray(x, np.float32))


# ------------------------------------------------------------ worked example

def test_worked_example_score_is_six():
    g = json.load(open(os.path.join(GOLDEN, "pt_3_1_two_head_example.json")))
    d = 128
    q = np.zeros((1, 1, 2, d), np.float32)
    q[0, 0, :, 0] = g["q"]
    K = np.zeros((1, 1, d), np.float32)
    K[0, 0, 0] = g["k"]
    w = np.array(g["w"], np.float32).reshape(1, 1, 2)
    prob = oracle.Problem(_bits(q), w, _bits(K), 0)
    idx, sc, rs = oracle.dsa(prob, topk=1, want_rowscore=True)
    assert idx[0, 0] == 0
    assert sc[0, 0] == g["score"]
    # the same example split into the head-fused linear term and the
    # per-head correction: g_t . k = 4.5, sum_j w_j ReLU(-q_j . k) = 1.5
    gq = sum(wj * qj for wj, qj in zip(g["w"], g["q"]))
    assert gq == g["fused_query_g"]
    assert gq * g["k"] == g["linear_term"]
    corr = sum(wj * max(-qj * g["k"], 0.0) for wj, qj in zip(g["w"], g["q"]))
    assert corr == g["nonlinear_correction"]
    assert rs[0, 0] == g["linear_term"] + g["nonlinear_correction"]


def test_linear_plus_correction_identity_random():
    """I = g.k + sum_j w_j ReLU(-q_j.k) with g = sum_j w_j q_j, on random data:
    a different formula for the same value (catches a dropped ReLU, a sign
    flip, a wrong head or key index)."""
    p, prob = _prob(11, Bt=2, T=3, L=40, H=5, d=16, offset=37)
    _, _, rs = oracle.dsa(prob, topk=4, want_rowscore=True)
    q = synth.bf16_bits_to_f32(p["q"]).astype(np.float64)
    K = synth.bf16_bits_to_f32(p["K"]).astype(np.float64)
    w = p["w"].astype(np.float64)
    for b in range(2):
        for i in range(3):
            t = p["offset"] + i
            z = q[b, i] @ K[b, : t + 1].T  # [H, n]
            g = w[b, i] @ q[b, i]
            alt = g @ K[b, : t + 1].T + (w[b, i][:, None] * np.maximum(-z, 0)).sum(0)
            got = rs[b * 3 + i, : t + 1]
            np.testing.assert_allclose(got, alt, rtol=1e-12, atol=1e-15)
            assert np.all(np.isnan(rs[b * 3 + i, t + 1:]))


def test_nonnegative_case_is_a_matrix_product():
    """All q, k >= 0 makes every ReLU the identity: I = (w^T Q) K^T."""
    p, _ = _prob(12, Bt=1, T=2, L=30, H=4, d=12, offset=28)
    qa = _bits(np.abs(synth.bf16_bits_to_f32(p["q"])))
    Ka = _bits(np.abs(synth.bf16_bits_to_f32(p["K"])))
    prob = oracle.Problem(qa, p["w"], Ka, 28)
    _, _, rs = oracle.dsa(prob, topk=3, want_rowscore=True)
    q = synth.bf16_bits_to_f32(qa).astype(np.float64)[0]
    K = synth.bf16_bits_to_f32(Ka).astype(np.float64)[0]
    w = p["w"].astype(np.float64)[0]
    for i in range(2):
        t = 28 + i
        ref = np.einsum("j,jx,sx->s", w[i], q[i], K[: t + 1])
        np.testing.assert_allclose(rs[i, : t + 1], ref, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------ brute force

@pytest.mark.parametrize("seed,T,L,H,d,k,offset", [
    (21, 1, 9, 3, 6, 4, 8),
    (22, 3, 10, 2, 5, 3, 7),
    (23, 4, 6, 4, 4, 2, 0),   # rows shorter than k at the sequence start
    (24, 2, 8, 3, 8, 8, 6),   # k larger than every prefix
])
def test_dsa_matches_exact_brute_force(seed, T, L, H, d, k, offset):
    p, prob = _prob(seed, Bt=2, T=T, L=L, H=H, d=d, offset=offset)
    idx, sc, rs = oracle.dsa(prob, topk=k, want_rowscore=True)
    for b in range(2):
        qe, we, ke = brute.exact_vectors(p["q"][b], p["w"][b], p["K"][b])
        for i in range(T):
            t = offset + i
            sel, scores = brute.dsa_row(qe, we, ke, i, t, k)
            row = b * T + i
            got = [int(s) for s in idx[row] if s >= 0]
            assert frozenset(got) == sel
            assert len(got) == min(k, t + 1)
            assert np.all(idx[row, len(got):] == -1)
            for s in range(t + 1):
                assert rs[row, s] == pytest.approx(float(scores[s]), rel=1e-12, abs=1e-18)


def test_dsa_ties_take_lowest_indices():
    """Duplicate keys tie exactly; the lower positions win."""
    d, H, L = 8, 2, 9
    rng = np.random.default_rng(5)
    base = rng.standard_normal((3, d)).astype(np.float32)
    K = np.stack([base[s % 3] for s in range(L)])[None]
    q = rng.standard_normal((1, 1, H, d)).astype(np.float32)
    w = np.abs(rng.standard_normal((1, 1, H))).astype(np.float32)
    prob = oracle.Problem(_bits(q), w, _bits(K), L - 1)
    idx, sc = oracle.dsa(prob, topk=4)
    qe, we, ke = brute.exact_vectors(_bits(q)[0], w[0], _bits(K)[0])
    sel, _ = brute.dsa_row(qe, we, ke, 0, L - 1, 4)
    assert frozenset(idx[0].tolist()) == sel
    # whichever key pattern wins, its three copies tie and the earliest go first
    order = idx[0].tolist()
    for a, b2 in zip(order, order[1:]):
        if sc[0, order.index(a)] == sc[0, order.index(b2)]:
            assert a < b2


def test_all_equal_keys_select_prefix_start():
    d, H, L, k = 16, 4, 50, 7
    rng = np.random.default_rng(6)
    K = np.repeat(rng.standard_normal((1, 1, d)).astype(np.float32), L, axis=1)
    q = rng.standard_normal((1, 2, H, d)).astype(np.float32)
    w = rng.standard_normal((1, 2, H)).astype(np.float32)
    idx, _ = oracle.dsa(oracle.Problem(_bits(q), w, _bits(K), 30), topk=k)
    assert idx.tolist() == [list(range(k))] * 2


def test_causal_and_whole_prefix_rows():
    p, prob = _prob(31, Bt=2, T=20, L=40, H=4, d=32, offset=20, needles=8)
    idx, sc = oracle.dsa(prob, topk=25)
    for row in range(40):
        t = 20 + row % 20
        got = idx[row][idx[row] >= 0]
        assert got.max() <= t
        assert len(got) == min(25, t + 1)
        if t + 1 <= 25:
            assert sorted(got.tolist()) == list(range(t + 1))
        assert np.all(np.diff(sc[row, : len(got)]) <= 0)


def test_future_needle_is_never_selected():
    """A key that matches the query perfectly but sits at s = t+1 is masked."""
    d, H, L = 32, 4, 12
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, H, d)).astype(np.float32) * 0.1
    w = np.ones((1, 1, H), np.float32)
    K = rng.standard_normal((1, L, d)).astype(np.float32) * 0.1
    K[0, 6] = 50 * q[0, 0, 0]
    prob = oracle.Problem(_bits(q), w, _bits(K), 5)  # t = 5
    idx, _ = oracle.dsa(prob, topk=3)
    assert 6 not in idx[0].tolist()
    prob = oracle.Problem(_bits(q), w, _bits(K), 6)  # t = 6: now visible and first
    idx, _ = oracle.dsa(prob, topk=3)
    assert idx[0, 0] == 6


def test_head_permutation_and_positive_scaling():
    p, prob = _prob(41, Bt=1, T=4, L=64, H=6, d=32, offset=60)
    idx0, sc0 = oracle.dsa(prob, topk=10)
    perm = np.random.default_rng(1).permutation(6)
    prob_p = oracle.Problem(p["q"][:, :, perm], p["w"][:, :, perm], p["K"], 60)
    idx1, sc1 = oracle.dsa(prob_p, topk=10)
    assert np.array_equal(idx0, idx1)
    np.testing.assert_allclose(sc0, sc1, rtol=1e-12)
    prob_s = oracle.Problem(p["q"], p["w"] * np.float32(4.0), p["K"], 60)
    idx2, sc2 = oracle.dsa(prob_s, topk=10)
    assert np.array_equal(idx0, idx2)
    assert np.array_equal(sc2, 4.0 * sc0)


def test_negative_weights_lower_scores():
    """A head with w < 0 pushes its matching key down, not up."""
    d, H, L = 16, 2, 20
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, H, d)).astype(np.float32) * 0.1
    K = rng.standard_normal((1, L, d)).astype(np.float32) * 0.1
    K[0, 3] = 20 * q[0, 0, 0]
    w = np.array([[[-1.0, 0.5]]], np.float32)
    idx, sc = oracle.dsa(oracle.Problem(_bits(q), w, _bits(K), L - 1), topk=L)
    assert idx[0, -1] == 3


# ------------------------------------------------------------------- MISA

@pytest.mark.parametrize("seed,T,L,H,d,k,B,h,kp,offset", [
    (51, 1, 9, 4, 5, 3, 3, 2, 0, 8),
    (52, 2, 8, 4, 4, 2, 3, 1, 0, 6),
    (53, 1, 10, 4, 4, 3, 4, 2, 5, 9),
    (54, 3, 7, 3, 4, 2, 2, 2, 4, 4),
])
def test_misa_matches_exact_brute_force(seed, T, L, H, d, k, B, h, kp, offset):
    p, prob = _prob(seed, Bt=1, T=T, L=L, H=H, d=d, offset=offset)
    out = oracle.misa(prob, topk=k, B=B, h=h, kprime=kp, want_hatrow=True)
    qe, we, ke = brute.exact_vectors(p["q"][0], p["w"][0], p["K"][0])
    for i in range(T):
        t = offset + i
        ref = brute.misa_row(qe, we, ke, i, t, k, B, h, kp)
        assert frozenset(out["heads"][i].tolist()) == ref["heads"]
        assert list(out["heads"][i]) == sorted(out["heads"][i])
        for j in range(H):
            assert out["E"][i, j] == pytest.approx(float(ref["E"][j]), rel=1e-12, abs=1e-18)
        got = frozenset(int(s) for s in out["idx"][i] if s >= 0)
        assert got == ref["sel"]
        for s in range(t + 1):
            assert out["hatrow"][i, s] == pytest.approx(float(ref["hat"][s]), rel=1e-12,
                                                        abs=1e-18)
        if kp:
            assert frozenset(int(s) for s in out["pool"][i] if s >= 0) == ref["pool"]
            for u, s in enumerate(out["idx"][i]):
                if s >= 0:
                    assert out["score"][i, u] == pytest.approx(float(ref["full"][s]),
                                                               rel=1e-12, abs=1e-18)


def test_misa_all_heads_equals_dsa_exactly():
    p, prob = _prob(61, Bt=2, T=5, L=300, H=8, d=32, offset=295, needles=6)
    idx, sc = oracle.dsa(prob, topk=20)
    out = oracle.misa(prob, topk=20, B=64, h=8)
    assert np.array_equal(out["idx"], idx)
    assert np.array_equal(out["score"], sc)


def test_misa_dagger_limits():
    p, prob = _prob(62, Bt=1, T=4, L=200, H=8, d=32, offset=150, needles=6)
    idx, sc = oracle.dsa(prob, topk=16)
    # k' covering every legal token: the rerank sees the whole prefix -> DSA
    dag = oracle.misa(prob, topk=16, B=32, h=2, kprime=200)
    assert np.array_equal(dag["idx"], idx)
    assert np.array_equal(dag["score"], sc)
    # k' = k: the rerank only reorders the 1-stage set
    one = oracle.misa(prob, topk=16, B=32, h=2)
    same = oracle.misa(prob, topk=16, B=32, h=2, kprime=16)
    for r in range(4):
        assert set(one["idx"][r].tolist()) == set(same["idx"][r].tolist())


def test_misa_override_heads_is_respected():
    p, prob = _prob(63, Bt=1, T=2, L=100, H=8, d=16, offset=98)
    forced = np.array([[0, 5, 7], [1, 2, 3]], np.int32)
    out = oracle.misa(prob, topk=5, B=16, h=3, override_heads=forced, want_hatrow=True)
    assert np.array_equal(out["heads"], forced)
    q = synth.bf16_bits_to_f32(p["q"]).astype(np.float64)[0]
    K = synth.bf16_bits_to_f32(p["K"]).astype(np.float64)[0]
    w = p["w"].astype(np.float64)[0]
    for i in range(2):
        t = 98 + i
        hs = forced[i]
        ref = (w[i, hs][:, None] * np.maximum(q[i, hs] @ K[: t + 1].T, 0)).sum(0)
        np.testing.assert_allclose(out["hatrow"][i, : t + 1], ref, rtol=1e-12, atol=1e-15)


def test_misa_rejects_bad_budgets():
    _, prob = _prob(64, L=50, H=4, d=8, offset=49)
    with pytest.raises(ValueError):
        oracle.misa(prob, topk=8, B=16, h=5)
    with pytest.raises(ValueError):
        oracle.misa(prob, topk=8, B=16, h=2, kprime=4)


# ------------------------------------------------------------------- HISA

@pytest.mark.parametrize("seed,T,L,H,d,k,b,r,offset", [
    (71, 1, 10, 3, 5, 3, 3, 2, 9),
    (72, 2, 9, 2, 4, 2, 2, 2, 7),
    (73, 3, 8, 3, 4, 3, 3, 1, 5),
])
def test_hisa_matches_exact_brute_force(seed, T, L, H, d, k, b, r, offset):
    p, prob = _prob(seed, Bt=1, T=T, L=L, H=H, d=d, offset=offset)
    out = oracle.hisa(prob, topk=k, b=b, r=r)
    qe, we, ke = brute.exact_vectors(p["q"][0], p["w"][0], p["K"][0])
    for i in range(T):
        t = offset + i
        ref = brute.hisa_row(qe, we, ke, i, t, k, b, r)
        assert frozenset(int(m) for m in out["blocks"][i] if m >= 0) == ref["blocks"]
        for m in range(t // b + 1):
            assert out["J"][i, m] == pytest.approx(float(ref["J"][m]), rel=1e-12, abs=1e-18)
        assert frozenset(int(s) for s in out["idx"][i] if s >= 0) == ref["sel"]


def test_hisa_limits_equal_dsa():
    p, prob = _prob(81, Bt=2, T=6, L=256, H=8, d=32, offset=250, needles=8)
    idx, sc = oracle.dsa(prob, topk=24)
    # every block kept -> DSA
    allb = oracle.hisa(prob, topk=24, b=16, r=16)
    assert np.array_equal(allb["idx"], idx)
    assert np.array_equal(allb["score"], sc)
    # blocks of one token with r >= k -> the coarse stage is DSA itself
    one = oracle.hisa(prob, topk=24, b=1, r=24)
    assert np.array_equal(one["idx"], idx)


def test_hisa_rejects_short_candidate_pool():
    _, prob = _prob(82, L=64, H=4, d=8, offset=63)
    with pytest.raises(ValueError):
        oracle.hisa(prob, topk=33, b=8, r=4)


def test_block_means_closed_form():
    """K[s] = s (small integers, exact in bf16): block mean = (lo + hi - 1) / 2."""
    L, d, blk = 100, 4, 16
    K = _bits(np.repeat(np.arange(L, dtype=np.float32)[:, None], d, axis=1))[None]
    pm = oracle.pool(K, blk)
    for m in range(pm.shape[1]):
        lo, hi = m * blk, min((m + 1) * blk, L)
        assert np.all(pm[0, m] == (lo + hi - 1) / 2.0)


def test_misa_router_constant_blocks():
    """Blocks of identical keys pool to that key: E_j is then a plain mean of
    |w_j| ReLU(q_j . v_m) over blocks, checked against hand-built values."""
    H, d, B = 3, 4, 4
    v = np.array([[1, 0, 0, 0], [0, 2, 0, 0], [0, 0, -1, 0]], np.float32)
    K = np.repeat(v, B, axis=0)[None]  # 3 blocks x 4 keys
    q = np.array([[[[1, 1, 1, 0], [0, 0, -2, 0], [-1, 0, 0, 0]]]], np.float32)
    w = np.array([[[0.5, -1.0, 2.0]]], np.float32)
    out = oracle.misa(oracle.Problem(_bits(q), w, _bits(K), 11), topk=2, B=B, h=1)
    # head 0: dots with v = 1, 2, -1 -> |0.5|*(1+2+0)/3 = 0.5
    # head 1: dots 0, 0, 2 -> 1*(2)/3; head 2: dots -1, 0, 0 -> 0
    np.testing.assert_allclose(out["E"][0], [0.5, 2.0 / 3.0, 0.0], rtol=1e-15)
    assert out["heads"][0].tolist() == [1]


# -------------------------------------------------------------- generator

def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -7], np.float32)
    back = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0 + 2 ** -7]


def test_generator_is_seeded_and_plants_needles():
    a = synth.make_problem(5, Bt=2, T=1, L=256, H=8, d=128, needles=4, needle_mode="decode")
    b = synth.make_problem(5, Bt=2, T=1, L=256, H=8, d=128, needles=4, needle_mode="decode")
    assert np.array_equal(a["K"], b["K"]) and np.array_equal(a["q"], b["q"])
    assert len(a["needle_pos"]) == 8
    qf = synth.bf16_bits_to_f32(a["q"])
    for bb, s in a["needle_pos"]:
        key = synth.bf16_bits_to_f32(a["K"][bb, s])
        ratios = [np.allclose(key, synth.bf16_bits_to_f32(synth.to_bf16_bits(3 * qf[bb, 0, j])))
                  for j in range(8)]
        assert any(ratios)


def test_hisa_generator_clusters_needles():
    p = synth.make_problem(9, Bt=1, T=1, L=4096, H=4, d=128, needles=8, needle_mode="hisa",
                           b=128)
    blocks = [s // 128 for _, s in p["needle_pos"]]
    assert blocks[:4] == [blocks[0]] * 4
    assert len(set(blocks[4:])) == 4 and blocks[0] not in blocks[4:]
