"""Pins for the oracle's MISA x HISA composition (no GPU).

The composition ([MISA] "core method": head routing and HISA's token
hierarchy are orthogonal and can run in series; PaperTrace / the indexer
survey pages: MISA combined with HISA as routing plus two stages): the MISA
router picks h heads from pooled blocks of B, HISA's block scores sum only
those heads, and the legal tokens of the r best blocks are rescored with every
head before the token top-k.

Pinned by: the limits h = H (HISA exactly) and r >= #blocks (DSA exactly);
exact rational brute force of the whole chain on tiny causal inputs; the
routed block scores against a library evaluation of sum_{j in heads}
w_j ReLU(q_j . mean(block)); staged overrides reproduce the unstaged result.
"""
from __future__ import annotations

import numpy as np
import pytest

import brute
import oracle
from sparse_attention_token_dsa_amd import synth


def _prob(p):
    return oracle.Problem(p["q"], p["w"], p["K"], p["offset"])


@pytest.mark.parametrize("seed", [51, 52])
def test_all_heads_is_hisa(seed):
    p = synth.make_problem(seed, Bt=2, T=2, L=900, H=8, offset=898)
    prob = _prob(p)
    a = oracle.misa_hisa(prob, 20, 256, 8, 64, 4)
    b = oracle.hisa(prob, 20, 64, 4)
    assert np.array_equal(a["heads"], np.tile(np.arange(8), (4, 1)))
    for key in ("idx", "score", "blocks"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(np.isnan(a["J"]), np.isnan(b["J"]))
    assert np.array_equal(a["J"][~np.isnan(a["J"])], b["J"][~np.isnan(b["J"])])


def test_all_blocks_is_dsa():
    p = synth.make_problem(53, Bt=1, T=3, L=500, H=8, offset=497)
    prob = _prob(p)
    a = oracle.misa_hisa(prob, 30, 128, 2, 32, 16)   # 16 blocks of 32 cover all 500 keys
    di, ds = oracle.dsa(prob, 30)
    assert np.array_equal(a["idx"], di) and np.array_equal(a["score"], ds)


@pytest.mark.parametrize("seed,T,L,H,B,h,b,r,k", [
    (61, 2, 9, 4, 4, 2, 3, 2, 3),
    (62, 3, 10, 3, 5, 1, 2, 3, 4),
    (63, 1, 8, 5, 8, 3, 4, 1, 2),
])
def test_brute_force(seed, T, L, H, B, h, b, r, k):
    d = 4
    p = synth.make_problem(seed, Bt=1, T=T, L=L, H=H, d=d, offset=L - T)
    out = oracle.misa_hisa(_prob(p), k, B, h, b, r)
    qe, we, ke = brute.exact_vectors(p["q"][0], p["w"][0], p["K"][0])
    for i in range(T):
        t = p["offset"] + i
        ref = brute.misa_hisa_row(qe, we, ke, i, t, k, B, h, b, r)
        assert set(out["heads"][i].tolist()) == set(ref["heads"])
        nb = t // b + 1
        assert np.allclose(out["J"][i, :nb], [float(ref["J"][m]) for m in range(nb)],
                           rtol=1e-12, atol=1e-15)
        assert set(out["blocks"][i][out["blocks"][i] >= 0].tolist()) == set(ref["blocks"])
        assert set(out["idx"][i][out["idx"][i] >= 0].tolist()) == set(ref["sel"])


def test_routed_block_scores_by_library():
    p = synth.make_problem(64, Bt=1, T=2, L=700, H=16, offset=698)
    prob = _prob(p)
    b = 50
    out = oracle.misa_hisa(prob, 10, 128, 4, b, 6)
    q = synth.bf16_bits_to_f32(p["q"][0]).astype(np.float64)
    K = synth.bf16_bits_to_f32(p["K"][0]).astype(np.float64)
    w = p["w"][0].astype(np.float64)
    for i in range(2):
        t = p["offset"] + i
        nb = t // b + 1
        reps = np.stack([K[m * b:min((m + 1) * b, t + 1)].mean(0) for m in range(nb)])
        hs = out["heads"][i]
        J = (w[i, hs][:, None] * np.maximum(q[i, hs] @ reps.T, 0)).sum(0)
        assert np.allclose(out["J"][i, :nb], J, rtol=1e-12, atol=1e-14 * np.abs(J).max())


def test_staged_overrides_reproduce_the_chain():
    p = synth.make_problem(65, Bt=1, T=4, L=1200, H=16, offset=1196)
    prob = _prob(p)
    a = oracle.misa_hisa(prob, 40, 256, 4, 64, 8)
    b = oracle.misa_hisa(prob, 40, 256, 4, 64, 8, override_heads=a["heads"],
                         override_blocks=a["blocks"])
    for key in ("idx", "score", "blocks"):
        assert np.array_equal(a[key], b[key])
