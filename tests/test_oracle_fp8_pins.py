"""Pins for the oracle's FP8 key path (no GPU).

What fixes the FP8 functions, other than the functions themselves:
* the OCP E4M3 format's landmark values (1, 2, the largest finite 448, the
  smallest normal 2^-6, the smallest subnormal 2^-9, NaN at 0x7F, -0 at 0x80)
  and its structure (sign symmetry, strictly increasing magnitudes);
* rounding: every code round-trips, midpoints between neighbouring codes go
  to the even code, values beyond 448 saturate;
* quantization: the largest element of a key maps to +-448 exactly, zero keys
  stay zero, and the dequantized key is within half a code step of the key;
* the score error bound of PaperTrace section 2.3 (ReLU is 1-Lipschitz, so
  |I_fp8 - I| <= sum_j |w_j| |q_j|_2 |e_s|_2 for the key error e_s), checked
  against the bf16 oracle, and its consequence: when 2E is below the gap m
  between the k-th and (k+1)-th score, the FP8 top-k set is the bf16 one;
* a key quantized without error (values already on the FP8 grid times a
  power of two) gives exactly the bf16 oracle's scores.

The query converted to E4M3 too (dsa_fp8q) is pinned by: a pure-Python
brute force (format table built from the definition, nearest-code search,
Python-float scores) on a tiny case; query heads already on the grid with
448 as their largest element giving exactly the dsa_fp8 scores; exact 2^e
scaling of every score under q -> 2^e q; and the Lipschitz bound on the
query's quantization error against dsa_fp8.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from sparse_attention_token_dsa_amd import synth


def test_e4m3_landmark_values():
    v = oracle.fp8_decode(np.arange(256))
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x3C] == 1.5
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6 and v[0x07] == 7 * 2.0 ** -9 and v[0x01] == 2.0 ** -9
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) < 0
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    mag = v[:0x7F]
    assert np.all(np.diff(mag) > 0), "magnitudes must increase strictly over 0x00..0x7E"
    assert np.array_equal(v[0x80:0xFF], -mag)


def test_e4m3_round_trip_and_ties_to_even():
    v = oracle.fp8_decode(np.arange(0x7F))
    codes = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(oracle.fp8_encode(v.astype(np.float32)), codes)
    assert np.array_equal(oracle.fp8_encode(-v[1:].astype(np.float32)), codes[1:] | 0x80)
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (v[:-1] + v[1:]) / 2), "midpoints exact in fp32"
    got = oracle.fp8_encode(mid)
    want = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(got, want)
    # just off the midpoint: the nearer code
    above = np.nextafter(mid, np.float32(np.inf))
    below = np.nextafter(mid, np.float32(-np.inf))
    assert np.array_equal(oracle.fp8_encode(above), codes[1:])
    assert np.array_equal(oracle.fp8_encode(below), codes[:-1])


def test_e4m3_saturates():
    x = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, -500.0], np.float32)
    assert oracle.fp8_encode(x).tolist() == [0x7E] * 6 + [0xFE]


def test_quantize_keys_maps_the_largest_element_to_448():
    p = synth.make_problem(81, Bt=2, T=1, L=40, H=4)
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    Kf = synth.bf16_bits_to_f32(p["K"]).astype(np.float64)
    amax = np.abs(Kf).max(-1)
    assert np.array_equal(scales, (amax.astype(np.float32) / np.float32(448.0)))
    vals = oracle.fp8_decode(codes)
    top = np.abs(vals).max(-1)
    assert np.all(top == 448.0)
    deq = vals * scales[..., None].astype(np.float64)
    # within half a code step: relative 2^-4 for normals, 2^-10 * scale below
    err = np.abs(deq - Kf)
    bound = np.maximum(np.abs(Kf) * 2.0 ** -4, scales[..., None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))


def test_quantize_zero_key():
    K = np.zeros((1, 3, 128), np.uint16)
    codes, scales = oracle.quantize_keys_fp8(K)
    assert np.all(codes == 0) and np.all(scales == 1.0)


def _fp8_vs_bf16(seed, T, L, H, d, k):
    p = synth.make_problem(seed, Bt=1, T=T, L=L, H=H, d=d, offset=L - T)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    i8, s8, r8 = oracle.dsa_fp8(prob, codes, scales, k, want_rowscore=True)
    ib, sb, rb = oracle.dsa(prob, k, want_rowscore=True)
    return p, prob, codes, scales, (i8, r8), (ib, rb)


@pytest.mark.parametrize("seed", [82, 83, 84])
def test_fp8_score_error_bound(seed):
    T, L, H, d, k = 3, 300, 8, 128, 20
    p, prob, codes, scales, (i8, r8), (ib, rb) = _fp8_vs_bf16(seed, T, L, H, d, k)
    q = synth.bf16_bits_to_f32(p["q"][0]).astype(np.float64)            # [T, H, d]
    w = p["w"][0].astype(np.float64)                                     # [T, H]
    Kf = synth.bf16_bits_to_f32(p["K"][0]).astype(np.float64)           # [L, d]
    deq = oracle.fp8_decode(codes[0]) * scales[0][:, None].astype(np.float64)
    e = np.linalg.norm(deq - Kf, axis=1)                                 # |e_s|_2
    qn = np.linalg.norm(q, axis=2)                                       # |q_j|_2
    for i in range(T):
        t = p["offset"] + i
        E_s = (np.abs(w[i]) * qn[i]).sum() * e[: t + 1]
        diff = np.abs(r8[i, : t + 1] - rb[i, : t + 1])
        assert np.all(diff <= E_s * (1 + 1e-9) + 1e-12), "error bound violated"
        assert np.any(diff > 0), "quantization should perturb some score"


def test_fp8_keeps_the_set_when_the_margin_allows():
    # When every winner's score minus its error bound E_s stays above every
    # other position's score plus its bound (2E < m in the uniform form), the
    # FP8 top-k set equals the bf16 one.  Each row gets k strong keys (3 q
    # summed over its heads, positive w) well above the random rest, so the
    # condition holds; it is asserted before the sets are compared.
    rng = np.random.default_rng(88)
    T, L, H, d, k = 4, 300, 4, 128, 6
    p = synth.make_problem(88, Bt=1, T=T, L=L, H=H, d=d, offset=L - T)
    p["w"][:] = np.abs(p["w"]) + np.float32(0.01)
    q = synth.bf16_bits_to_f32(p["q"][0]).astype(np.float64)
    K = synth.bf16_bits_to_f32(p["K"][0]).copy()
    allpos = rng.choice(L - T, size=T * k, replace=False)  # distinct across rows
    for i in range(T):
        pos = allpos[i * k:(i + 1) * k]
        K[pos] = (3.0 * q[i].sum(0)).astype(np.float32)[None, :] * (1 + 0.01 * np.arange(k))[:, None]
    p["K"][0] = synth.to_bf16_bits(K)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    i8, s8 = oracle.dsa_fp8(prob, codes, scales, k)
    ib, sb, rb = oracle.dsa(prob, k, want_rowscore=True)
    Kf = synth.bf16_bits_to_f32(p["K"][0]).astype(np.float64)
    deq = oracle.fp8_decode(codes[0]) * scales[0][:, None].astype(np.float64)
    e = np.linalg.norm(deq - Kf, axis=1)
    w = p["w"][0].astype(np.float64)
    for i in range(T):
        t = p["offset"] + i
        # per-position form of the argument: winners drop by at most E_s,
        # the rest rise by at most E_s
        E_s = e[: t + 1] * (np.abs(w[i]) * np.linalg.norm(q[i], axis=1)).sum()
        inside = np.zeros(t + 1, bool)
        inside[ib[i]] = True
        lo_in = (rb[i, : t + 1] - E_s)[inside].min()
        hi_out = (rb[i, : t + 1] + E_s)[~inside].max()
        assert lo_in > hi_out, "the construction must satisfy the margin condition"
        assert set(i8[i].tolist()) == set(ib[i].tolist())


def test_fp8_exact_keys_give_the_bf16_scores():
    # Keys whose values are E4M3 values times a common power of two, with one
    # element at 448 * 2^e: the scale is that power of two exactly, every
    # element quantizes without error, and the FP8 scores equal the bf16 ones.
    rng = np.random.default_rng(86)
    Bt, T, L, H, d, k = 1, 2, 50, 4, 128, 7
    v = oracle.fp8_decode(np.arange(0x7F))
    K = np.empty((Bt, L, d), np.float32)
    for s in range(L):
        e = int(rng.integers(-6, 4))
        row = rng.choice(v, size=d) * rng.choice([-1.0, 1.0], size=d)
        row[int(rng.integers(0, d))] = 448.0
        K[0, s] = (row * 2.0 ** e).astype(np.float32)
    Kb = synth.to_bf16_bits(K)
    assert np.array_equal(synth.bf16_bits_to_f32(Kb), K), "test keys must be bf16-exact"
    p = synth.make_problem(87, Bt=Bt, T=T, L=L, H=H, d=d, offset=L - T)
    prob = oracle.Problem(p["q"], p["w"], Kb, p["offset"])
    codes, scales = oracle.quantize_keys_fp8(Kb)
    i8, s8 = oracle.dsa_fp8(prob, codes, scales, k)
    ib, sb = oracle.dsa(prob, k)
    assert np.array_equal(i8, ib) and np.array_equal(s8, sb)


# ---------------------------------------------------------------- FP8 query
# The query converted to E4M3 as well (dsa_fp8q): each head vector by the
# key-cache rule; the score is the indexer formula on the dequantized query
# and key.

def _e4m3_values():
    """The 127 non-negative finite E4M3 values, code order, from the format's
    definition (bias 7, 3 mantissa bits, subnormals below 2^-6)."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(2.0 ** (e - 7) * (1 + m / 8) if e else 2.0 ** -6 * m / 8)
    return out


def _encode_py(x, vals):
    """Nearest E4M3 code of x (ties to the even code, saturating), by search."""
    s = 0x80 if x < 0 or (x == 0 and math.copysign(1.0, x) < 0) else 0
    a = min(abs(x), 448.0)
    best = min(range(len(vals)), key=lambda c: (abs(vals[c] - a), c & 1))
    return s | best, (-1 if s else 1) * vals[best]


def test_fp8q_brute_force_tiny():
    # Pure-Python quantization of q and k (fp32 divisions by fp32 scales) and
    # the score in Python floats, against the oracle.
    vals = _e4m3_values()
    T, L, H, d, k = 2, 12, 3, 128, 4
    p = synth.make_problem(91, Bt=1, T=T, L=L, H=H, d=d, offset=L - T)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    idx, sc, rs = oracle.dsa_fp8q(prob, codes, scales, k, want_rowscore=True)
    f32 = np.float32

    def quant(vec):
        m = max(abs(float(v)) for v in vec)
        a = f32(f32(m) / f32(448.0)) if m > 0 else f32(1.0)
        return a, [_encode_py(float(f32(v) / a), vals)[1] for v in vec]

    K = synth.bf16_bits_to_f32(p["K"][0])
    keys = [quant(K[s]) for s in range(L)]
    q = synth.bf16_bits_to_f32(p["q"][0])
    for i in range(T):
        t = p["offset"] + i
        heads = [quant(q[i, j]) for j in range(H)]
        # w_j * b_j as an exact double product (no rounding to fp32)
        wf = [float(p["w"][0, i, j]) * float(heads[j][0]) for j in range(H)]
        for s in range(t + 1):
            a, kv = keys[s]
            tot = 0.0
            for j in range(H):
                dot = sum(x * y for x, y in zip(heads[j][1], kv))
                tot += wf[j] * max(dot, 0.0)
            ref = float(a) * tot
            assert abs(rs[i, s] - ref) <= 1e-12 * max(1.0, abs(ref)), (i, s, rs[i, s], ref)
        order = sorted(range(t + 1), key=lambda s: (-rs[i, s], s))[:k]
        assert idx[i].tolist() == order


def test_fp8q_exact_queries_give_the_fp8_scores():
    # Query heads whose values are E4M3 values with one element at 448: the
    # scale is 1, nothing is lost, and the scores are those of dsa_fp8.
    rng = np.random.default_rng(92)
    Bt, T, L, H, d, k = 1, 3, 60, 5, 128, 8
    v = oracle.fp8_decode(np.arange(0x7F))
    p = synth.make_problem(92, Bt=Bt, T=T, L=L, H=H, d=d, offset=L - T)
    q = np.empty((Bt, T, H, d), np.float32)
    for i in range(T):
        for j in range(H):
            row = rng.choice(v, size=d) * rng.choice([-1.0, 1.0], size=d)
            row[int(rng.integers(0, d))] = 448.0
            q[0, i, j] = row
    qb = synth.to_bf16_bits(q)
    prob = oracle.Problem(qb, p["w"], p["K"], p["offset"])
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    iq, sq, rq = oracle.dsa_fp8q(prob, codes, scales, k, want_rowscore=True)
    i8, s8, r8 = oracle.dsa_fp8(prob, codes, scales, k, want_rowscore=True)
    assert np.array_equal(iq, i8) and np.array_equal(sq, s8)


@pytest.mark.parametrize("e", [-3, 2])
def test_fp8q_power_of_two_query_scaling(e):
    # q -> 2^e q leaves every code alone and scales every b by 2^e exactly, so
    # every score scales by 2^e exactly.
    T, L, H, d, k = 2, 90, 6, 128, 9
    p = synth.make_problem(93, Bt=1, T=T, L=L, H=H, d=d, offset=L - T)
    q2 = synth.to_bf16_bits(synth.bf16_bits_to_f32(p["q"]) * np.float32(2.0 ** e))
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    a = oracle.dsa_fp8q(oracle.Problem(p["q"], p["w"], p["K"], p["offset"]), codes, scales, k,
                        want_rowscore=True)
    b = oracle.dsa_fp8q(oracle.Problem(q2, p["w"], p["K"], p["offset"]), codes, scales, k,
                        want_rowscore=True)
    assert np.array_equal(a[0], b[0])
    for i in range(T):
        t = p["offset"] + i
        assert np.array_equal(a[2][i, : t + 1] * 2.0 ** e, b[2][i, : t + 1])


@pytest.mark.parametrize("seed", [94, 95])
def test_fp8q_error_bound_against_fp8(seed):
    # ReLU is 1-Lipschitz: against the bf16 query on the same FP8 keys, a
    # score moves by at most a_s sum_j |w_j| |b_j qhat_j - q_j|_2 |khat_s|_2
    # (plus fp64 rounding).
    T, L, H, d, k = 3, 200, 8, 128, 16
    p = synth.make_problem(seed, Bt=1, T=T, L=L, H=H, d=d, offset=L - T)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    _, _, rq = oracle.dsa_fp8q(prob, codes, scales, k, want_rowscore=True)
    _, _, r8 = oracle.dsa_fp8(prob, codes, scales, k, want_rowscore=True)
    qc, qs = oracle.quantize_keys_fp8(p["q"])
    q = synth.bf16_bits_to_f32(p["q"][0]).astype(np.float64)
    eq = np.linalg.norm(oracle.fp8_decode(qc[0]) * qs[0][..., None] - q, axis=2)  # [T, H]
    qhat = oracle.fp8_decode(qc[0]) * qs[0][..., None]
    khat = oracle.fp8_decode(codes[0])                                            # [L, d]
    kn = np.linalg.norm(khat, axis=1)
    a = scales[0].astype(np.float64)
    w = np.abs(p["w"][0].astype(np.float64))
    for i in range(T):
        t = p["offset"] + i
        dots = np.abs(qhat[i] @ khat[: t + 1].T)                                 # [H, t+1]
        bound = a[: t + 1] * ((w[i] * eq[i])[:, None] * kn[None, : t + 1]
                              + 2.0 ** -50 * w[i][:, None] * dots).sum(0)
        diff = np.abs(rq[i, : t + 1] - r8[i, : t + 1])
        assert np.all(diff <= bound * (1 + 1e-9) + 1e-15)
        assert np.any(diff > 0), "quantizing q should perturb some score"


# ------------------------------------------------- FP8 keys in MISA and HISA
# oracle.Problem with codes/scales: DSA, MISA and HISA read the dequantized
# keys.  Pinned by the reductions that hold for any keys (h = H is DSA; r = all
# blocks is DSA; the generic DSA equals dsa_fp8) and by keys already on the
# E4M3 grid, where the FP8 problem is the bf16 problem.

def _fp8_problem(seed, T, L, H, d=128):
    p = synth.make_problem(seed, Bt=1, T=T, L=L, H=H, d=d, offset=L - T)
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    prob8 = oracle.Problem(p["q"], p["w"], None, p["offset"], codes=codes, scales=scales)
    return p, codes, scales, prob8


def test_fp8_problem_dsa_equals_dsa_fp8():
    T, L, H, k = 3, 400, 8, 25
    p, codes, scales, prob8 = _fp8_problem(101, T, L, H)
    i1, s1, r1 = oracle.dsa(prob8, k, want_rowscore=True)
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    i2, s2, r2 = oracle.dsa_fp8(prob, codes, scales, k, want_rowscore=True)
    for i in range(T):
        n = p["offset"] + i + 1
        assert np.allclose(r1[i, :n], r2[i, :n], rtol=1e-12, atol=1e-300)
    assert np.array_equal(i1, i2)


def test_fp8_misa_all_heads_and_hisa_all_blocks_are_dsa():
    T, L, H, k = 2, 700, 8, 30
    p, codes, scales, prob8 = _fp8_problem(102, T, L, H)
    di, ds = oracle.dsa(prob8, k)
    m = oracle.misa(prob8, k, 128, H, 0)
    assert np.array_equal(m["idx"], di)
    md = oracle.misa(prob8, k, 128, 2, kprime=L)      # k' >= t+1: the full-head DSA
    assert np.array_equal(md["idx"], di)
    h = oracle.hisa(prob8, k, 64, (L + 63) // 64)
    assert np.array_equal(h["idx"], di)


def test_fp8_misa_hisa_on_grid_keys_equal_bf16():
    # Keys already on the E4M3 grid with 448 * 2^e as their largest element:
    # the FP8 cache holds them exactly, so every stage sees the bf16 keys.
    rng = np.random.default_rng(103)
    T, L, H, k = 2, 300, 8, 20
    v = oracle.fp8_decode(np.arange(0x7F))
    K = np.empty((1, L, 128), np.float32)
    for s in range(L):
        e = int(rng.integers(-8, -3))
        row = rng.choice(v, size=128) * rng.choice([-1.0, 1.0], size=128)
        row[int(rng.integers(0, 128))] = 448.0
        K[0, s] = row * 2.0 ** e
    Kb = synth.to_bf16_bits(K)
    p = synth.make_problem(103, Bt=1, T=T, L=L, H=H, offset=L - T)
    codes, scales = oracle.quantize_keys_fp8(Kb)
    prob = oracle.Problem(p["q"], p["w"], Kb, p["offset"])
    prob8 = oracle.Problem(p["q"], p["w"], None, p["offset"], codes=codes, scales=scales)
    for kp in (0, 64):
        a, b = oracle.misa(prob, k, 64, 3, kp), oracle.misa(prob8, k, 64, 3, kp)
        assert np.array_equal(a["heads"], b["heads"]) and np.array_equal(a["idx"], b["idx"])
        assert np.array_equal(a["score"], b["score"])
    a, b = oracle.hisa(prob, k, 32, 4), oracle.hisa(prob8, k, 32, 4)
    assert np.array_equal(a["blocks"], b["blocks"]) and np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["score"], b["score"])
