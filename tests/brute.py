"""Exact brute force for tiny selector problems (test pin for the oracle).

Independent of the C oracle in both arithmetic and algorithm:

* every value is an exact rational (``fractions.Fraction``) built from the
  bf16 / fp32 bit patterns, so dot products, ReLU, head sums and block means
  carry no rounding at all;
* selection does not sort: it enumerates every subset of the required size
  and keeps the one with the largest total score, breaking equal totals by the
  smallest sum of indices.  For distinct scores that is the unique top-k; with
  ties at the cutoff it is the set that takes the lowest tied indices, which is
  the tie reading the oracle uses.

Only usable for a handful of candidates (the enumeration is combinatorial).
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np


def _bf16(bits) -> Fraction:
    u = np.array([bits], dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return Fraction(float(u.view(np.float32)[0]))


def _f32(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def exact_vectors(q, w, K):
    """q [T,H,d] bits, w [T,H], K [L,d] bits (one sequence) -> Fraction lists."""
    T, H, d = q.shape
    L = K.shape[0]
    qe = [[[_bf16(q[i, j, x]) for x in range(d)] for j in range(H)] for i in range(T)]
    we = [[_f32(w[i, j]) for j in range(H)] for i in range(T)]
    ke = [[_bf16(K[s, x]) for x in range(d)] for s in range(L)]
    return qe, we, ke


def dot(a, b):
    return sum((x * y for x, y in zip(a, b)), Fraction(0))


def relu(z):
    return z if z > 0 else Fraction(0)


def score(qrow, wrow, key, heads=None):
    hs = range(len(qrow)) if heads is None else heads
    return sum((wrow[j] * relu(dot(qrow[j], key)) for j in hs), Fraction(0))


def mean(vectors):
    n = len(vectors)
    return [sum((v[x] for v in vectors), Fraction(0)) / n for x in range(len(vectors[0]))]


def best_subset(values, items, size):
    """Subset of `items` (ids) of the given size maximising the total of
    values[id]; equal totals -> smallest id sum.  Returns a frozenset."""
    size = min(size, len(items))
    best = None
    for comb in itertools.combinations(items, size):
        key = (sum((values[i] for i in comb), Fraction(0)), -sum(comb))
        if best is None or key > best[0]:
            best = (key, comb)
    return frozenset(best[1])


def dsa_row(qe, we, ke, i, t, k):
    scores = {s: score(qe[i], we[i], ke[s]) for s in range(t + 1)}
    return best_subset(scores, list(range(t + 1)), k), scores


def misa_row(qe, we, ke, i, t, k, B, h, kprime=0):
    H = len(qe[i])
    Mt = t // B + 1
    pooled = [mean(ke[m * B:min((m + 1) * B, t + 1)]) for m in range(Mt)]
    E = {}
    for j in range(H):
        tot = Fraction(0)
        for m in range(Mt):
            tot += abs(we[i][j] * relu(dot(qe[i][j], pooled[m])))
        E[j] = tot / Mt
    heads = best_subset(E, list(range(H)), h)
    hat = {s: score(qe[i], we[i], ke[s], sorted(heads)) for s in range(t + 1)}
    if kprime == 0:
        return dict(heads=heads, E=E, sel=best_subset(hat, list(range(t + 1)), k), hat=hat)
    pool = best_subset(hat, list(range(t + 1)), kprime)
    full = {s: score(qe[i], we[i], ke[s]) for s in pool}
    return dict(heads=heads, E=E, pool=pool, sel=best_subset(full, sorted(pool), k),
                hat=hat, full=full)


def hisa_row(qe, we, ke, i, t, k, b, r):
    nb = t // b + 1
    J = {}
    for m in range(nb):
        rep = mean(ke[m * b:min((m + 1) * b, t + 1)])
        J[m] = score(qe[i], we[i], rep)
    blocks = best_subset(J, list(range(nb)), r)
    cand = [s for m in sorted(blocks) for s in range(m * b, min((m + 1) * b, t + 1))]
    full = {s: score(qe[i], we[i], ke[s]) for s in cand}
    return dict(blocks=blocks, J=J, sel=best_subset(full, cand, k), full=full)


def lisa_row(qe, we, ke, i, t, k):
    """LISA: the per-head linear sum sum_j w_j (q_j . k), exact."""
    H = len(qe[i])
    lin = {s: sum((we[i][j] * dot(qe[i][j], ke[s]) for j in range(H)), Fraction(0))
           for s in range(t + 1)}
    return best_subset(lin, list(range(t + 1)), k), lin


def box_max_negdot(q, lo, hi):
    """max of -(q . k) over the box lo <= k <= hi, coordinate by coordinate:
    -q_d k_d is largest at k_d = lo_d when q_d > 0 and at hi_d when q_d < 0."""
    tot = Fraction(0)
    for qd, a, b in zip(q, lo, hi):
        if qd > 0:
            tot += -qd * a
        elif qd < 0:
            tot += -qd * b
    return tot


def resmisa_row(qe, we, ke, i, t, k, block, r):
    """ResMiSA, exact: route by |w_h| * max over legal blocks of the box
    maximum of -(q_h . k); score the routed heads through ReLU and the other
    heads linearly (sum_{h not in A} w_h z_h + sum_{h in A} w_h ReLU(z_h),
    which equals l + sum_{h in A} w_h ReLU(-z_h))."""
    H = len(qe[i])
    nb = t // block + 1
    S = {}
    for j in range(H):
        best = Fraction(0)
        for m in range(nb):
            keys = ke[m * block:min((m + 1) * block, t + 1)]
            lo = [min(v[x] for v in keys) for x in range(len(keys[0]))]
            hi = [max(v[x] for v in keys) for x in range(len(keys[0]))]
            best = max(best, abs(we[i][j]) * relu(box_max_negdot(qe[i][j], lo, hi)))
        S[j] = best
    heads = best_subset(S, list(range(H)), r) if r else frozenset()
    R = {}
    for s in range(t + 1):
        tot = Fraction(0)
        for j in range(H):
            z = dot(qe[i][j], ke[s])
            tot += we[i][j] * (relu(z) if j in heads else z)
        R[s] = tot
    return dict(heads=heads, S=S, sel=best_subset(R, list(range(t + 1)), k), R=R)


def misa_hisa_row(qe, we, ke, i, t, k, B, h, b, r):
    """MISA x HISA, exact: the MISA router's h heads score the b-blocks, the r
    best blocks' legal tokens are scored with every head."""
    routed = misa_row(qe, we, ke, i, t, 1, B, h)
    heads = sorted(routed["heads"])
    nb = t // b + 1
    J = {m: score(qe[i], we[i], mean(ke[m * b:min((m + 1) * b, t + 1)]), heads)
         for m in range(nb)}
    blocks = best_subset(J, list(range(nb)), r)
    cand = [s for m in sorted(blocks) for s in range(m * b, min((m + 1) * b, t + 1))]
    full = {s: score(qe[i], we[i], ke[s]) for s in cand}
    return dict(heads=routed["heads"], E=routed["E"], blocks=blocks, J=J,
                sel=best_subset(full, cand, k), full=full)
