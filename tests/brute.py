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
