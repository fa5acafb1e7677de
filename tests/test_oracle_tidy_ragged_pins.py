"""Pins for the oracle's index tidy-up and ragged-batch DSA (no GPU).

Tidy-up (PaperTrace 2.2.2, sections 2.2 / 2.3): a hand-worked row, loops
written out position by position for the page mapping and the counts, and
invariances (input order, duplicates, -1 entries).  Ragged batches: every
sequence equals the plain DSA problem on its own prefix, and a batch of equal
lengths equals the padded DSA call.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from sparse_attention_token_dsa_amd import synth


def test_tidy_hand_example():
    # page size 64; positions 5, 3, 64, 65, 3 (duplicate), 200 and two empties
    idx = np.array([[5, 3, 64, 65, 3, 200, -1, -1]])
    slots, stats = oracle.tidy(idx, 1, page_size=64)
    assert slots[0].tolist() == [3, 5, 64, 65, 200, -1, -1, -1]
    # pages {0, 1, 3}; runs [3], [5], [64, 65], [200]
    assert stats[0].tolist() == [5, 3, 4]
    # a table that maps logical pages 0, 1, 3 to physical 7, 2, 0 (page 2 unmapped)
    table = np.array([[7, 2, -1, 0]])
    slots, stats = oracle.tidy(idx, 1, block_table=table, page_size=64)
    # 5 -> 453, 3 -> 451, 64 -> 128, 65 -> 129, 200 -> 8
    assert slots[0].tolist() == [8, 128, 129, 451, 453, -1, -1, -1]
    assert stats[0].tolist() == [5, 3, 4]
    # a pool of 200 slots: 451 and 453 are dropped
    slots, stats = oracle.tidy(idx, 1, block_table=table, page_size=64, max_slots=200)
    assert slots[0].tolist() == [8, 128, 129, -1, -1, -1, -1, -1]
    assert stats[0].tolist() == [3, 2, 2]


def test_tidy_against_loops_and_invariances():
    rng = np.random.default_rng(5)
    T, k, page, npages = 2, 50, 16, 40
    idx = rng.integers(-1, page * npages + 20, size=(3 * T, k))    # some past the table
    table = rng.permutation(200)[: 3 * npages].reshape(3, npages)
    table[rng.random(table.shape) < 0.1] = -1
    slots, stats = oracle.tidy(idx, T, block_table=table, page_size=page)
    for row in range(3 * T):
        b = row // T
        seen = set()
        for s in idx[row]:
            if s < 0 or s // page >= npages or table[b, s // page] < 0:
                continue
            seen.add(int(table[b, s // page]) * page + int(s % page))
        want = sorted(seen)
        assert slots[row][: len(want)].tolist() == want and np.all(slots[row][len(want):] == -1)
        pages = len({v // page for v in want})
        runs = sum(1 for i, v in enumerate(want) if i == 0 or want[i - 1] + 1 != v)
        assert stats[row].tolist() == [len(want), pages, runs]
    shuffled = np.array([rng.permutation(r) for r in idx])
    s2, st2 = oracle.tidy(shuffled, T, block_table=table, page_size=page)
    assert np.array_equal(s2, slots) and np.array_equal(st2, stats)


def test_ragged_equals_per_sequence_and_padded():
    p = synth.make_problem(71, Bt=3, T=2, L=900, H=16, offset=898)
    lens = np.array([900, 437, 2], np.int32)
    idx, sc, rs = oracle.dsa_ragged(p["q"], p["w"], p["K"], lens, 40)
    for b, n in enumerate(lens):
        pb = oracle.Problem(p["q"][b:b + 1], p["w"][b:b + 1], p["K"][b:b + 1, :n], n - 2)
        i, s = oracle.dsa(pb, 40)
        assert np.array_equal(idx[2 * b:2 * b + 2], i) and np.array_equal(sc[2 * b:2 * b + 2], s)
        assert np.all(idx[2 * b:2 * b + 2] < n)
    # all lengths equal to the capacity: the ordinary call
    full = np.full(3, 900, np.int32)
    i2, s2, _ = oracle.dsa_ragged(p["q"], p["w"], p["K"], full, 40)
    i3, s3 = oracle.dsa(oracle.Problem(p["q"], p["w"], p["K"], 898), 40)
    assert np.array_equal(i2, i3) and np.array_equal(s2, s3)


def test_ragged_brute_force_with_needles_past_each_length():
    # Exact rational brute force (tests/brute.py), written from the reading
    # of seq_lens alone: sequence b's history is keys 0 .. n_b - 1 and its row
    # i sits at t = n_b - T + i.  Keys at and after n_b are planted to beat
    # every legal key of every row, so reading past a sequence's length (or
    # placing the rows at the capacity) would select them.
    import brute
    Bt, T, L, H, d, k = 3, 2, 11, 3, 8, 3
    p = synth.make_problem(72, Bt=Bt, T=T, L=L, H=H, d=d, offset=L - T)
    w = np.abs(p["w"]).astype(np.float32)
    K = p["K"].copy()
    lens = np.array([11, 7, 3], np.int32)
    qf = synth.bf16_bits_to_f32(p["q"])
    for b in range(Bt):
        for s in range(lens[b], L):
            K[b, s] = synth.to_bf16_bits(8.0 * (qf[b, 0, 0] + qf[b, 1, 0]))
    idx, sc, rs = oracle.dsa_ragged(p["q"], w, K, lens, k)
    for b in range(Bt):
        n = int(lens[b])
        qe, we, ke = brute.exact_vectors(p["q"][b], w[b], K[b])
        for i in range(T):
            row, t = b * T + i, n - T + i
            sel, scores = brute.dsa_row(qe, we, ke, i, t, k)
            got = [int(s) for s in idx[row] if s >= 0]
            assert len(got) == min(k, t + 1)
            assert set(got) == set(sel), (b, i, got, sorted(sel))
            assert all(s <= t for s in got)
            for u, s in enumerate(idx[row]):
                if s >= 0:
                    assert sc[row, u] == pytest.approx(float(scores[int(s)]), rel=1e-12, abs=1e-300)
            assert np.all(np.isnan(rs[row, t + 1:]))
            # the planted keys would have won: their exact score beats the kept ones
            if n < L:
                planted = brute.score(qe[i], we[i], ke[n])
                assert all(planted > scores[s] for s in got)
