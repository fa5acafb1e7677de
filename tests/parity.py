"""Parity rule between the HIP path and the CPU oracle, plus GPU run helpers.

Rule per query row (tolerance tol = 2e-3 * max |oracle score| over the row's
candidates):
* the GPU row holds exactly min(k, #candidates) distinct indices, all legal
  (0 <= s <= t), padded with -1 / -inf;
* every returned score is within tol of the oracle's score of that index;
* the GPU set equals the oracle set, or else every GPU index has oracle score
  >= S_k - tol (S_k = the oracle's k-th score) and every oracle index with
  score > S_k + tol is in the GPU set (near-tie exchanges only).
Discrete intermediate choices (MISA heads, the MISA-dagger k' pool, HISA
blocks) are checked with the same near-tie rule on their own statistic, then
the oracle is re-run with the GPU's choice ("override") for the next stage.
"""
from __future__ import annotations

import numpy as np

import oracle
from sparse_attention_token_dsa_amd import synth

TOL_REL = 2e-3


# ------------------------------------------------------------------ rule

def check_set(gidx, gsc, ref_idx, ref_sc, score_of, ncand, k, tol, t=None, cand_set=None,
              what="row"):
    """Check one GPU top-k row.  score_of(indices) -> oracle scores (float64).
    Returns the number of near-tie exchanges."""
    gidx = np.asarray(gidx)
    m = min(k, ncand)
    valid = gidx >= 0
    sel = gidx[valid]
    assert len(sel) == m, "%s: %d indices, expected %d" % (what, len(sel), m)
    assert len(np.unique(sel)) == m, "%s: duplicate indices" % what
    if gsc is not None:
        gsc = np.asarray(gsc)
        assert np.all(np.isneginf(gsc[~valid])), "%s: padding scores not -inf" % what
    if m == 0:
        return 0
    if t is not None:
        assert sel.min() >= 0 and sel.max() <= t, "%s: index outside [0, %d]" % (what, t)
    if cand_set is not None:
        extra = set(sel.tolist()) - cand_set
        assert not extra, "%s: indices outside the candidate set: %s" % (what, sorted(extra)[:8])
    osc = np.asarray(score_of(sel), dtype=np.float64)
    if gsc is not None:
        err = np.abs(gsc[valid].astype(np.float64) - osc)
        assert np.all(err <= tol), "%s: score error %.3g > tol %.3g" % (what, err.max(), tol)
    ref = np.asarray(ref_idx)[:m]
    rsc = np.asarray(ref_sc)[:m]
    assert np.all(ref >= 0)
    gs, rs = set(sel.tolist()), set(ref.tolist())
    if gs == rs:
        return 0
    s_k = rsc[-1]
    low = osc < s_k - tol
    assert not np.any(low), "%s: GPU index %s scores %.6g below S_k - tol = %.6g" % (
        what, sel[low][:4], osc[low].min(), s_k - tol)
    must = set(ref[rsc > s_k + tol].tolist())
    missing = must - gs
    assert not missing, "%s: clearly-in oracle indices missing: %s" % (what, sorted(missing)[:8])
    return len(rs - gs)


def check_choice(chosen, stat, n_legal, h, what):
    """Near-tie rule for a discrete choice of h items ranked by stat (desc)."""
    stat = np.asarray(stat, np.float64)[:n_legal]
    chosen = np.asarray(chosen)
    chosen = chosen[chosen >= 0]
    m = min(h, n_legal)
    assert len(chosen) == m and len(np.unique(chosen)) == m, "%s: bad choice %s" % (what, chosen)
    assert chosen.max() < n_legal
    tol = TOL_REL * np.max(np.abs(stat)) if stat.size else 0.0
    order = np.lexsort((np.arange(n_legal), -stat))
    kth = stat[order[m - 1]]
    assert np.all(stat[chosen] >= kth - tol), "%s: chosen item far below the cutoff" % what
    must = set(np.nonzero(stat > kth + tol)[0].tolist())
    assert must <= set(chosen.tolist()), "%s: clearly-in items missing" % what


# ------------------------------------------------------------ GPU helpers

def to_device(p, device):
    import torch
    q = torch.from_numpy(np.ascontiguousarray(p["q"]).view(np.int16)).to(device)
    w = torch.from_numpy(np.ascontiguousarray(p["w"])).to(device)
    K = torch.from_numpy(np.ascontiguousarray(p["K"]).view(np.int16)).to(device)
    return q, w, K


def _np(t):
    return None if t is None else t.cpu().numpy()


class Guarded:
    """A device buffer with guard bytes on both sides: `view` is what the
    library gets, the guards hold a fixed byte pattern that check() confirms
    is untouched after the call (a write past either end of an output or a
    workspace would change it)."""

    GUARD = 4096
    PATTERN = 0xA5

    def __init__(self, shape, dtype, device):
        import torch
        n = 1
        for x in shape:
            n *= int(x)
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((nbytes + 2 * self.GUARD,), self.PATTERN, dtype=torch.uint8,
                              device=device)
        self.nbytes = nbytes
        self.view = self.raw[self.GUARD:self.GUARD + nbytes].view(dtype).view(*shape)

    def check(self, what="buffer"):
        g = self.raw.cpu().numpy()
        lo, hi = g[:self.GUARD], g[self.GUARD + self.nbytes:]
        assert np.all(lo == self.PATTERN), "%s: guard bytes before it were written" % what
        assert np.all(hi == self.PATTERN), "%s: guard bytes after it were written" % what


def guarded_outputs(q, k, device, ws_bytes):
    """Guarded out_idx [B, T, k] int32, out_score fp32 and a uint8 workspace."""
    import torch
    B, T = q.shape[0], q.shape[1]
    return (Guarded((B, T, k), torch.int32, device), Guarded((B, T, k), torch.float32, device),
            Guarded((max(ws_bytes, 1),), torch.uint8, device))


def check_guards(*bufs):
    for i, b in enumerate(bufs):
        b.check("buffer %d" % i)


def rows_of(p, sample=None, seed=0):
    R = p["Bt"] * p["T"]
    if sample is None or sample >= R:
        return np.arange(R, dtype=np.int32)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(R, size=sample, replace=False).tolist())
    pick |= {0, R - 1}
    return np.array(sorted(pick), dtype=np.int32)


def t_of_row(p, row):
    return p["offset"] + row % p["T"]


# ------------------------------------------------------------ per method

def check_dsa(p, k, gidx, gsc, rows):
    """gidx/gsc: GPU outputs [Bt, T, k]; rows: flat rows to check."""
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    oidx, osc, rs = oracle.dsa(prob, k, rows=rows, want_rowscore=True)
    gi = gidx.reshape(-1, k)
    gs = None if gsc is None else gsc.reshape(-1, k)
    swaps = 0
    for u, row in enumerate(rows):
        t = t_of_row(p, row)
        srow = rs[u, : t + 1]
        tol = TOL_REL * np.max(np.abs(srow))
        swaps += check_set(gi[row], None if gs is None else gs[row], oidx[u], osc[u],
                           lambda s, srow=srow: srow[s], t + 1, k, tol, t=t,
                           what="dsa row %d" % row)
    return swaps


def check_dsa_fp8(p, codes, scales, k, gidx, gsc, rows):
    """As check_dsa, against the oracle's scores on the dequantized FP8 keys."""
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    oidx, osc, rs = oracle.dsa_fp8(prob, codes, scales, k, rows=rows, want_rowscore=True)
    gi = gidx.reshape(-1, k)
    gs = None if gsc is None else gsc.reshape(-1, k)
    swaps = 0
    for u, row in enumerate(rows):
        t = t_of_row(p, row)
        srow = rs[u, : t + 1]
        tol = TOL_REL * np.max(np.abs(srow))
        swaps += check_set(gi[row], None if gs is None else gs[row], oidx[u], osc[u],
                           lambda s, srow=srow: srow[s], t + 1, k, tol, t=t,
                           what="dsa-fp8 row %d" % row)
    return swaps


def check_dsa_fp8q(p, codes, scales, k, gidx, gsc, rows):
    """As check_dsa_fp8, with the query converted to E4M3 too (dsa_fp8q)."""
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    oidx, osc, rs = oracle.dsa_fp8q(prob, codes, scales, k, rows=rows, want_rowscore=True)
    return _check_rows(p, k, gidx, gsc, rows, oidx, osc, rs, "dsa-fp8q")


def _check_rows(p, k, gidx, gsc, rows, ref_idx, ref_sc, rowscore, what):
    gi = gidx.reshape(-1, k)
    gs = None if gsc is None else gsc.reshape(-1, k)
    swaps = 0
    for u, row in enumerate(rows):
        t = t_of_row(p, row)
        srow = rowscore[u, : t + 1]
        tol = TOL_REL * np.max(np.abs(srow))
        swaps += check_set(gi[row], None if gs is None else gs[row], ref_idx[u], ref_sc[u],
                           lambda s, srow=srow: srow[s], t + 1, k, tol, t=t,
                           what="%s row %d" % (what, row))
    return swaps


def check_lisa(p, k, gidx, gsc, rows):
    """LISA: against the oracle's linear score g . k."""
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    oidx, osc, rs = oracle.lisa(prob, k, rows=rows, want_rowscore=True)
    return _check_rows(p, k, gidx, gsc, rows, oidx, osc, rs, "lisa")


def check_resmisa(p, k, block, r, gidx, gsc, gheads, rows):
    """ResMiSA: the routed heads by the near-tie rule on S, then the tokens
    against the oracle run with the GPU's heads."""
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    over = None
    if r > 0:
        base = oracle.resmisa(prob, k, block, r, rows=rows)
        gh = gheads.reshape(-1, r)
        for u, row in enumerate(rows):
            assert np.all(np.diff(gh[row]) > 0), "resmisa heads row %d not ascending" % row
            check_choice(gh[row], base["S"][u], p["H"], r, "resmisa heads row %d" % row)
        over = np.ascontiguousarray(gh[rows])
    staged = oracle.resmisa(prob, k, block, r, rows=rows, override_heads=over, want_rowscore=True)
    return _check_rows(p, k, gidx, gsc, rows, staged["idx"], staged["score"], staged["rowscore"],
                       "resmisa")


def _problem(p, fp8):
    """The oracle's problem: bf16 keys, or with fp8 = (codes, scales) the FP8
    key cache."""
    if fp8 is None:
        return oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    return oracle.Problem(p["q"], p["w"], None, p["offset"], codes=fp8[0], scales=fp8[1])


def check_misa(p, k, B, h, kprime, gidx, gsc, gheads, gpool, rows, fp8=None):
    prob = _problem(p, fp8)
    base = oracle.misa(prob, k, B, h, kprime=0, rows=rows)
    gh = gheads.reshape(-1, h)
    for u, row in enumerate(rows):
        check_choice(gh[row], base["E"][u], p["H"], h, "misa heads row %d" % row)
    over_h = np.ascontiguousarray(gh[rows])
    staged = oracle.misa(prob, k, B, h, kprime=kprime, rows=rows, override_heads=over_h,
                         want_hatrow=True)
    gi = gidx.reshape(-1, k)
    gs = None if gsc is None else gsc.reshape(-1, k)
    swaps = 0
    if kprime == 0:
        for u, row in enumerate(rows):
            t = t_of_row(p, row)
            hat = staged["hatrow"][u, : t + 1]
            tol = TOL_REL * np.max(np.abs(hat))
            swaps += check_set(gi[row], None if gs is None else gs[row], staged["idx"][u],
                               staged["score"][u], lambda s, hat=hat: hat[s], t + 1, k, tol, t=t,
                               what="misa row %d" % row)
        return swaps
    # MISA-dagger: the k' pool by the routed score, then the rerank.
    gp = gpool.reshape(-1, kprime)
    for u, row in enumerate(rows):
        t = t_of_row(p, row)
        hat = staged["hatrow"][u, : t + 1]
        tol = TOL_REL * np.max(np.abs(hat))
        opool = staged["pool"][u]
        check_set(gp[row], None, opool, hat[opool[opool >= 0]], lambda s, hat=hat: hat[s],
                  t + 1, kprime, tol, t=t, what="misa-dagger pool row %d" % row)
    over_p = np.ascontiguousarray(gp[rows])
    final = oracle.misa(prob, k, B, h, kprime=kprime, rows=rows, override_heads=over_h,
                        override_pool=over_p)
    # all-heads score of every pool member (top-k' of the pool = the whole pool)
    every = oracle.misa(prob, kprime, B, h, kprime=kprime, rows=rows, override_heads=over_h,
                        override_pool=over_p)
    for u, row in enumerate(rows):
        t = t_of_row(p, row)
        pool = gp[row][gp[row] >= 0]
        sc_of = dict(zip(every["idx"][u].tolist(), every["score"][u].tolist()))
        sc_of.pop(-1, None)
        tol = TOL_REL * max(abs(v) for v in sc_of.values())
        swaps += check_set(gi[row], None if gs is None else gs[row], final["idx"][u],
                           final["score"][u], lambda s, d=sc_of: np.array([d[int(x)] for x in s]),
                           len(pool), k, tol, t=t, cand_set=set(pool.tolist()),
                           what="misa-dagger row %d" % row)
    return swaps


def check_hisa(p, k, b, r, gidx, gsc, gblocks, rows, coarse_heads=None, fp8=None):
    """coarse_heads [len(rows), h]: block scores over those heads (MISA x HISA,
    staged with the GPU's routed heads)."""
    prob = _problem(p, fp8)
    base = oracle.hisa(prob, k, b, r, rows=rows, coarse_heads=coarse_heads)
    gb = gblocks.reshape(-1, r)
    for u, row in enumerate(rows):
        t = t_of_row(p, row)
        check_choice(gb[row], base["J"][u], t // b + 1, r, "hisa blocks row %d" % row)
    over = np.ascontiguousarray(gb[rows])
    staged = oracle.hisa(prob, k, b, r, rows=rows, override_blocks=over,
                         coarse_heads=coarse_heads)
    gi = gidx.reshape(-1, k)
    gs = None if gsc is None else gsc.reshape(-1, k)
    swaps = 0
    for u, row in enumerate(rows):
        t = t_of_row(p, row)
        blocks = gb[row][gb[row] >= 0]
        cand = np.concatenate([np.arange(m * b, min((m + 1) * b, t + 1)) for m in blocks])
        # exact scores of the candidates: from the staged oracle top-k over
        # exactly these candidates (k = #candidates gives every score)
        allc = oracle.hisa(prob, len(cand), b, r, rows=np.array([row], np.int32),
                           override_blocks=over[u: u + 1],
                           coarse_heads=None if coarse_heads is None else coarse_heads[u: u + 1])
        sc_of = dict(zip(allc["idx"][0].tolist(), allc["score"][0].tolist()))
        tol = TOL_REL * max(abs(v) for v in sc_of.values())
        swaps += check_set(gi[row], None if gs is None else gs[row], staged["idx"][u],
                           staged["score"][u], lambda s, d=sc_of: np.array([d[int(x)] for x in s]),
                           len(cand), k, tol, t=t, cand_set=set(cand.tolist()),
                           what="hisa row %d" % row)
    return swaps


def check_misa_hisa(p, k, B, h, b, r, gidx, gsc, gheads, gblocks, rows):
    """MISA x HISA, staged: the routed heads by the near-tie rule on E, the
    blocks on the block scores over the GPU's heads, then the tokens over the
    GPU's blocks."""
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    base = oracle.misa(prob, 1, B, h, rows=rows)
    gh = gheads.reshape(-1, h)
    for u, row in enumerate(rows):
        assert np.all(np.diff(gh[row]) > 0), "misa-hisa heads row %d not ascending" % row
        check_choice(gh[row], base["E"][u], p["H"], h, "misa-hisa heads row %d" % row)
    return check_hisa(p, k, b, r, gidx, gsc, gblocks, rows,
                      coarse_heads=np.ascontiguousarray(gh[rows]))


# ------------------------------------------------------------------ smoke

def smoke_run(device):
    """One small call of every entry point on `device`, checked against the oracle."""
    import torch
    from sparse_attention_token_dsa_amd import api

    p = synth.make_problem(7, Bt=2, T=1, L=3000, H=64, needles=8, needle_mode="decode")
    q, w, K = to_device(p, device)
    rows = rows_of(p)
    idx, sc = api.indexer_score_topk(q, w, K, p["offset"], 64)
    torch.cuda.synchronize(device)
    check_dsa(p, 64, _np(idx), _np(sc), rows)

    idx, sc, heads, pool = api.misa_route(q, w, K, p["offset"], 64, 256, 8, k_prime=256,
                                          want_pool=True)
    torch.cuda.synchronize(device)
    check_misa(p, 64, 256, 8, 256, _np(idx), _np(sc), _np(heads), _np(pool), rows)

    idx, sc, blocks = api.hisa_coarse_fine(q, w, K, p["offset"], 64, 64, 8)
    torch.cuda.synchronize(device)
    check_hisa(p, 64, 64, 8, _np(idx), _np(sc), _np(blocks), rows)

    codes, scales = api.quantize_keys_fp8(K)
    torch.cuda.synchronize(device)
    oc, os_ = oracle.quantize_keys_fp8(p["K"])
    assert np.array_equal(_np(codes), oc) and np.array_equal(_np(scales), os_), "fp8 codes"
    idx, sc = api.indexer_score_topk_fp8(q, w, codes, scales, p["offset"], 64)
    torch.cuda.synchronize(device)
    check_dsa_fp8(p, oc, os_, 64, _np(idx), _np(sc), rows)
    idx, sc = api.indexer_score_topk_fp8q(q, w, codes, scales, p["offset"], 64)
    torch.cuda.synchronize(device)
    check_dsa_fp8q(p, oc, os_, 64, _np(idx), _np(sc), rows)
    idx, sc, heads, pool = api.misa_route_fp8(q, w, codes, scales, p["offset"], 64, 256, 8,
                                              k_prime=256, want_pool=True)
    torch.cuda.synchronize(device)
    check_misa(p, 64, 256, 8, 256, _np(idx), _np(sc), _np(heads), _np(pool), rows,
               fp8=(oc, os_))
    idx, sc, blocks = api.hisa_coarse_fine_fp8(q, w, codes, scales, p["offset"], 64, 64, 8)
    torch.cuda.synchronize(device)
    check_hisa(p, 64, 64, 8, _np(idx), _np(sc), _np(blocks), rows, fp8=(oc, os_))

    idx, sc = api.lisa_score_topk(q, w, K, p["offset"], 64)
    torch.cuda.synchronize(device)
    check_lisa(p, 64, _np(idx), _np(sc), rows)
    idx, sc, heads = api.resmisa_route(q, w, K, p["offset"], 64, 128, 7)
    torch.cuda.synchronize(device)
    check_resmisa(p, 64, 128, 7, _np(idx), _np(sc), _np(heads), rows)
    idx, sc, heads, blocks = api.misa_hisa(q, w, K, p["offset"], 64, 256, 8, 64, 8)
    torch.cuda.synchronize(device)
    check_misa_hisa(p, 64, 256, 8, 64, 8, _np(idx), _np(sc), _np(heads), _np(blocks), rows)

    slots, stats = api.tidy_indices(idx, 1, page_size=16, max_slots=p["L"])
    torch.cuda.synchronize(device)
    os2, ost = oracle.tidy(_np(idx).reshape(-1, 64), 1, page_size=16, max_slots=p["L"])
    assert np.array_equal(_np(slots).reshape(os2.shape), os2), "tidy slots"
    assert np.array_equal(_np(stats).reshape(ost.shape), ost), "tidy counts"
    lens = np.array([3000, 1234], np.int32)
    idx, sc = api.indexer_score_topk_ragged(q, w, K, torch.from_numpy(lens).to(device), 64,
                                            total_len=int(lens.sum()))
    torch.cuda.synchronize(device)
    oi, osc, rs = oracle.dsa_ragged(p["q"], p["w"], p["K"], lens, 64)
    gi, gs = _np(idx).reshape(-1, 64), _np(sc).reshape(-1, 64)
    for row in range(2):
        t = int(lens[row]) - 1
        srow = rs[row, : t + 1]
        check_set(gi[row], gs[row], oi[row], osc[row], lambda s, srow=srow: srow[s], t + 1, 64,
                  TOL_REL * np.max(np.abs(srow)), t=t, what="ragged row %d" % row)

    pp = synth.make_problem(8, Bt=1, T=64, L=700, H=64, needles=8, needle_mode="rows")
    q, w, K = to_device(pp, device)
    idx, sc = api.indexer_score_topk(q, w, K, pp["offset"], 48)
    torch.cuda.synchronize(device)
    check_dsa(pp, 48, _np(idx), _np(sc), rows_of(pp))
    print("smoke ok: DSA, FP8 keys (q bf16 and E4M3; MISA-dagger and HISA too), MISA-dagger, "
          "HISA, LISA, ResMiSA, MISA x HISA, tidy-up, "
          "ragged batches and the fused prefill match the oracle")


def prefill_group_rows(T, seed):
    """One random row of each 8-row group: the fused prefill's workgroup x
    runs group x (its short causal range) and group G - 1 - x (its long one),
    so this covers both groups of every workgroup."""
    rng = np.random.default_rng(seed)
    G = (T + 7) // 8
    return np.array(sorted(min(8 * g + int(rng.integers(0, 8)), T - 1) for g in range(G)),
                    dtype=np.int32)
