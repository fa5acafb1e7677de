"""Work counters of the indexer selectors: legal (query, key) pairs, dot
products, multiply-adds and the bytes a call must move.

Plain integer arithmetic on shapes, shared by the benchmark (its throughput
and roofline numerators) and the tests that pin it to the cost figures the
pages work by hand (PaperTrace, "2.2.2 MISA, LISA and ResMiSA": section 2.3,
the per-item cost of one decode step; section 3.2, the dot-product counts of
the head axis).  Nothing here runs a selector.
"""
from __future__ import annotations


# ------------------------------------------------------------ pairs, MACs

def legal_pairs(T: int, offset: int, batch: int = 1) -> int:
    """Causal (query, key) pairs: row i sits at t = offset + i and scores the
    t + 1 keys 0..t, so one sequence has T * offset + T (T + 1) / 2."""
    return batch * (T * offset + T * (T + 1) // 2)


def ragged_pairs(T: int, seq_lens) -> int:
    """Legal pairs of a ragged batch: sequence b's rows sit at
    seq_lens[b] - T + i."""
    return sum(legal_pairs(T, int(n) - T) for n in seq_lens)


def indexer_macs(pairs: int, heads: int, d: int) -> int:
    """Multiply-adds of the indexer dot products: one length-d dot product per
    (pair, head).  The ReLU and the weighted head sum are not counted (section
    2.3 counts t * H * d for one decode query)."""
    return pairs * heads * d


def misa_macs(pairs: int, h: int, d: int, rows: int = 0, H: int = 0, blocks: int = 0) -> int:
    """MISA: the token scoring with the h routed heads (section 2.3's
    t * h * d), plus the router's H x blocks dot products per query row when
    rows, H and blocks are given."""
    return pairs * h * d + rows * H * blocks * d


def hisa_counts(n: int, b: int, r: int) -> dict:
    """HISA on one query with n legal keys: block representatives scored
    (ceil(n / b)), tokens rescored (r * b), and the rescored share of the
    history (section 2.3: b = 64 over 131072 keys gives 2048 blocks; r = 128
    gives 8192 tokens, 6.25 percent)."""
    return {"reps": (n + b - 1) // b, "tokens": r * b, "percent": 100.0 * r * b / n}


# ---------------------------------------------------- head-axis dot counts

def dsa_dots(N: int, H: int) -> int:
    """Dot products of one DSA query over N keys (section 3.2: N * H_I)."""
    return N * H


def lisa_dots(N: int) -> int:
    """LISA: the fused query scores every key once."""
    return N


def resmisa_dots(N: int, r: int) -> int:
    """ResMiSA: the shared linear term plus r residual heads per key."""
    return N * (r + 1)


def lisa_dagger_dots(N: int, M: int, H: int) -> int:
    """LISA-dagger: one linear scan of N keys, then the M-candidate pool
    rescored with all H heads."""
    return N + M * H


def lisa_ddagger_dots(N: int, M: int, H: int, G: int) -> float:
    """LISA-double-dagger: the linear scan shared by a group of G layers, the
    pool rescoring per layer (average dot products per layer)."""
    return N / G + M * H


# ------------------------------------------------------------------ bytes

def key_bytes(batch: int, L: int, d: int, fp8: bool = False) -> int:
    """The key cache: bf16, 2 d bytes per key; FP8 codes plus one fp32 scale,
    d + 4 bytes per key."""
    return batch * L * (d + 4 if fp8 else 2 * d)


def scan_bytes(rows: int, batch: int, L: int, H: int, d: int, fp8: bool = False) -> int:
    """Algorithmic bytes of one decode scan: the keys once, each row's q
    (bf16 [H, d]) and w (fp32 [H]).  The heads a routed scan reads are H = h."""
    return key_bytes(batch, L, d, fp8) + rows * H * (2 * d + 4)


def score_row_bytes(rows: int, L: int) -> int:
    """The fp32 score row a decode scan of this design writes per query row
    (its own staging for the top-k, not part of the method's bytes)."""
    return rows * L * 4


def topk_out_bytes(rows: int, k: int, with_scores: bool = True) -> int:
    """int32 indices (and fp32 scores) of the selected set."""
    return rows * k * (8 if with_scores else 4)


def prefill_bytes(batch: int, T: int, L: int, H: int, d: int, k: int) -> int:
    """Algorithmic bytes of one fused prefill call: q, w, the keys once and
    the int32 indices out."""
    return batch * T * H * (2 * d + 4) + key_bytes(batch, L, d) + batch * T * k * 4


def pool_bytes(batch: int, L: int, d: int, blocks: int) -> int:
    """One pooling pass: the keys once, `blocks` hi/lo bf16 representatives
    per sequence out (4 d bytes each)."""
    return key_bytes(batch, L, d) + batch * blocks * 4 * d


def gather_bytes(rows: int, cand: int, d: int, fp8: bool = False) -> int:
    """A rescoring pass over `cand` gathered keys per row."""
    return rows * cand * (d + 4 if fp8 else 2 * d)
