"""CPU oracle for the DSA lightning-indexer selector (DSA, MISA, HISA).

TEST INFRASTRUCTURE ONLY.  The plain fp64 C definition lives in ``oracle.c``;
this module compiles it with gcc (a second or so) and wraps it for numpy.
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the HIP library and never
imports it.

Every function takes the seeded host arrays directly: ``q`` as uint16 bf16 bit
patterns ``[Bt, T, H, d]``, ``w`` float32 ``[Bt, T, H]``, ``K`` uint16
``[Bt, L, d]``.  Outputs per evaluated row are sorted by (score desc, index
asc) and padded with -1 / -inf.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so next to its source (plain gcc, -O2, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("w", ctypes.c_void_p), ("K", ctypes.c_void_p),
                ("Bt", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("d", ctypes.c_int32), ("L", ctypes.c_int32),
                ("causal_offset", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i = ctypes.c_int
        _lib.oracle_dsa.argtypes = [P, i, P, i, P, P, P, i]
        _lib.oracle_misa.argtypes = [P, i, i, i, i, P, i, P, P, P, P, P, P, P, P, i]
        _lib.oracle_hisa.argtypes = [P, i, i, i, P, i, P, P, i, P, P, P, P, i]
        _lib.oracle_pool.argtypes = [P, i, i, i, i, P]
        _lib.oracle_quantize_keys_fp8.argtypes = [P, ctypes.c_long, i, P, P, i]
        _lib.oracle_dsa_fp8.argtypes = [P, P, P, i, P, i, P, P, P, i]
        _lib.oracle_dsa_fp8q.argtypes = [P, P, P, i, P, i, P, P, P, i]
        _lib.oracle_lisa.argtypes = [P, i, P, i, P, P, P, i]
        _lib.oracle_resmisa.argtypes = [P, i, i, i, P, i, P, P, P, P, P, P, i]
        _lib.oracle_box_bound.argtypes = [P, P, P, i]
        _lib.oracle_box_bound.restype = ctypes.c_double
        _lib.oracle_fp8_e4m3_decode.argtypes = [ctypes.c_uint8]
        _lib.oracle_fp8_e4m3_decode.restype = ctypes.c_double
        _lib.oracle_fp8_e4m3_encode.argtypes = [ctypes.c_float]
        _lib.oracle_fp8_e4m3_encode.restype = ctypes.c_uint8
        for f in (_lib.oracle_dsa, _lib.oracle_misa, _lib.oracle_hisa, _lib.oracle_pool,
                  _lib.oracle_quantize_keys_fp8, _lib.oracle_dsa_fp8, _lib.oracle_dsa_fp8q,
                  _lib.oracle_lisa,
                  _lib.oracle_resmisa):
            f.restype = ctypes.c_int
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Problem:
    """Holds contiguous copies of (q, w, K) and the causal offset.  With
    codes/scales (an FP8 key cache, K = None) DSA, MISA and HISA read key s of
    sequence b as scales[b, s] * e4m3(codes[b, s])."""

    def __init__(self, q, w, K, causal_offset, codes=None, scales=None):
        self.q = np.ascontiguousarray(q, dtype=np.uint16)
        self.w = np.ascontiguousarray(w, dtype=np.float32)
        self.K = None if K is None else np.ascontiguousarray(K, dtype=np.uint16)
        self.codes = None if codes is None else np.ascontiguousarray(codes, dtype=np.uint8)
        self.scales = None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)
        Bt, T, H, d = self.q.shape
        assert self.w.shape == (Bt, T, H), self.w.shape
        assert (self.K is None) != (self.codes is None), "K or (codes, scales)"
        kk = self.K if self.K is not None else self.codes
        assert kk.shape[0] == Bt and kk.shape[2] == d, kk.shape
        if self.codes is not None:
            assert self.scales is not None and self.scales.shape == kk.shape[:2]
        self.Bt, self.T, self.H, self.d = Bt, T, H, d
        self.L = kk.shape[1]
        self.offset = int(causal_offset)
        self._c = _Problem(_ptr(self.q), _ptr(self.w), _ptr(self.K), Bt, T, H, d, self.L,
                           self.offset, _ptr(self.codes), _ptr(self.scales))

    def rows(self, rows):
        if rows is None:
            return None, self.Bt * self.T
        r = np.ascontiguousarray(rows, dtype=np.int32)
        assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < self.Bt * self.T))
        return r, int(r.size)


def _threads(nthreads):
    if nthreads:
        return int(nthreads)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _check(rc, name):
    if rc != 0:
        raise ValueError("%s rejected its arguments (code %d)" % (name, rc))


def dsa(prob: Problem, topk: int, rows=None, want_rowscore=False, nthreads=0):
    """DSA score + causal mask + token top-k.  Returns (idx, score[, rowscore])."""
    lib = _load()
    r, n = prob.rows(rows)
    idx = np.empty((n, topk), np.int32)
    sc = np.empty((n, topk), np.float64)
    rs = np.empty((n, prob.L), np.float64) if want_rowscore else None
    _check(lib.oracle_dsa(ctypes.byref(prob._c), topk, _ptr(r), n, _ptr(idx), _ptr(sc),
                          _ptr(rs), _threads(nthreads)), "oracle_dsa")
    return (idx, sc, rs) if want_rowscore else (idx, sc)


def misa(prob: Problem, topk: int, B: int, h: int, kprime: int = 0, rows=None,
         override_heads=None, override_pool=None, want_hatrow=False, nthreads=0):
    """MISA / MISA-dagger.  Returns a dict with idx, score, heads, E, pool, hatrow."""
    lib = _load()
    r, n = prob.rows(rows)
    oh = None if override_heads is None else np.ascontiguousarray(override_heads, np.int32)
    op = None if override_pool is None else np.ascontiguousarray(override_pool, np.int32)
    if oh is not None:
        assert oh.shape == (n, h)
    if op is not None:
        assert kprime > 0 and op.shape == (n, kprime)
    out = {
        "idx": np.empty((n, topk), np.int32),
        "score": np.empty((n, topk), np.float64),
        "heads": np.empty((n, h), np.int32),
        "E": np.empty((n, prob.H), np.float64),
        "pool": np.empty((n, kprime), np.int32) if kprime else None,
        "hatrow": np.empty((n, prob.L), np.float64) if want_hatrow else None,
    }
    _check(lib.oracle_misa(ctypes.byref(prob._c), topk, B, h, kprime, _ptr(r), n, _ptr(oh),
                           _ptr(op), _ptr(out["heads"]), _ptr(out["E"]), _ptr(out["pool"]),
                           _ptr(out["hatrow"]), _ptr(out["idx"]), _ptr(out["score"]),
                           _threads(nthreads)), "oracle_misa")
    return out


def hisa(prob: Problem, topk: int, b: int, r: int, rows=None, override_blocks=None,
         coarse_heads=None, nthreads=0):
    """HISA coarse (blocks) + fine (tokens).  Returns a dict with idx, score, blocks, J.
    coarse_heads [n, h] (ascending): score the blocks with those heads only."""
    lib = _load()
    rr, n = prob.rows(rows)
    ob = None if override_blocks is None else np.ascontiguousarray(override_blocks, np.int32)
    if ob is not None:
        assert ob.shape == (n, r)
    ch = None if coarse_heads is None else np.ascontiguousarray(coarse_heads, np.int32)
    hsel = 0 if ch is None else ch.shape[1]
    if ch is not None:
        assert ch.shape == (n, hsel) and np.all(np.diff(ch, axis=1) > 0)
    nbmax = (prob.L + b - 1) // b
    out = {
        "idx": np.empty((n, topk), np.int32),
        "score": np.empty((n, topk), np.float64),
        "blocks": np.empty((n, r), np.int32),
        "J": np.empty((n, nbmax), np.float64),
    }
    _check(lib.oracle_hisa(ctypes.byref(prob._c), topk, b, r, _ptr(rr), n, _ptr(ob), _ptr(ch),
                           hsel, _ptr(out["blocks"]), _ptr(out["J"]), _ptr(out["idx"]),
                           _ptr(out["score"]), _threads(nthreads)), "oracle_hisa")
    return out


def pool(K, block: int):
    """Block means of K [Bt, L, d] (bf16 bits) -> float64 [Bt, ceil(L/block), d]."""
    lib = _load()
    K = np.ascontiguousarray(K, np.uint16)
    Bt, L, d = K.shape
    nb = (L + block - 1) // block
    out = np.empty((Bt, nb, d), np.float64)
    _check(lib.oracle_pool(_ptr(K), Bt, L, d, block, _ptr(out)), "oracle_pool")
    return out


def fp8_decode(codes):
    """OCP E4M3 values (float64) of uint8 codes (any shape)."""
    lib = _load()
    c = np.asarray(codes, np.uint8)
    table = np.array([lib.oracle_fp8_e4m3_decode(v) for v in range(256)], np.float64)
    return table[c]


def fp8_encode(x):
    """Nearest OCP E4M3 codes (ties to even, saturating) of float32 values."""
    lib = _load()
    x = np.asarray(x, np.float32)
    return np.array([lib.oracle_fp8_e4m3_encode(float(v)) for v in x.ravel()],
                    np.uint8).reshape(x.shape)


def quantize_keys_fp8(K, nthreads=0):
    """Per-key FP8 quantization of K [..., L, d] (bf16 bits) -> (codes uint8
    [..., L, d], scales float32 [..., L])."""
    lib = _load()
    K = np.ascontiguousarray(K, np.uint16)
    d = K.shape[-1]
    n = K.size // d
    codes = np.empty(K.shape, np.uint8)
    scales = np.empty(K.shape[:-1], np.float32)
    _check(lib.oracle_quantize_keys_fp8(_ptr(K), n, d, _ptr(codes), _ptr(scales),
                                        _threads(nthreads)),
           "oracle_quantize_keys_fp8")
    return codes, scales


def dsa_fp8(prob: Problem, codes, scales, topk: int, rows=None, want_rowscore=False,
            nthreads=0):
    """DSA on FP8 keys (codes [Bt, L, d], scales [Bt, L]); prob.K is not used.
    Returns (idx, score[, rowscore])."""
    lib = _load()
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    assert codes.shape == (prob.Bt, prob.L, prob.d) and scales.shape == (prob.Bt, prob.L)
    r, n = prob.rows(rows)
    idx = np.empty((n, topk), np.int32)
    sc = np.empty((n, topk), np.float64)
    rs = np.empty((n, prob.L), np.float64) if want_rowscore else None
    _check(lib.oracle_dsa_fp8(ctypes.byref(prob._c), _ptr(codes), _ptr(scales), topk, _ptr(r),
                              n, _ptr(idx), _ptr(sc), _ptr(rs), _threads(nthreads)),
           "oracle_dsa_fp8")
    return (idx, sc, rs) if want_rowscore else (idx, sc)


def dsa_fp8q(prob: Problem, codes, scales, topk: int, rows=None, want_rowscore=False,
             nthreads=0):
    """DSA on FP8 keys with the query converted to E4M3 as well, the compute
    type of the fp8 matrix product (PaperTrace section 2.3: the query is
    converted to the compute type in registers; its error counts on top of
    the key error).

    Each head vector q_{t,j} is quantized by the key-cache rule (b_j =
    max|q|/448 in fp32, 1 for a zero vector; codes of q/b_j), and the score is
    the indexer formula on the dequantized vectors, in fp64:
    I = sum_j w_j max((b_j decode(qc_j)) . (a_s decode(c_s)), 0).
    Returns (idx, score[, rowscore]).
    """
    lib = _load()
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    assert codes.shape == (prob.Bt, prob.L, prob.d) and scales.shape == (prob.Bt, prob.L)
    r, n = prob.rows(rows)
    idx = np.empty((n, topk), np.int32)
    sc = np.empty((n, topk), np.float64)
    rs = np.empty((n, prob.L), np.float64) if want_rowscore else None
    _check(lib.oracle_dsa_fp8q(ctypes.byref(prob._c), _ptr(codes), _ptr(scales), topk, _ptr(r),
                               n, _ptr(idx), _ptr(sc), _ptr(rs), _threads(nthreads)),
           "oracle_dsa_fp8q")
    return (idx, sc, rs) if want_rowscore else (idx, sc)


def lisa(prob: Problem, topk: int, rows=None, want_rowscore=False, nthreads=0):
    """LISA: top-k by the linear score g . k.  Returns (idx, score[, rowscore])."""
    lib = _load()
    r, n = prob.rows(rows)
    idx = np.empty((n, topk), np.int32)
    sc = np.empty((n, topk), np.float64)
    rs = np.empty((n, prob.L), np.float64) if want_rowscore else None
    _check(lib.oracle_lisa(ctypes.byref(prob._c), topk, _ptr(r), n, _ptr(idx), _ptr(sc), _ptr(rs),
                           _threads(nthreads)), "oracle_lisa")
    return (idx, sc, rs) if want_rowscore else (idx, sc)


def resmisa(prob: Problem, topk: int, block: int, r: int, rows=None, override_heads=None,
            want_rowscore=False, nthreads=0):
    """ResMiSA: shared linear score + r routed residual heads.  Returns a dict
    with idx, score, heads [n, r] (ascending), S [n, H], rowscore."""
    lib = _load()
    rw, n = prob.rows(rows)
    oh = None if override_heads is None else np.ascontiguousarray(override_heads, np.int32)
    if oh is not None:
        assert oh.shape == (n, r)
    out = {
        "idx": np.empty((n, topk), np.int32),
        "score": np.empty((n, topk), np.float64),
        "heads": np.empty((n, r), np.int32) if r else None,
        "S": np.empty((n, prob.H), np.float64) if r else None,
        "rowscore": np.empty((n, prob.L), np.float64) if want_rowscore else None,
    }
    _check(lib.oracle_resmisa(ctypes.byref(prob._c), topk, block, r, _ptr(rw), n, _ptr(oh),
                              _ptr(out["heads"]), _ptr(out["S"]), _ptr(out["rowscore"]),
                              _ptr(out["idx"]), _ptr(out["score"]), _threads(nthreads)),
           "oracle_resmisa")
    return out


def box_bound(q, kmin, kmax):
    """U- = sum_d (max(-q,0) kmax - max(q,0) kmin) for one head and one box."""
    lib = _load()
    q = np.ascontiguousarray(q, np.float64)
    kmin = np.ascontiguousarray(kmin, np.float64)
    kmax = np.ascontiguousarray(kmax, np.float64)
    assert q.shape == kmin.shape == kmax.shape and q.ndim == 1
    return lib.oracle_box_bound(_ptr(q), _ptr(kmin), _ptr(kmax), q.shape[0])


def misa_hisa(prob: Problem, topk: int, B: int, h: int, b: int, r: int, rows=None,
              override_heads=None, override_blocks=None, nthreads=0):
    """MISA x HISA: the MISA router picks h heads (pooled blocks of B), HISA's
    block scores use only those heads (blocks of b), the legal tokens of the r
    best blocks are rescored with every head, top-k.  Returns a dict with
    heads, E, blocks, J, idx, score."""
    m = misa(prob, 1, B, h, rows=rows, nthreads=nthreads)
    heads = m["heads"] if override_heads is None else np.ascontiguousarray(override_heads, np.int32)
    out = hisa(prob, topk, b, r, rows=rows, override_blocks=override_blocks, coarse_heads=heads,
               nthreads=nthreads)
    out["heads"] = heads
    out["E"] = m["E"]
    return out


def dsa_ragged(q, w, K, seq_lens, topk, nthreads=0):
    """DSA over sequences of different lengths: sequence b's history is
    K[b, :seq_lens[b]] and its T query rows sit at seq_lens[b] - T + i; each
    sequence is the plain DSA problem on its own keys.  Returns (idx, score,
    rowscore) with rows b*T + i; rowscore [rows, L] is NaN past the row."""
    Bt, T = q.shape[0], q.shape[1]
    L = K.shape[1]
    idx = np.empty((Bt * T, topk), np.int32)
    sc = np.empty((Bt * T, topk), np.float64)
    rs = np.full((Bt * T, L), np.nan)
    for b in range(Bt):
        n = int(seq_lens[b])
        assert T <= n <= L
        pb = Problem(q[b:b + 1], w[b:b + 1], np.ascontiguousarray(K[b:b + 1, :n]), n - T)
        i, s, r = dsa(pb, topk, want_rowscore=True, nthreads=nthreads)
        idx[b * T:(b + 1) * T] = i
        sc[b * T:(b + 1) * T] = s
        rs[b * T:(b + 1) * T, :n] = r
    return idx, sc, rs


def tidy(idx, T, block_table=None, page_size=1, max_slots=0):
    """Index tidy-up ([PT] 2.2; counts of [PT] 2.3).  Per row of idx [rows, k]
    (-1 empty): the physical slots table[b][s // page] * page + s % page (s
    itself without a table), dropping positions past the table, on a negative
    entry, or (max_slots > 0) at or after max_slots; distinct, ascending, -1
    padded.  stats [rows, 3] = (distinct slots, distinct pages, maximal runs of
    consecutive slots)."""
    idx = np.asarray(idx).reshape(-1, np.asarray(idx).shape[-1])
    rows, k = idx.shape
    slots = np.full((rows, k), -1, np.int32)
    stats = np.zeros((rows, 3), np.int32)
    for row in range(rows):
        b = row // T
        v = idx[row][idx[row] >= 0].astype(np.int64)
        if block_table is not None:
            pg = v // page_size
            keep = pg < block_table.shape[1]
            v, pg = v[keep], pg[keep]
            phys = block_table[b][pg].astype(np.int64)
            keep = phys >= 0
            v = phys[keep] * page_size + v[keep] % page_size
        if max_slots > 0:
            v = v[v < max_slots]
        u = np.unique(v)
        slots[row, :len(u)] = u
        runs = 0 if len(u) == 0 else 1 + int(np.count_nonzero(np.diff(u) != 1))
        stats[row] = (len(u), len(np.unique(u // page_size)), runs)
    return slots, stats
