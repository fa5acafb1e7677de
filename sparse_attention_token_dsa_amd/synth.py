"""Seeded synthetic inputs for the indexer workloads.

This module only draws and lays out data; it holds none of the selector's
arithmetic.  Both the CPU oracle (tests, CPU baseline) and the GPU path take
their bytes from here, so the two see identical inputs.

Recipe (numpy ``Generator(PCG64(seed))``, draw order q, w, K, needles):

* q ~ N(0, sigma = 1/sqrt(128)) drawn in float32, rounded to bf16
  (round-to-nearest-even), shape [Bt, T, H, d];
* w ~ N(0, sigma = 1/64) float32, shape [Bt, T, H];
* K ~ N(0, sigma = 1/sqrt(128)) float32 -> bf16, shape [Bt, L, d], drawn one
  sequence at a time;
* needles: a needle at key position s copies 3 * q[t, j] (rounded to bf16)
  into K[s] for a random query row t that can see s and a random head j.

The workloads' sizes follow the pages' settings (H_I = 64 for DeepSeek-V3.2 and
32 for GLM-5, d = 128, k = 2048, MISA B = 1024 / h = 8 / k' = 8192, HISA
b = 128 / r = 64).  Needles stand in for needle-in-a-haystack structure; no
benchmark items are reproduced.
"""
from __future__ import annotations

import numpy as np

SIGMA_QK = 1.0 / np.sqrt(128.0)
SIGMA_W = 1.0 / 64.0

# name -> workload description.  offset = absolute position of query row 0.
CONFIGS = {
    "prefill_tiny": dict(seed=1010, Bt=1, T=1024, L=1024, H=64, d=128, offset=0, topk=128,
                         needles=16, needle_mode="rows"),
    "decode_32k": dict(seed=1020, Bt=32, T=1, L=32768, H=64, d=128, offset=32767, topk=2048,
                       needles=64, needle_mode="decode"),
    "prefill_chunked": dict(seed=1030, Bt=1, T=4096, L=32768, H=64, d=128, offset=28672,
                            topk=2048, needles=16, needle_mode="rows"),
    "misa_128k_h64": dict(seed=1040, Bt=8, T=1, L=131072, H=64, d=128, offset=131071,
                          topk=2048, B=1024, h=8, kprime=8192, needles=64, needle_mode="decode"),
    "misa_128k_h32": dict(seed=1041, Bt=8, T=1, L=131072, H=32, d=128, offset=131071,
                          topk=2048, B=1024, h=8, kprime=8192, needles=64, needle_mode="decode"),
    "hisa_128k": dict(seed=1050, Bt=8, T=1, L=131072, H=64, d=128, offset=131071, topk=2048,
                      b=128, r=64, needles=64, needle_mode="hisa"),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_bf16(rng, shape, sigma):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def make_problem(seed, Bt, T, L, H, d=128, offset=None, needles=0, needle_mode="rows",
                 block=None, **extra):
    """Draw one problem.  Returns dict(q, w, K, offset, needle_pos, ...meta)."""
    if offset is None:
        offset = L - T
    assert 0 <= offset and offset + T <= L
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _draw_bf16(rng, (Bt, T, H, d), SIGMA_QK)
    w = (rng.standard_normal((Bt, T, H), dtype=np.float32) * np.float32(SIGMA_W)).astype(
        np.float32)
    K = np.empty((Bt, L, d), np.uint16)
    for b in range(Bt):
        K[b] = _draw_bf16(rng, (L, d), SIGMA_QK)
    qf = None
    needle_pos = []

    def plant(b, s, row, j):
        nonlocal qf
        if qf is None:
            qf = {}
        key = (b, row, j)
        if key not in qf:
            qf[key] = bf16_bits_to_f32(q[b, row, j])
        K[b, s] = to_bf16_bits(qf[key] * np.float32(3.0))

    if needles:
        if needle_mode == "rows":
            # needles spread over positions; each is aimed at one query row
            # that can see it (t >= s) and one head.
            for b in range(Bt):
                pos = rng.choice(L, size=min(needles, L), replace=False)
                for s in pos:
                    lo = max(int(s), offset)
                    t = int(rng.integers(lo, offset + T)) if lo < offset + T else offset + T - 1
                    j = int(rng.integers(0, H))
                    plant(b, int(s), t - offset, j)
                    needle_pos.append((b, int(s)))
        elif needle_mode == "decode":
            for b in range(Bt):
                pos = rng.choice(L, size=min(needles, L), replace=False)
                for s in pos:
                    j = int(rng.integers(0, H))
                    plant(b, int(s), T - 1, j)
                    needle_pos.append((b, int(s)))
        elif needle_mode == "hisa":
            bs = block or extra.get("b", 128)
            nblk = (L + bs - 1) // bs
            half = needles // 2
            for b in range(Bt):
                blocks = rng.choice(nblk, size=1 + (needles - half), replace=False)
                # clustered: `half` distinct positions inside one block
                lo = int(blocks[0]) * bs
                width = min(bs, L - lo)
                for s in lo + rng.choice(width, size=min(half, width), replace=False):
                    j = int(rng.integers(0, H))
                    plant(b, int(s), T - 1, j)
                    needle_pos.append((b, int(s)))
                # scattered: one needle in each of the other blocks
                for m in blocks[1:]:
                    lo = int(m) * bs
                    width = min(bs, L - lo)
                    s = lo + int(rng.integers(0, width))
                    j = int(rng.integers(0, H))
                    plant(b, s, T - 1, j)
                    needle_pos.append((b, s))
        else:
            raise ValueError(needle_mode)
    out = dict(q=q, w=w, K=K, offset=int(offset), Bt=Bt, T=T, L=L, H=H, d=d,
               needle_pos=needle_pos)
    out.update(extra)
    return out


def make_config(name: str, **overrides):
    """Draw a named workload; overrides replace fields (e.g. a smaller L)."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    return make_problem(**cfg)
