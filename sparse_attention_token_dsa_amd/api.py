"""Thin torch binding of the C ABI in include/sa_indexer.h.

Argument marshalling only: tensors are checked for device, dtype and layout,
their data pointers and the current HIP stream are handed to
``libsaindexer.so``, and every step of the selector runs in its HIP kernels.
The library must have been built (``__graft_entry__.build()``); there is no
fallback path.

Tensor conventions (all on one GPU, contiguous):
  q    bf16 [batch, T, H, 128]      (or int16/uint16 holding bf16 bits)
  w    fp32 [batch, T, H]
  keys bf16 [batch, L, 128]
Outputs: idx int32 [batch, T, topk] (set per row, -1 padded) and score fp32.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsaindexer.so")

SA_OK = 0
SA_EINVAL = -1
SA_EUNSUPPORTED = -2
SA_EWORKSPACE = -3
SA_EHIP = -4

# Every symbol include/sa_indexer.h declares.
EXPORTS = (
    "indexer_score_topk_ws", "indexer_score_topk", "sa_pool_blocks", "sa_pool_blocks2",
    "misa_route_ws", "misa_route", "hisa_coarse_fine_ws", "hisa_coarse_fine",
    "sa_last_error", "sa_profile_enable", "sa_profile_read", "sa_kernel_count",
    "sa_kernel_name", "sa_quantize_keys_fp8", "indexer_score_topk_fp8_ws",
    "indexer_score_topk_fp8", "lisa_score_topk_ws", "lisa_score_topk", "sa_block_extrema",
    "resmisa_route_ws", "resmisa_route", "misa_hisa_ws", "misa_hisa", "sa_tidy_indices",
    "indexer_score_topk_ragged_ws", "indexer_score_topk_ragged", "indexer_score_topk_fp8q_ws",
    "indexer_score_topk_fp8q", "misa_route_fp8_ws", "misa_route_fp8", "hisa_coarse_fine_fp8_ws",
    "hisa_coarse_fine_fp8", "indexer_score_topk_fp8_ragged_ws", "indexer_score_topk_fp8_ragged",
)


class SaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "T", "H", "d", "L", "causal_offset", "topk")]


_lib = None


def load():
    """Load libsaindexer.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libsaindexer.so is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    SP = ctypes.POINTER(Shape)
    lib.indexer_score_topk_ws.argtypes = [SP, ctypes.POINTER(S)]
    lib.indexer_score_topk.argtypes = [P, P, P, SP, P, P, P, S, P]
    lib.sa_pool_blocks.argtypes = [P, I, I, I, I, P, P]
    lib.sa_pool_blocks2.argtypes = [P, I, I, I, I, I, P, P, P]
    lib.misa_route_ws.argtypes = [SP, I, I, I, I, ctypes.POINTER(S)]
    lib.misa_route.argtypes = [P, P, P, SP, I, I, I, P, P, P, P, P, P, S, P]
    lib.hisa_coarse_fine_ws.argtypes = [SP, I, I, I, ctypes.POINTER(S)]
    lib.hisa_coarse_fine.argtypes = [P, P, P, SP, I, I, P, P, P, P, P, S, P]
    lib.sa_quantize_keys_fp8.argtypes = [P, I, I, I, P, P, P]
    lib.indexer_score_topk_fp8_ws.argtypes = [SP, ctypes.POINTER(S)]
    lib.indexer_score_topk_fp8.argtypes = [P, P, P, P, SP, P, P, P, S, P]
    lib.misa_route_fp8_ws.argtypes = lib.misa_route_ws.argtypes
    lib.misa_route_fp8.argtypes = [P, P, P, P, SP, I, I, I, P, P, P, P, P, P, S, P]
    lib.hisa_coarse_fine_fp8_ws.argtypes = lib.hisa_coarse_fine_ws.argtypes
    lib.hisa_coarse_fine_fp8.argtypes = [P, P, P, P, SP, I, I, P, P, P, P, P, S, P]
    lib.indexer_score_topk_fp8_ragged_ws.argtypes = [SP, ctypes.POINTER(S)]
    lib.indexer_score_topk_fp8_ragged.argtypes = [P, P, P, P, P, ctypes.c_int64, I, SP, P, P, P,
                                                  S, P]
    lib.indexer_score_topk_fp8q_ws.argtypes = [SP, ctypes.POINTER(S)]
    lib.indexer_score_topk_fp8q.argtypes = [P, P, P, P, SP, P, P, P, S, P]
    lib.sa_tidy_indices.argtypes = [P, I, I, I, P, I, I, I, P, P, P]
    lib.indexer_score_topk_ragged_ws.argtypes = [SP, ctypes.POINTER(S)]
    lib.indexer_score_topk_ragged.argtypes = [P, P, P, P, ctypes.c_int64, SP, P, P, P, S, P]
    lib.misa_hisa_ws.argtypes = [SP, I, I, I, I, I, I, ctypes.POINTER(S)]
    lib.misa_hisa.argtypes = [P, P, P, SP, I, I, I, I, P, P, P, P, P, P, P, S, P]
    lib.lisa_score_topk_ws.argtypes = [SP, ctypes.POINTER(S)]
    lib.lisa_score_topk.argtypes = [P, P, P, SP, P, P, P, S, P]
    lib.sa_block_extrema.argtypes = [P, I, I, I, I, P, P]
    lib.resmisa_route_ws.argtypes = [SP, I, I, I, ctypes.POINTER(S)]
    lib.resmisa_route.argtypes = [P, P, P, SP, I, I, P, P, P, P, P, S, P]
    lib.sa_last_error.restype = ctypes.c_char_p
    lib.sa_profile_enable.argtypes = [I]
    lib.sa_profile_read.argtypes = [I, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)]
    lib.sa_kernel_count.restype = I
    lib.sa_kernel_name.argtypes = [I]
    lib.sa_kernel_name.restype = ctypes.c_char_p
    for name in ("indexer_score_topk_ws", "indexer_score_topk", "sa_pool_blocks",
                 "sa_pool_blocks2", "misa_route_ws", "misa_route", "hisa_coarse_fine_ws",
                 "hisa_coarse_fine", "sa_profile_enable", "sa_profile_read",
                 "sa_quantize_keys_fp8", "indexer_score_topk_fp8_ws", "indexer_score_topk_fp8",
                 "lisa_score_topk_ws", "lisa_score_topk", "sa_block_extrema", "resmisa_route_ws",
                 "resmisa_route", "misa_hisa_ws", "misa_hisa", "sa_tidy_indices",
                 "indexer_score_topk_ragged_ws", "indexer_score_topk_ragged",
                 "indexer_score_topk_fp8q_ws", "indexer_score_topk_fp8q", "misa_route_fp8_ws",
                 "misa_route_fp8", "hisa_coarse_fine_fp8_ws", "hisa_coarse_fine_fp8",
                 "indexer_score_topk_fp8_ragged_ws", "indexer_score_topk_fp8_ragged"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc, name):
    if rc != SA_OK:
        msg = load().sa_last_error().decode(errors="replace")
        raise SaError(rc, "%s: %s" % (name, msg))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _bf16(t, name, ndim):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("%s must hold bf16 bits (bfloat16/int16/uint16), got %s" % (name, t.dtype))
    if t.dim() != ndim or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %d-d GPU tensor" % (name, ndim))
    return t


def _shape(q, w, keys, causal_offset, topk):
    _bf16(q, "q", 4)
    _bf16(keys, "keys", 3)
    if w.dtype != torch.float32 or not w.is_cuda or not w.is_contiguous():
        raise TypeError("w must be a contiguous float32 GPU tensor")
    B, T, H, d = q.shape
    if tuple(w.shape) != (B, T, H) or keys.shape[0] != B or keys.shape[2] != d:
        raise ValueError("shapes disagree: q %s w %s keys %s" % (tuple(q.shape), tuple(w.shape),
                                                                  tuple(keys.shape)))
    if not (q.device == w.device == keys.device):
        raise ValueError("q, w and keys must be on one device")
    return Shape(B, T, H, d, keys.shape[1], int(causal_offset), int(topk))


def _outputs(q, topk, out_idx, out_score, want_score):
    B, T = q.shape[0], q.shape[1]
    if out_idx is None:
        out_idx = torch.empty((B, T, topk), dtype=torch.int32, device=q.device)
    if out_score is None and want_score:
        out_score = torch.empty((B, T, topk), dtype=torch.float32, device=q.device)
    return out_idx, out_score


def _workspace(nbytes, device, ws):
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small: %d < %d" % (ws.numel() * ws.element_size(),
                                                              nbytes))
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def indexer_score_topk_ws(shape: Shape) -> int:
    n = ctypes.c_size_t()
    _check(load().indexer_score_topk_ws(ctypes.byref(shape), ctypes.byref(n)),
           "indexer_score_topk_ws")
    return n.value


def indexer_score_topk(q, w, keys, causal_offset, topk, out_idx=None, out_score=None,
                       want_score=True, ws=None):
    """DSA lightning indexer: causal scores with all heads + token top-k."""
    s = _shape(q, w, keys, causal_offset, topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(indexer_score_topk_ws(s), q.device, ws)
    _check(load().indexer_score_topk(_p(q), _p(w), _p(keys), ctypes.byref(s), _p(out_idx),
                                     _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
           "indexer_score_topk")
    return out_idx, out_score


def pool_blocks(keys, block, out=None):
    """Block means of keys -> [batch, ceil(L/block), 2, 128] bf16 hi/lo pairs."""
    _bf16(keys, "keys", 3)
    B, L, d = keys.shape
    nb = (L + block - 1) // block
    if out is None:
        out = torch.empty((B, nb, 2, d), dtype=torch.int16, device=keys.device)
    _check(load().sa_pool_blocks(_p(keys), B, L, d, int(block), _p(out), _stream(keys.device)),
           "sa_pool_blocks")
    return out


def pool_blocks2(keys, small, large, out_small=None, out_large=None):
    """Both block pools in one pass over the keys."""
    _bf16(keys, "keys", 3)
    B, L, d = keys.shape
    if out_small is None:
        out_small = torch.empty((B, (L + small - 1) // small, 2, d), dtype=torch.int16,
                                device=keys.device)
    if out_large is None:
        out_large = torch.empty((B, (L + large - 1) // large, 2, d), dtype=torch.int16,
                                device=keys.device)
    _check(load().sa_pool_blocks2(_p(keys), B, L, d, int(small), int(large), _p(out_small),
                                  _p(out_large), _stream(keys.device)), "sa_pool_blocks2")
    return out_small, out_large


def misa_route_ws(shape: Shape, block_B, h, k_prime, pooled_given) -> int:
    n = ctypes.c_size_t()
    _check(load().misa_route_ws(ctypes.byref(shape), int(block_B), int(h), int(k_prime),
                                int(bool(pooled_given)), ctypes.byref(n)), "misa_route_ws")
    return n.value


def misa_route(q, w, keys, causal_offset, topk, block_B, h, k_prime=0, pooled=None,
               want_heads=True, want_pool=False, out_idx=None, out_score=None,
               want_score=True, ws=None):
    """MISA routed indexer (k_prime=0) or MISA-dagger (k_prime >= topk).
    Returns (idx, score, heads, pool)."""
    s = _shape(q, w, keys, causal_offset, topk)
    B, T = q.shape[0], q.shape[1]
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    heads = torch.empty((B, T, h), dtype=torch.int32, device=q.device) if want_heads else None
    pool = (torch.empty((B, T, k_prime), dtype=torch.int32, device=q.device)
            if (want_pool and k_prime) else None)
    ws = _workspace(misa_route_ws(s, block_B, h, k_prime, pooled is not None), q.device, ws)
    _check(load().misa_route(_p(q), _p(w), _p(keys), ctypes.byref(s), int(block_B), int(h),
                             int(k_prime), _p(pooled), _p(heads), _p(pool), _p(out_idx),
                             _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
           "misa_route")
    return out_idx, out_score, heads, pool


def hisa_coarse_fine_ws(shape: Shape, block_b, r, reps_given) -> int:
    n = ctypes.c_size_t()
    _check(load().hisa_coarse_fine_ws(ctypes.byref(shape), int(block_b), int(r),
                                      int(bool(reps_given)), ctypes.byref(n)),
           "hisa_coarse_fine_ws")
    return n.value


def hisa_coarse_fine(q, w, keys, causal_offset, topk, block_b, r, reps=None,
                     want_blocks=True, out_idx=None, out_score=None, want_score=True, ws=None):
    """HISA block-then-token search.  Returns (idx, score, blocks)."""
    s = _shape(q, w, keys, causal_offset, topk)
    B, T = q.shape[0], q.shape[1]
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    blocks = torch.empty((B, T, r), dtype=torch.int32, device=q.device) if want_blocks else None
    ws = _workspace(hisa_coarse_fine_ws(s, block_b, r, reps is not None), q.device, ws)
    _check(load().hisa_coarse_fine(_p(q), _p(w), _p(keys), ctypes.byref(s), int(block_b),
                                   int(r), _p(reps), _p(blocks), _p(out_idx), _p(out_score),
                                   _p(ws), ws.numel(), _stream(q.device)), "hisa_coarse_fine")
    return out_idx, out_score, blocks


# ------------------------------------------------------------- FP8 keys

def quantize_keys_fp8(keys, out_codes=None, out_scales=None):
    """Per-key E4M3 codes and fp32 scales: codes uint8 [batch, L, 128],
    scales fp32 [batch, L] with key = scale * decode(codes)."""
    _bf16(keys, "keys", 3)
    B, L, d = keys.shape
    if out_codes is None:
        out_codes = torch.empty((B, L, d), dtype=torch.uint8, device=keys.device)
    if out_scales is None:
        out_scales = torch.empty((B, L), dtype=torch.float32, device=keys.device)
    _check(load().sa_quantize_keys_fp8(_p(keys), B, L, d, _p(out_codes), _p(out_scales),
                                       _stream(keys.device)), "sa_quantize_keys_fp8")
    return out_codes, out_scales


def _fp8_shape(q, w, codes, scales, causal_offset, topk):
    _bf16(q, "q", 4)
    if codes.dtype != torch.uint8 or codes.dim() != 3 or not codes.is_cuda \
            or not codes.is_contiguous():
        raise TypeError("codes must be a contiguous uint8 [batch, L, 128] GPU tensor")
    if scales.dtype != torch.float32 or not scales.is_cuda or not scales.is_contiguous():
        raise TypeError("scales must be a contiguous float32 GPU tensor")
    if w.dtype != torch.float32 or not w.is_cuda or not w.is_contiguous():
        raise TypeError("w must be a contiguous float32 GPU tensor")
    B, T, H, d = q.shape
    if tuple(w.shape) != (B, T, H) or codes.shape[0] != B or codes.shape[2] != d \
            or tuple(scales.shape) != tuple(codes.shape[:2]):
        raise ValueError("shapes disagree: q %s w %s codes %s scales %s"
                         % (tuple(q.shape), tuple(w.shape), tuple(codes.shape),
                            tuple(scales.shape)))
    if not (q.device == w.device == codes.device == scales.device):
        raise ValueError("q, w, codes and scales must be on one device")
    return Shape(B, T, H, d, codes.shape[1], int(causal_offset), int(topk))


def indexer_score_topk_fp8_ws(shape: Shape) -> int:
    n = ctypes.c_size_t()
    _check(load().indexer_score_topk_fp8_ws(ctypes.byref(shape), ctypes.byref(n)),
           "indexer_score_topk_fp8_ws")
    return n.value


def indexer_score_topk_fp8(q, w, codes, scales, causal_offset, topk, out_idx=None,
                           out_score=None, want_score=True, ws=None):
    """DSA indexer over E4M3 keys with per-key scales (rows T < 16)."""
    s = _fp8_shape(q, w, codes, scales, causal_offset, topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(indexer_score_topk_fp8_ws(s), q.device, ws)
    _check(load().indexer_score_topk_fp8(_p(q), _p(w), _p(codes), _p(scales), ctypes.byref(s),
                                         _p(out_idx), _p(out_score), _p(ws), ws.numel(),
                                         _stream(q.device)), "indexer_score_topk_fp8")
    return out_idx, out_score


def indexer_score_topk_fp8q_ws(shape: Shape) -> int:
    n = ctypes.c_size_t()
    _check(load().indexer_score_topk_fp8q_ws(ctypes.byref(shape), ctypes.byref(n)),
           "indexer_score_topk_fp8q_ws")
    return n.value


def indexer_score_topk_fp8q(q, w, codes, scales, causal_offset, topk, out_idx=None,
                            out_score=None, want_score=True, ws=None):
    """As indexer_score_topk_fp8 with the query converted to E4M3 in the
    kernel (per-head scale) and the dot products on the fp8 MFMA."""
    s = _fp8_shape(q, w, codes, scales, causal_offset, topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(indexer_score_topk_fp8q_ws(s), q.device, ws)
    _check(load().indexer_score_topk_fp8q(_p(q), _p(w), _p(codes), _p(scales), ctypes.byref(s),
                                          _p(out_idx), _p(out_score), _p(ws), ws.numel(),
                                          _stream(q.device)), "indexer_score_topk_fp8q")
    return out_idx, out_score


def indexer_score_topk_fp8_ragged(q, w, codes, scales, seq_lens, topk, total_len=0, q_fp8=False,
                                  out_idx=None, out_score=None, want_score=True, ws=None):
    """Ragged batches over an FP8 key cache (capacity codes.shape[1]); q_fp8
    picks the E4M3-query scores of indexer_score_topk_fp8q."""
    if seq_lens.dtype != torch.int32 or not seq_lens.is_cuda or seq_lens.numel() != q.shape[0]:
        raise TypeError("seq_lens must be an int32 GPU tensor with one entry per sequence")
    s = _fp8_shape(q, w, codes, scales, codes.shape[1] - q.shape[1], topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    n = ctypes.c_size_t()
    _check(load().indexer_score_topk_fp8_ragged_ws(ctypes.byref(s), ctypes.byref(n)),
           "indexer_score_topk_fp8_ragged_ws")
    ws = _workspace(n.value, q.device, ws)
    _check(load().indexer_score_topk_fp8_ragged(_p(q), _p(w), _p(codes), _p(scales),
                                                _p(seq_lens.contiguous()), int(total_len),
                                                int(bool(q_fp8)), ctypes.byref(s), _p(out_idx),
                                                _p(out_score), _p(ws), ws.numel(),
                                                _stream(q.device)),
           "indexer_score_topk_fp8_ragged")
    return out_idx, out_score


def misa_route_fp8(q, w, codes, scales, causal_offset, topk, block_B, h, k_prime=0, pooled=None,
                   want_heads=True, want_pool=False, out_idx=None, out_score=None,
                   want_score=True, ws=None):
    """misa_route over an FP8 key cache.  Returns (idx, score, heads, pool)."""
    s = _fp8_shape(q, w, codes, scales, causal_offset, topk)
    B, T = q.shape[0], q.shape[1]
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    heads = torch.empty((B, T, h), dtype=torch.int32, device=q.device) if want_heads else None
    pool = (torch.empty((B, T, k_prime), dtype=torch.int32, device=q.device)
            if (want_pool and k_prime) else None)
    n = ctypes.c_size_t()
    _check(load().misa_route_fp8_ws(ctypes.byref(s), int(block_B), int(h), int(k_prime),
                                    int(pooled is not None), ctypes.byref(n)), "misa_route_fp8_ws")
    ws = _workspace(n.value, q.device, ws)
    _check(load().misa_route_fp8(_p(q), _p(w), _p(codes), _p(scales), ctypes.byref(s),
                                 int(block_B), int(h), int(k_prime), _p(pooled), _p(heads),
                                 _p(pool), _p(out_idx), _p(out_score), _p(ws), ws.numel(),
                                 _stream(q.device)), "misa_route_fp8")
    return out_idx, out_score, heads, pool


def hisa_coarse_fine_fp8(q, w, codes, scales, causal_offset, topk, block_b, r, reps=None,
                         want_blocks=True, out_idx=None, out_score=None, want_score=True,
                         ws=None):
    """hisa_coarse_fine over an FP8 key cache.  Returns (idx, score, blocks)."""
    s = _fp8_shape(q, w, codes, scales, causal_offset, topk)
    B, T = q.shape[0], q.shape[1]
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    blocks = torch.empty((B, T, r), dtype=torch.int32, device=q.device) if want_blocks else None
    n = ctypes.c_size_t()
    _check(load().hisa_coarse_fine_fp8_ws(ctypes.byref(s), int(block_b), int(r),
                                          int(reps is not None), ctypes.byref(n)),
           "hisa_coarse_fine_fp8_ws")
    ws = _workspace(n.value, q.device, ws)
    _check(load().hisa_coarse_fine_fp8(_p(q), _p(w), _p(codes), _p(scales), ctypes.byref(s),
                                       int(block_b), int(r), _p(reps), _p(blocks), _p(out_idx),
                                       _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
           "hisa_coarse_fine_fp8")
    return out_idx, out_score, blocks


# ------------------------------------------------- tidy-up, ragged rows

def tidy_indices(idx, T, block_table=None, page_size=1, max_slots=0, out_slots=None,
                 out_stats=None, want_stats=True):
    """Selected positions [batch, T, k] (or [rows, k]) -> distinct physical
    slots in ascending order, -1 padded, and per-row (slots, pages, runs)."""
    if idx.dtype != torch.int32 or not idx.is_cuda or not idx.is_contiguous():
        raise TypeError("idx must be a contiguous int32 GPU tensor")
    k = idx.shape[-1]
    rows = idx.numel() // k
    if block_table is not None:
        if (block_table.dtype != torch.int32 or not block_table.is_cuda
                or not block_table.is_contiguous() or block_table.dim() != 2):
            raise TypeError("block_table must be a contiguous int32 [batch, pages] GPU tensor")
        if block_table.shape[0] * int(T) != rows:
            raise ValueError("block_table needs one row per sequence (rows / T = %d), has %d"
                             % (rows // int(T), block_table.shape[0]))
    if out_slots is None:
        out_slots = torch.empty_like(idx)
    if out_stats is None and want_stats:
        out_stats = torch.empty(idx.shape[:-1] + (3,), dtype=torch.int32, device=idx.device)
    _check(load().sa_tidy_indices(_p(idx), rows, int(T), k, _p(block_table),
                                  0 if block_table is None else block_table.shape[1],
                                  int(page_size), int(max_slots), _p(out_slots), _p(out_stats),
                                  _stream(idx.device)), "sa_tidy_indices")
    return out_slots, out_stats


def indexer_score_topk_ragged_ws(shape: Shape) -> int:
    n = ctypes.c_size_t()
    _check(load().indexer_score_topk_ragged_ws(ctypes.byref(shape), ctypes.byref(n)),
           "indexer_score_topk_ragged_ws")
    return n.value


def indexer_score_topk_ragged(q, w, keys, seq_lens, topk, total_len=0, out_idx=None,
                              out_score=None, want_score=True, ws=None):
    """DSA over sequences of different lengths: keys [batch, L_cap, 128],
    seq_lens int32 [batch] on the GPU; row i of sequence b sits at
    seq_lens[b] - T + i.  total_len: the host's sum of the lengths (0 if
    unknown), used only to size the work per workgroup."""
    if seq_lens.dtype != torch.int32 or not seq_lens.is_cuda or seq_lens.numel() != q.shape[0]:
        raise TypeError("seq_lens must be an int32 GPU tensor with one entry per sequence")
    s = _shape(q, w, keys, keys.shape[1] - q.shape[1], topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(indexer_score_topk_ragged_ws(s), q.device, ws)
    _check(load().indexer_score_topk_ragged(_p(q), _p(w), _p(keys), _p(seq_lens.contiguous()),
                                            int(total_len), ctypes.byref(s), _p(out_idx), _p(out_score), _p(ws),
                                            ws.numel(), _stream(q.device)),
           "indexer_score_topk_ragged")
    return out_idx, out_score


# ---------------------------------------------------------- MISA x HISA

def misa_hisa_ws(shape: Shape, block_B, h, block_b, r, pooled_given, reps_given) -> int:
    n = ctypes.c_size_t()
    _check(load().misa_hisa_ws(ctypes.byref(shape), int(block_B), int(h), int(block_b), int(r),
                               int(bool(pooled_given)), int(bool(reps_given)), ctypes.byref(n)),
           "misa_hisa_ws")
    return n.value


def misa_hisa(q, w, keys, causal_offset, topk, block_B, h, block_b, r, pooled=None, reps=None,
              want_heads=True, want_blocks=True, out_heads=None, out_blocks=None, out_idx=None,
              out_score=None, want_score=True, ws=None):
    """MISA router heads -> HISA block scores over those heads -> every-head
    rescoring of the r best blocks' tokens.  Returns (idx, score, heads, blocks)."""
    s = _shape(q, w, keys, causal_offset, topk)
    B, T = q.shape[0], q.shape[1]
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    heads = out_heads
    if heads is None and want_heads:
        heads = torch.empty((B, T, h), dtype=torch.int32, device=q.device)
    blocks = out_blocks
    if blocks is None and want_blocks:
        blocks = torch.empty((B, T, r), dtype=torch.int32, device=q.device)
    ws = _workspace(misa_hisa_ws(s, block_B, h, block_b, r, pooled is not None, reps is not None),
                    q.device, ws)
    _check(load().misa_hisa(_p(q), _p(w), _p(keys), ctypes.byref(s), int(block_B), int(h),
                            int(block_b), int(r), _p(pooled), _p(reps), _p(heads), _p(blocks),
                            _p(out_idx), _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
           "misa_hisa")
    return out_idx, out_score, heads, blocks


# ------------------------------------------------------- LISA / ResMiSA

def lisa_score_topk_ws(shape: Shape) -> int:
    n = ctypes.c_size_t()
    _check(load().lisa_score_topk_ws(ctypes.byref(shape), ctypes.byref(n)), "lisa_score_topk_ws")
    return n.value


def lisa_score_topk(q, w, keys, causal_offset, topk, out_idx=None, out_score=None,
                    want_score=True, ws=None):
    """LISA: top-k by the linear score g . k, g = sum_j w_j q_j."""
    s = _shape(q, w, keys, causal_offset, topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(lisa_score_topk_ws(s), q.device, ws)
    _check(load().lisa_score_topk(_p(q), _p(w), _p(keys), ctypes.byref(s), _p(out_idx),
                                  _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
           "lisa_score_topk")
    return out_idx, out_score


def block_extrema(keys, block, out=None):
    """Per-block key max then min -> [batch, ceil(L/block), 2, 128] bf16 bits."""
    _bf16(keys, "keys", 3)
    B, L, d = keys.shape
    nb = (L + block - 1) // block
    if out is None:
        out = torch.empty((B, nb, 2, d), dtype=torch.int16, device=keys.device)
    _check(load().sa_block_extrema(_p(keys), B, L, d, int(block), _p(out), _stream(keys.device)),
           "sa_block_extrema")
    return out


def resmisa_route_ws(shape: Shape, block, r, extrema_given) -> int:
    n = ctypes.c_size_t()
    _check(load().resmisa_route_ws(ctypes.byref(shape), int(block), int(r),
                                   int(bool(extrema_given)), ctypes.byref(n)), "resmisa_route_ws")
    return n.value


def resmisa_route(q, w, keys, causal_offset, topk, block, r, extrema=None, want_heads=True,
                  out_heads=None, out_idx=None, out_score=None, want_score=True, ws=None):
    """ResMiSA: shared linear score + r routed residual heads.  Returns
    (idx, score, heads)."""
    s = _shape(q, w, keys, causal_offset, topk)
    B, T = q.shape[0], q.shape[1]
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    heads = out_heads
    if heads is None and want_heads and r > 0:
        heads = torch.empty((B, T, r), dtype=torch.int32, device=q.device)
    ws = _workspace(resmisa_route_ws(s, block, r, extrema is not None), q.device, ws)
    _check(load().resmisa_route(_p(q), _p(w), _p(keys), ctypes.byref(s), int(block), int(r),
                                _p(extrema), _p(heads), _p(out_idx), _p(out_score), _p(ws),
                                ws.numel(), _stream(q.device)), "resmisa_route")
    return out_idx, out_score, heads


# ------------------------------------------------------------ diagnostics

def kernel_names():
    lib = load()
    return [lib.sa_kernel_name(i).decode() for i in range(lib.sa_kernel_count())]


def profile_enable(on=True):
    _check(load().sa_profile_enable(1 if on else 0), "sa_profile_enable")


def profile_read():
    """{kernel name: (total_ms, launches)} for every kernel with launches."""
    lib = load()
    out = {}
    for i, name in enumerate(kernel_names()):
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        _check(lib.sa_profile_read(i, ctypes.byref(ms), ctypes.byref(n)), "sa_profile_read")
        if n.value:
            out[name] = (ms.value, n.value)
    return out


def last_error():
    return load().sa_last_error().decode(errors="replace")
