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
    "indexer_score_topk_noalloc", "indexer_score_topk_pooled_ws", "indexer_score_topk_pooled",
    "indexer_score_topk_pooled_phase", "misa_route_phase",
)

# Bytes of the static device scratch behind indexer_score_topk_noalloc
# (SA_NOALLOC_SCRATCH_BYTES in include/sa_indexer.h).
NOALLOC_SCRATCH_BYTES = 32 << 20


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
    lib.indexer_score_topk_noalloc.argtypes = [P, P, P, SP, P, P, P]
    lib.indexer_score_topk_pooled_ws.argtypes = [SP, I, I, ctypes.POINTER(S)]
    lib.indexer_score_topk_pooled.argtypes = [P, P, P, SP, I, I, P, P, P, P, P, S, P, P]
    lib.indexer_score_topk_pooled_phase.argtypes = [P, P, P, SP, I, I, P, P, P, P, P, S, I, P]
    lib.sa_pool_blocks.argtypes = [P, I, I, I, I, P, P]
    lib.sa_pool_blocks2.argtypes = [P, I, I, I, I, I, P, P, P]
    lib.misa_route_ws.argtypes = [SP, I, I, I, I, ctypes.POINTER(S)]
    lib.misa_route.argtypes = [P, P, P, SP, I, I, I, P, P, P, P, P, P, S, P]
    lib.misa_route_phase.argtypes = [P, P, P, SP, I, I, I, P, P, P, P, P, P, S, I, P]
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
                 "indexer_score_topk_fp8_ragged_ws", "indexer_score_topk_fp8_ragged",
                 "indexer_score_topk_noalloc", "indexer_score_topk_pooled_ws",
                 "indexer_score_topk_pooled"):
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


def _event(ev, dev):
    """Raw hipEvent_t of a torch.cuda.Event (created on first use), or None."""
    if ev is None:
        return None
    if not isinstance(ev, torch.cuda.Event):
        raise TypeError("pools_ready must be a torch.cuda.Event")
    if not ev.cuda_event:
        ev.record(torch.cuda.current_stream(dev))  # creates the event
    return ctypes.c_void_p(ev.cuda_event)


BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _bf16(t, name, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.dtype not in BF16:
        raise TypeError("%s must hold bf16 bits (bfloat16/int16/uint16), got %s" % (name, t.dtype))
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %d-d tensor" % (name, ndim))
    return t


def _tensor(t, name, dtypes, shape, device):
    """Check a caller-supplied tensor the library will read or write through a
    raw pointer: dtype, exact shape, contiguity and device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s must be %s, got %s" % (name, "/".join(str(d) for d in dtypes),
                                                   t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    return t


def _opt(t, name, dtypes, shape, device):
    return None if t is None else _tensor(t, name, dtypes, shape, device)


def _gpu(t):
    """Every pointer handed to the library must be device memory."""
    if not t.is_cuda:
        raise ValueError("tensors must be on a GPU (got %s)" % t.device)


def _blocks(L, blk):
    return (L + int(blk) - 1) // int(blk)


def _shape(q, w, keys, causal_offset, topk):
    _bf16(q, "q", 4)
    _bf16(keys, "keys", 3)
    B, T, H, d = q.shape
    _tensor(w, "w", (torch.float32,), (B, T, H), q.device)
    if keys.shape[0] != B or keys.shape[2] != d:
        raise ValueError("shapes disagree: q %s w %s keys %s" % (tuple(q.shape), tuple(w.shape),
                                                                  tuple(keys.shape)))
    if keys.device != q.device:
        raise ValueError("q, w and keys must be on one device")
    return Shape(B, T, H, d, keys.shape[1], int(causal_offset), int(topk))


def _outputs(q, topk, out_idx, out_score, want_score):
    B, T = q.shape[0], q.shape[1]
    if out_idx is None:
        out_idx = torch.empty((B, T, topk), dtype=torch.int32, device=q.device)
    else:
        _tensor(out_idx, "out_idx", (torch.int32,), (B, T, topk), q.device)
    if out_score is None and want_score:
        out_score = torch.empty((B, T, topk), dtype=torch.float32, device=q.device)
    elif out_score is not None:
        _tensor(out_score, "out_score", (torch.float32,), (B, T, topk), q.device)
    return out_idx, out_score


def _workspace(nbytes, device, ws):
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8:
            raise TypeError("ws must be a uint8 tensor")
        if not ws.is_contiguous() or ws.device != device:
            raise ValueError("ws must be contiguous and on %s" % device)
        if ws.numel() < nbytes:
            raise ValueError("workspace too small: %d < %d" % (ws.numel(), nbytes))
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _seq_lens(seq_lens, B, device):
    return _tensor(seq_lens, "seq_lens", (torch.int32,), (B,), device)


def _ws_query(fn, name, *args):
    n = ctypes.c_size_t()
    _check(fn(*args, ctypes.byref(n)), name)
    return n.value


def indexer_score_topk_ws(shape: Shape) -> int:
    return _ws_query(load().indexer_score_topk_ws, "indexer_score_topk_ws", ctypes.byref(shape))


def indexer_score_topk(q, w, keys, causal_offset, topk, out_idx=None, out_score=None,
                       want_score=True, ws=None):
    """DSA lightning indexer: causal scores with all heads + token top-k."""
    s = _shape(q, w, keys, causal_offset, topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(indexer_score_topk_ws(s), q.device, ws)
    _gpu(q)
    _check(load().indexer_score_topk(_p(q), _p(w), _p(keys), ctypes.byref(s), _p(out_idx),
                                     _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
           "indexer_score_topk")
    return out_idx, out_score


def indexer_score_topk_noalloc(q, w, keys, causal_offset, topk, out_idx, out_score=None):
    """indexer_score_topk with the library's static device scratch in place of
    a workspace: the call allocates nothing, so out_idx (and out_score, or
    None) must be given.  Calls that overlap on one GPU race (they share the
    scratch); shapes needing more than NOALLOC_SCRATCH_BYTES are rejected."""
    s = _shape(q, w, keys, causal_offset, topk)
    if out_idx is None:
        raise ValueError("indexer_score_topk_noalloc allocates nothing: pass out_idx")
    _outputs(q, topk, out_idx, out_score, False)
    _gpu(q)
    _check(load().indexer_score_topk_noalloc(_p(q), _p(w), _p(keys), ctypes.byref(s),
                                             _p(out_idx), _p(out_score), _stream(q.device)),
           "indexer_score_topk_noalloc")
    return out_idx, out_score


def indexer_score_topk_pooled_ws(shape: Shape, small, large) -> int:
    return _ws_query(load().indexer_score_topk_pooled_ws, "indexer_score_topk_pooled_ws",
                     ctypes.byref(shape), int(small), int(large))


# Phases of the decode selectors (SA_PHASE_SCAN, SA_PHASE_SELECT; both = the
# whole call).  The select call repeats the scan call's arguments, outputs
# and workspace.
PHASE_SCAN, PHASE_SELECT, PHASE_ALL = 1, 2, 3


def _phases(phases):
    if phases not in (PHASE_SCAN, PHASE_SELECT, PHASE_ALL):
        raise ValueError("phases must be PHASE_SCAN, PHASE_SELECT or PHASE_ALL")
    return int(phases)


def indexer_score_topk_pooled(q, w, keys, causal_offset, topk, small, large, out_small=None,
                              out_large=None, out_idx=None, out_score=None, want_score=True,
                              ws=None, pools_ready=None, phases=PHASE_ALL):
    """DSA decode selector that also writes the block means of the keys
    (sa_pool_blocks2 layout) in the same pass.  pools_ready: a
    torch.cuda.Event recorded on the current stream once the means are
    written (before the call's top-k kernels).  phases: PHASE_SCAN and then
    PHASE_SELECT split the call in two (same arguments and workspace).
    Returns (idx, score, small pools, large pools)."""
    phases = _phases(phases)
    if phases != PHASE_ALL and pools_ready is not None:
        raise ValueError("pools_ready belongs to the whole call (phases=PHASE_ALL)")
    if phases != PHASE_ALL and ws is None:
        raise ValueError("a call in phases needs the caller's workspace (ws)")
    s = _shape(q, w, keys, causal_offset, topk)
    out_small = _reps_out(keys, small, out_small, "out_small")
    out_large = _reps_out(keys, large, out_large, "out_large")
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(indexer_score_topk_pooled_ws(s, small, large), q.device, ws)
    _gpu(q)
    if phases == PHASE_ALL:
        _check(load().indexer_score_topk_pooled(_p(q), _p(w), _p(keys), ctypes.byref(s),
                                                int(small), int(large), _p(out_small),
                                                _p(out_large), _p(out_idx), _p(out_score), _p(ws),
                                                ws.numel(), _event(pools_ready, q.device),
                                                _stream(q.device)),
               "indexer_score_topk_pooled")
    else:
        _check(load().indexer_score_topk_pooled_phase(_p(q), _p(w), _p(keys), ctypes.byref(s),
                                                      int(small), int(large), _p(out_small),
                                                      _p(out_large), _p(out_idx),
                                                      _p(out_score), _p(ws), ws.numel(), phases,
                                                      _stream(q.device)),
               "indexer_score_topk_pooled_phase")
    return out_idx, out_score, out_small, out_large


def _reps_out(keys, block, out, name):
    B, L, d = keys.shape
    shape = (B, _blocks(L, block), 2, d)
    if out is None:
        return torch.empty(shape, dtype=torch.int16, device=keys.device)
    return _tensor(out, name, BF16, shape, keys.device)


def pool_blocks(keys, block, out=None):
    """Block means of keys -> [batch, ceil(L/block), 2, 128] bf16 hi/lo pairs."""
    _bf16(keys, "keys", 3)
    if int(block) < 1:
        raise ValueError("block must be >= 1")
    B, L, d = keys.shape
    out = _reps_out(keys, block, out, "out")
    _gpu(keys)
    _check(load().sa_pool_blocks(_p(keys), B, L, d, int(block), _p(out), _stream(keys.device)),
           "sa_pool_blocks")
    return out


def pool_blocks2(keys, small, large, out_small=None, out_large=None):
    """Both block pools in one pass over the keys."""
    _bf16(keys, "keys", 3)
    if int(small) < 1 or int(large) < 1:
        raise ValueError("block sizes must be >= 1")
    B, L, d = keys.shape
    out_small = _reps_out(keys, small, out_small, "out_small")
    out_large = _reps_out(keys, large, out_large, "out_large")
    _gpu(keys)
    _check(load().sa_pool_blocks2(_p(keys), B, L, d, int(small), int(large), _p(out_small),
                                  _p(out_large), _stream(keys.device)), "sa_pool_blocks2")
    return out_small, out_large


def _reps_in(t, name, q, L, block):
    """Block representatives given by the caller: [batch, ceil(L/block), 2, 128]."""
    if t is None:
        return None
    if int(block) < 1:
        raise ValueError("block size must be >= 1")
    return _tensor(t, name, BF16, (q.shape[0], _blocks(L, block), 2, q.shape[3]), q.device)


def _rows_out(t, name, q, n, want):
    """int32 [batch, T, n] per-row output (heads, blocks, pool), or None."""
    if t is not None:
        return _tensor(t, name, (torch.int32,), (q.shape[0], q.shape[1], n), q.device)
    if want and n > 0:
        return torch.empty((q.shape[0], q.shape[1], n), dtype=torch.int32, device=q.device)
    return None


def misa_route_ws(shape: Shape, block_B, h, k_prime, pooled_given) -> int:
    return _ws_query(load().misa_route_ws, "misa_route_ws", ctypes.byref(shape), int(block_B),
                     int(h), int(k_prime), int(bool(pooled_given)))


def misa_route(q, w, keys, causal_offset, topk, block_B, h, k_prime=0, pooled=None,
               want_heads=True, want_pool=False, out_idx=None, out_score=None,
               want_score=True, ws=None, out_heads=None, out_pool=None, phases=PHASE_ALL):
    """MISA routed indexer (k_prime=0) or MISA-dagger (k_prime >= topk).
    phases: PHASE_SCAN and then PHASE_SELECT split the call in two (decode
    rows with whole pooling blocks; same arguments, outputs and workspace).
    Returns (idx, score, heads, pool)."""
    phases = _phases(phases)
    if phases != PHASE_ALL and ws is None:
        raise ValueError("a call in phases needs the caller's workspace (ws)")
    s = _shape(q, w, keys, causal_offset, topk)
    pooled = _reps_in(pooled, "pooled", q, s.L, block_B)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    heads = _rows_out(out_heads, "out_heads", q, int(h), want_heads)
    pool = _rows_out(out_pool, "out_pool", q, int(k_prime), want_pool) if k_prime else None
    ws = _workspace(misa_route_ws(s, block_B, h, k_prime, pooled is not None), q.device, ws)
    _gpu(q)
    if phases == PHASE_ALL:
        _check(load().misa_route(_p(q), _p(w), _p(keys), ctypes.byref(s), int(block_B), int(h),
                                 int(k_prime), _p(pooled), _p(heads), _p(pool), _p(out_idx),
                                 _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
               "misa_route")
    else:
        _check(load().misa_route_phase(_p(q), _p(w), _p(keys), ctypes.byref(s), int(block_B),
                                       int(h), int(k_prime), _p(pooled), _p(heads), _p(pool),
                                       _p(out_idx), _p(out_score), _p(ws), ws.numel(), phases,
                                       _stream(q.device)),
               "misa_route_phase")
    return out_idx, out_score, heads, pool


def hisa_coarse_fine_ws(shape: Shape, block_b, r, reps_given) -> int:
    return _ws_query(load().hisa_coarse_fine_ws, "hisa_coarse_fine_ws", ctypes.byref(shape),
                     int(block_b), int(r), int(bool(reps_given)))


def hisa_coarse_fine(q, w, keys, causal_offset, topk, block_b, r, reps=None,
                     want_blocks=True, out_idx=None, out_score=None, want_score=True, ws=None,
                     out_blocks=None):
    """HISA block-then-token search.  Returns (idx, score, blocks)."""
    s = _shape(q, w, keys, causal_offset, topk)
    reps = _reps_in(reps, "reps", q, s.L, block_b)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    blocks = _rows_out(out_blocks, "out_blocks", q, int(r), want_blocks)
    ws = _workspace(hisa_coarse_fine_ws(s, block_b, r, reps is not None), q.device, ws)
    _gpu(q)
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
    else:
        _tensor(out_codes, "out_codes", (torch.uint8,), (B, L, d), keys.device)
    if out_scales is None:
        out_scales = torch.empty((B, L), dtype=torch.float32, device=keys.device)
    else:
        _tensor(out_scales, "out_scales", (torch.float32,), (B, L), keys.device)
    _gpu(keys)
    _check(load().sa_quantize_keys_fp8(_p(keys), B, L, d, _p(out_codes), _p(out_scales),
                                       _stream(keys.device)), "sa_quantize_keys_fp8")
    return out_codes, out_scales


def _fp8_shape(q, w, codes, scales, causal_offset, topk):
    _bf16(q, "q", 4)
    B, T, H, d = q.shape
    if not isinstance(codes, torch.Tensor) or codes.dtype != torch.uint8 or codes.dim() != 3:
        raise TypeError("codes must be a uint8 [batch, L, 128] tensor")
    L = codes.shape[1]
    _tensor(codes, "codes", (torch.uint8,), (B, L, d), q.device)
    _tensor(scales, "scales", (torch.float32,), (B, L), q.device)
    _tensor(w, "w", (torch.float32,), (B, T, H), q.device)
    return Shape(B, T, H, d, L, int(causal_offset), int(topk))


def indexer_score_topk_fp8_ws(shape: Shape) -> int:
    return _ws_query(load().indexer_score_topk_fp8_ws, "indexer_score_topk_fp8_ws",
                     ctypes.byref(shape))


def indexer_score_topk_fp8(q, w, codes, scales, causal_offset, topk, out_idx=None,
                           out_score=None, want_score=True, ws=None):
    """DSA indexer over E4M3 keys with per-key scales (rows T < 16)."""
    s = _fp8_shape(q, w, codes, scales, causal_offset, topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(indexer_score_topk_fp8_ws(s), q.device, ws)
    _gpu(q)
    _check(load().indexer_score_topk_fp8(_p(q), _p(w), _p(codes), _p(scales), ctypes.byref(s),
                                         _p(out_idx), _p(out_score), _p(ws), ws.numel(),
                                         _stream(q.device)), "indexer_score_topk_fp8")
    return out_idx, out_score


def indexer_score_topk_fp8q_ws(shape: Shape) -> int:
    return _ws_query(load().indexer_score_topk_fp8q_ws, "indexer_score_topk_fp8q_ws",
                     ctypes.byref(shape))


def indexer_score_topk_fp8q(q, w, codes, scales, causal_offset, topk, out_idx=None,
                            out_score=None, want_score=True, ws=None):
    """As indexer_score_topk_fp8 with the query converted to E4M3 in the
    kernel (per-head scale) and the dot products on the fp8 MFMA."""
    s = _fp8_shape(q, w, codes, scales, causal_offset, topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(indexer_score_topk_fp8q_ws(s), q.device, ws)
    _gpu(q)
    _check(load().indexer_score_topk_fp8q(_p(q), _p(w), _p(codes), _p(scales), ctypes.byref(s),
                                          _p(out_idx), _p(out_score), _p(ws), ws.numel(),
                                          _stream(q.device)), "indexer_score_topk_fp8q")
    return out_idx, out_score


def indexer_score_topk_fp8_ragged(q, w, codes, scales, seq_lens, topk, total_len=0, q_fp8=False,
                                  out_idx=None, out_score=None, want_score=True, ws=None):
    """Ragged batches over an FP8 key cache (capacity codes.shape[1]); q_fp8
    picks the E4M3-query scores of indexer_score_topk_fp8q."""
    _bf16(q, "q", 4)
    if not isinstance(codes, torch.Tensor) or codes.dim() != 3:
        raise TypeError("codes must be a uint8 [batch, L, 128] tensor")
    s = _fp8_shape(q, w, codes, scales, codes.shape[1] - q.shape[1], topk)
    _seq_lens(seq_lens, q.shape[0], q.device)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    n = _ws_query(load().indexer_score_topk_fp8_ragged_ws, "indexer_score_topk_fp8_ragged_ws",
                  ctypes.byref(s))
    ws = _workspace(n, q.device, ws)
    _gpu(q)
    _check(load().indexer_score_topk_fp8_ragged(_p(q), _p(w), _p(codes), _p(scales),
                                                _p(seq_lens), int(total_len),
                                                int(bool(q_fp8)), ctypes.byref(s), _p(out_idx),
                                                _p(out_score), _p(ws), ws.numel(),
                                                _stream(q.device)),
           "indexer_score_topk_fp8_ragged")
    return out_idx, out_score


def misa_route_fp8(q, w, codes, scales, causal_offset, topk, block_B, h, k_prime=0, pooled=None,
                   want_heads=True, want_pool=False, out_idx=None, out_score=None,
                   want_score=True, ws=None, out_heads=None, out_pool=None):
    """misa_route over an FP8 key cache.  Returns (idx, score, heads, pool)."""
    s = _fp8_shape(q, w, codes, scales, causal_offset, topk)
    pooled = _reps_in(pooled, "pooled", q, s.L, block_B)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    heads = _rows_out(out_heads, "out_heads", q, int(h), want_heads)
    pool = _rows_out(out_pool, "out_pool", q, int(k_prime), want_pool) if k_prime else None
    n = _ws_query(load().misa_route_fp8_ws, "misa_route_fp8_ws", ctypes.byref(s), int(block_B),
                  int(h), int(k_prime), int(pooled is not None))
    ws = _workspace(n, q.device, ws)
    _gpu(q)
    _check(load().misa_route_fp8(_p(q), _p(w), _p(codes), _p(scales), ctypes.byref(s),
                                 int(block_B), int(h), int(k_prime), _p(pooled), _p(heads),
                                 _p(pool), _p(out_idx), _p(out_score), _p(ws), ws.numel(),
                                 _stream(q.device)), "misa_route_fp8")
    return out_idx, out_score, heads, pool


def hisa_coarse_fine_fp8(q, w, codes, scales, causal_offset, topk, block_b, r, reps=None,
                         want_blocks=True, out_idx=None, out_score=None, want_score=True,
                         ws=None, out_blocks=None):
    """hisa_coarse_fine over an FP8 key cache.  Returns (idx, score, blocks)."""
    s = _fp8_shape(q, w, codes, scales, causal_offset, topk)
    reps = _reps_in(reps, "reps", q, s.L, block_b)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    blocks = _rows_out(out_blocks, "out_blocks", q, int(r), want_blocks)
    n = _ws_query(load().hisa_coarse_fine_fp8_ws, "hisa_coarse_fine_fp8_ws", ctypes.byref(s),
                  int(block_b), int(r), int(reps is not None))
    ws = _workspace(n, q.device, ws)
    _gpu(q)
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
    if not isinstance(idx, torch.Tensor) or idx.dtype != torch.int32 or not idx.is_contiguous():
        raise TypeError("idx must be a contiguous int32 tensor")
    if idx.dim() < 1 or idx.numel() == 0:
        raise ValueError("idx must have at least one row")
    k = idx.shape[-1]
    rows = idx.numel() // k
    if int(T) < 1 or rows % int(T):
        raise ValueError("T must divide the number of rows (%d)" % rows)
    if block_table is not None:
        if (not isinstance(block_table, torch.Tensor) or block_table.dtype != torch.int32
                or block_table.dim() != 2):
            raise TypeError("block_table must be an int32 [batch, pages] tensor")
        _tensor(block_table, "block_table", (torch.int32,), (rows // int(T), block_table.shape[1]),
                idx.device)
    if out_slots is None:
        out_slots = torch.empty_like(idx)
    else:
        _tensor(out_slots, "out_slots", (torch.int32,), tuple(idx.shape), idx.device)
    if out_stats is None and want_stats:
        out_stats = torch.empty(idx.shape[:-1] + (3,), dtype=torch.int32, device=idx.device)
    elif out_stats is not None:
        _tensor(out_stats, "out_stats", (torch.int32,), tuple(idx.shape[:-1]) + (3,), idx.device)
    _gpu(idx)
    _check(load().sa_tidy_indices(_p(idx), rows, int(T), k, _p(block_table),
                                  0 if block_table is None else block_table.shape[1],
                                  int(page_size), int(max_slots), _p(out_slots), _p(out_stats),
                                  _stream(idx.device)), "sa_tidy_indices")
    return out_slots, out_stats


def indexer_score_topk_ragged_ws(shape: Shape) -> int:
    return _ws_query(load().indexer_score_topk_ragged_ws, "indexer_score_topk_ragged_ws",
                     ctypes.byref(shape))


def indexer_score_topk_ragged(q, w, keys, seq_lens, topk, total_len=0, out_idx=None,
                              out_score=None, want_score=True, ws=None):
    """DSA over sequences of different lengths: keys [batch, L_cap, 128],
    seq_lens int32 [batch] on the GPU; row i of sequence b sits at
    seq_lens[b] - T + i.  total_len: the host's sum of the lengths (0 if
    unknown), used only to size the work per workgroup."""
    _bf16(q, "q", 4)
    _bf16(keys, "keys", 3)
    s = _shape(q, w, keys, keys.shape[1] - q.shape[1], topk)
    _seq_lens(seq_lens, q.shape[0], q.device)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(indexer_score_topk_ragged_ws(s), q.device, ws)
    _gpu(q)
    _check(load().indexer_score_topk_ragged(_p(q), _p(w), _p(keys), _p(seq_lens),
                                            int(total_len), ctypes.byref(s), _p(out_idx),
                                            _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
           "indexer_score_topk_ragged")
    return out_idx, out_score


# ---------------------------------------------------------- MISA x HISA

def misa_hisa_ws(shape: Shape, block_B, h, block_b, r, pooled_given, reps_given) -> int:
    return _ws_query(load().misa_hisa_ws, "misa_hisa_ws", ctypes.byref(shape), int(block_B),
                     int(h), int(block_b), int(r), int(bool(pooled_given)),
                     int(bool(reps_given)))


def misa_hisa(q, w, keys, causal_offset, topk, block_B, h, block_b, r, pooled=None, reps=None,
              want_heads=True, want_blocks=True, out_heads=None, out_blocks=None, out_idx=None,
              out_score=None, want_score=True, ws=None):
    """MISA router heads -> HISA block scores over those heads -> every-head
    rescoring of the r best blocks' tokens.  Returns (idx, score, heads, blocks)."""
    s = _shape(q, w, keys, causal_offset, topk)
    pooled = _reps_in(pooled, "pooled", q, s.L, block_B)
    reps = _reps_in(reps, "reps", q, s.L, block_b)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    heads = _rows_out(out_heads, "out_heads", q, int(h), want_heads)
    blocks = _rows_out(out_blocks, "out_blocks", q, int(r), want_blocks)
    ws = _workspace(misa_hisa_ws(s, block_B, h, block_b, r, pooled is not None, reps is not None),
                    q.device, ws)
    _gpu(q)
    _check(load().misa_hisa(_p(q), _p(w), _p(keys), ctypes.byref(s), int(block_B), int(h),
                            int(block_b), int(r), _p(pooled), _p(reps), _p(heads), _p(blocks),
                            _p(out_idx), _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
           "misa_hisa")
    return out_idx, out_score, heads, blocks


# ------------------------------------------------------- LISA / ResMiSA

def lisa_score_topk_ws(shape: Shape) -> int:
    return _ws_query(load().lisa_score_topk_ws, "lisa_score_topk_ws", ctypes.byref(shape))


def lisa_score_topk(q, w, keys, causal_offset, topk, out_idx=None, out_score=None,
                    want_score=True, ws=None):
    """LISA: top-k by the linear score g . k, g = sum_j w_j q_j."""
    s = _shape(q, w, keys, causal_offset, topk)
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    ws = _workspace(lisa_score_topk_ws(s), q.device, ws)
    _gpu(q)
    _check(load().lisa_score_topk(_p(q), _p(w), _p(keys), ctypes.byref(s), _p(out_idx),
                                  _p(out_score), _p(ws), ws.numel(), _stream(q.device)),
           "lisa_score_topk")
    return out_idx, out_score


def block_extrema(keys, block, out=None):
    """Per-block key max then min -> [batch, ceil(L/block), 2, 128] bf16 bits."""
    _bf16(keys, "keys", 3)
    if int(block) < 1:
        raise ValueError("block must be >= 1")
    B, L, d = keys.shape
    out = _reps_out(keys, block, out, "out")
    _gpu(keys)
    _check(load().sa_block_extrema(_p(keys), B, L, d, int(block), _p(out), _stream(keys.device)),
           "sa_block_extrema")
    return out


def resmisa_route_ws(shape: Shape, block, r, extrema_given) -> int:
    return _ws_query(load().resmisa_route_ws, "resmisa_route_ws", ctypes.byref(shape),
                     int(block), int(r), int(bool(extrema_given)))


def resmisa_route(q, w, keys, causal_offset, topk, block, r, extrema=None, want_heads=True,
                  out_heads=None, out_idx=None, out_score=None, want_score=True, ws=None):
    """ResMiSA: shared linear score + r routed residual heads.  Returns
    (idx, score, heads)."""
    s = _shape(q, w, keys, causal_offset, topk)
    extrema = _reps_in(extrema, "extrema", q, s.L, block) if int(r) > 0 else None
    out_idx, out_score = _outputs(q, topk, out_idx, out_score, want_score)
    heads = _rows_out(out_heads, "out_heads", q, int(r), want_heads) if int(r) > 0 else None
    ws = _workspace(resmisa_route_ws(s, block, r, extrema is not None), q.device, ws)
    _gpu(q)
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
