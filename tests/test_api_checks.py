"""The binding checks every tensor it hands to the library as a raw pointer
(dtype, exact shape, contiguity, device) before any call, so that a wrong
caller buffer is an exception on the host rather than an out-of-bounds read or
write on the device.  CPU tensors reach every check; a call that passes them
all is still refused because its tensors are not on a GPU."""
import pytest

torch = pytest.importorskip("torch")

from sparse_attention_token_dsa_amd import api  # noqa: E402

B, T, H, D, L, K = 2, 1, 16, 128, 300, 8


@pytest.fixture(scope="module", autouse=True)
def lib():
    try:
        return api.load()
    except RuntimeError as e:
        pytest.skip(str(e))


def qwk(T=T):
    q = torch.zeros((B, T, H, D), dtype=torch.int16)
    w = torch.zeros((B, T, H), dtype=torch.float32)
    k = torch.zeros((B, L, D), dtype=torch.int16)
    return q, w, k


def reps(block, dtype=torch.int16, nb=None):
    return torch.zeros((B, (L + block - 1) // block if nb is None else nb, 2, D), dtype=dtype)


def _raises(fn, exc, text):
    with pytest.raises(exc) as e:
        fn()
    assert text in str(e.value), str(e.value)


def test_valid_cpu_call_is_refused_as_not_on_gpu():
    q, w, k = qwk()
    _raises(lambda: api.indexer_score_topk(q, w, k, L - 1, K), ValueError, "on a GPU")
    _raises(lambda: api.misa_route(q, w, k, L - 1, K, 64, 4, pooled=reps(64)), ValueError,
            "on a GPU")
    _raises(lambda: api.hisa_coarse_fine(q, w, k, L - 1, K, 16, 4, reps=reps(16)), ValueError,
            "on a GPU")


@pytest.mark.parametrize("bad, text", [
    (lambda: torch.zeros((B, T, K), dtype=torch.int64), "out_idx must be"),
    (lambda: torch.zeros((B, T, K - 1), dtype=torch.int32), "out_idx must have shape"),
    (lambda: torch.zeros((B, T, 2 * K), dtype=torch.int32)[:, :, ::2], "contiguous"),
])
def test_out_idx_checked(bad, text):
    q, w, k = qwk()
    _raises(lambda: api.indexer_score_topk(q, w, k, L - 1, K, out_idx=bad()),
            (TypeError, ValueError), text)


def test_out_score_checked():
    q, w, k = qwk()
    _raises(lambda: api.indexer_score_topk(q, w, k, L - 1, K,
                                           out_score=torch.zeros((B, T, K), dtype=torch.float16)),
            TypeError, "out_score must be")
    _raises(lambda: api.indexer_score_topk(q, w, k, L - 1, K,
                                           out_score=torch.zeros((B, T + 1, K))),
            ValueError, "out_score must have shape")


def test_workspace_checked():
    q, w, k = qwk()
    _raises(lambda: api.indexer_score_topk(q, w, k, L - 1, K, ws=torch.zeros(1 << 20)),
            TypeError, "ws must be a uint8")
    _raises(lambda: api.indexer_score_topk(q, w, k, L - 1, K,
                                           ws=torch.zeros(16, dtype=torch.uint8)),
            ValueError, "workspace too small")


def test_weights_checked():
    q, w, k = qwk()
    _raises(lambda: api.indexer_score_topk(q, w.double(), k, L - 1, K), TypeError, "w must be")
    _raises(lambda: api.indexer_score_topk(q, w[:, :, :-1], k, L - 1, K), ValueError,
            "w must have shape")


def test_pooled_and_reps_checked():
    q, w, k = qwk()
    # the layout of another block size: reading it as B = 64 would run past it
    _raises(lambda: api.misa_route(q, w, k, L - 1, K, 64, 4, pooled=reps(16)), ValueError,
            "pooled must have shape")
    _raises(lambda: api.misa_route(q, w, k, L - 1, K, 64, 4,
                                   pooled=reps(64, dtype=torch.float32)), TypeError,
            "pooled must be")
    _raises(lambda: api.hisa_coarse_fine(q, w, k, L - 1, K, 16, 4, reps=reps(64)), ValueError,
            "reps must have shape")
    _raises(lambda: api.misa_hisa(q, w, k, L - 1, K, 64, 4, 16, 4, pooled=reps(64),
                                  reps=reps(32)), ValueError, "reps must have shape")
    _raises(lambda: api.resmisa_route(q, w, k, L - 1, K, 16, 3, extrema=reps(8)), ValueError,
            "extrema must have shape")


def test_row_outputs_checked():
    q, w, k = qwk()
    _raises(lambda: api.misa_route(q, w, k, L - 1, K, 64, 4, out_heads=torch.zeros(
        (B, T, 3), dtype=torch.int32)), ValueError, "out_heads must have shape")
    _raises(lambda: api.misa_route(q, w, k, L - 1, K, 64, 4, k_prime=16, out_pool=torch.zeros(
        (B, T, 8), dtype=torch.int32)), ValueError, "out_pool must have shape")
    _raises(lambda: api.hisa_coarse_fine(q, w, k, L - 1, K, 16, 4, out_blocks=torch.zeros(
        (B, T, 4), dtype=torch.int64)), TypeError, "out_blocks must be")
    _raises(lambda: api.misa_hisa(q, w, k, L - 1, K, 64, 4, 16, 4, out_blocks=torch.zeros(
        (B, T, 5), dtype=torch.int32)), ValueError, "out_blocks must have shape")


def test_pool_and_extrema_outputs_checked():
    _, _, k = qwk()
    _raises(lambda: api.pool_blocks(k, 64, out=reps(32)), ValueError, "out must have shape")
    _raises(lambda: api.pool_blocks2(k, 16, 64, out_small=reps(16), out_large=reps(16)),
            ValueError, "out_large must have shape")
    _raises(lambda: api.block_extrema(k, 16, out=reps(16, dtype=torch.int32)), TypeError,
            "out must be")
    _raises(lambda: api.quantize_keys_fp8(k, out_codes=torch.zeros((B, L, D - 1),
                                                                   dtype=torch.uint8)),
            ValueError, "out_codes must have shape")
    _raises(lambda: api.quantize_keys_fp8(k, out_scales=torch.zeros((B, L),
                                                                    dtype=torch.float64)),
            TypeError, "out_scales must be")


def test_fp8_cache_checked():
    q, w, _ = qwk()
    codes = torch.zeros((B, L, D), dtype=torch.uint8)
    scales = torch.zeros((B, L))
    _raises(lambda: api.indexer_score_topk_fp8(q, w, codes, scales[:, :-1], L - 1, K),
            ValueError, "scales must have shape")
    _raises(lambda: api.indexer_score_topk_fp8q(q, w, codes.int(), scales, L - 1, K),
            TypeError, "codes must be")
    _raises(lambda: api.hisa_coarse_fine_fp8(q, w, codes, scales, L - 1, K, 16, 4,
                                             reps=reps(8)), ValueError, "reps must have shape")


def test_seq_lens_checked():
    q, w, k = qwk()
    _raises(lambda: api.indexer_score_topk_ragged(q, w, k, torch.zeros(B, dtype=torch.int64), K),
            TypeError, "seq_lens must be")
    _raises(lambda: api.indexer_score_topk_ragged(q, w, k, torch.zeros(B + 1, dtype=torch.int32),
                                                  K), ValueError, "seq_lens must have shape")


def test_tidy_outputs_checked():
    idx = torch.zeros((B, T, K), dtype=torch.int32)
    _raises(lambda: api.tidy_indices(idx, T, out_slots=torch.zeros((B, T, K - 1),
                                                                   dtype=torch.int32)),
            ValueError, "out_slots must have shape")
    _raises(lambda: api.tidy_indices(idx, T, out_stats=torch.zeros((B, T, 2), dtype=torch.int32)),
            ValueError, "out_stats must have shape")
    _raises(lambda: api.tidy_indices(idx, T, block_table=torch.zeros((B + 1, 4),
                                                                     dtype=torch.int32)),
            ValueError, "block_table must have shape")
