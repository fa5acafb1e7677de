"""Workspace sizes on the host: the prefill paths keep O(rows * k) survivor
entries per call, never an O(rows * n) score matrix (PaperTrace, "2.2.2 MISA,
LISA and ResMiSA", section 2.2: the score matrix is not written back)."""
import pytest

from sparse_attention_token_dsa_amd import api


@pytest.fixture(scope="module", autouse=True)
def lib():
    try:
        return api.load()
    except RuntimeError as e:
        pytest.skip(str(e))


@pytest.mark.parametrize("T,L,k", [(4096, 32768, 2048), (16384, 131072, 2048), (1024, 131072, 64)])
def test_prefill_workspace_is_below_the_score_matrix(T, L, k):
    s = api.Shape(1, T, 64, 128, L, L - T, k)
    n2 = T * L * 4  # fp32 scores of every (row, key) pair
    dsa = api.indexer_score_topk_ws(s)
    assert dsa < n2 and dsa <= T * max(6 * k, 8192) * 8 + (1 << 20)
    misa = api.misa_route_ws(s, 1024, 8, 0, True)
    assert misa < n2
    # MISA-dagger keeps a pool of k' = 4k per row: O(rows * k') survivors and
    # pool lists (here k' may reach a quarter of the row)
    kp = 4 * k
    dagger = api.misa_route_ws(s, 1024, 8, kp, True)
    heads = T * 8 * (2 * 128 + 4 + 4) + T * (4 * 128 + 1)  # routed q rows, weights, ids; cut-block means
    assert dagger <= T * min(L, max(6 * kp, 8192)) * 8 + T * kp * 12 + heads + (2 << 20)
    # HISA and MISA x HISA: block scores and the r*b rescored tokens per row
    b, r = 128, 64
    lists = T * ((L + b - 1) // b * 4 + r * 4 + r * b * 8)
    assert api.hisa_coarse_fine_ws(s, b, r, True) <= lists + T * 2 * 128 * 2 + (1 << 20)
    # (plus the routed heads and the cut-block means of both block sizes)
    assert api.misa_hisa_ws(s, 1024, 8, b, r, True, True) <= lists + T * (8 * 4 + 2 * 512 + 2) \
        + (1 << 20)
    # the fused prefill on the FP8 cache: the same survivor lists as bf16 keys
    assert api.indexer_score_topk_fp8q_ws(s) == dsa


def test_short_rows_keep_every_key():
    # rows with fewer legal keys than the bound: one slot per legal key
    s = api.Shape(1, 1024, 64, 128, 1024, 0, 128)
    assert api.indexer_score_topk_ws(s) <= 1024 * 1024 * 8 + (1 << 20)
