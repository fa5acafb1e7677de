"""The benchmark's work counters against the cost figures the pages work by
hand (PaperTrace, "2.2.2 MISA, LISA and ResMiSA": section 2.3, the per-item
cost of one decode step; section 3.2, dot-product counts on the head and
layer axes), and against closed forms.

bench.py computes its throughput numerators (legal pairs, MACs) and roofline
bytes with these same functions, so a mistake in them fails here first.
"""
import json
import os

import pytest

from sparse_attention_token_dsa_amd import workload as wl

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


def test_decode_cost_of_section_2_3():
    g = _golden("pt_2_3_decode_cost.json")
    t, H, d, k = g["decode_t"], g["decode_H"], g["decode_d"], g["decode_topk"]
    # one decode query at context length t scores all t keys
    pairs = wl.legal_pairs(1, t - 1)
    assert pairs == t
    assert wl.indexer_macs(pairs, H, d) == g["dsa_macs"] == 268435456
    assert wl.misa_macs(pairs, g["misa_h"], d) == g["misa_macs"] == 33554432
    assert 100.0 * k / t == pytest.approx(g["sparse_mla_fraction_percent"], abs=1e-12)
    hc = wl.hisa_counts(t, g["hisa_b"], g["hisa_r"])
    assert hc["reps"] == g["hisa_reps"] == 2048
    assert hc["tokens"] == g["hisa_tokens"] == 8192
    assert hc["percent"] == pytest.approx(g["hisa_fraction_percent"], abs=1e-12)
    # r = 32 leaves exactly k tokens to rescore (no slack, section 2.3)
    assert wl.hisa_counts(t, g["hisa_b"], 32)["tokens"] == k


def test_head_axis_counts_of_section_3_2():
    g = _golden("pt_2_3_decode_cost.json")
    N, H = g["axes_N"], g["axes_H"]
    dsa = wl.dsa_dots(N, H)
    assert dsa == g["axes_dots_dsa"] == 8388608
    assert wl.lisa_dots(N) * H == dsa                      # 1/64 of DSA
    assert wl.resmisa_dots(N, g["resmisa_r"]) == g["resmisa_dots"] == 1048576
    assert wl.resmisa_dots(N, g["resmisa_r"]) * 8 == dsa   # 1/8 of DSA
    ld = wl.lisa_dagger_dots(N, g["lisa_dagger_pool"], H)
    assert ld == g["lisa_dagger_dots"] == 655360
    assert round(100.0 * ld / dsa, 2) == g["lisa_dagger_percent"]


def test_layer_axis_of_section_3_2():
    g = _golden("pt_3_2_layer_axis.json")
    v = wl.lisa_ddagger_dots(g["N"], g["M"], g["H"], g["G"])
    assert round(100.0 * v / wl.dsa_dots(g["N"], g["H"]), 2) == g["lisa_ddagger_percent"]
    # G = 1 is LISA-dagger
    assert wl.lisa_ddagger_dots(g["N"], g["M"], g["H"], 1) == wl.lisa_dagger_dots(g["N"], g["M"], g["H"])


def test_legal_pairs_closed_form_and_brute_force():
    # the chunked-prefill workload: T = 4096 rows over P = 28672 cached keys
    assert wl.legal_pairs(4096, 28672) == 125831168
    for T, off in ((1, 0), (1, 31), (7, 0), (5, 11), (64, 100)):
        assert wl.legal_pairs(T, off) == sum(off + i + 1 for i in range(T))
    assert wl.legal_pairs(3, 5, batch=4) == 4 * wl.legal_pairs(3, 5)
    lens = [40, 17, 9]
    assert wl.ragged_pairs(4, lens) == sum(n - 4 + i + 1 for n in lens for i in range(4))
    # the prefill MAC count the MFMA roofline divides by
    assert wl.indexer_macs(wl.legal_pairs(4096, 28672), 64, 128) == 1030808928256  # 1.031e12 MAC, 2.0616e12 flop


def test_bytes():
    # the L = 131072, batch-8 decode scan: keys + q + w
    assert wl.scan_bytes(8, 8, 131072, 64, 128) == 268435456 + 131072 + 2048 == 268568576
    assert wl.score_row_bytes(8, 131072) == 4194304
    # FP8 cache: 128 code bytes + one fp32 scale per key
    assert wl.key_bytes(8, 131072, 128, fp8=True) == 8 * 131072 * 132
    # config-2 decode (32 x 32768): K 256 MiB, q 512 KiB, w 8 KiB, idx 256 KiB
    assert wl.key_bytes(32, 32768, 128) == 268435456
    assert wl.scan_bytes(32, 32, 32768, 64, 128) - wl.key_bytes(32, 32768, 128) == 524288 + 8192
    assert wl.topk_out_bytes(32, 2048, with_scores=False) == 262144
    assert wl.gather_bytes(8, 8192, 128) == 16 * 2 ** 20
