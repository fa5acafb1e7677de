"""GPU parity of the FP8 key path (PaperTrace section 2.3: the indexer's keys
held as E4M3 codes with one fp32 scale per key).

* sa_quantize_keys_fp8 is byte work: its codes and scales must equal the
  oracle's bit for bit, including subnormal codes, signed zeros, exact
  midpoints between codes and all-zero keys.
* indexer_score_topk_fp8 is compared with the oracle's DSA on the dequantized
  keys under the rule of tests/parity.py, on the oracle's own codes, so the two
  stages are checked independently.
* indexer_score_topk_fp8q (the query converted to E4M3 in the kernel, fp8
  MFMA) is compared with the oracle's dsa_fp8q the same way; its query codes,
  a decision taken in fp32 on both sides, are checked exactly through unit
  keys that read one code each.
* misa_route_fp8 and hisa_coarse_fine_fp8 are staged against the oracle's
  MISA and HISA over the same FP8 cache (heads, pool and blocks by the
  near-tie rule, then tokens on the GPU's choices).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from parity import (_np, check_dsa_fp8, check_dsa_fp8q, check_hisa, check_misa,
                    prefill_group_rows, rows_of, to_device)
from sparse_attention_token_dsa_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_token_dsa_amd import api as a
    a.load()
    return a


def gpu_quantize(api, K):
    Kd = torch.from_numpy(np.ascontiguousarray(K).view(np.int16)).to(DEV)
    codes, scales = api.quantize_keys_fp8(Kd)
    torch.cuda.synchronize()
    return _np(codes), _np(scales)


def assert_quantize_exact(api, K):
    gc, gs = gpu_quantize(api, K)
    oc, os_ = oracle.quantize_keys_fp8(K)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, "codes differ at %s: gpu %s oracle %s" % (
        bad[:4].tolist(), gc[tuple(bad[:4].T)].tolist(), oc[tuple(bad[:4].T)].tolist())


@pytest.mark.parametrize("Bt,L,seed", [(1, 1, 1), (3, 1000, 2), (2, 4099, 3)])
def test_quantize_random_keys(api, Bt, L, seed):
    say("quantize random Bt=%d L=%d" % (Bt, L))
    p = synth.make_problem(300 + seed, Bt=Bt, T=1, L=L, H=4)
    assert_quantize_exact(api, p["K"])


def test_quantize_edge_values(api):
    # Keys built so that k_x / a lands on chosen values: every E4M3 magnitude,
    # the midpoints between neighbouring codes (ties to even), values just off
    # them, subnormals, values that round to zero, signed zeros and all-zero keys.
    say("quantize edge values")
    v = oracle.fp8_decode(np.arange(0x7F))
    mids = (v[:-1] + v[1:]) / 2
    vals = np.concatenate([v, mids, mids * (1 + 2.0 ** -7), mids * (1 - 2.0 ** -7),
                           [2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11, 0.0]])
    rng = np.random.default_rng(5)
    rows = []
    for e in (-20, -3, 0, 5):
        for start in range(0, len(vals), 127):
            row = np.zeros(128)
            chunk = vals[start:start + 127]
            row[:len(chunk)] = chunk * rng.choice([-1.0, 1.0], size=len(chunk))
            row[127] = 448.0              # a = 2^e exactly
            rows.append(row * 2.0 ** e)
    K = synth.to_bf16_bits(np.array(rows, np.float32))[None]
    K[0, 1, 5] = 0x8000                   # -0
    zero = np.zeros((1, 3, 128), np.uint16)
    zero[0, 1, :] = 0x8000                # a key of -0 only
    K = np.concatenate([K, zero], axis=1)
    assert_quantize_exact(api, K)


@pytest.mark.parametrize("Bt,T,L,H,k", [
    (3, 1, 5000, 64, 100),        # decode, ragged L
    (2, 3, 9001, 64, 257),        # several decode rows per sequence
    (1, 15, 3000, 64, 300),       # the most rows the FP8 path takes
    (2, 1, 300, 64, 512),         # k > t+1: the whole prefix
    (1, 2, 20000, 32, 2048),      # H = 32
    (2, 1, 4100, 40, 64),         # H not a multiple of 16
    (1, 1, 1, 64, 8),             # a single key
])
def test_dsa_fp8(api, Bt, T, L, H, k):
    say("dsa fp8 Bt=%d T=%d L=%d H=%d k=%d" % (Bt, T, L, H, k))
    p = synth.make_problem(400 + L % 89, Bt=Bt, T=T, L=L, H=H, needles=8,
                           needle_mode="decode" if T == 1 else "rows")
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    q, w, _ = to_device(p, DEV)
    idx, sc = api.indexer_score_topk_fp8(q, w, torch.from_numpy(codes).to(DEV),
                                         torch.from_numpy(scales).to(DEV), p["offset"], k)
    torch.cuda.synchronize()
    check_dsa_fp8(p, codes, scales, k, _np(idx), _np(sc), rows_of(p))


def test_dsa_fp8_zero_keys(api):
    # All-zero keys (scale 1, codes 0) score exactly 0 next to real keys.
    say("dsa fp8 zero keys")
    p = synth.make_problem(410, Bt=1, T=1, L=3000, H=64)
    p["K"][0, ::3] = 0
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    assert np.all(scales[0, ::3] == 1.0)
    q, w, _ = to_device(p, DEV)
    idx, sc = api.indexer_score_topk_fp8(q, w, torch.from_numpy(codes).to(DEV),
                                         torch.from_numpy(scales).to(DEV), p["offset"], 1500)
    torch.cuda.synchronize()
    check_dsa_fp8(p, codes, scales, 1500, _np(idx), _np(sc), rows_of(p))


def test_dsa_fp8_128k_quantized_on_gpu(api):
    # The 128k decode workload (8 sequences, 64 heads, k = 2048): GPU-quantized
    # keys (checked bit-exact first), then every row against the oracle.
    say("dsa fp8 128k b8 h64")
    p = synth.make_config("misa_128k_h64")
    q, w, K = to_device(p, DEV)
    codes, scales = api.quantize_keys_fp8(K)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_keys_fp8(p["K"])
    assert np.array_equal(_np(codes), oc) and np.array_equal(_np(scales), os_)
    idx, sc = api.indexer_score_topk_fp8(q, w, codes, scales, p["offset"], 2048)
    torch.cuda.synchronize()
    check_dsa_fp8(p, oc, os_, 2048, _np(idx), _np(sc), rows_of(p))


def test_dsa_fp8_rejects_prefill_rows(api):
    say("dsa fp8 T=16 rejected")
    p = synth.make_problem(420, Bt=1, T=16, L=100, H=16)
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    q, w, _ = to_device(p, DEV)
    with pytest.raises(api.SaError) as e:
        api.indexer_score_topk_fp8(q, w, torch.from_numpy(codes).to(DEV),
                                   torch.from_numpy(scales).to(DEV), p["offset"], 8)
    assert e.value.code == api.SA_EUNSUPPORTED


# ------------------------------------------------------------ FP8 query

@pytest.mark.parametrize("Bt,T,L,H,k", [
    (3, 1, 5000, 64, 100),
    (2, 3, 9001, 64, 257),
    (1, 15, 3000, 64, 300),
    (2, 1, 300, 64, 512),
    (1, 2, 20000, 32, 2048),
    (2, 1, 4100, 40, 64),
    (1, 1, 1, 64, 8),
    (1, 4, 700, 1, 50),           # a single head
])
def test_dsa_fp8q(api, Bt, T, L, H, k):
    say("dsa fp8q Bt=%d T=%d L=%d H=%d k=%d" % (Bt, T, L, H, k))
    p = synth.make_problem(430 + L % 89, Bt=Bt, T=T, L=L, H=H, needles=8,
                           needle_mode="decode" if T == 1 else "rows")
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    q, w, _ = to_device(p, DEV)
    idx, sc = api.indexer_score_topk_fp8q(q, w, torch.from_numpy(codes).to(DEV),
                                          torch.from_numpy(scales).to(DEV), p["offset"], k)
    torch.cuda.synchronize()
    check_dsa_fp8q(p, codes, scales, k, _np(idx), _np(sc), rows_of(p))


def test_dsa_fp8q_query_codes_exact(api):
    # Keys +-448 e_x (scale 1) read one query code each: with a single head of
    # weight 1, key x scores b * 448 * max(qhat_x, 0) and key 128 + x scores
    # b * 448 * max(-qhat_x, 0).  Rows put q / b on E4M3 values, midpoints
    # between codes (ties to even), points just off them, subnormals and
    # values that round to zero; one row is all zero (b = 1).  Every score
    # must match the oracle's to fp32 rounding, which no wrong code does.
    say("dsa fp8q query codes")
    v = oracle.fp8_decode(np.arange(0x7F))
    mids = (v[:-1] + v[1:]) / 2
    pool = np.concatenate([v, mids, mids * (1 + 2.0 ** -7), mids * (1 - 2.0 ** -7),
                           [2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11]])
    rng = np.random.default_rng(11)
    T, L = 8, 256
    q = np.zeros((1, T, 1, 128), np.float32)
    for i in range(T - 1):
        row = rng.choice(pool, size=128) * rng.choice([-1.0, 1.0], size=128)
        row[int(rng.integers(0, 128))] = 448.0 * (1 if i % 2 else -1)
        q[0, i, 0] = row * 2.0 ** (-12 + 3 * i)
    qb = synth.to_bf16_bits(q)
    K = np.zeros((1, L, 128), np.float32)
    for x in range(128):
        K[0, x, x] = 448.0
        K[0, 128 + x, x] = -448.0
    p = {"q": qb, "w": np.ones((1, T, 1), np.float32), "K": synth.to_bf16_bits(K),
         "offset": L - T, "Bt": 1, "T": T, "H": 1, "L": L}
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    assert np.all(scales == 1.0)
    qd = torch.from_numpy(qb.view(np.int16)).to(DEV)
    wd = torch.from_numpy(p["w"]).to(DEV)
    idx, sc = api.indexer_score_topk_fp8q(qd, wd, torch.from_numpy(codes).to(DEV),
                                          torch.from_numpy(scales).to(DEV), p["offset"], L)
    torch.cuda.synchronize()
    prob = oracle.Problem(p["q"], p["w"], p["K"], p["offset"])
    _, _, rs = oracle.dsa_fp8q(prob, codes, scales, L, want_rowscore=True)
    gi, gs = _np(idx).reshape(T, L), _np(sc).reshape(T, L)
    for i in range(T):
        n = p["offset"] + i + 1      # k >= n: the whole prefix, in no set order
        assert np.array_equal(np.sort(gi[i, :n]), np.arange(n)), "row %d set" % i
        assert np.all(gi[i, n:] == -1)
        ref = rs[i, gi[i, :n]]
        assert np.allclose(gs[i, :n], ref, rtol=2e-7, atol=0), "row %d scores" % i
    assert np.any(rs[:, :128] > 0) and np.any(rs[:, 128:] > 0)


def test_dsa_fp8q_128k(api):
    # The 128k decode workload with GPU-quantized keys, every row.
    say("dsa fp8q 128k b8 h64")
    p = synth.make_config("misa_128k_h64")
    q, w, K = to_device(p, DEV)
    codes, scales = api.quantize_keys_fp8(K)
    idx, sc = api.indexer_score_topk_fp8q(q, w, codes, scales, p["offset"], 2048)
    torch.cuda.synchronize()
    check_dsa_fp8q(p, _np(codes), _np(scales), 2048, _np(idx), _np(sc), rows_of(p))


# ------------------------------------------- FP8 prefill (fused, fp8 MFMA)

def _fp8q_prefill(api, p, k):
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    q, w, _ = to_device(p, DEV)
    idx, sc = api.indexer_score_topk_fp8q(q, w, torch.from_numpy(codes).to(DEV),
                                          torch.from_numpy(scales).to(DEV), p["offset"], k)
    torch.cuda.synchronize()
    return codes, scales, _np(idx), _np(sc)


@pytest.mark.parametrize("Bt,T,L,H,k", [
    (1, 16, 100, 16, 8),           # the smallest prefill chunk
    (1, 1024, 1024, 64, 128),      # the whole sequence as one chunk
    (2, 200, 3000, 64, 257),       # ragged tail of 8-row groups and 64-key tiles
    (1, 96, 20000, 32, 2048),      # H = 32, k above the LDS candidate buffer
    (1, 120, 2500, 40, 100),       # H = 40: three head tiles, the last partial
    (1, 40, 700, 1, 50),           # a single head
])
def test_dsa_fp8q_prefill(api, Bt, T, L, H, k):
    say("dsa fp8q prefill Bt=%d T=%d L=%d H=%d k=%d" % (Bt, T, L, H, k))
    p = synth.make_problem(440 + L % 83, Bt=Bt, T=T, L=L, H=H, needles=8, needle_mode="rows")
    codes, scales, idx, sc = _fp8q_prefill(api, p, k)
    check_dsa_fp8q(p, codes, scales, k, idx, sc, rows_of(p))


def test_dsa_fp8q_prefill_bounded_lists(api):
    # More legal keys than list slots: the lists are compacted while sweeping.
    say("dsa fp8q prefill bounded lists")
    T, L, H, k = 64, 40000, 16, 100
    shape = api.Shape(1, T, H, 128, L, L - T, k)
    assert api.indexer_score_topk_fp8q_ws(shape) < T * L * 8
    p = synth.make_problem(447, Bt=1, T=T, L=L, H=H, offset=L - T, needles=8,
                           needle_mode="rows")
    codes, scales, idx, sc = _fp8q_prefill(api, p, k)
    check_dsa_fp8q(p, codes, scales, k, idx, sc, rows_of(p))


def test_dsa_fp8q_prefill_chunked_rows(api):
    # The chunked-prefill workload (4096 queries over 28672 cached keys) on
    # the FP8 cache; one row of every eighth 8-row group checked.
    say("dsa fp8q prefill_chunked 64 rows")
    p = synth.make_config("prefill_chunked")
    q, w, K = to_device(p, DEV)
    codes, scales = api.quantize_keys_fp8(K)
    idx, sc = api.indexer_score_topk_fp8q(q, w, codes, scales, p["offset"], 2048)
    torch.cuda.synchronize()
    rows = prefill_group_rows(p["T"], 5)[::8]
    check_dsa_fp8q(p, _np(codes), _np(scales), 2048, _np(idx), _np(sc), rows)


def test_dsa_fp8_bf16_query_rejects_prefill_rows(api):
    say("dsa fp8 ragged T=16 with a bf16 query rejected")
    p = synth.make_problem(422, Bt=2, T=16, L=100, H=16, offset=84)
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    q, w, _ = to_device(p, DEV)
    lens = torch.tensor([100, 50], dtype=torch.int32, device=DEV)
    with pytest.raises(api.SaError) as e:
        api.indexer_score_topk_fp8_ragged(q, w, torch.from_numpy(codes).to(DEV),
                                          torch.from_numpy(scales).to(DEV), lens, 8,
                                          q_fp8=False)
    assert e.value.code == api.SA_EUNSUPPORTED


# --------------------------------------------------- MISA / HISA on FP8 keys

def _fp8_case(p):
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    q, w, _ = to_device(p, DEV)
    return q, w, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), (codes, scales)


@pytest.mark.parametrize("Bt,T,L,H,B,h,k,kp", [
    (2, 1, 5000, 64, 256, 8, 64, 0),
    (2, 1, 5000, 64, 256, 8, 64, 320),       # MISA-dagger
    (1, 3, 7000, 32, 1024, 8, 100, 0),       # cut last block, H = 32
    (1, 4, 4000, 64, 300, 4, 50, 200),       # block not a power of two
    (1, 15, 900, 64, 128, 8, 40, 100),       # many decode-style rows
])
def test_misa_fp8(api, Bt, T, L, H, B, h, k, kp):
    say("misa fp8 Bt=%d T=%d L=%d H=%d B=%d h=%d k=%d kp=%d" % (Bt, T, L, H, B, h, k, kp))
    p = synth.make_problem(450 + L % 97 + kp, Bt=Bt, T=T, L=L, H=H, needles=8,
                           needle_mode="decode" if T == 1 else "rows")
    q, w, cd, sd, fp8 = _fp8_case(p)
    idx, sc, heads, pool = api.misa_route_fp8(q, w, cd, sd, p["offset"], k, B, h, k_prime=kp,
                                              want_pool=True)
    torch.cuda.synchronize()
    check_misa(p, k, B, h, kp, _np(idx), _np(sc), _np(heads), None if pool is None else _np(pool),
               rows_of(p), fp8=fp8)


def test_misa_fp8_rejects_prefill_rows(api):
    say("misa fp8 T=16 rejected")
    p = synth.make_problem(461, Bt=1, T=16, L=300, H=16)
    q, w, cd, sd, _ = _fp8_case(p)
    with pytest.raises(api.SaError) as e:
        api.misa_route_fp8(q, w, cd, sd, p["offset"], 8, 64, 4)
    assert e.value.code == api.SA_EUNSUPPORTED


def test_misa_fp8_all_heads_equals_dsa_fp8(api):
    say("misa fp8 h = H")
    p = synth.make_problem(460, Bt=2, T=1, L=6000, H=32, needles=8, needle_mode="decode")
    q, w, cd, sd, fp8 = _fp8_case(p)
    mi, _, _, _ = api.misa_route_fp8(q, w, cd, sd, p["offset"], 128, 512, 32)
    di, _ = api.indexer_score_topk_fp8(q, w, cd, sd, p["offset"], 128)
    torch.cuda.synchronize()
    assert np.array_equal(np.sort(_np(mi).reshape(-1, 128), 1), np.sort(_np(di).reshape(-1, 128), 1))


@pytest.mark.parametrize("Bt,T,L,H,b,r,k", [
    (2, 1, 5000, 64, 64, 8, 64),
    (1, 3, 9000, 64, 128, 16, 300),           # cut last block
    (1, 20, 1000, 32, 32, 6, 100),
])
def test_hisa_fp8(api, Bt, T, L, H, b, r, k):
    say("hisa fp8 Bt=%d T=%d L=%d H=%d b=%d r=%d k=%d" % (Bt, T, L, H, b, r, k))
    p = synth.make_problem(470 + L % 89, Bt=Bt, T=T, L=L, H=H, needles=8,
                           needle_mode="decode" if T == 1 else "rows")
    q, w, cd, sd, fp8 = _fp8_case(p)
    idx, sc, blocks = api.hisa_coarse_fine_fp8(q, w, cd, sd, p["offset"], k, b, r)
    torch.cuda.synchronize()
    check_hisa(p, k, b, r, _np(idx), _np(sc), _np(blocks), rows_of(p), fp8=fp8)


def test_misa_hisa_fp8_128k(api):
    # The 128k decode workload's MISA (B 1024, h 8, k' 8192) and HISA (b 128,
    # r 64) on GPU-quantized keys, every row.
    say("misa-dagger / hisa fp8 128k b8 h64")
    p = synth.make_config("misa_128k_h64")
    q, w, K = to_device(p, DEV)
    cd, sd = api.quantize_keys_fp8(K)
    torch.cuda.synchronize()
    fp8 = (_np(cd), _np(sd))
    idx, sc, heads, pool = api.misa_route_fp8(q, w, cd, sd, p["offset"], 2048, 1024, 8,
                                              k_prime=8192, want_pool=True)
    torch.cuda.synchronize()
    check_misa(p, 2048, 1024, 8, 8192, _np(idx), _np(sc), _np(heads), _np(pool), rows_of(p),
               fp8=fp8)
    idx, sc, blocks = api.hisa_coarse_fine_fp8(q, w, cd, sd, p["offset"], 2048, 128, 64)
    torch.cuda.synchronize()
    check_hisa(p, 2048, 128, 64, _np(idx), _np(sc), _np(blocks), rows_of(p), fp8=fp8)


@pytest.mark.parametrize("Bt,T,L,H,k,lens,q_fp8", [
    (4, 1, 20000, 64, 512, [20000, 9001, 37, 1], False),
    (4, 1, 20000, 64, 512, [20000, 9001, 37, 1], True),
    (3, 3, 5000, 32, 100, [5000, 1200, 3], False),
    (3, 3, 5000, 32, 100, [5000, 1200, 3], True),
    (3, 32, 5000, 64, 100, [5000, 1200, 40], True),   # prefill rows: the fused prefill
])
def test_dsa_fp8_ragged(api, Bt, T, L, H, k, lens, q_fp8):
    # Each sequence against the oracle's FP8 DSA on its own prefix.
    from parity import TOL_REL, check_set
    say("dsa fp8 ragged Bt=%d T=%d L=%d lens=%s q_fp8=%s" % (Bt, T, L, lens, q_fp8))
    p = synth.make_problem(480 + Bt, Bt=Bt, T=T, L=L, H=H, offset=L - T, needles=8)
    codes, scales = oracle.quantize_keys_fp8(p["K"])
    q, w, _ = to_device(p, DEV)
    lens = np.array(lens, np.int32)
    idx, sc = api.indexer_score_topk_fp8_ragged(q, w, torch.from_numpy(codes).to(DEV),
                                                torch.from_numpy(scales).to(DEV),
                                                torch.from_numpy(lens).to(DEV), k,
                                                total_len=int(lens.sum()), q_fp8=q_fp8)
    torch.cuda.synchronize()
    gi, gs = _np(idx).reshape(-1, k), _np(sc).reshape(-1, k)
    fn = oracle.dsa_fp8q if q_fp8 else oracle.dsa_fp8
    for b in range(Bt):
        n = max(int(lens[b]), T)
        pb = oracle.Problem(p["q"][b:b + 1], p["w"][b:b + 1],
                            np.ascontiguousarray(p["K"][b:b + 1, :n]), n - T)
        oi, osc, rs = fn(pb, np.ascontiguousarray(codes[b:b + 1, :n]),
                         np.ascontiguousarray(scales[b:b + 1, :n]), k, want_rowscore=True)
        for i in range(T):
            row, t = b * T + i, n - T + i
            srow = rs[i, : t + 1]
            tol = TOL_REL * np.max(np.abs(srow))
            check_set(gi[row], gs[row], oi[i], osc[i], lambda s, srow=srow: srow[s], t + 1, k,
                      tol, t=t, what="fp8 ragged row %d" % row)
