"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle step to a fixed point: a hand-worked example (golden
fixture), a library routine on a special case, a closed form, an invariant the
pages imply, or an independent brute-force restatement on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import lsa_oracle as O
from oracle import loops as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- P1 decode

def test_e4m3fn_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_e4m3fn_closed_forms():
    d = O.decode_e4m3fn(np.array([0x7E, 0x08, 0x01, 0x7F, 0xFF, 0x80, 0x38, 0xFE], dtype=np.uint8))
    assert d[0] == 448.0
    assert d[1] == 2.0 ** -6
    assert d[2] == 2.0 ** -9
    assert math.isnan(d[3]) and math.isnan(d[4])
    assert d[5] == 0.0 and math.copysign(1.0, d[5]) == -1.0
    assert d[6] == 1.0
    assert d[7] == -448.0


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4096).astype(np.float32) * 100
    b = torch.from_numpy(x).to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.decode_bf16(bits), b.to(torch.float64).numpy())


def test_fp8_dequant_scale_multiplies():
    codes = np.array([[0x38, 0x40, 0xB8]], dtype=np.uint8)        # 1.0, 2.0, -1.0
    k = O.index_keys_f64(codes, np.array([0.25], dtype=np.float32))
    assert np.array_equal(k, np.array([[0.25, 0.5, -0.25]]))


# ----------------------------------------------------------------------------- P2 indexer

def test_indexer_single_head_is_relu_dot():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 16))
    keys = rng.standard_normal((50, 16))
    s = O.indexer_scores(q, np.array([1.0]), keys, 49)
    assert np.allclose(s, np.maximum(np.dot(keys, q[0]), 0.0), rtol=0, atol=1e-13)


def test_indexer_zero_weights_and_masking():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 8))
    keys = rng.standard_normal((20, 8))
    s = O.indexer_scores(q, np.zeros(4), keys, 11)
    assert np.all(s[:12] == 0.0) and np.all(np.isneginf(s[12:]))


def test_indexer_weight_linearity_and_head_additivity():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 8))
    w = rng.random(3)
    keys = rng.standard_normal((30, 8))
    tot = O.indexer_scores(q, w, keys, 29)
    per_head = sum(O.indexer_scores(q[h:h + 1], w[h:h + 1], keys, 29) for h in range(3))
    assert np.allclose(tot, per_head, atol=1e-13)
    assert np.allclose(O.indexer_scores(q, 2 * w, keys, 29), 2 * tot, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_indexer_matches_brute_force(seed):
    rng = np.random.default_rng(10 + seed)
    H, D, N = 3, 5, 40
    q = rng.standard_normal((H, D))
    w = rng.random(H) - 0.3                 # any sign is accepted
    keys = rng.standard_normal((N, D))
    p = N - 1 - seed
    s = O.indexer_scores(q, w, keys, p)
    for i in range(N):
        want = L.score(q.tolist(), w.tolist(), keys[i].tolist()) if i <= p else -math.inf
        assert s[i] == pytest.approx(want, abs=1e-12) if i <= p else s[i] == want


# ----------------------------------------------------------------------------- golden

def test_golden_hand_worked_flat_and_hi():
    g = _golden("hand_worked_select.json")
    q, w, keys = np.array(g["q"]), np.array(g["w"]), np.array(g["keys"])
    s = O.indexer_scores(q, w, keys, len(keys) - 1)
    assert np.array_equal(s, np.array(g["scores"]))
    for c in g["flat_cases"]:
        sc = O.indexer_scores(q, w, keys[: c["p"] + 1], c["p"])
        idx = O.select_tokens(sc, c["p"], c["K"], c["S"], c["W"])
        assert idx.tolist() == c["idx"], c["why"]
    for c in g["hi_cases"]:
        nb = len(keys) // c["Bs"]
        kbar = O.block_means(keys, c["Bs"], nb)
        idx, kept, _, _ = O.select_tokens_hi(q, w, keys, kbar, c["p"], c["K"], c["S"], c["W"],
                                             c["Bs"], c["n_keep"])
        assert kept[kept >= 0].tolist() == c["kept"], c["why"]
        assert idx.tolist() == c["idx"], c["why"]
    c = g["hi_max_case"]
    k2 = np.array(c["keys"])
    kbar = O.block_means(k2, c["Bs"], len(k2) // c["Bs"])
    idx, kept, _, _ = O.select_tokens_hi(q, w, k2, kbar, c["p"], c["K"], c["S"], c["W"],
                                         c["Bs"], c["n_keep"])
    assert kept[kept >= 0].tolist() == c["kept"], c["why"]
    assert idx.tolist() == c["idx"], c["why"]


# ----------------------------------------------------------------------------- P3 selection

def _rand_scores(rng, n, ties=False):
    if ties:
        return rng.integers(0, 6, size=n).astype(np.float64)
    return rng.standard_normal(n)


@pytest.mark.parametrize("seed", range(12))
def test_selection_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 300))
    p = n - 1
    K = int(rng.integers(1, 80))
    S = int(rng.integers(0, K + 1))
    W = int(rng.integers(0, K - S + 1))
    sc = _rand_scores(rng, n, ties=seed % 2 == 0)
    idx = O.select_tokens(sc, p, K, S, W)
    valid = idx[idx >= 0]
    F = set(range(min(S, p + 1))) | set(range(max(0, p - W + 1), p + 1))
    assert len(idx) == K
    assert np.all(idx[len(valid):] == -1)
    assert np.all(np.diff(valid) > 0)                          # ascending, unique
    assert len(valid) == min(K, p + 1)                          # budget filled
    assert F <= set(valid.tolist())                             # sink and window always in
    C = [s for s in range(p + 1) if s not in F]
    chosen = [s for s in valid if s not in F]
    rest = [s for s in C if s not in set(chosen)]
    if chosen and rest:
        assert min(sc[chosen]) >= max(sc[rest])
        # ties at the boundary go to the lower position
        lo = min(sc[chosen])
        tied_out = [s for s in rest if sc[s] == lo]
        tied_in = [s for s in chosen if sc[s] == lo]
        if tied_out:
            assert max(tied_in) < min(tied_out)


@pytest.mark.parametrize("seed", range(6))
def test_selection_without_forced_is_lexsort_and_partition(seed):
    rng = np.random.default_rng(200 + seed)
    n, K = 257, 31
    sc = rng.standard_normal(n)
    idx = O.select_tokens(sc, n - 1, K, 0, 0)
    want = np.sort(np.lexsort((np.arange(n), -sc))[:K])
    assert np.array_equal(idx, want)
    kth = -np.partition(-sc, K - 1)[K - 1]
    assert sc[idx].min() == kth


@pytest.mark.parametrize("seed", range(10))
def test_selection_matches_rank_counting(seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 60))
    p = n - 1 - int(rng.integers(0, min(n, 5)))
    K = int(rng.integers(1, 20))
    S = int(rng.integers(0, K + 1))
    W = int(rng.integers(0, K - S + 1))
    sc = _rand_scores(rng, n, ties=True)
    got = O.select_tokens(sc, p, K, S, W)
    want = L.select({i: sc[i] for i in range(n)}, p, K, S, W)
    assert got.tolist() == want


def test_selection_budget_precondition():
    with pytest.raises(ValueError):
        O.select_tokens(np.zeros(10), 9, 4, 3, 2)


# ----------------------------------------------------------------------------- P4 HI

def test_block_means_is_numpy_mean():
    rng = np.random.default_rng(7)
    keys = rng.standard_normal((640, 8))
    kb = O.block_means(keys, 64, 10)
    for j in range(10):
        assert np.allclose(kb[j], np.mean(keys[j * 64:(j + 1) * 64], axis=0), atol=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_hi_all_blocks_kept_equals_flat(seed):
    rng = np.random.default_rng(400 + seed)
    Bs = 8
    N = int(rng.integers(4, 40)) * Bs + int(rng.integers(0, Bs))
    H, D = 3, 6
    q, w = rng.standard_normal((H, D)), rng.random(H)
    keys = rng.standard_normal((N, D))
    p = N - 1
    K, S, W = 24, 3, Bs + 2                   # W >= Bs - 1: the incomplete block is forced
    kbar = O.block_means(keys, Bs, N // Bs)
    flat = O.select_tokens(O.indexer_scores(q, w, keys, p), p, K, S, W)
    hi, kept, _, _ = O.select_tokens_hi(q, w, keys, kbar, p, K, S, W, Bs, N // Bs)
    assert np.array_equal(flat, hi)


@pytest.mark.parametrize("seed", range(6))
def test_hi_matches_brute_force(seed):
    rng = np.random.default_rng(500 + seed)
    Bs = 4
    N = int(rng.integers(3, 12)) * Bs + int(rng.integers(0, Bs))
    H, D = 2, 3
    q, w = rng.standard_normal((H, D)), rng.random(H)
    keys = rng.standard_normal((N, D))
    p = N - 1 - int(rng.integers(0, 3))
    K, S, W, n_keep = 9, 2, int(rng.integers(1, 6)), int(rng.integers(1, 4))
    kbar = O.block_means(keys, Bs, N // Bs)
    idx, kept, _, _ = O.select_tokens_hi(q, w, keys, kbar, p, K, S, W, Bs, n_keep)
    bidx, bkept = L.hi_select(q.tolist(), w.tolist(), keys.tolist(), p, K, S, W, Bs, n_keep)
    assert kept.tolist() == bkept
    assert idx.tolist() == bidx


def test_hi_recovers_planted_blocks():
    rng = np.random.default_rng(8)
    Bs, nb, H, D = 16, 64, 2, 16
    keys = rng.standard_normal((Bs * nb, D)) / 4
    q = rng.standard_normal((H, D))
    planted = [5, 17, 33, 40]
    for j in planted:
        keys[j * Bs:(j + 1) * Bs] += 2.0 * q[0] / np.linalg.norm(q[0])
    kbar = O.block_means(keys, Bs, nb)
    p = Bs * nb - 1
    c = O.coarse_block_scores(q, np.array([1.0, 0.0]), kbar, p, 4, 16, Bs)
    kept = O.keep_blocks(c, 4)
    assert kept.tolist() == planted


# ----------------------------------------------------------------------------- P5 attention

def _sdpa_dense(q, k, v, tau):
    qt = torch.from_numpy(q)[None, :, None, :]           # [1, H, 1, d]
    kt = torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(v)[None, None].expand(1, q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=tau)[0, :, 0].numpy()


@pytest.mark.parametrize("seed", range(4))
def test_budget_covers_context_equals_dense_causal(seed):
    rng = np.random.default_rng(600 + seed)
    N, Hq, Hkv, d = 37, 4, 2, 8
    keys_i = rng.standard_normal((N, 5))
    qi, wi = rng.standard_normal((2, 5)), rng.random(2)
    k = rng.standard_normal((N, Hkv, d))
    v = rng.standard_normal((N, Hkv, d))
    q = rng.standard_normal((Hq, d))
    p = N - 1 - seed
    idx = O.select_tokens(O.indexer_scores(qi, wi, keys_i[: p + 1], p), p, N + 3, 2, 3)
    assert idx[idx >= 0].tolist() == list(range(p + 1))
    o, lse = O.attend(q, k, v, idx, 0.3)
    g = Hq // Hkv
    for hq in range(Hq):
        kvh = hq // g
        want = _sdpa_dense(q[hq:hq + 1], k[: p + 1, kvh], v[: p + 1, kvh], 0.3)[0]
        assert np.allclose(o[hq], want, atol=1e-12)
        z = 0.3 * k[: p + 1, kvh] @ q[hq]
        assert lse[hq] == pytest.approx(np.log(np.sum(np.exp(z))), abs=1e-12)


def test_attention_closed_forms():
    # one selected row: o = V[s]
    k = np.arange(12, dtype=np.float64).reshape(6, 1, 2)
    v = np.arange(18, dtype=np.float64).reshape(6, 1, 3) * 0.5
    q = np.array([[0.3, -0.2]])
    o, _ = O.attend(q, k, v, np.array([4, -1, -1]), 1.0)
    assert np.array_equal(o[0], v[4, 0])
    # equal logits (q = 0): o = mean of selected V rows, lse = log(count)
    o, lse = O.attend(np.zeros((1, 2)), k, v, np.array([0, 2, 5, -1]), 1.0)
    assert np.allclose(o[0], v[[0, 2, 5], 0].mean(axis=0), atol=1e-15)
    assert lse[0] == pytest.approx(math.log(3))
    # logits 0,1,2 and one-hot values: o = e^s / (1 + e + e^2)
    k1 = np.array([[[0.0]], [[1.0]], [[2.0]]])
    v1 = np.eye(3)[:, None, :]
    o, lse = O.attend(np.array([[1.0]]), k1, v1, np.array([0, 1, 2]), 1.0)
    den = 1 + math.e + math.e ** 2
    assert np.allclose(o[0], [1 / den, math.e / den, math.e ** 2 / den], atol=1e-15)
    assert lse[0] == pytest.approx(math.log(den), abs=1e-14)


def test_attention_permutation_invariant_and_gqa_mapping():
    rng = np.random.default_rng(9)
    N, Hq, Hkv, d = 20, 8, 2, 4
    k, v = rng.standard_normal((N, Hkv, d)), rng.standard_normal((N, Hkv, d + 1))
    q = rng.standard_normal((Hq, d))
    idx = np.array([1, 3, 4, 9, 15, -1])
    o1, l1 = O.attend(q, k, v, idx, 0.5)
    o2, l2 = O.attend(q, k, v, np.array([15, 4, 1, 9, 3, -1]), 0.5)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)
    lo, ll = L.attend(q.tolist(), k.tolist(), v.tolist(), idx.tolist(), 0.5, Hkv)
    assert np.allclose(o1, np.array(lo), atol=1e-12) and np.allclose(l1, ll, atol=1e-12)
    # head 3 reads KV head 0, head 4 reads KV head 1 (kvh = hq // g)
    o_h3, _ = O.attend(q[3:4], k[:, :1], v[:, :1], idx, 0.5)
    o_h4, _ = O.attend(q[4:5], k[:, 1:], v[:, 1:], idx, 0.5)
    assert np.allclose(o1[3], o_h3[0]) and np.allclose(o1[4], o_h4[0])


def test_mla_value_is_row_prefix():
    rows = np.arange(2 * 1 * 6, dtype=np.float64).reshape(2, 1, 6)
    kr, vr = O.mla_kv(rows, 4)
    assert np.array_equal(vr, rows[..., :4]) and kr is rows


# ----------------------------------------------------------------------------- P6 CLI

def test_cli_reuse_equals_per_layer_recompute():
    from synth import config, make_inputs
    cfg = config(5, B=2, N=300, K=40, S=4, W=8, Hq=8, Hkv=2, H_I=4, D_I=16, d_qk=16, d_v=16)
    inp = make_inputs(cfg)
    res = O.reference_step(inp)
    for layer in range(cfg.layers):
        one = dict(inp)
        one["q"], one["k"], one["v"] = inp["q"][layer:layer + 1], inp["k"][layer:layer + 1], inp["v"][layer:layer + 1]
        one["cfg"] = cfg.scaled(layers=1)
        r1 = O.reference_step(one)
        for b in range(cfg.B):
            assert np.array_equal(r1["idx"][(b, 0)], res["idx"][(b, 0)])
            assert np.array_equal(r1["out"][(0, b, 0)], res["out"][(layer, b, 0)])
    # distinct layers do give distinct outputs for the same selection
    assert not np.allclose(res["out"][(0, 0, 0)], res["out"][(1, 0, 0)])


def test_reference_step_small_c1_shape_consistency():
    from synth import config, make_inputs
    cfg = config(1, N=600, K=64, S=4, W=16)
    inp = make_inputs(cfg)
    res = O.reference_step(inp)
    P = O.query_positions(inp["ctx_len"], cfg.T)
    for t in range(cfg.T):
        idx = res["idx"][(0, t)]
        assert idx.max() == P[0, t]
        assert res["out"][(0, 0, t)].shape == (cfg.Hq, cfg.d_v)
    # salient keys are chosen far above the chance rate of the fill
    sal = set(inp["salient"][0].tolist())
    chosen = set(res["idx"][(0, 0)].tolist())
    chance = (cfg.K - cfg.S - cfg.W) / (cfg.N - cfg.T - cfg.S - cfg.W)
    assert len(sal & chosen) / len(sal) > 4 * chance


# ----------------------------------------------------------------------------- cache append (R12, R25)

def test_e4m3fn_encode_round_trips_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.decode_e4m3fn(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(O.encode_e4m3fn(vals[fin]), codes[fin])  # -0.0 -> 0x80 included


def test_e4m3fn_encode_ties_to_even_and_saturation():
    # midpoints between neighbours go to the even code (mantissa LSB 0)
    cases = {
        1.0625: 0x38,            # between 1.0 (0x38) and 1.125 (0x39)
        1.1875: 0x3A,            # between 1.125 (0x39) and 1.25 (0x3A)
        2.0 ** -10: 0x00,        # between 0 and the smallest subnormal 2^-9 (0x01)
        1.5 * 2.0 ** -9: 0x02,   # between 2^-9 (0x01) and 2^-8 (0x02)
        2.0 ** -6 - 2.0 ** -10: 0x08,  # between the largest subnormal 7*2^-9 (0x07) and 2^-6 (0x08)
        432.0: 0x7E,             # between 416 (0x7D) and 448 (0x7E)
        1.0e6: 0x7E,             # beyond the range: the largest finite value
        -1.0625: 0xB8,
        -1.0e-30: 0x80,          # rounds to -0
    }
    x = np.array(list(cases), dtype=np.float64)
    assert np.array_equal(O.encode_e4m3fn(x), np.array(list(cases.values()), dtype=np.uint8))
    # just off a midpoint: to the nearer side
    assert O.encode_e4m3fn(np.array([1.0625 + 1e-9, 1.1875 - 1e-9])).tolist() == [0x39, 0x39]


def test_e4m3fn_encode_matches_torch_cast():
    # a library routine on the special case of in-range float32 values, subnormals included
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 1e-2,
                        rng.standard_normal(5000) * 3e-3]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_e4m3fn(x), ref)


def test_quantize_key_rows_scale_and_extremes():
    rng = np.random.default_rng(8)
    k = (rng.standard_normal((64, 128)) / np.sqrt(128)).astype(np.float32)
    k[3] = 0.0
    codes, scale = O.quantize_key_rows(k)
    amax = np.abs(k).max(axis=1)
    assert scale.dtype == np.float32
    assert scale[3] == np.float32(np.float32(1e-12) / np.float32(448.0)) and not codes[3].any()
    rows = np.arange(64) != 3
    # the largest magnitude of each row lands on +-448 (0x7E / 0xFE)
    j = np.abs(k).argmax(axis=1)
    assert np.all((codes[rows, j[rows]] & 0x7F) == 0x7E)
    # dequantised keys within half a step of 3 mantissa bits (relative 2^-4), or of the
    # subnormal spacing 2^-9 * scale near zero
    deq = O.decode_e4m3fn(codes) * scale[:, None].astype(np.float64)
    err = np.abs(deq - k)
    bound = np.maximum(np.abs(k) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(err[rows] <= bound[rows])
    # agrees with the generator's reading of the same quantisation (torch's cast)
    y = np.clip(k / scale[:, None], -448, 448).astype(np.float32)
    assert np.array_equal(codes, torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_cache_append_positions_rows_and_completed_blocks():
    rng = np.random.default_rng(9)
    B, N, D, T, E = 3, 256, 8, 5, 6
    caches = {"k": np.zeros((B, N, D), np.uint8), "scale": np.zeros((B, N), np.float32),
              "rows": [np.zeros((B, N, E), np.uint16)]}
    k_new = rng.standard_normal((B, T, D)).astype(np.float32)
    rows_new = [rng.integers(0, 65535, (B, T, E), dtype=np.uint16)]
    pos0 = np.array([0, 60, 253])  # sequence 2: the last two new tokens fall past N
    written = O.cache_append(caches, k_new, rows_new, pos0, fp8=True)
    assert written == [(0, s) for s in range(5)] + [(1, s) for s in range(60, 65)] + [(2, 253), (2, 254), (2, 255)]
    assert np.array_equal(caches["rows"][0][1, 60:65], rows_new[0][1])
    assert not caches["rows"][0][1, 65:].any() and not caches["rows"][0][1, :60].any()
    codes, sc = O.quantize_key_rows(k_new[2, :3])
    assert np.array_equal(caches["k"][2, 253:256], codes) and np.array_equal(caches["scale"][2, 253:256], sc)
    # blocks of 64: sequence 1 completes block 0 (row 63), sequence 2 completes block 3 (row 255)
    assert O.completed_blocks(written, 64, 4) == [(1, 0), (2, 3)]
    assert O.completed_blocks(written, 64, 3) == [(1, 0)]


# ----------------------------------------------------------------------------- fp8-query indexer (R27)

def _bf16_bits(x):
    x = np.asarray(x, dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.decode_bf16(bits), x.astype(np.float64)), "value not exact in bf16"
    return bits


def test_fp8_query_worked_example():
    # q = (2, -1, 0.5, 13/128): amax 2, scale s = 2/448 in fp32; q/s = 448, -224, 112,
    # 22.75 -> codes 448, -224, 112 and 22 (22.75 lies between the grid points 22 and 24)
    bits = _bf16_bits([2.0, -1.0, 0.5, 0.1015625])
    s = float(np.float32(2.0) / np.float32(448.0))
    deq = O.index_query_f64(bits[None], True)[0]
    assert np.array_equal(deq, np.array([448.0, -224.0, 112.0, 22.0]) * s)
    assert np.array_equal(O.index_query_f64(bits[None], False)[0], [2.0, -1.0, 0.5, 0.1015625])
    # one head of weight 0.5 against the key (1, 1, 1, 1): 0.5 * (448 - 224 + 112 + 22) * s
    sc = O.indexer_scores(deq[None], np.array([0.5]), np.ones((1, 4)), 0)
    assert sc[0] == 0.5 * 358.0 * s


def test_fp8_query_exact_for_representable_rows():
    # rows that are e4m3 values times 2^-6 with a 448 * 2^-6 entry: scale 2^-6 exactly,
    # every code reproduces its element, so the quantised query equals the bf16 query
    rng = np.random.default_rng(27)
    codes = rng.integers(0, 256, (3, 5, 64)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C            # no NaN codes
    codes[..., 7] = 0x7E                             # +448
    q = O.decode_e4m3fn(codes) * 2.0 ** -6
    bits = _bf16_bits(q.astype(np.float32))
    assert np.array_equal(O.index_query_f64(bits, True), O.decode_bf16(bits))


def test_fp8_query_error_bound_rows_and_scaling():
    rng = np.random.default_rng(28)
    x = rng.standard_normal((4, 8, 128)).astype(np.float32)
    x *= (2.0 ** rng.integers(-10, 10, (4, 8, 1))).astype(np.float32)   # row magnitudes differ
    bits = _bf16_bits_round(x)
    q = O.decode_bf16(bits)
    deq = O.index_query_f64(bits, True)
    s = np.maximum(np.abs(q).max(axis=-1, keepdims=True), 1e-12) / 448.0
    # round to nearest on the e4m3 grid: relative 2^-4 (normal codes), 2^-10 * s (subnormal)
    assert np.all(np.abs(deq - q) <= np.maximum(2.0 ** -4 * np.abs(q), 2.0 ** -10 * s) * (1 + 1e-6))
    # each row on its own scale: quantising rows one at a time changes nothing
    for t in range(4):
        for h in range(8):
            assert np.array_equal(O.index_query_f64(bits[t, h][None], True)[0], deq[t, h])
    # doubling a row (exact in bf16) doubles its dequantised values exactly
    bits2 = _bf16_bits((q * 2.0).astype(np.float32))
    assert np.array_equal(O.index_query_f64(bits2, True), 2.0 * deq)


def _bf16_bits_round(x):
    """float32 -> bf16 bits, round to nearest even (torch's cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_fp8_query_score_is_the_fp8_contraction():
    # scale_k * sum_h (w_h * s_q,h) * ReLU(codes_h . codes_k) in exact arithmetic on the
    # decoded codes (every product of two e4m3 values and their 128-term sums are exact
    # in float64) equals the score of the dequantised rows
    rng = np.random.default_rng(29)
    H, D, n = 16, 128, 40
    bits = _bf16_bits_round(rng.standard_normal((H, D)).astype(np.float32))
    w = rng.random(H)
    kc, ks = O.quantize_key_rows(rng.standard_normal((n, D)).astype(np.float32))
    qc, qs = O.quantize_key_rows(O.decode_bf16(bits).astype(np.float32))
    dots = O.decode_e4m3fn(kc) @ O.decode_e4m3fn(qc).T                    # [n, H], exact
    want = ks.astype(np.float64) * (np.maximum(dots, 0.0) @ (w * qs.astype(np.float64)))
    got = O.indexer_scores(O.index_query_f64(bits, True), w, O.index_keys_f64(kc, ks), n - 1)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


# ----------------------------------------------------------------------------- attention backward (R28)

def _torch_sparse_attention(q, k_rows, v_rows, idx, tau):
    """Sparse attention written with torch ops (gather, softmax), float64, for autograd."""
    sel = torch.as_tensor(np.asarray(idx)[np.asarray(idx) >= 0], dtype=torch.long)
    Hq, Hkv = q.shape[0], k_rows.shape[1]
    g = Hq // Hkv
    kv_of_head = torch.arange(Hq) // g
    Ks = k_rows[sel][:, kv_of_head, :].permute(1, 0, 2)        # [Hq, n, dqk]
    Vs = v_rows[sel][:, kv_of_head, :].permute(1, 0, 2)        # [Hq, n, dv]
    z = tau * torch.einsum("hd,hnd->hn", q, Ks)
    return torch.einsum("hn,hnd->hd", torch.softmax(z, dim=1), Vs), torch.logsumexp(z, dim=1)


def _bwd_case(rng, Hq, Hkv, dqk, dv, N, K, n_pad=0):
    q = rng.standard_normal((Hq, dqk)) / np.sqrt(dqk)
    k = rng.standard_normal((N, Hkv, dqk))
    v = rng.standard_normal((N, Hkv, dv))
    idx = np.full(K, -1, np.int64)
    idx[: K - n_pad] = np.sort(rng.choice(N, K - n_pad, replace=False))
    dout = rng.standard_normal((Hq, dv))
    return q, k, v, idx, dout


@pytest.mark.parametrize("Hq,Hkv,dqk,dv,mla", [(8, 2, 16, 16, False), (6, 1, 24, 16, True), (4, 4, 8, 12, False)])
def test_attention_backward_matches_autograd(Hq, Hkv, dqk, dv, mla):
    rng = np.random.default_rng(31 + Hq)
    N, K, tau = 40, 12, 0.3
    q, k, v, idx, dout = _bwd_case(rng, Hq, Hkv, dqk, dv, N, K, n_pad=3)
    if mla:
        v = k[..., :dv]
    out, lse = O.attend(q, k, v, idx, tau)
    dq, dK, dV = O.attend_backward(q, k, v, idx, tau, out, lse, dout)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = tk[..., :dv] if mla else torch.tensor(v, requires_grad=True)
    to, tl = _torch_sparse_attention(tq, tk, tv, idx, tau)
    assert np.allclose(to.detach().numpy(), out, atol=1e-12) and np.allclose(tl.detach().numpy(), lse, atol=1e-12)
    grads = torch.autograd.grad((to * torch.tensor(dout)).sum(), (tq, tk) if mla else (tq, tk, tv))
    assert np.allclose(dq, grads[0].numpy(), atol=1e-12)
    if mla:
        assert np.allclose(O.mla_row_grad(dK, dV), grads[1].numpy(), atol=1e-12)
    else:
        assert np.allclose(dK, grads[1].numpy(), atol=1e-12)
        assert np.allclose(dV, grads[2].numpy(), atol=1e-12)


def test_attention_backward_finite_differences():
    rng = np.random.default_rng(32)
    q, k, v, idx, dout = _bwd_case(rng, 2, 1, 4, 3, 7, 4, n_pad=1)
    tau = 0.7

    def loss(q_, k_, v_):
        o, _ = O.attend(q_, k_, v_, idx, tau)
        return float(np.sum(o * dout))
    out, lse = O.attend(q, k, v, idx, tau)
    dq, dK, dV = O.attend_backward(q, k, v, idx, tau, out, lse, dout)
    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dK, 1), (v, dV, 2)):
        for pos in np.ndindex(arr.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][pos] += eps
            up = loss(*args)
            args[which][pos] -= 2 * eps
            dn = loss(*args)
            assert abs((up - dn) / (2 * eps) - grad[pos]) < 1e-7, (which, pos)


def test_attention_backward_closed_forms():
    rng = np.random.default_rng(33)
    q, k, v, _, dout = _bwd_case(rng, 4, 2, 8, 8, 10, 1)
    # one selected row: the softmax is constant 1, so q and K get no gradient and V's
    # row receives the sum of its heads' output gradients
    idx = np.array([6, -1, -1])
    out, lse = O.attend(q, k, v, idx, 0.5)
    dq, dK, dV = O.attend_backward(q, k, v, idx, 0.5, out, lse, dout)
    assert np.allclose(dq, 0, atol=1e-15) and np.allclose(dK, 0, atol=1e-15)
    assert np.allclose(dV[6, 0], dout[0] + dout[1]) and np.allclose(dV[6, 1], dout[2] + dout[3])
    assert np.count_nonzero(dV[np.arange(10) != 6]) == 0
    # nothing selected: every gradient is zero
    dq0, dK0, dV0 = O.attend_backward(q, k, v, np.full(3, -1), 0.5, np.zeros_like(out), np.full(4, -np.inf), dout)
    assert not dq0.any() and not dK0.any() and not dV0.any()
    # zero output gradient: zero everywhere
    z = O.attend_backward(q, k, v, np.array([1, 4, 9]), 0.5, *O.attend(q, k, v, np.array([1, 4, 9]), 0.5),
                          np.zeros_like(dout))
    assert all(not a.any() for a in z)


# ----------------------------------------------------------------------------- shared selection (R29)

def test_shared_selection_rows_worked_example():
    # context 12, three draft tokens at positions 9, 10, 11 sharing the row (0, 5, 9, 10, 11, -1)
    rows = O.shared_selection_rows([0, 5, 9, 10, 11, -1], 12, 3)
    assert rows.tolist() == [[0, 5, 9, -1, -1, -1], [0, 5, 9, 10, -1, -1], [0, 5, 9, 10, 11, -1]]
    # one token: its own position is the last one, nothing is masked
    assert O.shared_selection_rows([3, 7, -1], 8, 1).tolist() == [[3, 7, -1]]
    # a token before every entry keeps nothing, and its attention is empty
    r = O.shared_selection_rows([6, 7], 8, 3)
    assert r[0].tolist() == [-1, -1]
    o, lse = O.attend(np.ones((2, 4)), np.ones((8, 1, 4)), np.ones((8, 1, 4)), r[0], 0.5)
    assert not o.any() and np.all(np.isneginf(lse))


# ----------------------------------------------------------------------------- indexer distillation target (R30)

def test_indexer_target_is_head_mean_of_attention():
    # closed forms: the target sums to 1 over the valid entries; with one head it is that
    # head's softmax; with identical heads the mean is any one of them
    rng = np.random.default_rng(71)
    N, K, tau = 30, 9, 0.4
    k = rng.standard_normal((N, 2, 8))
    idx = np.full(K, -1)
    idx[:7] = np.sort(rng.choice(N, 7, replace=False))
    q = rng.standard_normal((4, 8))
    _, lse = O.attend(q, k, k, idx, tau)
    p = O.indexer_target(q, k, idx, tau, lse)
    assert abs(p.sum() - 1.0) < 1e-12 and np.all(p[7:] == 0)
    q1 = q[:1]
    _, lse1 = O.attend(q1, k[:, :1], k[:, :1], idx, tau)
    z = tau * (k[idx[:7], 0] @ q1[0])
    soft = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    assert np.allclose(O.indexer_target(q1, k[:, :1], idx, tau, lse1)[:7], soft, atol=1e-15)
    q2 = np.repeat(q[:1], 2, axis=0)
    _, lse2 = O.attend(q2, k[:, :1], k[:, :1], idx, tau)
    assert np.allclose(O.indexer_target(q2, k[:, :1], idx, tau, lse2)[:7], soft, atol=1e-15)


def test_indexer_kl_zero_minimum_and_finite_differences():
    rng = np.random.default_rng(72)
    K = 8
    valid = np.array([True] * 6 + [False] * 2)
    t = np.zeros(K)
    t[:6] = rng.random(6)
    t[:6] /= t[:6].sum()
    # scores equal to log target (plus a constant): the indexer matches, loss and gradient 0
    loss, grad = O.indexer_kl(t, np.concatenate([np.log(t[:6]) + 3.0, [5.0, -2.0]]), valid)
    assert abs(loss) < 1e-12 and np.allclose(grad, 0, atol=1e-12)
    # elsewhere the loss is positive and the gradient is the derivative of the loss
    sc = rng.standard_normal(K)
    loss, grad = O.indexer_kl(t, sc, valid)
    assert loss > 0 and grad[6] == 0 and grad[7] == 0 and abs(grad.sum()) < 1e-12
    eps = 1e-6
    for j in range(K):
        up, dn = sc.copy(), sc.copy()
        up[j] += eps
        dn[j] -= eps
        fd = (O.indexer_kl(t, up, valid)[0] - O.indexer_kl(t, dn, valid)[0]) / (2 * eps)
        assert abs(fd - grad[j]) < 1e-8, j
    # two entries by hand: target (1, 0), scores (0, 0): loss log 2, gradient (-1/2, 1/2)
    loss, grad = O.indexer_kl([1.0, 0.0], [0.0, 0.0], [True, True])
    assert abs(loss - np.log(2.0)) < 1e-15 and np.allclose(grad, [-0.5, 0.5])


# ----------------------------------------------------------------------------- positions, MLA value, HI fine stage

def test_query_positions_hand_worked():
    # R11 worked on paper: a sequence with ctx visible rows and T query tokens puts token t
    # at position ctx - T + t, so the T queries are the last T rows in token order
    # (ctx 12, T 3 -> 9 10 11; ctx 7 -> 4 5 6; ctx 3 -> 0 1 2).
    got = O.query_positions(np.array([12, 7, 3]), 3)
    assert got.tolist() == [[9, 10, 11], [4, 5, 6], [0, 1, 2]]
    assert O.query_positions(np.array([5]), 1).tolist() == [[4]]


def _dense_prefix_sdpa(q, k, v, tau, n):
    """torch's float64 scaled dot-product attention of one query token's heads over rows
    [0, n) (a library routine; the causal prefix written out by its length)."""
    Hq, Hkv = q.shape[0], k.shape[1]
    g = Hq // Hkv
    out = np.zeros((Hq, v.shape[2]))
    for hq in range(Hq):
        out[hq] = _sdpa_dense(q[hq:hq + 1], k[:n, hq // g], v[:n, hq // g], tau)[0]
    return out


def test_reference_step_positions_are_causal_prefixes():
    # Budget >= context: token t of T attends over exactly its causal prefix [0, N-T+t]
    # (R11 with ctx = N), which the library's dense attention over that many rows fixes.
    from synth import config, make_inputs
    cfg = config(1, N=40, T=3, K=64, S=4, W=8, H_I=2, D_I=8, Hq=4, d_qk=16, d_v=16)
    inp = make_inputs(cfg)
    res = O.reference_step(inp)
    k, v = O.decode_bf16(inp["k"][0, 0]), O.decode_bf16(inp["v"][0, 0])
    for t in range(cfg.T):
        n = cfg.N - cfg.T + t + 1
        assert res["idx"][(0, t)][res["idx"][(0, t)] >= 0].tolist() == list(range(n))
        q = O.decode_bf16(inp["q"][0, 0, t])
        want = _dense_prefix_sdpa(q, k, v, cfg.tau, n)
        assert np.allclose(res["out"][(0, 0, t)], want, atol=1e-12)


def _mla_cfg(**kw):
    from synth import config
    base = dict(B=1, N=30, T=1, H_I=2, D_I=8, Hq=4, d_qk=24, d_v=16, salient="none")
    base.update(kw)
    return config(2, **base)


def test_reference_step_mla_one_selected_row_is_its_value_prefix():
    # One selected row (budget K = 1 taken by a sink of 1): o = V[0] exactly for every head,
    # and V of an MLA latent row is its first d_v columns (R15: the configuration's 512
    # latent + 64 rope columns, the rope part entering only q.K); lse = z_0.
    from synth import make_inputs
    cfg = _mla_cfg(K=1, S=1, W=0)
    inp = make_inputs(cfg)
    res = O.reference_step(inp)
    assert res["idx"][(0, 0)].tolist() == [0]
    row0 = O.decode_bf16(inp["k"][0, 0, 0, 0])
    q = O.decode_bf16(inp["q"][0, 0, 0])
    for h in range(cfg.Hq):
        assert np.array_equal(res["out"][(0, 0, 0)][h], row0[: cfg.d_v])
        assert res["lse"][(0, 0, 0)][h] == pytest.approx(cfg.tau * float(np.dot(q[h], row0)), abs=1e-12)


def test_reference_step_mla_dense_matches_sdpa():
    # Budget >= context on MLA rows: the library's dense attention with K = the whole
    # latent row and V = its first d_v columns.
    from synth import make_inputs
    cfg = _mla_cfg(K=40, S=2, W=4)
    inp = make_inputs(cfg)
    res = O.reference_step(inp)
    rows = O.decode_bf16(inp["k"][0, 0])                 # [N, 1, d_qk]
    q = O.decode_bf16(inp["q"][0, 0, 0])
    want = _dense_prefix_sdpa(q, rows, rows[..., : cfg.d_v], cfg.tau, cfg.N)
    assert np.allclose(res["out"][(0, 0, 0)], want, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_fine_given_all_eligible_kept_equals_flat(seed):
    # R9: with every eligible block kept, the fine stage on that kept list is the flat
    # selection, bit for bit.
    rng = np.random.default_rng(700 + seed)
    Bs = 8
    N = int(rng.integers(4, 40)) * Bs + int(rng.integers(0, Bs))
    H, D = 3, 6
    q, w = rng.standard_normal((H, D)), rng.random(H)
    keys = rng.standard_normal((N, D))
    p = N - 1 - int(rng.integers(0, 3))
    K, S, W = 24, 3, Bs + 2
    flat = O.select_tokens(O.indexer_scores(q, w, keys[: p + 1], p), p, K, S, W)
    elig = np.nonzero(O.eligible_blocks(p, S, W, Bs, N // Bs))[0]
    kept = O.pad_sorted(elig, elig.size + 2)            # -1 padding is ignored
    got, cand, sc = O.select_fine_given_kept(q, w, keys, kept, p, K, S, W, Bs)
    assert np.array_equal(got, flat)
    assert np.allclose(sc, O.indexer_scores(q, w, keys[: p + 1], p)[cand], atol=1e-12)


def test_fine_given_kept_hand_worked():
    # The hand-worked HI cases: the fine stage run on the kept list worked on paper gives
    # the idx worked on paper.
    g = _golden("hand_worked_select.json")
    q, w, keys = np.array(g["q"]), np.array(g["w"]), np.array(g["keys"])
    for c in g["hi_cases"]:
        kept = np.array(c["kept"] + [-1], dtype=np.int64)
        idx, _, _ = O.select_fine_given_kept(q, w, keys, kept, c["p"], c["K"], c["S"], c["W"], c["Bs"])
        assert idx.tolist() == c["idx"], c["why"]


def test_hi_candidates_hand_worked():
    # Reading R9 on paper: the fine candidates are the positions of the kept blocks and of
    # the incomplete visible block, at or before p, minus the forced set.
    # p = 10, blocks of 4, sink 1, window 1: forced {0, 10}; kept block 0 gives 0..3, the
    # incomplete block (positions 8..11, visible up to 10) gives 8..10.
    assert O.hi_candidates(10, 1, 1, 4, np.array([0, -1])).tolist() == [1, 2, 3, 8, 9]
    # kept blocks 2 and 0 (any order), p = 13, sink 2, window 3: forced {0, 1, 11, 12, 13};
    # blocks 0 and 2 give 0..3 and 8..11, the incomplete block 12..13 is all forced.
    assert O.hi_candidates(13, 2, 3, 4, np.array([2, 0])).tolist() == [2, 3, 8, 9, 10]
    # positions past p are dropped: block 3 covers 12..15 and p = 12 leaves only 12, which
    # the window forces
    assert O.hi_candidates(12, 0, 1, 4, np.array([3])).tolist() == []
