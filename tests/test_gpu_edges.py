"""GPU edge cases and invariants of the HIP path (through the C ABI), against the oracle.

Short and ragged contexts, per-sequence context lengths, ties everywhere (zero
weights: every score equal), an empty fill (K = sink + window), K = 1, padded and
out-of-range idx entries, explicit split counts, HI with every block kept equal to
flat selection, CLI reuse equal to per-layer calls, fp32 output, workspace reuse, the
split merge in several rounds, and the attention shapes with up to 16 query heads per KV
head (MLA and GQA rows, 2- and 3-stage rings).
"""
import numpy as np
import pytest
import torch

import long_context_sparse_07_amd as L
from oracle import lsa_oracle as O
from synth import config, make_inputs
from gpu_harness import upload, gpu_index_select, gpu_attend, check_band, check_attn

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def _flat_check(inp, d, r):
    cfg = inp["cfg"]
    ora = O.reference_step(inp)
    P = O.query_positions(inp["ctx_len"], cfg.T)
    idx = _np(r["idx"])
    for b in range(cfg.B):
        for t in range(cfg.T):
            p = int(P[b, t])
            F = O.forced_positions(p, cfg.S, cfg.W)
            C = np.setdiff1d(np.arange(max(p + 1, 0)), F)
            check_band(idx[b, t], C, ora["scores"][(b, t)][C] if C.size else np.zeros(0), F, cfg.K,
                       what=f"{cfg.name} {b},{t}")
    out, _ = gpu_attend(d, r["idx"])
    o = _np(out)
    for layer in range(cfg.layers):
        for b in range(cfg.B):
            for t in range(cfg.T):
                check_attn(o[layer, b, t], ora["out"][(layer, b, t)], f"{cfg.name} L{layer} {b},{t}")
    return ora


@pytest.mark.parametrize("N", [50, 200, 511, 700])
def test_short_context(N):
    # p < K (everything visible selected), p < S + W (sink and window overlap)
    cfg = config(1, N=N, K=512, S=16, W=128, salient="none")
    inp = make_inputs(cfg)
    d = upload(inp)
    r = gpu_index_select(d)
    _flat_check(inp, d, r)


def test_per_sequence_context_lengths():
    cfg = config(5, B=3, T=2, N=3000, K=256, S=16, W=64, layers=1)
    inp = make_inputs(cfg)
    inp["ctx_len"] = np.array([3000, 1234, 130], dtype=np.int32)
    d = upload(inp)
    r = gpu_index_select(d)
    _flat_check(inp, d, r)


def test_all_scores_equal_tie_break_and_list_overflow():
    # w = 0: every score is 0; the fill is the lowest candidate positions. 40000 equal
    # keys overflow the composite list, so the resolve stage rescans the row.
    cfg = config(1, N=40000, K=512, S=16, W=128, salient="none", T=2)
    inp = make_inputs(cfg)
    inp["w"][:] = 0.0
    d = upload(inp)
    r = gpu_index_select(d)
    idx = _np(r["idx"])
    P = O.query_positions(inp["ctx_len"], cfg.T)
    for t in range(cfg.T):
        p = int(P[0, t])
        want = O.select_tokens(np.zeros(p + 1), p, cfg.K, cfg.S, cfg.W)
        assert np.array_equal(idx[0, t], want)


def test_fill_empty_and_k_one():
    cfg = config(1, N=1000, K=144, S=16, W=128, salient="none")     # K == S + W: no fill
    inp = make_inputs(cfg)
    d = upload(inp)
    r = gpu_index_select(d)
    _flat_check(inp, d, r)
    sc = L.lsa_index(d["qI"], d["w"], d["kI"], ctx_len=d["ctx_len"])
    one = _np(L.lsa_select(sc, 1, 0, 0, ctx_len=d["ctx_len"]))
    ora = O.reference_step(inp, with_attend=False)
    for t in range(cfg.T):
        s = ora["scores"][(0, t)]
        best = int(np.lexsort((np.arange(len(s)), -s))[0])
        assert one[0, t, 0] == best


def test_attend_padding_and_out_of_range_rows():
    cfg = config(5, B=2, N=2000, K=300, S=16, W=64, layers=1)
    inp = make_inputs(cfg)
    d = upload(inp)
    rng = np.random.default_rng(5)
    idx = np.full((cfg.B, 1, cfg.K), -1, dtype=np.int32)
    idx[0, 0, :100] = np.sort(rng.choice(cfg.N, 100, replace=False))
    idx[0, 0, 100:110] = cfg.N + 5            # out of range: skipped like -1
    # sequence 1: every entry padding -> out 0, lse -inf
    out, lse = gpu_attend(d, torch.from_numpy(idx).cuda(), n_splits=3)
    o, l = _np(out), _np(lse)
    want, wl = O.attend(O.decode_bf16(inp["q"][0, 0, 0]), O._LazyRows(inp["k"][0, 0]),
                        O._LazyRows(inp["v"][0, 0]), idx[0, 0, :100], cfg.tau)
    check_attn(o[0, 0, 0], want, "padded")
    assert np.allclose(l[0, 0, 0], wl, atol=2e-3)
    assert np.all(o[0, 1, 0] == 0) and np.all(np.isneginf(l[0, 1, 0]))


@pytest.mark.parametrize("splits", [1, 2, 7, 16, 0])
def test_attend_split_counts(splits):
    cfg = config(2, B=2, N=6000, K=512, S=32, W=128)
    inp = make_inputs(cfg)
    d = upload(inp)
    r = gpu_index_select(d)
    ora = O.reference_step(inp)
    idx_o = torch.from_numpy(np.stack([[ora["idx"][(b, 0)] for b in range(cfg.B)]]).transpose(1, 0, 2).astype(np.int32)).cuda()
    out, lse = gpu_attend(d, idx_o, n_splits=splits)
    o = _np(out)
    for b in range(cfg.B):
        check_attn(o[0, b, 0], ora["out"][(0, b, 0)], f"splits={splits} b={b}")


def test_fp32_output_matches_bf16_output():
    cfg = config(5, B=2, N=3000, K=256, S=16, W=64, layers=2)
    inp = make_inputs(cfg)
    d = upload(inp)
    r = gpu_index_select(d)
    ob, lb = gpu_attend(d, r["idx"])
    of, lf = gpu_attend(d, r["idx"], out_dtype=torch.float32)
    assert torch.equal(lb, lf)
    assert torch.equal(of.to(torch.bfloat16), ob)


def test_hi_with_all_blocks_kept_equals_flat():
    base = config(3, N=64 * 200, K=512, S=64, W=128, n_keep=200)
    inp = make_inputs(base)
    d = upload(inp)
    r_hi = gpu_index_select(d)
    flat = dict(d)
    flat["cfg"] = base.scaled(hi=False)
    r_flat = gpu_index_select(flat)
    assert torch.equal(r_hi["idx"], r_flat["idx"])


@pytest.mark.parametrize("splits", [1, 8, 16])
def test_cli_reuse_equals_per_layer_calls(splits):
    # the same split count on both sides (the default count depends on the number of
    # layers in the launch, and the split merge's order on the count)
    cfg = config(5, B=4, N=4000, K=512, S=32, W=128)
    inp = make_inputs(cfg)
    d = upload(inp)
    r = gpu_index_select(d)
    out, lse = gpu_attend(d, r["idx"], n_splits=splits)
    for layer in range(cfg.layers):
        o1, l1 = L.lsa_attend(d["q"][layer:layer + 1], d["k"][layer:layer + 1], d["v"][layer:layer + 1],
                              r["idx"], cfg.tau, n_splits=splits)
        assert torch.equal(o1[0], out[layer]) and torch.equal(l1[0], lse[layer])


def test_select_workspace_reuse_is_clean():
    cfg = config(2, B=2, N=7000, K=512, S=32, W=128)
    inp = make_inputs(cfg)
    d = upload(inp)
    sc = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"])
    a = L.lsa_select(sc, cfg.K, cfg.S, cfg.W)
    b = L.lsa_select(sc, cfg.K, cfg.S, cfg.W)
    c = L.lsa_select(sc[:, :, :5000].contiguous(), 300, 10, 20)   # a different shape on the same workspace
    e = L.lsa_select(sc, cfg.K, cfg.S, cfg.W)
    assert torch.equal(a, b) and torch.equal(a, e)
    assert c.shape == (2, 1, 300)


@pytest.mark.parametrize("cid", [2, 5])
def test_attend_128_splits_merge_in_rounds(cid):
    # 4096 selected rows in 128 splits of 32: the merge's split groups take several rounds
    # of loads (MLA rows: 2 groups of 64 splits; 128-wide rows: 16 groups of 8)
    kw = dict(B=2, N=9000, K=4096, S=64, W=512)
    if cid == 5:
        kw["layers"] = 1
    cfg = config(cid, **kw)
    inp = make_inputs(cfg)
    d = upload(inp)
    ora = O.reference_step(inp)
    idx_o = torch.from_numpy(np.stack([[ora["idx"][(b, 0)] for b in range(cfg.B)]]).transpose(1, 0, 2).astype(np.int32)).cuda()
    out, lse = gpu_attend(d, idx_o, n_splits=128)
    o, l = _np(out), _np(lse)
    for b in range(cfg.B):
        check_attn(o[0, b, 0], ora["out"][(0, b, 0)], f"c{cid} 128 splits b={b}")
        assert np.allclose(l[0, b, 0], ora["lse"][(0, b, 0)], atol=2e-3), f"c{cid} lse b={b}"


@pytest.mark.parametrize("cid,Hq,Hkv,K,splits", [
    (2, 16, 1, 512, 0),     # MLA rows, one wave of heads: four waves load, 36 KB stages
    (2, 8, 1, 1024, 1),     # MLA, one long split: the 2-stage ring
    (5, 64, 4, 2048, 1),    # GQA 16 heads per KV head, one 2048-row split: the 2-stage ring
    (5, 8, 4, 2048, 3),     # GQA 2 heads per KV head, 3 splits: the 3-stage ring
    (5, 32, 4, 1024, 0),    # GQA 8 heads per KV head, the default split count
])
def test_attend_one_head_wave_shapes(cid, Hq, Hkv, K, splits):
    # up to 16 query heads per KV head: a workgroup of four waves of which one computes;
    # the ring depth follows the split length
    kw = dict(B=2, N=6000, K=K, S=32, W=128, Hq=Hq, Hkv=Hkv)
    if cid == 5:
        kw["layers"] = 1
    cfg = config(cid, **kw)
    inp = make_inputs(cfg)
    d = upload(inp)
    ora = O.reference_step(inp)
    idx_o = torch.from_numpy(np.stack([[ora["idx"][(b, 0)] for b in range(cfg.B)]]).transpose(1, 0, 2).astype(np.int32)).cuda()
    out, lse = gpu_attend(d, idx_o, n_splits=splits)
    o, l = _np(out), _np(lse)
    for b in range(cfg.B):
        check_attn(o[0, b, 0], ora["out"][(0, b, 0)], f"c{cid} Hq={Hq} Hkv={Hkv} b={b}")
        assert np.allclose(l[0, b, 0], ora["lse"][(0, b, 0)], atol=2e-3), f"lse b={b}"


def test_index_launch_events_time_one_indexer_launch():
    # the measurement hook: the next token-indexer launch records its own start and end;
    # the scores are those of a plain call, and the hook is used up by that one launch
    cfg = config(2, B=2, N=65536)
    d = upload(make_inputs(cfg))
    kw = dict(k_scale=d["kI_scale"], ctx_len=d["ctx_len"])
    sc0 = L.lsa_index(d["qI"], d["w"], d["kI"], **kw)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    L.lsa_index_launch_events(e0, e1)
    sc1 = L.lsa_index(d["qI"], d["w"], d["kI"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(sc1, sc0)
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < 50.0
    L.lsa_index(d["qI"], d["w"], d["kI"], **kw)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == ms


@pytest.mark.parametrize("splits", [0, 1])
def test_attend_launch_events_time_one_call(splits):
    # the attention's measurement hook: the next call's first kernel records the start, its
    # last (the merge, or the attention itself with one split) the end; same output as a
    # plain call, and the hook is used up by that call
    cfg = config(2, B=2, N=8192, K=512, S=32, W=128)
    d = upload(make_inputs(cfg))
    idx = L.lsa_select(L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"]), cfg.K, cfg.S, cfg.W)
    out0, lse0 = L.lsa_attend(d["q"], d["k"], d["v"], idx, cfg.tau, n_splits=splits)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    L.lsa_attend_launch_events(e0, e1)
    out1, lse1 = L.lsa_attend(d["q"], d["k"], d["v"], idx, cfg.tau, n_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out0.view(torch.int16)) and torch.equal(lse1, lse0)
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < 50.0
    L.lsa_attend(d["q"], d["k"], d["v"], idx, cfg.tau, n_splits=splits)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == ms
