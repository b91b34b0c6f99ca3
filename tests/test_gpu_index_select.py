"""lsa_index_select (the indexer priming the selection, then the selection, as one call;
the scores may stay in the workspace) against lsa_index followed by lsa_select on the same
inputs: the index lists must be identical (both decide in fp32 on the same scores), and so
must the scores when they are written. Cases: the 128K decode shape (64 heads, fp8 keys),
32 heads, bf16 keys of 64 dims, several query tokens per sequence, ragged context lengths,
contexts shorter than the budget (everything visible taken), a budget of one, no sink or
window, scores not written, fp8 queries, rows where every score is equal (the whole row
ties), workspace reuse, two calls giving the same bytes, and many query rows. Prefill
shapes (thousands of query tokens) take the candidate-list path, where the indexer lists
each row's candidates that can still reach its fill and the selection ranks only those:
the same comparison there, with ragged, short and sub-T contexts, a query count that is
not a multiple of four, an empty fill, a budget of one, fp8 queries, whole-row ties
(every candidate listed, in LDS and beyond it). Against the oracle: the band rule on a
reduced shape of both paths.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_07_amd as L
from oracle import lsa_oracle as O
from synth import config, make_inputs
from gpu_harness import upload, check_band

pytestmark = pytest.mark.gpu


def _run(cfg, inp, **kw):
    d = upload(inp)
    ks = d["kI_scale"]
    q8 = kw.pop("q_fp8", False)
    ws_ = kw.pop("with_scores", True)
    sc_ref = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=ks, ctx_len=d["ctx_len"], q_fp8=q8)
    idx_ref = L.lsa_select(sc_ref, cfg.K, cfg.S, cfg.W, ctx_len=d["ctx_len"])
    sc, idx = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=ks, ctx_len=d["ctx_len"],
                                 q_fp8=q8, with_scores=ws_, **kw)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref), "idx differs from lsa_index + lsa_select"
    if sc is not None:
        assert torch.equal(sc, sc_ref), "scores differ from lsa_index"
    return d, sc_ref, idx


CASES = {
    "c2_full": (2, {}),
    "h64_fp8_ragged": (2, dict(B=3, N=20000, K=512, S=32, W=128)),
    "h32_fp8": (5, dict(B=4, N=30000, layers=1)),
    "h32_bf16_d64_T4": (2, dict(B=2, T=4, N=9000, H_I=32, D_I=64, k_fp8=False, K=256, S=16, W=64)),
    "h64_bf16_d128": (2, dict(B=2, N=7000, k_fp8=False, K=300, S=8, W=40)),
    "short_ctx": (2, dict(B=4, N=3000, K=2048, S=64, W=512)),
    "k1_sink": (2, dict(B=2, N=5000, K=1, S=1, W=0)),
    "k1_fill": (2, dict(B=2, N=5000, K=1, S=0, W=0)),
    "no_forced": (5, dict(B=2, N=8000, K=700, S=0, W=0, layers=1)),
    "many_rows_unfused": (5, dict(B=300, N=1000, K=100, S=8, W=16, layers=1)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_index_select_matches_separate_calls(name):
    cid, kw = CASES[name]
    cfg = config(cid, **kw)
    inp = make_inputs(cfg, with_kv=False)
    if name in ("h64_fp8_ragged", "short_ctx", "h32_bf16_d64_T4"):
        rng = np.random.default_rng(17)
        inp["ctx_len"] = np.array([cfg.N - int(rng.integers(0, cfg.N // 2)) * (b % 2) for b in range(cfg.B)], np.int32)
        if name == "short_ctx":
            inp["ctx_len"] = np.array([3000, 40, 700, 2049][: cfg.B], np.int32)
    _run(cfg, inp)
    # second call: the workspace left clean, same bytes; then without the scores
    d, sc_ref, idx = _run(cfg, inp)
    sc2, idx2 = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                   ctx_len=d["ctx_len"], with_scores=False)
    torch.cuda.synchronize()
    assert sc2 is None and torch.equal(idx2, idx), "idx without the score write differs"


def test_index_select_fp8_queries():
    cfg = config(2, B=4, N=40000, K=1024, S=32, W=256, q_fp8=True)
    _run(cfg, make_inputs(cfg, with_kv=False), q_fp8=True)


def test_index_select_all_scores_equal_whole_row_ties():
    # w = 0: every score is 0, every candidate sits in one bin and the fill is the
    # lowest candidate positions (ties go to the lower position)
    for N in (12000, 131072):
        cfg = config(2, B=2, N=N, K=2048, S=64, W=512)
        inp = make_inputs(cfg, with_kv=False)
        inp["w"] = np.zeros_like(inp["w"])
        d, sc, idx = _run(cfg, inp)
        g = idx.cpu().numpy()
        for b in range(cfg.B):
            want = O.select_tokens(np.zeros(N), N - 1, cfg.K, cfg.S, cfg.W)
            assert np.array_equal(g[b, 0], want)


def test_index_select_against_oracle_band():
    cfg = config(2, B=2, N=24000, K=1024, S=32, W=256)
    inp = make_inputs(cfg, with_kv=False)
    d = upload(inp)
    _, idx = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                ctx_len=d["ctx_len"], with_scores=False)
    torch.cuda.synchronize()
    ora = O.reference_step(inp, with_attend=False)
    P = O.query_positions(inp["ctx_len"], cfg.T)
    g = idx.cpu().numpy()
    for b in range(cfg.B):
        p = int(P[b, 0])
        F = O.forced_positions(p, cfg.S, cfg.W)
        C = np.setdiff1d(np.arange(p + 1), F)
        check_band(g[b, 0], C, ora["scores"][(b, 0)][C], F, cfg.K, what=f"fused {b}")


# Prefill shapes where the indexer writes each row's candidate list (whole rows, four
# query tokens a workgroup, at least 512 groups of four) and the selection ranks the
# lists instead of the scores; the lists' bounded prefix of each row must give the same
# selection as the full row.
EMIT_CASES = {
    "pre_h64_fp8": (4, dict(T=2048, N=8192)),
    "pre_h32_bf16_d64_ragged": (4, dict(B=4, T=512, N=5000, H_I=32, D_I=64, k_fp8=False, K=256, S=16, W=64)),
    "pre_T_not_multiple_of_4": (4, dict(T=2046, N=6000, K=512, S=16, W=64)),
    "pre_short_ctx": (4, dict(B=2, T=1024, N=3000, K=2048, S=64, W=512)),
    "pre_fill_zero": (4, dict(T=2048, N=6000, K=576, S=64, W=512)),
    "pre_k1_fill": (4, dict(T=2048, N=4000, K=1, S=0, W=0)),
}


@pytest.mark.parametrize("name", list(EMIT_CASES))
def test_index_select_candidate_lists(name):
    cid, kw = EMIT_CASES[name]
    cfg = config(cid, **kw)
    inp = make_inputs(cfg, with_kv=False)
    if name == "pre_h32_bf16_d64_ragged":
        inp["ctx_len"] = np.array([5000, 3100, 4999, 512], np.int32)
    if name == "pre_short_ctx":
        inp["ctx_len"] = np.array([3000, 700], np.int32)  # rows before position 0 see nothing
    print(f"[emit] {name}", flush=True)
    _run(cfg, inp)
    d, sc_ref, idx = _run(cfg, inp)
    sc2, idx2 = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                   ctx_len=d["ctx_len"], with_scores=False)
    torch.cuda.synchronize()
    assert sc2 is None and torch.equal(idx2, idx), "idx without the score write differs"


def test_index_select_candidate_lists_fp8_queries():
    cfg = config(4, T=2048, N=9000, q_fp8=True)
    _run(cfg, make_inputs(cfg, with_kv=False), q_fp8=True)


@pytest.mark.parametrize("N", [9000, 20000])
def test_index_select_candidate_lists_whole_row_ties(N):
    # w = 0: every score is 0, the running threshold never leaves the one bin, so every
    # candidate is listed (at N = 20000 more ties than the selection holds in LDS)
    cfg = config(4, T=2048, N=N)
    inp = make_inputs(cfg, with_kv=False)
    inp["w"] = np.zeros_like(inp["w"])
    d, sc, idx = _run(cfg, inp, with_scores=False)
    g = idx.cpu().numpy()
    P = O.query_positions(inp["ctx_len"], cfg.T)
    for t in (0, 1, 1000, 2047):
        p = int(P[0, t])
        assert np.array_equal(g[0, t], O.select_tokens(np.zeros(p + 1), p, cfg.K, cfg.S, cfg.W)), t


def test_index_select_candidate_lists_against_oracle_band():
    cfg = config(4, T=2048, N=6144)
    inp = make_inputs(cfg, with_kv=False)
    d = upload(inp)
    _, idx = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                ctx_len=d["ctx_len"], with_scores=False)
    torch.cuda.synchronize()
    rows = [(0, t) for t in (0, 1, 2, 3, 777, 2044, 2047)]
    ora = O.reference_step(inp, rows=rows, with_attend=False)
    P = O.query_positions(inp["ctx_len"], cfg.T)
    g = idx.cpu().numpy()
    for b, t in rows:
        p = int(P[b, t])
        F = O.forced_positions(p, cfg.S, cfg.W)
        C = np.setdiff1d(np.arange(p + 1), F)
        check_band(g[b, t], C, ora["scores"][(b, t)][C], F, cfg.K, what=f"lists {b},{t}")
