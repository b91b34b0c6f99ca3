"""SI selection on the GPU (lsa_select through the C ABI) on designed fp32 score rows,
against the oracle's selection of the same fp32 values, and the primed selection
(lsa_index preparing the selection workspace) against the unprimed one.

The designed rows exercise every path of the selection's row pass: the position bitmap
(N <= 2^18) and the sorted list (N > 2^18); rows whose length is not a multiple of 4;
threshold groups ranked directly, by radix passes over the tie list (more than 1024
equal scores), from the workspace copy of the tie list (more ties than the resolve holds
in LDS), and by rescanning the row (more ties than the list holds); -0.0 next to +0.0;
-inf entries (never candidates); fewer candidates than the fill.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_07_amd as L
from oracle import lsa_oracle as O
from synth import config, make_inputs
from gpu_harness import upload

pytestmark = pytest.mark.gpu


def _gpu_select(rows: np.ndarray, K: int, S: int, W: int) -> np.ndarray:
    """rows fp32 [R, N]: one query token per row (T = 1, p = N - 1)."""
    R, N = rows.shape
    sc = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.float32)).cuda().view(R, 1, N)
    return L.lsa_select(sc, K, S, W).cpu().numpy()[:, 0]


def _oracle_select(row32: np.ndarray, K: int, S: int, W: int) -> np.ndarray:
    """Selection of the ABI: candidates are the finite scores at visible positions
    outside the forced set; the oracle's fill rule on the same fp32 values."""
    p = row32.size - 1
    s = row32.astype(np.float64)
    F = O.forced_positions(p, S, W)
    C = np.setdiff1d(np.arange(p + 1), F)
    C = C[np.isfinite(s[C])]
    fill = O.top_fill(C, s[C], K - F.size)
    return O.pad_sorted(np.concatenate([F, fill]), K)


def _check_rows(rows, K, S, W):
    got = _gpu_select(rows, K, S, W)
    for i, row in enumerate(rows):
        want = _oracle_select(row.astype(np.float32), K, S, W)
        assert np.array_equal(got[i], want), f"row {i}: {np.count_nonzero(got[i] != want)} entries differ"


def test_random_rows_bitmap_and_unaligned_lengths():
    rng = np.random.default_rng(11)
    for N in (4096, 5003, 131071):
        rows = rng.standard_normal((3, N)).astype(np.float32)
        _check_rows(rows, 2048, 64, 512)


def test_random_rows_beyond_bitmap():
    rng = np.random.default_rng(12)
    rows = rng.standard_normal((2, 300000)).astype(np.float32)
    _check_rows(rows, 2048, 64, 512)


def test_many_equal_scores_in_threshold_group():
    # 600 clear winners, then 3000 scores exactly 1.0 sharing the threshold group: the
    # position order decides, via radix passes over the LDS tie list
    rng = np.random.default_rng(13)
    N = 20000
    row = (rng.standard_normal(N) * 0.01 - 5.0).astype(np.float32)
    pos = rng.permutation(np.arange(16, N - 64))
    row[pos[:600]] = 10.0 + rng.random(600).astype(np.float32)
    row[pos[600:3600]] = 1.0
    _check_rows(row[None], 2048, 16, 64)


def test_equal_scores_beyond_lds_tie_list():
    # 10000 scores exactly 2.0 (more than the resolve keeps in LDS: ranked from the
    # workspace list) with part of them needed
    rng = np.random.default_rng(14)
    N = 40000
    row = (rng.standard_normal(N) * 0.01 - 5.0).astype(np.float32)
    pos = rng.permutation(np.arange(16, N - 64))
    row[pos[:500]] = 3.0 + rng.random(500).astype(np.float32)
    row[pos[500:10500]] = 2.0
    _check_rows(row[None], 2048, 16, 64)


def test_tie_list_overflow_rescans_row():
    # 2048 rows x 16384 columns: the per-row tie list holds 8192 entries, so a row whose
    # threshold bin holds 10000 equal scores is resolved by rescanning the row
    rng = np.random.default_rng(17)
    R, N = 2048, 16384
    rows = rng.standard_normal((R, N)).astype(np.float32)
    hot = 7
    rows[hot] = (rng.standard_normal(N) * 0.01 - 5.0).astype(np.float32)
    pos = rng.permutation(np.arange(16, N - 64))
    rows[hot, pos[:500]] = 3.0 + rng.random(500).astype(np.float32)
    rows[hot, pos[500:10500]] = 2.0
    got = _gpu_select(rows, 2048, 16, 64)
    for i in (hot, 0, 1234, R - 1):
        want = _oracle_select(rows[i], 2048, 16, 64)
        assert np.array_equal(got[i], want), f"row {i}"


def test_signed_zeros_and_masked_entries():
    rng = np.random.default_rng(15)
    N = 3000
    row = np.where(rng.random(N) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    hot = rng.choice(np.arange(16, N - 64), 100, replace=False)
    row[hot] = rng.random(100).astype(np.float32) + 0.5
    masked = rng.choice(np.arange(16, N - 64), 400, replace=False)
    row[masked] = -np.inf
    _check_rows(row[None], 256, 16, 64)


def test_fewer_candidates_than_fill():
    rng = np.random.default_rng(16)
    N = 5000
    row = np.full(N, -np.inf, dtype=np.float32)
    live = rng.choice(np.arange(16, N - 64), 100, replace=False)
    row[live] = rng.standard_normal(100).astype(np.float32)
    _check_rows(row[None], 512, 16, 64)


# ----------------------------------------------------------------------------- primed

def _primed_vs_plain(cfg, seed_offset=0):
    inp = make_inputs(cfg)
    d = upload(inp)
    sc = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], ctx_len=d["ctx_len"])
    idx = L.lsa_select(sc, cfg.K, cfg.S, cfg.W, ctx_len=d["ctx_len"])
    for _ in range(2):  # the second call reuses the workspace the first one left clean
        sc2, idx2 = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                       ctx_len=d["ctx_len"])
        assert torch.equal(sc2, sc)
        assert torch.equal(idx2, idx)
    return d


@pytest.mark.parametrize("cid,kw", [
    (2, dict(B=2, N=9000, K=512, S=32, W=128)),          # 64 heads fp8: histogram in the indexer epilogue
    (5, dict(B=3, N=5000, K=512, S=32, W=128, layers=1)),  # 32 heads fp8: histogram in the indexer epilogue
    (1, dict(N=3000, K=256, S=16, W=64)),                 # 4 heads, 8 queries per workgroup: histogram pass
    (4, dict(T=64, N=4064, K=256, S=16, W=64)),            # prefill: histogram pass
])
def test_primed_selection_equals_plain(cid, kw):
    _primed_vs_plain(config(cid, **kw))


def test_primed_selection_per_sequence_context_lengths():
    cfg = config(5, B=3, T=2, N=3000, K=256, S=16, W=64, layers=1)
    inp = make_inputs(cfg)
    inp["ctx_len"] = np.array([3000, 1234, 130], dtype=np.int32)
    d = upload(inp)
    sc = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], ctx_len=d["ctx_len"])
    idx = L.lsa_select(sc, cfg.K, cfg.S, cfg.W, ctx_len=d["ctx_len"])
    _, idx2 = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                 ctx_len=d["ctx_len"])
    assert torch.equal(idx2, idx)


def test_primed_hi_fine_selection_equals_plain():
    cfg = config(3, N=19200, K=512, S=64, W=128, n_keep=32)
    inp = make_inputs(cfg)
    d = upload(inp)
    kbar = L.lsa_block_means(d["kI"], cfg.Bs, k_scale=d["kI_scale"])
    cs = L.lsa_index(d["qI"], d["w"], kbar, mode=L.LSA_INDEX_BLOCKS, N=cfg.N, ctx_len=d["ctx_len"],
                     block_size=cfg.Bs, sink=cfg.S, window=cfg.W)
    kept = L.lsa_select(cs, cfg.n_keep, 0, 0, causal=False)
    fs = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], kept=kept, block_size=cfg.Bs,
                     ctx_len=d["ctx_len"])
    idx = L.lsa_select(fs, cfg.K, cfg.S, cfg.W, N=cfg.N, ctx_len=d["ctx_len"], kept=kept, block_size=cfg.Bs)
    fs2, idx2 = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                   ctx_len=d["ctx_len"], kept=kept, block_size=cfg.Bs)
    assert torch.equal(fs2, fs)
    assert torch.equal(idx2, idx)


@pytest.mark.parametrize("B,N,n_keep", [(1, 1048576, 256), (2, 320037, 256), (3, 19200, 32)])
def test_primed_block_selection_equals_plain(B, N, n_keep):
    # the BLOCKS indexer primes the coarse block selection (causal = 0, no forced set):
    # scores and kept lists equal those of the plain calls, from a dirty workspace (cleared
    # first) and from the clean one the selection leaves; 16384 blocks (the 1M cache),
    # 5000 (a partial last workgroup of block scores, ragged contexts) and 300 (the
    # one-launch selection: nothing primed)
    cfg = config(3, B=B, N=N, n_keep=n_keep)
    inp = make_inputs(cfg)
    d = upload(inp)
    kbar = L.lsa_block_means(d["kI"], cfg.Bs, k_scale=d["kI_scale"])
    kw = dict(mode=L.LSA_INDEX_BLOCKS, N=cfg.N, ctx_len=d["ctx_len"], block_size=cfg.Bs, sink=cfg.S, window=cfg.W)
    cs = L.lsa_index(d["qI"], d["w"], kbar, **kw)
    kept = L.lsa_select(cs, cfg.n_keep, 0, 0, causal=False)
    nbytes = L.lsa_select_workspace_bytes(cs, cfg.n_keep, causal=False)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    for state in (L.LSA_WS_UNKNOWN, L.LSA_WS_CLEAN, L.LSA_WS_CLEAN):
        cs2 = L.lsa_index(d["qI"], d["w"], kbar, select_ws=ws, select_ws_state=state, **kw)
        kept2 = L.lsa_select(cs2, cfg.n_keep, 0, 0, causal=False, workspace=ws, workspace_state=L.LSA_WS_PRIMED)
        torch.cuda.synchronize()
        assert torch.equal(cs2, cs)
        assert torch.equal(kept2, kept)


def test_priming_clears_a_dirty_workspace():
    cfg = config(2, B=2, N=9000, K=512, S=32, W=128)
    inp = make_inputs(cfg)
    d = upload(inp)
    sc = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], ctx_len=d["ctx_len"])
    idx = L.lsa_select(sc, cfg.K, cfg.S, cfg.W, ctx_len=d["ctx_len"])
    probe = L.SelectDesc(B=cfg.B, T=cfg.T, N=cfg.N, scores=sc.data_ptr(), n_cols=cfg.N, K=cfg.K, sink=cfg.S,
                         window=cfg.W, causal=1, idx=idx.data_ptr())
    nbytes = L.lib().lsa_select_workspace_bytes(probe)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    idx2 = torch.empty_like(idx)
    sc2 = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], ctx_len=d["ctx_len"], sink=cfg.S,
                      window=cfg.W, select_ws=ws, select_ws_state=L.LSA_WS_UNKNOWN)
    sel = L.SelectDesc(B=cfg.B, T=cfg.T, N=cfg.N, scores=sc2.data_ptr(), n_cols=cfg.N, K=cfg.K, sink=cfg.S,
                       window=cfg.W, causal=1, idx=idx2.data_ptr(), workspace_state=L.LSA_WS_PRIMED)
    rc = L.lib().lsa_select(sel, ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert torch.equal(idx2, idx)
    # the selection leaves its workspace clean: a second priming may say so
    idx3 = torch.empty_like(idx)
    L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], ctx_len=d["ctx_len"], sink=cfg.S, window=cfg.W,
                scores=sc2, select_ws=ws, select_ws_state=L.LSA_WS_CLEAN)
    sel.idx = idx3.data_ptr()
    assert L.lib().lsa_select(sel, ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream) == 0
    assert torch.equal(idx3, idx)
